// Online softmax and the fp16-V weighted sum on the matrix cores.
//
// The weighted sum o[g][c] = sum_t p[g][t] V[t][c] of a 64-token chunk is a
// small matrix product (G query heads x 64 tokens x d channels).  It runs as
// v_mfma_f32_16x16x32_f16: A = the chunk's weights (rows = query heads,
// K = 32 tokens, fp16), B = the value rows (K = 32 tokens, N = 16 channels),
// fp32 accumulators.  Rows of A past G repeat real heads; their output rows are
// never read.
//
// The value cache is stored in the operand order of B ("32-token tiles"): a
// tile of 32 tokens x d channels is d/16 blocks of 1 KiB, block n holding
// channels 16n .. 16n+15, and inside a block lane l (0..63) owns 16 bytes: the
// 8 tokens 8(l/16) .. 8(l/16)+7 of channel 16n + l%16.  Element (t, c) of a
// stream is therefore at half-word
//   (t/32) * 32 d + ((c/16) * 4 + (t%32)/8) * 128 + (c%16) * 8 + t%8,
// one coalesced 1 KiB wave load per MFMA operand and no transposition.
//
// Weights keep fp32 accuracy on the fp16 matrix cores: each weight p (in
// [0, 1], the running maximum scores 1) is scaled by 2^15 (exact) and split
// into two fp16 parts, hi = fp16(p 2^15) and lo = fp16(p 2^15 - hi), both
// multiplied with the same value operand (two MFMAs).  hi + lo carries p to
// about 2^-22 relative (absolute 2^-40 where lo is subnormal), close to the
// fp32 weight; products are exact in fp32 and accumulate in fp32.  The
// denominator sums the scaled weights in fp32, so o / l is unchanged by the
// scale.
#pragma once

#include "device_common.hpp"

namespace pgkq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Half-word offset of element (t, c) in a stream of 32-token tiles of width d.
__host__ __device__ constexpr int64_t vtile_index(int64_t t, int c, int d) {
  return (t >> 5) * 32 * d + ((int64_t(c >> 4) * 4 + ((t >> 3) & 3)) * 128) + (c & 15) * 8 + (t & 7);
}

template <int D, int G, int WAVES>
struct MfmaPV {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "query heads per kv-head");
  static_assert(D % 16 == 0, "head dim");
  static constexpr int NT = D / 16;     // 16-channel blocks
  static constexpr int KS = kWave / 32;  // 32-token steps per chunk
  static constexpr int TILE_BYTES = 32 * D * 2;
  static constexpr int MERGE_FLOATS = WAVES * G * (D + 2);
  // LDS bytes of one wavefront's weight rows ([hi, lo][G][64] fp16)
  static constexpr int P_BYTES = 2 * G * kWave * 2;
  static constexpr float kPScale = 32768.f;  // 2^15: keeps hi in the normal fp16 range

  f32x4 acc[NT];
  float m_run[G], l_lane[G];
  int lane, wave;

  __device__ __forceinline__ void init(int tid) {
    lane = tid & 63;
    wave = tid >> 6;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  struct VChunk {
    u32x4 r[KS][NT];
  };

  // The B operands of the chunk at token c0 (a multiple of 32).  `vr` spans the
  // tiles [0, ceil(t_end / 32)) of the stream, so whole tiles past the split
  // read as zeros; inside the last tile, tokens at or beyond t_end may hold any
  // bits and are cleared here (their weight is zero, but 0 x NaN is NaN).
  __device__ __forceinline__ void load_v(VChunk& vc, int64_t c0, __amdgpu_buffer_rsrc_t vr,
                                         int64_t t_end) const {
    const uint32_t base = static_cast<uint32_t>(c0 >> 5) * TILE_BYTES + lane * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int n = 0; n < NT; ++n) vc.r[ks][n] = buf_load_b128(vr, base + ks * TILE_BYTES + n * 1024);
  }

  // Zero the value slots at or past t_end in a chunk that holds a ragged tile
  // (they hold whatever the cache's spare slots hold).  Kept apart from the
  // loads and called just before the chunk is used, so that issuing the loads
  // never waits for them.
  __device__ __forceinline__ void mask_v(VChunk& vc, int64_t c0, int64_t t_end) const {
    if (c0 + kWave > t_end && (t_end & 31) != 0) {  // wave-uniform: the chunk holds a ragged tile
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int64_t t8 = c0 + 32 * ks + 8 * (lane >> 4);  // first token of this lane's 8
        const int64_t live = t_end - t8;                   // tokens of the 8 that exist
        u32x4 keep;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          keep[j] = (live > 2 * j ? 0xFFFFu : 0u) | (live > 2 * j + 1 ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int n = 0; n < NT; ++n) vc.r[ks][n] &= keep;
      }
    }
  }

  // s: raw scores of token c0 + prow (ignored when !valid), prow a permutation
  // of the lanes (the lane index when scores arrive lane = token); p_lds: this
  // wavefront's P_BYTES of LDS.
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, void* p_lds) {
    chunk(s, valid, scale_log2, vc, p_lds, lane);
  }
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, void* p_lds, int prow) {
    _Float16* p16 = static_cast<_Float16*>(p_lds);
    float alpha[G];
    bool grew = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid ? s[g] * scale_log2 : -INFINITY;
      const float mnew = fmaxf(m_run[g], wave_max_uniform(z));
      alpha[g] = 1.f;
      if (mnew > m_run[g]) {  // wave-uniform
        alpha[g] = fast_exp2(m_run[g] - mnew);  // m_run = -inf gives 0
        l_lane[g] *= alpha[g];
        m_run[g] = mnew;
        grew = true;
      }
      const float ps = valid ? fast_exp2(z - m_run[g]) * kPScale : 0.f;
      const _Float16 hi = static_cast<_Float16>(ps);
      const _Float16 lo = static_cast<_Float16>(ps - static_cast<float>(hi));
      l_lane[g] += ps;
      p16[g * kWave + prow] = hi;
      p16[(G + g) * kWave + prow] = lo;
    }
    if (grew) {  // wave-uniform: rescale the accumulator rows of the heads whose maximum grew
      // lane l holds rows 4(l/16) + r of every block
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (G <= 4) {
          f[r] = r < G ? alpha[r] : 1.f;
        } else {
          f[r] = (lane >> 4) == 0 ? alpha[r] : ((lane >> 4) == 1 ? alpha[4 + r] : 1.f);
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[n][r] *= f[r];
    }
    wave_lds_sync();
    const int arow = (lane & 15) & (G - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = arow * kWave + 32 * ks + 8 * (lane >> 4);
      const f16x8 a_hi = *reinterpret_cast<const f16x8*>(p16 + k0);
      const f16x8 a_lo = *reinterpret_cast<const f16x8*>(p16 + G * kWave + k0);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const f16x8 b = __builtin_bit_cast(f16x8, vc.r[ks][n]);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b, acc[n], 0, 0, 0);
      }
    }
    wave_lds_sync();
  }

  // Lane l holds, for head g = 4(l/16) + r, channels 16n + l%16 of o in acc[n][r].
  __device__ __forceinline__ bool owns(int g) const { return (lane >> 4) == (g >> 2); }

  // Merge the wavefronts of the workgroup through `scratch` (MERGE_FLOATS
  // floats of LDS, free to reuse: the caller synchronizes before) and write
  // the final output rows (n_splits == 1) or partial `split` of each query head
  // row0 .. row0 + G - 1.
  __device__ __forceinline__ void finish(float* scratch, int tid, int n_splits, int split,
                                         float* __restrict__ out, float* __restrict__ partial,
                                         size_t row0) {
    float l_w[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l_w[g] = wave_sum(l_lane[g]);
    float* wm = scratch;                  // [WAVES][G]
    float* wl = scratch + WAVES * G;      // [WAVES][G]
    float* wo = scratch + 2 * WAVES * G;  // [WAVES][G][D]
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (owns(g)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) wo[(wave * G + g) * D + 16 * n + (lane & 15)] = acc[n][g & 3];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        wm[wave * G + g] = m_run[g];
        wl[wave * G + g] = l_w[g];
      }
    }
    __syncthreads();
    for (int e = tid; e < G * D; e += WAVES * kWave) {
      const int g = e / D, dd = e % D;
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) Mx = fmaxf(Mx, wm[w * G + g]);
      float num = 0.f, den = 0.f;
      if (Mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
          const float f = exp2f(wm[w * G + g] - Mx);
          num += f * wo[(w * G + g) * D + dd];
          den += f * wl[w * G + g];
        }
      }
      const size_t row = row0 + g;
      if (n_splits == 1) {
        out[row * D + dd] = den > 0.f ? num / den : 0.f;
      } else {
        float* part = partial + (row * n_splits + split) * (D + 4);
        part[4 + dd] = num;
        if (dd == 0) {
          part[0] = Mx;
          part[1] = den;
        }
      }
    }
  }
};

}  // namespace pgkq
