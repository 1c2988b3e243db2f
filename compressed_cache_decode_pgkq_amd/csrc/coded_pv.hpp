// Online softmax and the weighted sum of PGKQ-coded values (PGKQ-KV: the value
// cache coded by the key encoder without the transform; EdgeLLM-Nano paper
// page, PGKQ-KV paragraphs).
//
// The output sum_t p_t V-hat_t is accumulated in the code domain:
//   * pair part: lane = CPL channels (CPL / 2 pairs) of a token row; each
//     pair's joint code indexes a 2^P-entry LDS table of
//     (level[rc] cos thetahat[ac], level[rc] sin thetahat[ac]) and is weighted
//     by p_t;
//   * QJL part: a_j = sum_t p_t nu_t (2 bit_tj - 1) = 2 c_j - s with
//     c_j = sum_t p_t (bit_tj nu_t) and s = sum_t p_t nu_t.  c is a small
//     matrix product (G heads x 64 tokens x m sketch columns) and runs on the
//     matrix cores as v_mfma_f32_16x16x32_f16: A = the weights p split into
//     fp16 high and low parts (scaled by 2^15, as for fp16 values), B = the
//     fp16 norm nu_t where bit_tj is set and 0 elsewhere (exact: nu is stored
//     as fp16), fp32 accumulators; s is summed per token lane.  The product
//     kappa S^T a, linear in the partial states, is left to the merge kernel
//     (one matrix-vector product per query head instead of one per
//     partition).
// The chunk's code words arrive lane = token (coalesced dword loads) and are
// transposed through a wave-private LDS block.  The wavefronts' states
// (m, l, o[d], a[m]) are merged in the workgroup into one partial per split.
// A lane holds G CPL pair accumulators: CPL = 8 up to 4 query heads, 4 for 8
// heads (twice the rows per lane, half the registers).  With 8 heads the
// sketch sums stay on the vector ALU (lane = CPL sketch bits of a row: a_j
// accumulated directly): the matrix-core operands would push the registers and
// LDS of the workgroup past the limits of two workgroups per compute unit.
#pragma once

#include "mfma_pv.hpp"

namespace pgkq {

template <int D, int G, int WAVES, int BMV, bool QJLV>
struct CodedPV {
  static constexpr int N = D / 2;
  static constexpr int P = 2 * BMV - 1;        // b_main + b_angle of the values
  static constexpr int NCODES = 1 << P;
  static constexpr int M = QJLV ? D : 0;
  static constexpr int NC = N * P / 32;        // code words per token
  static constexpr int NW = NC + M / 32;       // words per token
  static constexpr int NROW = NW + (QJLV ? 1 : 0);  // LDS rows per chunk: words, norms
  static constexpr int CPL = G >= 8 ? 4 : 8;    // channels per lane
  static constexpr int PPL = CPL / 2;           // pairs per lane
  static constexpr int LPT = D / CPL;           // lanes per token row
  static constexpr bool SKM = QJLV && G <= 4;    // sketch sums on the matrix cores
  static constexpr bool SKV = QJLV && !SKM;      // sketch sums on the vector ALU
  static constexpr int NSWV = M / 32;           // sketch words per token
  static constexpr int NB = SKM ? M / 16 : 1;   // 16-column blocks of the sketch
  static constexpr int KS = kWave / 32;         // 32-token steps per chunk
  static constexpr float kPScale = 32768.f;     // 2^15: keeps hi in the normal fp16 range
  // LDS bytes of one wavefront's sketch weight rows ([hi, lo][G][64] fp16)
  static constexpr int P16_BYTES = SKM ? 2 * G * kWave * 2 : 16;
  static constexpr int TPI = kWave / LPT;      // rows per pass
  static constexpr int NIT = kWave / TPI;      // passes per chunk
  static constexpr int WIDTH = 2 * D + 4;      // partial row: m, l, -, -, o[D], a[D]
  // transposition block rows are padded by one word: the lanes of a token row
  // read different words of the same token, which would otherwise all fall in
  // one LDS bank
  static constexpr int VW_STRIDE = kWave + 1;
  static constexpr int LDS_WORDS = NROW * VW_STRIDE;
  static_assert(PPL * P <= 32, "a lane's pair codes span at most two words");
  static_assert(LPT <= kWave, "lanes per token row");

  float m_run[G], l_lane[G], o[G][CPL], spn[G];
  f32x4 sacc[NB];                            // c, C layout of the matrix product (scaled by 2^15)
  float acc[SKV ? G : 1][SKV ? CPL : 1];     // sum_t p_t nu_t bit_tj of this lane's bits
  int lane, wave, slot, dblk;
  uint32_t row_bytes, nu_off;

  struct VChunk {
    uint32_t w[NW];
    uint32_t nu;
  };

  __device__ __forceinline__ void init(int tid, int64_t capacity) {
    lane = tid & 63;
    wave = tid >> 6;
    slot = lane / LPT;
    dblk = lane % LPT;
    row_bytes = 4u * static_cast<uint32_t>(capacity);
    nu_off = NW * row_bytes;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
      spn[g] = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[g][k] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) sacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < (SKV ? G : 1); ++g)
#pragma unroll
      for (int k = 0; k < (SKV ? CPL : 1); ++k) acc[g][k] = 0.f;
  }

  // code words of token c0 + lane (the whole stream is the buffer range;
  // tokens past the split are masked when accumulated)
  __device__ __forceinline__ void load_v(VChunk& vc, int64_t c0, __amdgpu_buffer_rsrc_t vr) const {
    const uint32_t t4 = static_cast<uint32_t>(c0 + lane) * 4u;
#pragma unroll
    for (int w = 0; w < NW; ++w) vc.w[w] = buf_load_b32(vr, t4 + w * row_bytes);
    if constexpr (QJLV) vc.nu = buf_load_b16(vr, nu_off + t4 / 2);
  }

  // s: raw scores of token c0 + lane; p_rows: the wavefront's [64][G] weights;
  // vw: its LDS_WORDS transposition block; vtab: the pair table; p16: its
  // P16_BYTES of sketch weight rows; rows at or beyond c_end carry no weight
  // (their slots may hold any bits).
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, float* p_rows, uint32_t* vw,
                                        const float2* vtab, int64_t c0, int64_t c_end, void* p16v) {
    float pv[G], alpha[G];
    bool grew = false;
    const float nu_t = QJLV ? half_bits_to_float(static_cast<uint16_t>(vc.nu)) : 0.f;
    _Float16* p16 = static_cast<_Float16*>(p16v);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid ? s[g] * scale_log2 : -INFINITY;
      const float mnew = fmaxf(m_run[g], wave_max_uniform(z));
      alpha[g] = 1.f;
      if (mnew > m_run[g]) {  // wave-uniform
        alpha[g] = fast_exp2(m_run[g] - mnew);
        l_lane[g] *= alpha[g];
        spn[g] *= alpha[g];
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[g][k] *= alpha[g];
        if constexpr (SKV) {
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[g][k] *= alpha[g];
        }
        m_run[g] = mnew;
        grew = true;
      }
      pv[g] = valid ? fast_exp2(z - m_run[g]) : 0.f;
      l_lane[g] += pv[g];
      if constexpr (SKM) {
        if (valid) spn[g] = fmaf(pv[g], nu_t, spn[g]);
        const float ps = pv[g] * kPScale;
        const _Float16 hi = static_cast<_Float16>(ps);
        const _Float16 lo = static_cast<_Float16>(ps - static_cast<float>(hi));
        p16[g * kWave + lane] = hi;
        p16[(G + g) * kWave + lane] = lo;
      }
    }
    if constexpr (SKM) {
      if (grew) {  // wave-uniform: rescale the sketch rows of the heads whose maximum grew
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
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[n][r] *= f[r];
      }
    }
    if constexpr (G == 1) {
      p_rows[lane] = pv[0];
    } else if constexpr (G == 2) {
      *reinterpret_cast<float2*>(p_rows + lane * 2) = make_float2(pv[0], pv[1]);
    } else {
#pragma unroll
      for (int g = 0; g < G; g += 4)
        *reinterpret_cast<float4*>(p_rows + lane * G + g) = make_float4(pv[g], pv[g + 1], pv[g + 2], pv[g + 3]);
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) vw[w * VW_STRIDE + lane] = vc.w[w];
    if constexpr (SKM) vw[NW * VW_STRIDE + lane] = (c0 + lane < c_end) ? (vc.nu & 0xFFFFu) : 0u;
    if constexpr (SKV) vw[NW * VW_STRIDE + lane] = vc.nu;
    wave_lds_sync();

    const int o0 = PPL * P * dblk;  // first polar bit of this lane's pairs
    const int w0 = o0 >> 5, sh = o0 & 31;
    const int w1 = w0 + 1 < NROW ? w0 + 1 : NROW - 1;
    constexpr uint32_t mask = (1u << P) - 1u;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if ((it & 3) == 0) sched_fence();
      const int r = it * TPI + slot;
      float pp[G];
      lds_fetch<G>(p_rows + r * G, pp);
      const uint64_t bits = uint64_t(vw[w0 * VW_STRIDE + r]) | (uint64_t(vw[w1 * VW_STRIDE + r]) << 32);
#pragma unroll
      for (int j = 0; j < PPL; ++j) {
        const uint32_t code = static_cast<uint32_t>(bits >> (sh + P * j)) & mask;
        const float2 t = vtab[code];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          o[g][2 * j] = fmaf(pp[g], t.x, o[g][2 * j]);
          o[g][2 * j + 1] = fmaf(pp[g], t.y, o[g][2 * j + 1]);
        }
      }
      if constexpr (SKV) {
        constexpr uint32_t smask = (1u << CPL) - 1u;
        const uint32_t sb =
            (vw[(NC + (CPL * dblk) / 32) * VW_STRIDE + r] >> ((CPL * dblk) & 31)) & smask;
        const float nu = half_bits_to_float(static_cast<uint16_t>(vw[NW * VW_STRIDE + r]));
        const bool live = c0 + r < c_end;  // a slot past the cache may hold any bits
        float fb[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) fb[k] = static_cast<float>((sb >> k) & 1u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pn = live ? pp[g] * nu : 0.f;
          spn[g] += pn;
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[g][k] = fmaf(fb[k], pn, acc[g][k]);
        }
      }
    }
    if constexpr (SKM) {
      // c += P (bit * nu): lane l supplies A[head l % 16][tokens 8 (l / 16) ..]
      // and B[tokens 8 (l / 16) + j][sketch column 16 n + l % 16]; a token
      // past c_end has nu = 0 in the block, so its bits do not matter
      const int arow = (lane & 15) & (G - 1);
      const int bit = lane & 15;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r0 = 32 * ks + 8 * (lane >> 4);
        const f16x8 a_hi = *reinterpret_cast<const f16x8*>(p16 + arow * kWave + r0);
        const f16x8 a_lo = *reinterpret_cast<const f16x8*>(p16 + (G + arow) * kWave + r0);
        // nu of tokens (2q, 2q + 1) as one fp16 pair, then per column block a
        // 0 / -1 mask from each token's bit (sign-extending 1-bit extract)
        uint32_t nu2[4], sw[8][NSWV];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          nu2[q] = vw[NW * VW_STRIDE + r0 + 2 * q] | (vw[NW * VW_STRIDE + r0 + 2 * q + 1] << 16);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int w = 0; w < NSWV; ++w) sw[j][w] = vw[(NC + w) * VW_STRIDE + r0 + j];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int w = n >> 1, sft = 16 * (n & 1) + bit;
          u32x4 bq;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t m0 = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(sw[2 * q][w]), sft, 1));
            const uint32_t m1 = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(sw[2 * q + 1][w]), sft, 1));
            bq[q] = ((m0 & 0xFFFFu) | (m1 & 0xFFFF0000u)) & nu2[q];
          }
          const f16x8 b = __builtin_bit_cast(f16x8, bq);
          sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b, sacc[n], 0, 0, 0);
          sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b, sacc[n], 0, 0, 0);
        }
      }
    }
    wave_lds_sync();
  }

  // Sum the lane groups of the wavefront (every group scanned other rows).
  __device__ __forceinline__ void reduce_slots() {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[g][k] += __shfl_xor(o[g][k], off, kWave);
        if constexpr (SKV) {
          spn[g] += __shfl_xor(spn[g], off, kWave);
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[g][k] += __shfl_xor(acc[g][k], off, kWave);
        }
      }
    }
  }

  static constexpr int MERGE_FLOATS = WAVES * G * (2 * D + 2);

  // The wavefronts of the workgroup merged through `scratch` (MERGE_FLOATS
  // floats of LDS, free to reuse: the caller synchronizes before), written as
  // partial `split` of `n_parts`.
  __device__ __forceinline__ void finish(float* scratch, int tid, float* __restrict__ partial,
                                         size_t row0, int split, int n_parts) {
    reduce_slots();
    float l_w[G], s_w[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l_w[g] = wave_sum(l_lane[g]);
      s_w[g] = SKM ? wave_sum(spn[g]) : 0.f;  // (with SKV every lane group holds the wave's sum)
    }
    float* wm = scratch;                  // [WAVES][G]
    float* wl = scratch + WAVES * G;      // [WAVES][G]
    float* wo = scratch + 2 * WAVES * G;  // [WAVES][G][2D]: o, then a
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          wo[(wave * G + g) * 2 * D + dblk * CPL + k] = o[g][k];
          if constexpr (!SKM)
            wo[(wave * G + g) * 2 * D + D + dblk * CPL + k] = SKV ? 2.f * acc[g][k] - spn[g] : 0.f;
        }
    }
    if constexpr (SKM) {
      // a = 2 c - s; lane l holds c of head 4 (l / 16) + r, column 16 n + l % 16
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if ((lane >> 4) == (g >> 2)) {
#pragma unroll
          for (int n = 0; n < NB; ++n)
            wo[(wave * G + g) * 2 * D + D + 16 * n + (lane & 15)] =
                2.f * (sacc[n][g & 3] * (1.f / kPScale)) - s_w[g];
        }
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
    for (int e = tid; e < G * 2 * D; e += WAVES * kWave) {
      const int g = e / (2 * D), dd = e % (2 * D);
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) Mx = fmaxf(Mx, wm[w * G + g]);
      float num = 0.f, den = 0.f;
      if (Mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
          const float f = exp2f(wm[w * G + g] - Mx);
          num += f * wo[(w * G + g) * 2 * D + dd];
          den += f * wl[w * G + g];
        }
      }
      float* part = partial + ((row0 + g) * n_parts + split) * WIDTH;
      part[4 + dd] = num;
      if (dd == 0) {
        part[0] = Mx;
        part[1] = den;
      }
    }
  }
};

}  // namespace pgkq
