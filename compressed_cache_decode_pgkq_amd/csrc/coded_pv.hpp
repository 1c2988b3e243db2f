// Online softmax and the weighted sum of PGKQ-coded values (PGKQ-KV: the value
// cache coded by the key encoder without the transform; EdgeLLM-Nano paper
// page, PGKQ-KV paragraphs).
//
// The output sum_t p_t V-hat_t is accumulated in the code domain:
//   * pair part: lane = CPL channels (CPL / 2 pairs) of a token row; each
//     pair's joint code indexes a 2^P-entry LDS table of
//     (level[rc] cos thetahat[ac], level[rc] sin thetahat[ac]) and is weighted
//     by p_t;
//   * QJL part: the same lane owns CPL sketch bits; it accumulates
//     sum_t p_t nu_t bit_tj and sum_t p_t nu_t, giving
//     a_j = sum_t p_t nu_t (2 bit_tj - 1).  The product kappa S^T a, linear in
//     the partial states, is left to the merge kernel (one matrix-vector
//     product per query head instead of one per partition).
// The chunk's code words arrive lane = token (coalesced dword loads) and are
// transposed through a wave-private LDS block.  The wavefronts' states
// (m, l, o[d], a[m]) are merged in the workgroup into one partial per split.
// A lane holds 2 G CPL accumulators: CPL = 8 up to 4 query heads, 4 for 8 heads
// (twice the rows per lane, half the registers).
#pragma once

#include "device_common.hpp"

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

  float m_run[G], l_lane[G], o[G][CPL], acc[G][CPL], spn[G];
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
      for (int k = 0; k < CPL; ++k) {
        o[g][k] = 0.f;
        acc[g][k] = 0.f;
      }
    }
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
  // vw: its LDS_WORDS transposition block; vtab: the pair table; rows at or
  // beyond c_end carry no weight.
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, float* p_rows, uint32_t* vw,
                                        const float2* vtab, int64_t c0, int64_t c_end) {
    float pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid ? s[g] * scale_log2 : -INFINITY;
      const float mnew = fmaxf(m_run[g], wave_max_uniform(z));
      if (mnew > m_run[g]) {  // wave-uniform
        const float alpha = fast_exp2(m_run[g] - mnew);
        l_lane[g] *= alpha;
        spn[g] *= alpha;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          o[g][k] *= alpha;
          acc[g][k] *= alpha;
        }
        m_run[g] = mnew;
      }
      pv[g] = valid ? fast_exp2(z - m_run[g]) : 0.f;
      l_lane[g] += pv[g];
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
    if constexpr (QJLV) vw[NW * VW_STRIDE + lane] = vc.nu;
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
      if constexpr (QJLV) {
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
    wave_lds_sync();
  }

  // Sum the lane groups of the wavefront (every group scanned other rows).
  __device__ __forceinline__ void reduce_slots() {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        spn[g] += __shfl_xor(spn[g], off, kWave);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          o[g][k] += __shfl_xor(o[g][k], off, kWave);
          acc[g][k] += __shfl_xor(acc[g][k], off, kWave);
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
    float l_w[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l_w[g] = wave_sum(l_lane[g]);
    float* wm = scratch;                  // [WAVES][G]
    float* wl = scratch + WAVES * G;      // [WAVES][G]
    float* wo = scratch + 2 * WAVES * G;  // [WAVES][G][2D]: o, then a
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
          wo[(wave * G + g) * 2 * D + dblk * CPL + k] = o[g][k];
          wo[(wave * G + g) * 2 * D + D + dblk * CPL + k] = QJLV ? 2.f * acc[g][k] - spn[g] : 0.f;
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
