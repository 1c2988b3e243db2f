// Online softmax and fp16-V weighted sum shared by the decode scans.
//
// A wavefront owns chunks of 64 tokens.  Scores arrive lane = token; the chunk
// maximum is a wave reduction, the weights go through a wave-private LDS row,
// and the P.V accumulation runs lane = 8 channels of one token row (16-byte V
// loads).  At the end the wavefronts of the workgroup are merged in LDS and the
// state is written either as the final normalized output or as a split partial
// (m, l, o) in the log2 domain for the log-sum-exp merge.
#pragma once

#include "device_common.hpp"

namespace pgkq {

template <int G>
__device__ __forceinline__ void lds_fetch(const float* p, float (&v)[G]) {
  if constexpr (G == 1) {
    v[0] = p[0];
  } else if constexpr (G == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
#pragma unroll
    for (int k = 0; k < G; k += 4) {
      const float4 t = *reinterpret_cast<const float4*>(p + k);
      v[k] = t.x;
      v[k + 1] = t.y;
      v[k + 2] = t.z;
      v[k + 3] = t.w;
    }
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int G, int WAVES>
struct SoftmaxPV {
  static constexpr int LPT = D / 8;        // lanes per V row
  static constexpr int TPI = kWave / LPT;  // V rows per wavefront load
  static constexpr int MERGE_FLOATS = WAVES * G * (D + 2);

  float m_run[G], l_lane[G], o[G][8];
  int lane, wave, slot, dblk;

  __device__ __forceinline__ void init(int tid) {
    lane = tid & 63;
    wave = tid >> 6;
    slot = lane / LPT;
    dblk = lane % LPT;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[g][k] = 0.f;
    }
  }

  // V rows of one chunk held in registers: row it*TPI + slot, channels
  // dblk*8 .. dblk*8+7.  `vr` covers the split's rows [0, t_end) of the stream
  // (buffer range), so rows past the split end read as zeros; their weight is
  // zero as well.
  struct VChunk {
    u32x4 r[kWave / TPI];
  };

  __device__ __forceinline__ void load_v(VChunk& vc, int64_t c0, __amdgpu_buffer_rsrc_t vr) const {
    const uint32_t base = static_cast<uint32_t>(c0 + slot) * (D * 2) + dblk * 16;
#pragma unroll
    for (int it = 0; it < kWave / TPI; ++it) vc.r[it] = buf_load_b128(vr, base + it * TPI * D * 2);
  }

  // s: raw scores of token c0 + prow (ignored when !valid); p_rows: this
  // wavefront's [64][G] LDS rows.  prow is a permutation of the lanes (the
  // lane index when scores arrive lane = token).
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, float* p_rows) {
    chunk(s, valid, scale_log2, vc, p_rows, lane);
  }
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        const VChunk& vc, float* p_rows, int prow) {
    float pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid ? s[g] * scale_log2 : -INFINITY;
      const float mnew = fmaxf(m_run[g], wave_max_uniform(z));
      if (mnew > m_run[g]) {  // wave-uniform: rescale only when the maximum grows
        const float alpha = fast_exp2(m_run[g] - mnew);  // m_run = -inf gives 0
        l_lane[g] *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[g][k] *= alpha;
        m_run[g] = mnew;
      }
      pv[g] = valid ? fast_exp2(z - m_run[g]) : 0.f;
      l_lane[g] += pv[g];
    }
    if constexpr (G == 1) {
      p_rows[prow] = pv[0];
    } else if constexpr (G == 2) {
      *reinterpret_cast<float2*>(p_rows + prow * 2) = make_float2(pv[0], pv[1]);
    } else {
#pragma unroll
      for (int g = 0; g < G; g += 4)
        *reinterpret_cast<float4*>(p_rows + prow * G + g) = make_float4(pv[g], pv[g + 1], pv[g + 2], pv[g + 3]);
    }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < kWave / TPI; ++it) {
      if ((it & 3) == 0) sched_fence();  // at most 4 weight rows read ahead
      const int r = it * TPI + slot;
      __half2 hv[4];
      __builtin_memcpy(hv, &vc.r[it], sizeof(hv));
      float pp[G];
      lds_fetch<G>(p_rows + r * G, pp);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 f2 = __half22float2(hv[k]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          o[g][2 * k] = fmaf(pp[g], f2.x, o[g][2 * k]);
          o[g][2 * k + 1] = fmaf(pp[g], f2.y, o[g][2 * k + 1]);
        }
      }
    }
    wave_lds_sync();
  }

  // Write this wavefront's own state as partial `pidx` of `n_parts` for the
  // query heads row0 .. row0 + G - 1 (no LDS, no barrier): used when every
  // wavefront scans a partition of its own.
  __device__ __forceinline__ void finish_wave(float* __restrict__ partial, size_t row0, int pidx,
                                              int n_parts) {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[g][k] += __shfl_xor(o[g][k], off, kWave);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float l_w = wave_sum(l_lane[g]);
      float* part = partial + ((row0 + g) * n_parts + pidx) * (D + 4);
      if (lane < LPT) {
        *reinterpret_cast<float4*>(part + 4 + dblk * 8) = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
        *reinterpret_cast<float4*>(part + 8 + dblk * 8) = make_float4(o[g][4], o[g][5], o[g][6], o[g][7]);
      }
      if (lane == 0) {
        part[0] = m_run[g];
        part[1] = l_w;
      }
    }
  }

  // Merge the wavefronts through `scratch` (MERGE_FLOATS floats of LDS, free to
  // reuse: the caller synchronizes before) and write the state of query heads
  // hq0 .. hq0 + G - 1.  out: [.., D] rows at out_row(g); partial rows likewise.
  __device__ __forceinline__ void finish(float* scratch, int tid, int n_splits, int split,
                                         float* __restrict__ out, float* __restrict__ partial,
                                         size_t row0) {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) o[g][k] += __shfl_xor(o[g][k], off, kWave);
    }
    float l_w[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l_w[g] = wave_sum(l_lane[g]);
    float* wm = scratch;                      // [WAVES][G]
    float* wl = scratch + WAVES * G;          // [WAVES][G]
    float* wo = scratch + 2 * WAVES * G;      // [WAVES][G][D]
    if (lane < LPT) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < 8; ++k) wo[(wave * G + g) * D + dblk * 8 + k] = o[g][k];
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
      const size_t row = row0 + g;  // (sequence, query head) row
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
