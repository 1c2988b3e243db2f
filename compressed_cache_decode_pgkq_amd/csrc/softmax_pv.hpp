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

  // s: raw scores of token c0 + lane (ignored when !valid); p_row: this
  // wavefront's [64][G] LDS rows; vbase: V of the stream.
  __device__ __forceinline__ void chunk(const float (&s)[G], bool valid, float scale_log2,
                                        int64_t c0, int64_t t_end, const __half* __restrict__ vbase,
                                        float* p_rows) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float z = valid ? s[g] * scale_log2 : -INFINITY;
      const float cmax = wave_max(z);
      const float mnew = fmaxf(m_run[g], cmax);
      const float alpha = exp2f(m_run[g] - mnew);  // m_run = -inf gives 0
      const float p = valid ? exp2f(z - mnew) : 0.f;
      l_lane[g] = l_lane[g] * alpha + p;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[g][k] *= alpha;
      m_run[g] = mnew;
      p_rows[lane * G + g] = p;
    }
    wave_lds_sync();
#pragma unroll 4
    for (int it = 0; it < kWave / TPI; ++it) {
      const int r = it * TPI + slot;
      const int64_t tt = c0 + r;
      if (tt < t_end) {
        const uint4 raw = *reinterpret_cast<const uint4*>(vbase + size_t(tt) * D + dblk * 8);
        const __half2* hv = reinterpret_cast<const __half2*>(&raw);
        float vf[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 f2 = __half22float2(hv[k]);
          vf[2 * k] = f2.x;
          vf[2 * k + 1] = f2.y;
        }
        float pp[G];
        lds_fetch<G>(p_rows + r * G, pp);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int k = 0; k < 8; ++k) o[g][k] = fmaf(pp[g], vf[k], o[g][k]);
      }
    }
    wave_lds_sync();
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
