// FP16-cache decode attention for gfx950: the uncompressed comparator the
// EdgeLLM-Nano page measures fidelity against (its "FP16 wrapper" cache).
//
// Same split/online-softmax skeleton as the PGKQ scan: per (sequence, kv-head,
// token split) workgroup, lane = token for the scores (fp32 dot products of the
// fp16 key row with the G query heads held in LDS), then the shared softmax and
// P.V tail.  The query scale is applied as a log2-domain softmax scale.
#include "softmax_pv.hpp"

namespace pgkq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int D, int G>
__global__ void __launch_bounds__(kThreads)
fp16_scan_kernel(Fp16DecodeArgs a, const __half* __restrict__ K, const __half* __restrict__ V) {
  constexpr int MERGE_FLOATS = SoftmaxPV<D, G, kWaves>::MERGE_FLOATS;
  constexpr int QF = G * D;
  constexpr int MAIN = QF > MERGE_FLOATS ? QF : MERGE_FLOATS;
  __shared__ __align__(16) float s_main[MAIN];  // queries, then the merge
  __shared__ __align__(16) float s_p[kWaves][kWave][G];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  // s_main[c * G + g] = q of head h*G + g, channel c
  for (int e = tid; e < QF; e += kThreads) {
    const int g = e % G, c = e / G;
    s_main[e] = load_f(a.q, a.q_dtype, (size_t(b) * a.n_q + size_t(h) * G + g) * D + c);
  }
  __syncthreads();

  const int64_t t_begin = int64_t(split) * a.tokens_per_split;
  const int64_t t_end = min<int64_t>(t_begin + a.tokens_per_split, a.n_tokens);
  const int64_t stream = b * a.n_kv + h;
  const __half* kbase = K + size_t(stream) * a.capacity * D;
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(V + size_t(stream) * a.capacity * D, static_cast<uint32_t>(t_end * D * 2));

  SoftmaxPV<D, G, kWaves> sm;
  sm.init(tid);
  for (int64_t c0 = t_begin + int64_t(sm.wave) * kWave; c0 < t_end; c0 += kThreads) {
    const int64_t t = c0 + sm.lane;
    const bool valid = t < t_end;
    typename SoftmaxPV<D, G, kWaves>::VChunk vc;
    sm.load_v(vc, c0, vrs);
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
    if (valid) {
      const uint4* krow = reinterpret_cast<const uint4*>(kbase + size_t(t) * D);
#pragma unroll 4
      for (int c8 = 0; c8 < D / 8; ++c8) {
        const uint4 raw = krow[c8];
        const __half2* hk = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 f2 = __half22float2(hk[k]);
          float q0[G], q1[G];
          lds_fetch<G>(&s_main[(c8 * 8 + 2 * k) * G], q0);
          lds_fetch<G>(&s_main[(c8 * 8 + 2 * k + 1) * G], q1);
#pragma unroll
          for (int g = 0; g < G; ++g) s[g] = fmaf(f2.y, q1[g], fmaf(f2.x, q0[g], s[g]));
        }
      }
    }
    sm.chunk(s, valid, a.scale_log2, vc, &s_p[sm.wave][0][0]);
  }
  __syncthreads();
  sm.finish(s_main, tid, a.n_splits, split, a.out, a.partial, size_t(b) * a.n_q + size_t(h) * G);
}

template <int D, int G>
hipError_t fp16_t(const Fp16DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.n_splits), unsigned(a.n_kv), unsigned(a.n_seq));
  hipLaunchKernelGGL((fp16_scan_kernel<D, G>), grid, dim3(kThreads), 0, s, a, a.K, a.V);
  return hipGetLastError();
}

template <int D>
hipError_t fp16_g(const Fp16DecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 1: return fp16_t<D, 1>(a, s);
    case 2: return fp16_t<D, 2>(a, s);
    case 4: return fp16_t<D, 4>(a, s);
    case 8: return fp16_t<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fp16_decode(const Fp16DecodeArgs& a, hipStream_t s) {
  if (a.d == 64) return fp16_g<64>(a, s);
  if (a.d == 128) return fp16_g<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pgkq
