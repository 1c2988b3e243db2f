// PGKQ-KV decode attention for gfx950: PGKQ key codes for the logits (the
// PGKQ scan unchanged) and PGKQ-coded values for the weighted sum (EdgeLLM-Nano
// paper page, PGKQ-KV paragraphs: polar codes, Lloyd-Max table and QJL sketch
// applied to V, Hadamard disabled for V).
//
// Two kernels after the shared query preparation:
//   decode_scan_kernel<..., VB>  the scan of scan.hpp with the coded value path
//                                (CodedPV): per workgroup (its wavefronts
//                                merged in LDS) a partial state
//                                (m, l, o[d], a[d]) with o the weighted pair
//                                reconstructions and a_j = sum_t p_t nu_t
//                                (2 bit_tj - 1);
//   kv_merge_kernel              per (sequence, query head): log-sum-exp merge
//                                of the partials, then
//                                out = (o + kappa S_v^T a) / l.
#include "scan.hpp"

namespace pgkq {

namespace {

__global__ void __launch_bounds__(128)
kv_merge_kernel(const float* __restrict__ partial, float* __restrict__ out, const float* __restrict__ Sv,
                int d, int n_parts, int group, int qjl) {
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int nq = gridDim.x;
  const int h = hq / group;
  const int width = 2 * d + 4;
  const float* part = partial + (size_t(b) * nq + hq) * size_t(n_parts) * width;
  const int tid = threadIdx.x;
  __shared__ float s_a[128];
  float Mx = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < n_parts; ++p) Mx = fmaxf(Mx, part[size_t(p) * width]);
  float num = 0.f, an = 0.f, den = 0.f;
  if (tid < d && Mx != -INFINITY) {
#pragma unroll 4
    for (int p = 0; p < n_parts; ++p) {
      const float* pp = part + size_t(p) * width;
      const float f = exp2f(pp[0] - Mx);
      num += f * pp[4 + tid];
      an += f * pp[4 + d + tid];
      den += f * pp[1];
    }
  }
  if (tid < d) s_a[tid] = an;
  __syncthreads();
  if (tid < d) {
    float corr = 0.f;
    if (qjl) {
      // kappa S^T a: column tid of S_v[h], rows j < m = d
      const float* S = Sv + size_t(h) * d * d + tid;
#pragma unroll 8
      for (int j = 0; j < d; ++j) corr = fmaf(S[size_t(j) * d], s_a[j], corr);
      corr *= 1.2533141373155003f / float(d);  // sqrt(pi/2) / m
    }
    out[(size_t(b) * nq + hq) * d + tid] = den > 0.f ? (num + corr) / den : 0.f;
  }
}

template <int D, int BM, bool QJL, int G, int VB>
hipError_t kv_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.n_splits), unsigned(a.n_kv), unsigned(a.n_seq));
  hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, false, VB>), grid, dim3(kScanThreads), 0, s,
                     a, a.codes, a.V);
  return hipGetLastError();
}

template <int D, int BM, bool QJL, int VB>
hipError_t kv_g(const DecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 1: return kv_t<D, BM, QJL, 1, VB>(a, s);
    case 2: return kv_t<D, BM, QJL, 2, VB>(a, s);
    case 4: return kv_t<D, BM, QJL, 4, VB>(a, s);
    case 8: return kv_t<D, BM, QJL, 8, VB>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// (b_main of K, b_main of V): k2v2, k3v3, k4v4, k3v2, k4v2 (the configurations
// the PGKQ-KV paragraphs evaluate)
template <int D, bool QJL>
hipError_t kv_b(const Geometry& g, const DecodeArgs& a, hipStream_t s) {
  const int k = g.bm, v = a.bm_v;
  if (k == 2 && v == 2) return kv_g<D, 2, QJL, 2>(a, s);
  if (k == 3 && v == 3) return kv_g<D, 3, QJL, 3>(a, s);
  if (k == 4 && v == 4) return kv_g<D, 4, QJL, 4>(a, s);
  if (k == 3 && v == 2) return kv_g<D, 3, QJL, 2>(a, s);
  if (k == 4 && v == 2) return kv_g<D, 4, QJL, 2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_decode_scan(const Geometry& g, const DecodeArgs& a, hipStream_t s) {
  const bool q = g.m != 0;
  if (g.d == 64) return q ? kv_b<64, true>(g, a, s) : kv_b<64, false>(g, a, s);
  if (g.d == 128) return q ? kv_b<128, true>(g, a, s) : kv_b<128, false>(g, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_kv_merge(const DecodeArgs& a, int d, int n_parts, hipStream_t s) {
  if (d > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_merge_kernel, dim3(unsigned(a.n_q), unsigned(a.n_seq)), dim3(128), 0, s,
                     a.partial, a.out, a.S_v, d, n_parts, a.group, a.S_v ? 1 : 0);
  return hipGetLastError();
}

}  // namespace pgkq
