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
//                                out = (o + kappa S_v^T a) / l (512 threads:
//                                groups of d take every J-th partial, then
//                                d / J rows of S_v each).
#include "scan.hpp"

namespace pgkq {

namespace {

constexpr int kKvMergeThreads = 512;

// Per (sequence, query head): log-sum-exp merge of the partial states, then
// out = (o + kappa S_v^T a) / l.  The J = 512 / d thread groups take every
// J-th partial, and then d / J consecutive rows of S_v each; their sums are
// combined in LDS in group order (deterministic).  The S_v loads are issued
// first (they do not depend on the partials): the kernel is bound by latency.
template <int D>
__global__ void __launch_bounds__(kKvMergeThreads)
kv_merge_kernel(const float* __restrict__ partial, float* __restrict__ out, const float* __restrict__ Sv,
                int n_parts, int group, int qjl) {
  constexpr int J = kKvMergeThreads / D;  // thread groups
  constexpr int RPT = D / J;              // rows of S_v per thread
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int nq = gridDim.x;
  const int h = hq / group;
  constexpr int width = 2 * D + 4;
  const float* part = partial + (size_t(b) * nq + hq) * size_t(n_parts) * width;
  const int tid = threadIdx.x;
  const int c = tid % D, j = tid / D;
  __shared__ float s_num[J][D], s_an[J][D], s_den[J];
  __shared__ float s_a[D];
  float sv[RPT];
  if (qjl) {  // column c of S_v[h], rows [j RPT, (j + 1) RPT)
    const float* S = Sv + size_t(h) * D * D + size_t(j) * RPT * D + c;
#pragma unroll
    for (int r = 0; r < RPT; ++r) sv[r] = S[size_t(r) * D];
  }
  float Mx = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < n_parts; ++p) Mx = fmaxf(Mx, part[size_t(p) * width]);
  float num = 0.f, an = 0.f, den = 0.f;
  if (Mx != -INFINITY) {
#pragma unroll 4
    for (int p = j; p < n_parts; p += J) {
      const float* pp = part + size_t(p) * width;
      const float f = exp2f(pp[0] - Mx);
      num += f * pp[4 + c];
      an += f * pp[4 + D + c];
      den += f * pp[1];
    }
  }
  s_num[j][c] = num;
  s_an[j][c] = an;
  if (c == 0) s_den[j] = den;
  __syncthreads();
  if (j == 0) {
    float nt = 0.f, at = 0.f, dt = 0.f;
#pragma unroll
    for (int k = 0; k < J; ++k) {
      nt += s_num[k][c];
      at += s_an[k][c];
      dt += s_den[k];
    }
    s_num[0][c] = nt;
    s_a[c] = at;
    if (c == 0) s_den[0] = dt;
  }
  __syncthreads();
  float corr = 0.f;
  if (qjl) {  // this thread's rows of S_v^T a
#pragma unroll
    for (int r = 0; r < RPT; ++r) corr = fmaf(sv[r], s_a[j * RPT + r], corr);
  }
  s_an[j][c] = corr;  // (every read of s_an precedes the barrier above)
  __syncthreads();
  if (j == 0) {
    float ct = 0.f;
#pragma unroll
    for (int k = 0; k < J; ++k) ct += s_an[k][c];
    ct *= 1.2533141373155003f / float(D);  // kappa = sqrt(pi/2) / m, m = d
    const float dt = s_den[0];
    out[(size_t(b) * nq + hq) * D + c] = dt > 0.f ? (s_num[0][c] + ct) / dt : 0.f;
  }
}

template <int D, int BM, bool QJL, int G, int VB>
hipError_t kv_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.n_kv), unsigned(a.n_seq), unsigned(a.n_splits));
  hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, false, VB>), grid, dim3(kScanThreads), 0, s,
                     a, a.codes, as_half(a.V));
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
  const dim3 grid(static_cast<unsigned>(a.n_q), static_cast<unsigned>(a.n_seq));
  const int qjl = a.S_v ? 1 : 0;
  if (d == 64) {
    hipLaunchKernelGGL(kv_merge_kernel<64>, grid, dim3(kKvMergeThreads), 0, s, a.partial, a.out, a.S_v,
                       n_parts, a.group, qjl);
  } else if (d == 128) {
    hipLaunchKernelGGL(kv_merge_kernel<128>, grid, dim3(kKvMergeThreads), 0, s, a.partial, a.out,
                       a.S_v, n_parts, a.group, qjl);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pgkq
