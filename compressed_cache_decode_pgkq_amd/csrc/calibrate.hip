// Calibration over the keys to be encoded (gfx950): per-channel sums of
// squares, step (0) of the PGKQ pipeline (channel reorder by decreasing l2 norm
// with high/low interleaving; EdgeLLM-Nano paper page, "PGKQ pipeline") and the
// per-head scale of the Lloyd-Max radius table.
//
// Two kernels, deterministic (fixed summation order, no atomics):
//   calib_partial   one workgroup per (chunk of key rows, kv-head): float64 sums
//                   of squares per channel into a workspace row;
//   calib_finalize  one workgroup per kv-head: sums the chunk rows in order,
//                   derives s_h = sqrt(mean ||k||^2), scales the unit Lloyd-Max
//                   table by s_h / sqrt(d/2) (float64 product, one rounding to
//                   fp32) and, when asked, ranks the channels (stable, by
//                   descending sum of squares) into the interleaved order
//                   [pi_0, pi_{d-1}, pi_1, pi_{d-2}, ...].
#include "device_common.hpp"

namespace pgkq {

namespace {

constexpr int kThreads = 256;

template <int D>
__global__ void __launch_bounds__(kThreads) calib_partial_kernel(CalibArgs a) {
  constexpr int PH = kThreads / D;  // row phases per workgroup
  const int tid = threadIdx.x;
  const int c = tid % D, ph = tid / D;
  const int64_t ch = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t total = a.n_seq * a.n_tokens;
  const int64_t r0 = ch * a.rows_per_chunk;
  const int64_t r1 = min<int64_t>(r0 + a.rows_per_chunk, total);
  double acc = 0.0;
  for (int64_t r = r0 + ph; r < r1; r += PH) {
    const int64_t bb = r / a.n_tokens, t = r % a.n_tokens;
    const int64_t idx = ((bb * a.n_kv + h) * a.n_tokens + t) * D + c;
    const double v = double(load_f(a.K, a.k_dtype, idx));
    acc += v * v;
  }
  __shared__ double s_acc[kThreads];
  s_acc[tid] = acc;
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
#pragma unroll
    for (int p = 0; p < PH; ++p) s += s_acc[p * D + tid];
    a.partial[(size_t(h) * a.n_chunks + ch) * D + tid] = s;
  }
}

template <int D>
__global__ void __launch_bounds__(D) calib_finalize_kernel(CalibArgs a) {
  const int c = threadIdx.x;
  const int h = blockIdx.x;
  __shared__ double s_ss[D];
  __shared__ int s_pi[D];
  __shared__ double s_sigma;
  double s = 0.0;
  for (int64_t ch = 0; ch < a.n_chunks; ++ch) s += a.partial[(size_t(h) * a.n_chunks + ch) * D + c];
  s_ss[c] = s;
  a.sumsq[size_t(h) * D + c] = s;
  __syncthreads();
  if (c == 0) {
    double tot = 0.0;
    for (int k = 0; k < D; ++k) tot += s_ss[k];
    const double sh = sqrt(tot / double(a.n_seq * a.n_tokens));
    s_sigma = sh / sqrt(double(D / 2));
  }
  __syncthreads();
  const int L = a.L;
  float* cb = a.codebook + size_t(h) * 2 * L;
  if (c < L) cb[c] = static_cast<float>(a.base_levels[c] * s_sigma);
  if (c >= L && c < 2 * L - 1) cb[c] = static_cast<float>(a.base_thresholds[c - L] * s_sigma);
  if (c == 2 * L - 1) cb[c] = __int_as_float(0x7F800000);
  if (a.perm) {
    if (a.reorder) {
      int rank = 0;
      for (int k = 0; k < D; ++k) {
        const double o = s_ss[k];
        rank += (o > s || (o == s && k < c)) ? 1 : 0;
      }
      s_pi[rank] = c;
      __syncthreads();
      if (c < D / 2) {
        a.perm[size_t(h) * D + 2 * c] = static_cast<uint16_t>(s_pi[c]);
        a.perm[size_t(h) * D + 2 * c + 1] = static_cast<uint16_t>(s_pi[D - 1 - c]);
      }
    } else {
      a.perm[size_t(h) * D + c] = static_cast<uint16_t>(c);
    }
  }
}

template <int D>
hipError_t calib_t(const CalibArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((calib_partial_kernel<D>), dim3(unsigned(a.n_chunks), unsigned(a.n_kv)),
                     dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((calib_finalize_kernel<D>), dim3(unsigned(a.n_kv)), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  if (a.d == 64) return calib_t<64>(a, s);
  if (a.d == 128) return calib_t<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pgkq
