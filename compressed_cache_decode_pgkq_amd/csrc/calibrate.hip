// Calibration over the keys to be encoded (gfx950): per-channel sums of
// squares, step (0) of the PGKQ pipeline (channel reorder by decreasing l2 norm
// with high/low interleaving; EdgeLLM-Nano paper page, "PGKQ pipeline") and the
// per-head scale of the Lloyd-Max radius table.
//
// Two kernels, deterministic (fixed summation order, no atomics):
//   calib_partial   one workgroup per (chunk of token rows, kv-head, sequence):
//                   float64 sums of squares per channel into a workspace row;
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

// One workgroup per (chunk of rows_per_chunk token rows, kv-head, sequence):
// 16-byte loads, EPT consecutive channels per thread, float64 sums.
template <int D, int ESIZE>
__global__ void __launch_bounds__(kThreads) calib_partial_kernel(CalibArgs a) {
  constexpr int EPT = 16 / ESIZE;        // elements per 16-byte load
  constexpr int TPR = D / EPT;           // threads per row
  constexpr int RPP = kThreads / TPR;    // rows per pass
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rp = tid / TPR;
  const int64_t tc = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t t0 = tc * a.rows_per_chunk;
  const int64_t t1 = min<int64_t>(t0 + a.rows_per_chunk, a.n_tokens);
  const uint8_t* base = static_cast<const uint8_t*>(a.K) +
                        ((b * a.n_kv + h) * a.n_tokens) * int64_t(D) * ESIZE + cg * 16;
  double acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.0;
  auto row = [&](int64_t t) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + t * int64_t(D) * ESIZE));
  };
  auto add = [&](const u32x4& raw) {
    if constexpr (ESIZE == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float fx = __half2float(__ushort_as_half(static_cast<uint16_t>(raw[k])));
        const float fy = __half2float(__ushort_as_half(static_cast<uint16_t>(raw[k] >> 16)));
        acc[2 * k] += double(fx) * double(fx);
        acc[2 * k + 1] += double(fy) * double(fy);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float f = __uint_as_float(raw[k]);
        acc[k] += double(f) * double(f);
      }
    }
  };
  // four rows in flight per thread; the sums still run over the rows in order
  int64_t t = t0 + rp;
  for (; t + 3 * RPP < t1; t += 4 * RPP) {
    const u32x4 r0 = row(t), r1 = row(t + RPP), r2 = row(t + 2 * RPP), r3 = row(t + 3 * RPP);
    add(r0);
    add(r1);
    add(r2);
    add(r3);
  }
  for (; t < t1; t += RPP) add(row(t));
  __shared__ double s_acc[RPP][D];
#pragma unroll
  for (int e = 0; e < EPT; ++e) s_acc[rp][cg * EPT + e] = acc[e];
  __syncthreads();
  for (int c = tid; c < D; c += kThreads) {
    double s = 0.0;
#pragma unroll 8
    for (int r = 0; r < RPP; ++r) s += s_acc[r][c];
    const int64_t chunk = b * a.chunks_per_seq + tc;  // chunks of one head, in (b, tc) order
    a.partial[(size_t(h) * a.n_chunks + chunk) * D + c] = s;
  }
}

template <int D>
__global__ void __launch_bounds__(D) calib_finalize_kernel(CalibArgs a) {
  const int c = threadIdx.x;
  const int h = blockIdx.x;
  __shared__ double s_ss[D];
  __shared__ int s_pi[D];
  __shared__ double s_sigma;
  // eight interleaved partial sums (part[k] takes chunks k, k + 8, k + 16, ...
  // in order), combined in a fixed order: the result does not depend on
  // scheduling.  32 rows are requested per round trip (the kernel is bound by
  // load latency), then added in that order.
  double part[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const double* src = a.partial + size_t(h) * a.n_chunks * D + c;
  int64_t ch = 0;
  for (; ch + 32 <= a.n_chunks; ch += 32) {
    double v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) v[k] = src[(ch + k) * D];
#pragma unroll
    for (int k = 0; k < 32; ++k) part[k % 8] += v[k];
  }
  for (; ch + 8 <= a.n_chunks; ch += 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) part[k] += src[(ch + k) * D];
  }
  for (int k = 0; ch < a.n_chunks; ++ch, ++k) part[k] += src[ch * D];
  double s = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
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
  const dim3 grid(unsigned(a.chunks_per_seq), unsigned(a.n_kv), unsigned(a.n_seq));
  if (a.k_dtype == DT_F32) {
    hipLaunchKernelGGL((calib_partial_kernel<D, 4>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((calib_partial_kernel<D, 2>), grid, dim3(kThreads), 0, s, a);
  }
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
