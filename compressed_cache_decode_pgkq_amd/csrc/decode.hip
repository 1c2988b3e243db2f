// PGKQ decode attention for gfx950: analytic logits from the codes, softmax and
// the fp16-V weighted sum, split over the token axis (flash-decoding style).
//
// The decode side of the PGKQ pipeline (EdgeLLM-Nano paper page: codes are
// never inverted into K-hat; logits are computed analytically from Q, r-hat,
// theta-hat and the QJL sketch; the decode path applies the Hadamard rotation to
// Q, the polar reconstruction and the QJL correction; V stays FP16).
//
// Three kernels on one stream:
//   query_prep   per (sequence, query head): q~ = H (signs * q[perm]) / sqrt(d),
//                the per-pair angle table q~[2i] cos(c_a) + q~[2i+1] sin(c_a) for
//                every angle code a, and S_h q~ for the QJL term (done inside
//                the scan when each stream is one workgroup and G <= 2);
//   decode_scan  per (sequence, kv-head, token split): builds in LDS, for the G
//                query heads sharing the kv-head, a joint table indexed by the
//                pair's (radius, angle) code, J[i][code][g] = level[rc] *
//                angle_table_g[i][ac] (or level and angle tables separately when
//                the joint table would not fit), and 16-entry tables of signed
//                nibble sums of kappa * S_h q~ for the sketch.  Lane = token for
//                the score: one coalesced dword load per code word, one LDS read
//                per pair giving all G heads, one per sketch nibble.  Online
//                softmax per wavefront; the weighted sum of the fp16 values on
//                the matrix cores over the value cache in 32-token tiles;
//   merge        log-sum-exp merge of the split partial states.
#include "scan.hpp"

namespace pgkq {

namespace {

constexpr int kPrepThreads = 256;

// S_h staged in LDS for the per-thread products with S_h (S_h q~ in the query
// preparation, S_h eps~ in the append): thread t multiplies floats
// [t CPT, (t + 1) CPT) of S_h (row t / TPR, slice t % TPR), which sit in LDS
// segment t, padded by 16 bytes so that the segments' 16-byte reads fall in
// distinct banks.  S_h is read with coalesced 16-byte loads (a wave
// instruction covers 1 KiB of consecutive floats); loading each thread's
// contiguous slice directly would touch 64 cache lines per instruction.
template <int D, bool QJL>
struct SStage {
  static constexpr int M = QJL ? D : 0;
  static constexpr int TPR = QJL ? kPrepThreads / D : 1;  // threads per row of S_h
  static constexpr int CPT = D / TPR;                      // columns per thread
  static constexpr int SEG = CPT + 4;
  static constexpr int SLD = QJL ? M * D / 4 / kPrepThreads : 1;  // float4 loads per thread
  static constexpr int FLOATS = QJL ? kPrepThreads * SEG : 4;
  static_assert(!QJL || TPR == 2 || TPR == 4, "rows of S_h per workgroup");
  static_assert(!QJL || (M * D) % (4 * kPrepThreads) == 0, "S_h tiling");
  typedef float4 Loads[SLD];

  __device__ __forceinline__ static void load(Loads& v, const float* __restrict__ S, int h, int tid) {
    if constexpr (QJL) {
      const float4* Sh = reinterpret_cast<const float4*>(S + size_t(h) * M * D);
#pragma unroll
      for (int j = 0; j < SLD; ++j) v[j] = Sh[tid + kPrepThreads * j];
    }
  }
  // the caller synchronizes the workgroup before the segments are read
  __device__ __forceinline__ static void store(const Loads& v, float* s_S, int tid) {
    if constexpr (QJL) {
#pragma unroll
      for (int j = 0; j < SLD; ++j) {
        const int o = 4 * (tid + kPrepThreads * j);  // float offset in S_h
        *reinterpret_cast<float4*>(&s_S[(o / CPT) * SEG + o % CPT]) = v[j];
      }
    }
  }
  __device__ __forceinline__ static float4 slice(const float* s_S, int tid, int k) {
    return *reinterpret_cast<const float4*>(&s_S[tid * SEG + 4 * k]);
  }
};

// ------------------------------------------------------------------ append

// Encode one new key of stream (b, h) into slot a.append_slot and copy its
// value row: steps (1)-(4) of the pipeline for a single key, by the
// kPrepThreads threads of a workgroup of the preparation launch.  Decisions
// are taken on the unnormalized transform X = sqrt(d) k~ (exact in float64 for
// fp16 keys): X_x^2 + X_y^2 against d T_j^2 and the octant comparisons of
// (X_x, X_y), as in the bulk encoder; the residual, its norm and the QJL
// projection are float64 (each thread's slice of a row of S_h, the slices
// summed by DPP exchanges).  `sv` holds this thread's coalesced loads of S_h,
// staged into s_S with the key row.
template <int D, int BM, bool QJL>
__device__ __forceinline__ void append_key(const DecodeArgs& a, int64_t b, int h, int tid,
                           const typename SStage<D, QJL>::Loads& sv, float* s_S) {
  using ST = SStage<D, QJL>;
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int P = BM + BA;
  constexpr int L = 1 << BM;
  constexpr int A = 1 << BA;
  constexpr int M = QJL ? D : 0;
  constexpr int NC = N * P / 32;
  constexpr int NSW = M / 32;
  static_assert(D / 2 <= kWave, "one wavefront holds a level's butterflies");
  __shared__ float s_raw[D];
  __shared__ float s_cb[2 * L];
  __shared__ double2 s_grid[A];  // (cos, sin) of the angle grid
  __shared__ double s_x[D];
  __shared__ double s_ss[N];
  __shared__ uint32_t s_code[N];
  __shared__ uint32_t s_bit[D];
  const int64_t stream = b * a.n_kv + h;
  // independent loads first: the key row as stored, the value row, the channel
  // order, the signs and the codebook (the permuted gather then reads the row
  // from LDS); the angle grid is computed meanwhile
  int src = tid;
  bool neg = false;
  uint16_t vrow = 0;  // fp16 bits
  if (tid < D) {
    s_raw[tid] = load_f(a.k_new, a.k_dtype, size_t(stream) * D + tid);
    vrow = a.v_new[size_t(stream) * D + tid];
    if (a.perm) src = int(a.perm[size_t(h) * D + tid]);
    neg = a.hadamard && a.signs[size_t(h) * D + tid] < 0;
  }
  if (tid < 2 * L) s_cb[tid] = a.codebook[size_t(h) * 2 * L + tid];
  if (QJL && tid < A) {
    double sn, cs;
    sincospi(-1.0 + (2.0 * tid + 1.0) / double(A), &sn, &cs);
    s_grid[tid] = make_double2(cs, sn);
  }
  ST::store(sv, s_S, tid);  // S_h arrives with the key; staged before the transform
  __syncthreads();
  if (tid < D) {
    const double v = static_cast<double>(s_raw[src]);
    s_x[tid] = neg ? -v : v;
  }
  __syncthreads();
  if (a.hadamard && tid < kWave) {  // every butterfly of a level sits in wavefront 0
    for (int hh = 1; hh < D; hh <<= 1) {
      if (tid < D / 2) {
        const int c0 = (tid / hh) * 2 * hh + (tid % hh);
        const double u = s_x[c0], w = s_x[c0 + hh];
        s_x[c0] = u + w;
        s_x[c0 + hh] = u - w;
      }
      wave_lds_sync();  // the next level reads what other lanes wrote
    }
  }
  __syncthreads();
  if (tid < N) {
    const double x = s_x[2 * tid], y = s_x[2 * tid + 1];
    const double r2 = x * x + y * y;
    const double tscale = a.hadamard ? double(D) : 1.0;
    int rc = 0;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      const double t = static_cast<double>(s_cb[L + j]);
      rc += (tscale * t * t < r2) ? 1 : 0;
    }
    const int ac = octant_cell(x, y) >> (3 - BA);
    s_code[tid] = static_cast<uint32_t>(rc | (ac << BM));
    if constexpr (QJL) {
      const double inv_scale = a.hadamard ? 1.0 / sqrt(double(D)) : 1.0;
      const double2 cs = s_grid[ac];
      const double lv = static_cast<double>(s_cb[rc]);
      const double ex = x * inv_scale - lv * cs.x;
      const double ey = y * inv_scale - lv * cs.y;
      s_x[2 * tid] = ex;   // this thread's own pair: no other reader yet
      s_x[2 * tid + 1] = ey;
      s_ss[tid] = ex * ex + ey * ey;
    }
  }
  __syncthreads();
  if constexpr (QJL) {
    const int r = tid / ST::TPR, part = tid % ST::TPR;
    double u = 0.0;
#pragma unroll
    for (int k = 0; k < ST::CPT / 4; ++k) {
      const int c = part * ST::CPT + 4 * k;
      const float4 v = ST::slice(s_S, tid, k);
      u = fma(double(v.x), s_x[c], u);
      u = fma(double(v.y), s_x[c + 1], u);
      u = fma(double(v.z), s_x[c + 2], u);
      u = fma(double(v.w), s_x[c + 3], u);
    }
    u += quad_xor<1>(u);
    if constexpr (ST::TPR == 4) u += quad_xor<2>(u);
    if (part == 0) s_bit[r] = u >= 0.0 ? 1u : 0u;
    __syncthreads();
  }
  const int64_t slot = a.append_slot;
  uint8_t* base = a.codes_w + size_t(stream) * a.stream_bytes;
  uint32_t* rows = reinterpret_cast<uint32_t*>(base);
  if (tid < NC) {
    uint32_t word = 0;
    for (int i = (32 * tid) / P; i <= (32 * tid + 31) / P && i < N; ++i) {
      const int o = P * i - 32 * tid;
      word |= o >= 0 ? (s_code[i] << o) : (s_code[i] >> (-o));
    }
    rows[size_t(tid) * a.capacity + slot] = word;
  } else if (QJL && tid < NC + NSW) {
    const int w = tid - NC;
    uint32_t word = 0;
    for (int j = 0; j < 32; ++j) word |= s_bit[32 * w + j] << j;
    rows[size_t(tid) * a.capacity + slot] = word;
  }
  if (QJL && tid == 0) {
    double ss = 0.0;
    for (int i = 0; i < N; ++i) ss += s_ss[i];
    uint16_t* nu = reinterpret_cast<uint16_t*>(base + size_t(4) * (NC + NSW) * a.capacity);
    nu[slot] = f64_to_f16_rne_sat_nonneg(sqrt(ss));
  }
  if (tid < D)  // the value row goes into the stream's 32-token tiles
    a.V_w[size_t(stream) * a.capacity * D + vtile_index(slot, tid, D)] = vrow;
}

// ------------------------------------------------------------------ query prep

// One workgroup per query head: q~ = H (signs * q[perm]) / sqrt(d), the
// per-pair angle table q~[2i] cos thetahat_a + q~[2i+1] sin thetahat_a and,
// with QJL, S_h q~.  The kernel is latency-bound, so every global load that
// does not depend on another is issued at the start: S_h (staged in LDS,
// SStage), the query row, the signs and the channel order (the permuted gather
// then reads the query row from LDS).  For a decode step the launch has one
// more workgroup per (sequence, kv-head), which appends the stream's new token
// beside the preparation instead of before it.
template <int D, int BM, bool QJL>
__global__ void __launch_bounds__(kPrepThreads)
query_prep_kernel(DecodeArgs a, const float* __restrict__ S) {
  using ST = SStage<D, QJL>;
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int A = 1 << BA;
  constexpr int M = ST::M;
  constexpr int TPR = ST::TPR;
  constexpr int CPT = ST::CPT;
  static_assert(kPrepThreads % A == 0 && kPrepThreads >= D, "thread mapping");
  const PrepLayout pl{D, N, A, M};
  const int tid = threadIdx.x;
  // grid (sequence, row): a decode step's appending workgroups take the first
  // rows, so that they are dispatched before the preparation workgroups
  // (decode step 237 -> 233 us on the 32k-token workload)
  const int n_app = a.append_slot >= 0 ? int(a.n_kv) : 0;
  const int64_t b = blockIdx.x;
  const int hq = int(blockIdx.y) - n_app;
  __shared__ __align__(16) float s_S[ST::FLOATS];

  if (hq < 0) {  // decode step: the appending workgroup of kv-head blockIdx.y
    const int h = int(blockIdx.y);
    typename ST::Loads sv;
    ST::load(sv, S, h, tid);
    append_key<D, BM, QJL>(a, b, h, tid, sv, s_S);
    return;
  }
  const int h = hq / a.group;
  const int r = tid / TPR, part = tid % TPR;
  typename ST::Loads sv;
  ST::load(sv, S, h, tid);
  __shared__ float sraw[D];
  __shared__ float sx[D];
  __shared__ double sq64[D];
  float sgn = 1.f;
  int src = tid;
  if (tid < D) {
    sraw[tid] = load_f(a.q, a.q_dtype, (size_t(b) * a.n_q + hq) * D + tid);
    if (a.perm) src = int(a.perm[size_t(h) * D + tid]);
    if (a.hadamard) sgn = float(a.signs[size_t(h) * D + tid]);
  }
  // the angle grid of this thread's table entries (every entry it writes has
  // the angle code tid % A)
  double acs, asn;
  sincospi(-1.0 + (2.0 * (tid % A) + 1.0) / double(A), &asn, &acs);
  ST::store(sv, s_S, tid);
  __syncthreads();
  if (tid < D) sx[tid] = sraw[src] * sgn;
  __syncthreads();
  static_assert(N <= kWave, "one wavefront holds a level's butterflies");
  if (a.hadamard && tid < kWave) {  // every butterfly of a level sits in wavefront 0
    for (int hh = 1; hh < D; hh <<= 1) {
      if (tid < N) {
        const int c0 = (tid / hh) * 2 * hh + (tid % hh);
        const float u = sx[c0], w = sx[c0 + hh];
        sx[c0] = u + w;
        sx[c0 + hh] = u - w;
      }
      wave_lds_sync();  // the next level reads what other lanes wrote
    }
  }
  __syncthreads();
  float* out = a.prep + (size_t(b) * a.n_q + hq) * pl.stride();
  const float sc = a.hadamard ? 1.0f / sqrtf(float(D)) : 1.0f;
  if (tid < D) {
    const float qt = sx[tid] * sc;
    out[tid] = qt;
    sq64[tid] = double(qt);
  }
  __syncthreads();
  for (int e = tid; e < N * A; e += kPrepThreads) {
    const int i = e / A;
    out[pl.off_lut() + e] = static_cast<float>(sq64[2 * i] * acs + sq64[2 * i + 1] * asn);
  }
  if constexpr (QJL) {
    // S_h q~: TPR adjacent threads per row, each over a contiguous slice of
    // CPT columns; float64 products, the slices summed by DPP quad exchanges
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < CPT / 4; ++k) {
      const int c = part * CPT + 4 * k;
      const float4 v = ST::slice(s_S, tid, k);
      acc = fma(double(v.x), sq64[c], acc);
      acc = fma(double(v.y), sq64[c + 1], acc);
      acc = fma(double(v.z), sq64[c + 2], acc);
      acc = fma(double(v.w), sq64[c + 3], acc);
    }
    acc += quad_xor<1>(acc);
    if constexpr (TPR == 4) acc += quad_xor<2>(acc);
    if (part == 0) out[pl.off_sq() + r] = static_cast<float>(acc);
  }
}

// ------------------------------------------------------------------ merge

constexpr int kMergeThreads = 512;

// Log-sum-exp merge of the split partials (m, l, o) of one query head per
// workgroup.  The threads form J groups of d/4; a thread takes four channels
// of the partials j, j + J, j + 2J, ... of its group, four partials at a time
// with all their loads issued together (the kernel is latency-bound), merged
// online (the running maximum rescales what has been summed when it grows).
// The J group states are then combined through LDS.
template <int D>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const float* __restrict__ partial,
                                                              float* __restrict__ out, int n_splits) {
  constexpr int TPW = D / 4;                // threads per partial row
  constexpr int J = kMergeThreads / TPW;    // partial groups
  constexpr int kBlock = 4;
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int nq = gridDim.x;
  const int tid = threadIdx.x;
  const int q = tid % TPW, j = tid / TPW;
  const float* part = partial + (size_t(b) * nq + hq) * size_t(n_splits) * (D + 4);
  float Mx = -INFINITY, den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = j; p0 < n_splits; p0 += J * kBlock) {
    float mv[kBlock], lv[kBlock];
    float4 ov[kBlock];
#pragma unroll
    for (int k = 0; k < kBlock; ++k) {
      const int p = p0 + k * J;
      const float* pp = part + size_t(p) * (D + 4);
      const bool in = p < n_splits;
      mv[k] = in ? pp[0] : -INFINITY;
      lv[k] = in ? pp[1] : 0.f;
      ov[k] = in ? *reinterpret_cast<const float4*>(pp + 4 + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mb = Mx;
#pragma unroll
    for (int k = 0; k < kBlock; ++k) mb = fmaxf(mb, mv[k]);
    if (mb != -INFINITY) {
      const float f0 = exp2f(Mx - mb);  // 0 while nothing has been summed
      num.x *= f0;
      num.y *= f0;
      num.z *= f0;
      num.w *= f0;
      den *= f0;
#pragma unroll
      for (int k = 0; k < kBlock; ++k) {
        const float f = exp2f(mv[k] - mb);
        num.x += f * ov[k].x;
        num.y += f * ov[k].y;
        num.z += f * ov[k].z;
        num.w += f * ov[k].w;
        den += f * lv[k];
      }
      Mx = mb;
    }
  }
  __shared__ float s_m[J], s_l[J];
  __shared__ float4 s_o[J][TPW];
  s_o[j][q] = num;
  if (q == 0) {
    s_m[j] = Mx;
    s_l[j] = den;
  }
  __syncthreads();
  if (j == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < J; ++k) Mt = fmaxf(Mt, s_m[k]);
    float4 nt = make_float4(0.f, 0.f, 0.f, 0.f);
    float dt = 0.f;
    if (Mt != -INFINITY) {
#pragma unroll
      for (int k = 0; k < J; ++k) {
        const float f = exp2f(s_m[k] - Mt);
        const float4 o = s_o[k][q];
        nt.x += f * o.x;
        nt.y += f * o.y;
        nt.z += f * o.z;
        nt.w += f * o.w;
        dt += f * s_l[k];
      }
    }
    const float inv = dt > 0.f ? 1.f / dt : 0.f;
    *reinterpret_cast<float4*>(out + (size_t(b) * nq + hq) * D + 4 * q) =
        make_float4(nt.x * inv, nt.y * inv, nt.z * inv, nt.w * inv);
  }
}

// ------------------------------------------------------------------ dispatch

template <int D, int BM, bool QJL>
hipError_t prep_t(const DecodeArgs& a, hipStream_t s) {
  // a decode step adds one appending workgroup per (sequence, kv-head)
  const int64_t nx = a.n_q + (a.append_slot >= 0 ? a.n_kv : 0);
  hipLaunchKernelGGL((query_prep_kernel<D, BM, QJL>), dim3(unsigned(a.n_seq), unsigned(nx)),
                     dim3(kPrepThreads), 0, s, a, a.S);
  return hipGetLastError();
}

// Workgroups of the scan that prepares its query itself (one per stream): at
// head_dim 64 two wavefronts, so that the many short streams of that shape are
// resident at once (a 1536-stream, 512-token cache: one round instead of 1.2,
// whose second round ran alone at one workgroup per CU), else four.
template <int D>
constexpr int kFusedWaves = D == 64 ? 2 : kScanWaves;

template <int D, int BM, bool QJL, int G>
hipError_t scan_t(const DecodeArgs& a, bool logits_mode, hipStream_t s) {
  dim3 grid(unsigned(a.n_kv), unsigned(a.n_seq), unsigned(a.n_splits));
  if constexpr (G <= kFusedPrepMaxGroup) {
    if (a.fused_prep) {
      constexpr int W = kFusedWaves<D>;
      if (logits_mode) {
        hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, true, 0, true, W>), grid,
                           dim3(W * kWave), 0, s, a, a.codes, as_half(a.V));
      } else {
        hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, false, 0, true, W>), grid,
                           dim3(W * kWave), 0, s, a, a.codes, as_half(a.V));
      }
      return hipGetLastError();
    }
  }
  if (a.fused_prep) return hipErrorInvalidValue;
  if (logits_mode) {
    hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, true>), grid, dim3(kScanThreads), 0, s, a,
                       a.codes, as_half(a.V));
  } else {
    hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, false>), grid, dim3(kScanThreads), 0, s,
                       a, a.codes, as_half(a.V));
  }
  return hipGetLastError();
}

template <int D, int BM, bool QJL>
hipError_t scan_g(const DecodeArgs& a, bool lm, hipStream_t s) {
  switch (a.group) {
    case 1: return scan_t<D, BM, QJL, 1>(a, lm, s);
    case 2: return scan_t<D, BM, QJL, 2>(a, lm, s);
    case 4: return scan_t<D, BM, QJL, 4>(a, lm, s);
    case 8: return scan_t<D, BM, QJL, 8>(a, lm, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int BM>
hipError_t scan_q(const Geometry& g, const DecodeArgs& a, bool lm, hipStream_t s) {
  return g.m ? scan_g<D, BM, true>(a, lm, s) : scan_g<D, BM, false>(a, lm, s);
}

template <int D>
hipError_t scan_b(const Geometry& g, const DecodeArgs& a, bool lm, hipStream_t s) {
  switch (g.bm) {
    case 2: return scan_q<D, 2>(g, a, lm, s);
    case 3: return scan_q<D, 3>(g, a, lm, s);
    case 4: return scan_q<D, 4>(g, a, lm, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t prep_b(const Geometry& g, const DecodeArgs& a, hipStream_t s) {
  const bool q = g.m != 0;
  switch (g.bm) {
    case 2: return q ? prep_t<D, 2, true>(a, s) : prep_t<D, 2, false>(a, s);
    case 3: return q ? prep_t<D, 3, true>(a, s) : prep_t<D, 3, false>(a, s);
    case 4: return q ? prep_t<D, 4, true>(a, s) : prep_t<D, 4, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_query_prep(const Geometry& g, const DecodeArgs& a, hipStream_t s) {
  if (g.d == 64) return prep_b<64>(g, a, s);
  if (g.d == 128) return prep_b<128>(g, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_scan(const Geometry& g, const DecodeArgs& a, bool logits_mode,
                              hipStream_t s) {
  if (g.d == 64) return scan_b<64>(g, a, logits_mode, s);
  if (g.d == 128) return scan_b<128>(g, a, logits_mode, s);
  return hipErrorInvalidValue;
}

hipError_t launch_partial_merge(int d, int64_t n_seq, int64_t n_q, int n_splits,
                                const float* partial, float* out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_q), static_cast<unsigned>(n_seq));
  if (d == 64) {
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, s, partial, out, n_splits);
  } else if (d == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, s, partial, out, n_splits);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pgkq
