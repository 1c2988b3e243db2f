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
//                every angle code a, and S_h q~ for the QJL term;
//   decode_scan  per (sequence, kv-head, token split): builds in LDS, for the G
//                query heads sharing the kv-head, a joint table indexed by the
//                pair's (radius, angle) code, J[i][code][g] = level[rc] *
//                angle_table_g[i][ac] (or level and angle tables separately when
//                the joint table would not fit), and 16-entry tables of signed
//                nibble sums of kappa * S_h q~ for the sketch.  Lane = token for
//                the score: one coalesced dword load per code word, one LDS read
//                per pair giving all G heads, one per sketch nibble.  Online
//                softmax per wavefront, then lane = 8 channels of a token for
//                the P.V accumulation (16-byte fp16 V loads, fp32 accumulate);
//   merge        log-sum-exp merge of the split partial states.
#include "softmax_pv.hpp"

namespace pgkq {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanWaves = kScanThreads / kWave;
// waves per SIMD the register allocator must leave room for
#ifndef PGKQ_SCAN_MIN_WAVES
#define PGKQ_SCAN_MIN_WAVES 2
#endif
constexpr int kScanMinWavesPerEU = PGKQ_SCAN_MIN_WAVES;
// table lookups issued per scheduling group of the score loop
#ifndef PGKQ_PAIR_GROUP
#define PGKQ_PAIR_GROUP 8
#endif
constexpr int kPairGroup = PGKQ_PAIR_GROUP;


// ------------------------------------------------------------------ append

// Encode one new key of stream (b, h) into slot a.append_slot and copy its
// value row: steps (1)-(4) of the pipeline for a single key, by the 128
// threads of a query-prep workgroup.  Decisions are taken on the unnormalized
// transform X = sqrt(d) k~ (exact in float64 for fp16 keys): X_x^2 + X_y^2
// against d T_j^2 and the octant comparisons of (X_x, X_y), as in the bulk
// encoder; the residual, its norm and the QJL projection are float64.
template <int D, int BM, bool QJL>
__device__ void append_key(const DecodeArgs& a, const float* __restrict__ S, int64_t b, int h,
                           int tid) {
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int P = BM + BA;
  constexpr int L = 1 << BM;
  constexpr int A = 1 << BA;
  constexpr int M = QJL ? D : 0;
  constexpr int NC = N * P / 32;
  constexpr int NSW = M / 32;
  __shared__ double s_x[D];
  __shared__ double s_ss[N];
  __shared__ uint32_t s_code[N];
  __shared__ uint32_t s_bit[D];
  const int64_t stream = b * a.n_kv + h;
  const float* cb = a.codebook + size_t(h) * 2 * L;
  if (tid < D) {
    const int src = a.perm ? int(a.perm[size_t(h) * D + tid]) : tid;
    double v = static_cast<double>(load_f(a.k_new, a.k_dtype, size_t(stream) * D + src));
    if (a.hadamard && a.signs[size_t(h) * D + tid] < 0) v = -v;
    s_x[tid] = v;
  }
  __syncthreads();
  if (a.hadamard) {
    for (int hh = 1; hh < D; hh <<= 1) {
      double u = 0.0, w = 0.0;
      int c0 = 0;
      if (tid < D / 2) {
        c0 = (tid / hh) * 2 * hh + (tid % hh);
        u = s_x[c0];
        w = s_x[c0 + hh];
      }
      __syncthreads();
      if (tid < D / 2) {
        s_x[c0] = u + w;
        s_x[c0 + hh] = u - w;
      }
      __syncthreads();
    }
  }
  if (tid < N) {
    const double x = s_x[2 * tid], y = s_x[2 * tid + 1];
    const double r2 = x * x + y * y;
    const double tscale = a.hadamard ? double(D) : 1.0;
    int rc = 0;
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      const double t = static_cast<double>(cb[L + j]);
      rc += (tscale * t * t < r2) ? 1 : 0;
    }
    const int ac = octant_cell(x, y) >> (3 - BA);
    s_code[tid] = static_cast<uint32_t>(rc | (ac << BM));
    if constexpr (QJL) {
      const double inv_scale = a.hadamard ? 1.0 / sqrt(double(D)) : 1.0;
      double sn, cs;
      sincospi(-1.0 + (2.0 * ac + 1.0) / double(A), &sn, &cs);
      const double lv = static_cast<double>(cb[rc]);
      const double ex = x * inv_scale - lv * cs;
      const double ey = y * inv_scale - lv * sn;
      s_x[2 * tid] = ex;   // this thread's own pair: no other reader yet
      s_x[2 * tid + 1] = ey;
      s_ss[tid] = ex * ex + ey * ey;
    }
  }
  __syncthreads();
  if constexpr (QJL) {
    if (tid < M) {
      const float* Sr = S + (size_t(h) * M + tid) * D;
      double u = 0.0;
      for (int c = 0; c < D; ++c) u += static_cast<double>(Sr[c]) * s_x[c];
      s_bit[tid] = u >= 0.0 ? 1u : 0u;
    }
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
  if (tid < D) a.V_w[(size_t(stream) * a.capacity + slot) * D + tid] = a.v_new[size_t(stream) * D + tid];
}

// ------------------------------------------------------------------ query prep

template <int D, int BM, bool QJL>
__global__ void __launch_bounds__(128)
query_prep_kernel(DecodeArgs a, const float* __restrict__ S) {
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int A = 1 << BA;
  constexpr int M = QJL ? D : 0;
  const PrepLayout pl{D, N, A, M};
  const int tid = threadIdx.x;
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int h = hq / a.group;

  // decode step: the first query head of each kv-head appends its new token
  if (a.append_slot >= 0 && hq % a.group == 0) append_key<D, BM, QJL>(a, S, b, h, tid);

  __shared__ float sx[D];
  __shared__ double sq64[D];
  if (tid < D) {
    const int src = a.perm ? int(a.perm[size_t(h) * D + tid]) : tid;
    float v = load_f(a.q, a.q_dtype, (size_t(b) * a.n_q + hq) * D + src);
    if (a.hadamard) v *= float(a.signs[size_t(h) * D + tid]);
    sx[tid] = v;
  }
  __syncthreads();
  if (a.hadamard) {
    for (int hh = 1; hh < D; hh <<= 1) {
      float u = 0.f, w = 0.f;
      int c0 = 0;
      if (tid < D / 2) {
        c0 = (tid / hh) * 2 * hh + (tid % hh);
        u = sx[c0];
        w = sx[c0 + hh];
      }
      __syncthreads();
      if (tid < D / 2) {
        sx[c0] = u + w;
        sx[c0 + hh] = u - w;
      }
      __syncthreads();
    }
  }
  float* out = a.prep + (size_t(b) * a.n_q + hq) * pl.stride();
  const float sc = a.hadamard ? 1.0f / sqrtf(float(D)) : 1.0f;
  if (tid < D) {
    const float qt = sx[tid] * sc;
    out[tid] = qt;
    sq64[tid] = double(qt);
  }
  __syncthreads();
  for (int e = tid; e < N * A; e += blockDim.x) {
    const int i = e / A, ac = e % A;
    double sn, cs;
    sincospi(-1.0 + (2.0 * ac + 1.0) / double(A), &sn, &cs);
    out[pl.off_lut() + e] = static_cast<float>(sq64[2 * i] * cs + sq64[2 * i + 1] * sn);
  }
  if constexpr (QJL) {
    for (int r = tid; r < M; r += blockDim.x) {
      const float* Sr = S + (size_t(h) * M + r) * D;
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += double(Sr[c]) * sq64[c];
      out[pl.off_sq() + r] = static_cast<float>(acc);
    }
  }
}

// ------------------------------------------------------------------ scan

template <int D, int BM, int G>
struct ScanShape {
  static constexpr int N = D / 2;
  static constexpr int BA = BM - 1;
  static constexpr int P = BM + BA;
  static constexpr int L = 1 << BM;
  static constexpr int A = 1 << BA;
  static constexpr int NCODES = 1 << P;
  static constexpr bool JOINT = N * NCODES * G <= 8192;  // <= 32 KiB of LDS
  static constexpr int TABLE_FLOATS = JOINT ? N * NCODES * G : N * A * G + L;
};

template <int P>
__device__ __forceinline__ uint32_t code_at(const uint32_t* cw, int i) {
  const int off = P * i;
  const int w = off >> 5, s = off & 31;
  constexpr uint32_t mask = (1u << P) - 1u;
  if (s + P <= 32) return (cw[w] >> s) & mask;
  return __builtin_amdgcn_alignbit(cw[w + 1], cw[w], s) & mask;
}

template <int D, int BM, bool QJL, int G, bool LOGITS>
__global__ void __launch_bounds__(kScanThreads, kScanMinWavesPerEU)
decode_scan_kernel(DecodeArgs a, const uint8_t* __restrict__ codes, const __half* __restrict__ V) {
  using SS = ScanShape<D, BM, G>;
  constexpr int N = SS::N, BA = SS::BA, P = SS::P, L = SS::L, A = SS::A, NCODES = SS::NCODES;
  constexpr bool JOINT = SS::JOINT;
  constexpr int M = QJL ? D : 0;
  constexpr int NC = N * P / 32;
  constexpr int NW = NC + M / 32;
  constexpr int NQT = QJL ? (M / 4) * 16 * G : 1;
  constexpr int MERGE_FLOATS = SoftmaxPV<D, G, kScanWaves>::MERGE_FLOATS;
  constexpr int MAIN_FLOATS = SS::TABLE_FLOATS > MERGE_FLOATS ? SS::TABLE_FLOATS : MERGE_FLOATS;
  (void)BA;

  __shared__ __align__(16) float s_tab[MAIN_FLOATS];
  __shared__ __align__(16) float s_qt[NQT];
  __shared__ __align__(16) float s_p[kScanWaves][kWave][G];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const PrepLayout pl{D, N, A, M};
  const float* lv = a.codebook + size_t(h) * 2 * L;
  const float* prep0 = a.prep + (size_t(b) * a.n_q + size_t(h) * G) * pl.stride();

  const int64_t t_begin = int64_t(split) * a.tokens_per_split;
  const int64_t t_end = min<int64_t>(t_begin + a.tokens_per_split, a.n_tokens);
  const int64_t stream = b * a.n_kv + h;
  const uint8_t* cbase = codes + size_t(stream) * a.stream_bytes;
  // buffer ranges: the whole code stream, and this stream's V rows [0, t_end)
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cbase, static_cast<uint32_t>(a.stream_bytes));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(V + size_t(stream) * a.capacity * D, static_cast<uint32_t>(t_end * D * 2));
  const uint32_t nu_off = 4u * NW * static_cast<uint32_t>(a.capacity);
  const uint32_t row_bytes = 4u * static_cast<uint32_t>(a.capacity);

  SoftmaxPV<D, G, kScanWaves> sm;
  sm.init(tid);
  const int lane = sm.lane, wave = sm.wave;

  // Per chunk of 64 tokens, every load of the chunk (code words, norms, V rows)
  // is issued at its start; V is consumed only after the score, so its latency
  // hides behind the table lookups.
  uint32_t cw[NW];
  float nu = 0.f;
  typename SoftmaxPV<D, G, kScanWaves>::VChunk vc;
  // lanes past the split end read neighbouring (or, past the stream, zero)
  // words; their scores are masked
  auto load_codes = [&](int64_t c) {
    const uint32_t t4 = static_cast<uint32_t>(c + lane) * 4u;
#pragma unroll
    for (int w = 0; w < NW; ++w) cw[w] = buf_load_b32(crs, t4 + w * row_bytes);
    if constexpr (QJL) nu = half_bits_to_float(buf_load_b16(crs, nu_off + t4 / 2));
  };

  // ---- tables: one thread per (pair, query head)
  {
    float lvr[L];
#pragma unroll
    for (int r = 0; r < L; ++r) lvr[r] = lv[r];
    for (int ig = tid; ig < N * G; ig += kScanThreads) {
      const int i = ig / G, g = ig % G;
      const float* lut = prep0 + size_t(g) * pl.stride() + pl.off_lut() + i * A;
      float lt[A];
#pragma unroll
      for (int ac = 0; ac < A; ++ac) lt[ac] = lut[ac];
      if constexpr (JOINT) {
#pragma unroll
        for (int code = 0; code < NCODES; ++code)
          s_tab[(i * NCODES + code) * G + g] = lvr[code & (L - 1)] * lt[code >> BM];
      } else {
#pragma unroll
        for (int ac = 0; ac < A; ++ac) s_tab[(i * A + ac) * G + g] = lt[ac];
      }
    }
    if constexpr (!JOINT) {
      if (tid < L) s_tab[N * A * G + tid] = lvr[tid];
    }
  }
  if constexpr (QJL) {
    const float kappa = 1.2533141373155003f / float(M);  // sqrt(pi/2) / m
    for (int kg = tid; kg < (M / 4) * G; kg += kScanThreads) {
      const int k = kg / G, g = kg % G;
      const float* sq = prep0 + size_t(g) * pl.stride() + pl.off_sq() + 4 * k;
      const float q0 = sq[0], q1 = sq[1], q2 = sq[2], q3 = sq[3];
#pragma unroll
      for (int nib = 0; nib < 16; ++nib) {
        const float v = ((nib & 1) ? q0 : -q0) + ((nib & 2) ? q1 : -q1) + ((nib & 4) ? q2 : -q2) +
                        ((nib & 8) ? q3 : -q3);
        s_qt[(k * 16 + nib) * G + g] = kappa * v;
      }
    }
  }
  __syncthreads();

  // Token ranges: either the workgroup's split is shared by its wavefronts in
  // interleaved chunks, or (wave_parts) every wavefront scans a contiguous
  // partition of its own and writes its own partial state.
  int64_t c_first, c_end, c_step;
  if (a.wave_parts) {
    const int64_t tpw = a.tokens_per_split / kScanWaves;
    c_first = t_begin + int64_t(wave) * tpw;
    c_end = min<int64_t>(c_first + tpw, t_end);
    c_step = kWave;
  } else {
    c_first = t_begin + int64_t(wave) * kWave;
    c_end = t_end;
    c_step = kScanThreads;
  }
  for (int64_t c0 = c_first; c0 < c_end; c0 += c_step) {
    const int64_t t = c0 + lane;
    const bool valid = t < c_end;
    load_codes(c0);
    if constexpr (!LOGITS) sm.load_v(vc, c0, vrs);

    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      // bound the work in flight (registers): the code words of each group of
      // 8 pairs are pinned at the group's start, so neither their bit-field
      // extracts nor their table reads are hoisted above it
      if ((i % kPairGroup) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) pin_reg(s[g]);
#pragma unroll
        for (int w = (P * i) / 32; w <= (P * (i + kPairGroup) - 1) / 32 && w < NC; ++w) pin_reg(cw[w]);
      }
      const uint32_t code = code_at<P>(cw, i);
      float e[G];
      if constexpr (JOINT) {
        lds_fetch<G>(&s_tab[(i * NCODES + code) * G], e);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] += e[g];
      } else {
        const float lvl = s_tab[N * A * G + (code & (L - 1))];
        lds_fetch<G>(&s_tab[(i * A + (code >> BM)) * G], e);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(lvl, e[g], s[g]);
      }
    }
    if constexpr (QJL) {
      float qs[G];
#pragma unroll
      for (int g = 0; g < G; ++g) qs[g] = 0.f;
#pragma unroll
      for (int k = 0; k < M / 4; ++k) {
        if ((k % kPairGroup) == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) pin_reg(qs[g]);
          pin_reg(cw[NC + (k >> 3)]);
        }
        const uint32_t nib = (cw[NC + (k >> 3)] >> (4 * (k & 7))) & 15u;
        float e[G];
        lds_fetch<G>(&s_qt[(k * 16 + nib) * G], e);
#pragma unroll
        for (int g = 0; g < G; ++g) qs[g] += e[g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = fmaf(nu, qs[g], s[g]);
    }

    if constexpr (LOGITS) {
      if (valid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          a.logits[(size_t(b) * a.n_q + size_t(h) * G + g) * a.n_tokens + t] = s[g];
      }
    } else {
      sm.chunk(s, valid, a.scale_log2, vc, &s_p[wave][0][0]);
    }
  }
  if constexpr (!LOGITS) {
    const size_t row0 = size_t(b) * a.n_q + size_t(h) * G;
    if (a.wave_parts) {
      sm.finish_wave(a.partial, row0, split * kScanWaves + wave, a.n_splits * kScanWaves);
    } else {
      __syncthreads();  // tables are dead; their LDS holds the cross-wave merge
      sm.finish(s_tab, tid, a.n_splits, split, a.out, a.partial, row0);
    }
  }
}

// ------------------------------------------------------------------ merge

__global__ void __launch_bounds__(128) merge_kernel(const float* __restrict__ partial,
                                                    float* __restrict__ out, int d, int n_splits) {
  const int hq = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int nq = gridDim.x;
  const float* part = partial + (size_t(b) * nq + hq) * size_t(n_splits) * (d + 4);
  const int tid = threadIdx.x;
  float Mx = -INFINITY;
  for (int p = 0; p < n_splits; ++p) Mx = fmaxf(Mx, part[size_t(p) * (d + 4)]);
  for (int dd = tid; dd < d; dd += blockDim.x) {
    float num = 0.f, den = 0.f;
    if (Mx != -INFINITY) {
      for (int p = 0; p < n_splits; ++p) {
        const float* pp = part + size_t(p) * (d + 4);
        const float f = exp2f(pp[0] - Mx);
        num += f * pp[4 + dd];
        den += f * pp[1];
      }
    }
    out[(size_t(b) * nq + hq) * d + dd] = den > 0.f ? num / den : 0.f;
  }
}

// ------------------------------------------------------------------ dispatch

template <int D, int BM, bool QJL>
hipError_t prep_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((query_prep_kernel<D, BM, QJL>), dim3(unsigned(a.n_q), unsigned(a.n_seq)),
                     dim3(128), 0, s, a, a.S);
  return hipGetLastError();
}

template <int D, int BM, bool QJL, int G>
hipError_t scan_t(const DecodeArgs& a, bool logits_mode, hipStream_t s) {
  dim3 grid(unsigned(a.n_splits), unsigned(a.n_kv), unsigned(a.n_seq));
  if (logits_mode) {
    hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, true>), grid, dim3(kScanThreads), 0, s, a,
                       a.codes, a.V);
  } else {
    hipLaunchKernelGGL((decode_scan_kernel<D, BM, QJL, G, false>), grid, dim3(kScanThreads), 0, s,
                       a, a.codes, a.V);
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
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(n_q), unsigned(n_seq)), dim3(128), 0, s, partial,
                     out, d, n_splits);
  return hipGetLastError();
}

}  // namespace pgkq
