// The PGKQ decode scan kernel, shared by the decode of fp16 values
// (decode.hip) and of PGKQ-coded values (kv_decode.hip): analytic logits from
// the key codes, online softmax, and the weighted sum of the values.
//
// One workgroup per (token split, kv-head, sequence) builds in LDS, for the G
// query heads sharing the kv-head, a joint table indexed by a pair's (radius,
// angle) code, J[i][code][g] = level[rc] * angle_table_g[i][ac] (or level and
// angle tables separately when the joint table would not fit), and 16-entry
// tables of signed nibble sums of kappa * S_h q~ for the sketch.  Lane = token
// for the score: one coalesced dword load per code word, one LDS read per pair
// giving all G heads, one per sketch nibble.  The value path (template VB):
// VB = 0 reads fp16 values in 32-token tiles and sums them on the matrix cores
// (MfmaPV), VB > 0 reads values coded with b_main = VB (CodedPV).
#pragma once

#include <type_traits>

#include "coded_pv.hpp"
#include "mfma_pv.hpp"

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



template <int D, int BM, int G>
struct ScanShape {
  static constexpr int N = D / 2;
  static constexpr int BA = BM - 1;
  static constexpr int P = BM + BA;
  static constexpr int L = 1 << BM;
  static constexpr int A = 1 << BA;
  static constexpr int NCODES = 1 << P;
  static constexpr bool JOINT = N * NCODES * G <= 8192;  // <= 32 KiB of LDS
  // Floats per pair in the table: its block plus G floats of padding.  The
  // table is written by one thread per (pair, head); unpadded, the pairs of a
  // wavefront sit a multiple of 64 banks apart and every write is a 16-way
  // bank conflict.  With the padding consecutive pairs start G banks apart, so
  // the 64 / G pairs x G heads of a wavefront fill all 64 banks; the score's
  // reads of G consecutive floats stay aligned.
  static constexpr int PSTRIDE = (JOINT ? NCODES : A) * G + G;
  static constexpr int TABLE_FLOATS = JOINT ? N * PSTRIDE : N * PSTRIDE + L;
  static constexpr int QSTRIDE = 16 * G + G;  // floats per sketch nibble position, padded alike
};

template <int P>
__device__ __forceinline__ uint32_t code_at(const uint32_t* cw, int i) {
  const int off = P * i;
  const int w = off >> 5, s = off & 31;
  constexpr uint32_t mask = (1u << P) - 1u;
  if (s + P <= 32) return (cw[w] >> s) & mask;
  return __builtin_amdgcn_alignbit(cw[w + 1], cw[w], s) & mask;
}

template <int D, int G, int VB, bool QJL, int WAVES = kScanWaves>
using ValuePath = std::conditional_t<(VB > 0), CodedPV<D, G, WAVES, (VB > 0 ? VB : 2), QJL>,
                                     MfmaPV<D, G, WAVES>>;

// Query preparation inside the scan (FUSED): used when every (sequence,
// kv-head) stream is one workgroup, so that no preparation is repeated; the
// results are bit-identical to the separate preparation kernel (same
// operations in the same order).
template <int D, int BM, bool QJL, int G, int NT = kScanThreads>
struct FusedPrep {
  static constexpr int N = D / 2;
  static constexpr int A = 1 << (BM - 1);
  static constexpr int M = QJL ? D : 0;
  static constexpr int TPR = QJL ? NT / (QJL ? M : 1) : 1;  // threads per row of S_h
  static constexpr int CPT = D / TPR;                                  // columns per thread
  static_assert(!QJL || TPR == 2 || TPR == 4, "rows of S_h per workgroup");

  double q64[G][D];  // q~ as float64 (the raw query rows before)
  float qf[G][D];    // the gathered rows, transformed in place
  float sq[QJL ? G : 1][QJL ? M : 1];
  double2 grid[A];   // (cos, sin) of the angle grid

  static constexpr int QE = (G * D + NT - 1) / NT;

  // The global loads of the preparation, issued before anything else of the
  // workgroup (its first cache chunk among them, whose loads then queue behind
  // these): the thread's slice of a row of S_h, its query elements as stored,
  // their channel indices and signs.  All of them are unconditional buffer
  // loads (a lane past the rows, or a missing channel order, reads zero
  // through the range check), so that no branch or copy waits for one before
  // the chunk's loads are issued.
  struct Loads {
    float4 srow[QJL ? CPT / 4 : 1];
    uint32_t qlo[QE], qhi[QE];  // the element's low and high 16 bits (high: fp32 only)
    uint32_t pidx[QE];          // the channel order's entry (0 without one)
    uint32_t sgn[QE];           // the sign byte
  };
  __device__ __forceinline__ static void load(Loads& l, const DecodeArgs& a, int64_t b, int h,
                                              int tid) {
    if constexpr (QJL) {
      const float4* Sr = reinterpret_cast<const float4*>(a.S + (size_t(h) * M + tid / TPR) * D +
                                                         (tid % TPR) * CPT);
#pragma unroll
      for (int k = 0; k < CPT / 4; ++k) l.srow[k] = Sr[k];
    }
    const uint32_t esz = a.q_dtype == DT_F32 ? 4u : 2u;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(
        static_cast<const uint8_t*>(a.q) + (size_t(b) * a.n_q + size_t(h) * G) * D * esz, G * D * esz);
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(a.perm ? a.perm + size_t(h) * D : nullptr,
                                                 a.perm ? 2u * D : 0u);
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.signs + size_t(h) * D, D);
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const int e = tid + k * NT;
      const bool in = e < G * D;
      const uint32_t c = static_cast<uint32_t>(e % D);
      const uint32_t qo = in ? static_cast<uint32_t>(e) * esz : 0xFFFFFFF0u;
      l.qlo[k] = buf_load_b16(qrs, qo);
      l.qhi[k] = buf_load_b16(qrs, qo + 2);
      l.pidx[k] = buf_load_b16(prs, in ? 2 * c : 0xFFFFFFF0u);
      l.sgn[k] = buf_load_b8(srs, in ? c : 0xFFFFFFF0u);
    }
  }

  __device__ __forceinline__ void run(const Loads& l, const DecodeArgs& a, int tid) {
    {
      float* qraw = reinterpret_cast<float*>(&q64[0][0]);
      int src[QE];
      float sgn[QE];
#pragma unroll
      for (int k = 0; k < QE; ++k) {
        const int e = tid + k * NT;
        src[k] = 0;
        sgn[k] = 1.f;
        if (e < G * D) {
          const uint32_t lo = l.qlo[k];
          qraw[e] = a.q_dtype == DT_F32   ? __uint_as_float(lo | (l.qhi[k] << 16))
                    : a.q_dtype == DT_F16 ? __half2float(__ushort_as_half(static_cast<uint16_t>(lo)))
                                          : __uint_as_float(lo << 16);
          src[k] = (e / D) * D + (a.perm ? int(l.pidx[k]) : e % D);
          if (a.hadamard) sgn[k] = float(static_cast<int8_t>(l.sgn[k]));
        }
      }
      if (tid < A) {
        double sn, cs;
        sincospi(-1.0 + (2.0 * tid + 1.0) / double(A), &sn, &cs);
        grid[tid] = make_double2(cs, sn);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < QE; ++k) {
        const int e = tid + k * NT;
        if (e < G * D) (&qf[0][0])[e] = qraw[src[k]] * sgn[k];
      }
      __syncthreads();
    }
    if constexpr (G * N <= kWave) {
      // every butterfly of a level sits in wavefront 0: no workgroup barriers
      if (a.hadamard && tid < kWave) {
        for (int hh = 1; hh < D; hh <<= 1) {
          if (tid < G * N) {
            const int g = tid / N, j = tid % N;
            const int at = g * D + (j / hh) * 2 * hh + (j % hh);
            const float u = (&qf[0][0])[at], w = (&qf[0][0])[at + hh];
            (&qf[0][0])[at] = u + w;
            (&qf[0][0])[at + hh] = u - w;
          }
          wave_lds_sync();  // the next level reads what other lanes wrote
        }
      }
      __syncthreads();
    } else if (a.hadamard) {
      constexpr int BE = (G * N + NT - 1) / NT;
      for (int hh = 1; hh < D; hh <<= 1) {
        float u[BE], w[BE];
        int at[BE];
#pragma unroll
        for (int k = 0; k < BE; ++k) {
          const int e = tid + k * NT;
          at[k] = -1;
          if (e < G * N) {
            const int g = e / N, j = e % N;
            at[k] = g * D + (j / hh) * 2 * hh + (j % hh);
            u[k] = (&qf[0][0])[at[k]];
            w[k] = (&qf[0][0])[at[k] + hh];
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BE; ++k) {
          if (at[k] >= 0) {
            (&qf[0][0])[at[k]] = u[k] + w[k];
            (&qf[0][0])[at[k] + hh] = u[k] - w[k];
          }
        }
        __syncthreads();
      }
    }
    const float sc = a.hadamard ? 1.0f / sqrtf(float(D)) : 1.0f;
#pragma unroll
    for (int k = 0; k < QE; ++k) {
      const int e = tid + k * NT;
      if (e < G * D) (&q64[0][0])[e] = double((&qf[0][0])[e] * sc);
    }
    __syncthreads();
    if constexpr (QJL) {
      // S_h q~: float64 products over the thread's slice in column order, the
      // slices summed by DPP quad exchanges
      const int c0 = (tid % TPR) * CPT;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < CPT / 4; ++k) {
          float4 v = l.srow[k];
          pin_reg(v.x);  // converted where used, not all CPT doubles at once
          pin_reg(v.y);
          pin_reg(v.z);
          pin_reg(v.w);
          acc = fma(double(v.x), q64[g][c0 + 4 * k], acc);
          acc = fma(double(v.y), q64[g][c0 + 4 * k + 1], acc);
          acc = fma(double(v.z), q64[g][c0 + 4 * k + 2], acc);
          acc = fma(double(v.w), q64[g][c0 + 4 * k + 3], acc);
        }
        acc += quad_xor<1>(acc);
        if constexpr (TPR == 4) acc += quad_xor<2>(acc);
        if (tid % TPR == 0) sq[g][tid / TPR] = static_cast<float>(acc);
      }
    }
    __syncthreads();
  }

  // angle table entry of pair i, angle code ac, head g
  __device__ __forceinline__ float lut(int g, int i, int ac) const {
    return static_cast<float>(q64[g][2 * i] * grid[ac].x + q64[g][2 * i + 1] * grid[ac].y);
  }
};

template <int D, int BM, bool QJL, int G, bool LOGITS, int VB = 0, bool FUSED = false,
          int WAVES = kScanWaves>
__global__ void __launch_bounds__(WAVES * kWave, kScanMinWavesPerEU)
decode_scan_kernel(DecodeArgs a, const uint8_t* __restrict__ codes, const __half* __restrict__ V) {
  constexpr int NT = WAVES * kWave;  // threads of the workgroup
  using VP = ValuePath<D, G, VB, QJL, WAVES>;
  constexpr bool CODED_V = VB > 0;
  using SS = ScanShape<D, BM, G>;
  constexpr int N = SS::N, BA = SS::BA, P = SS::P, L = SS::L, A = SS::A, NCODES = SS::NCODES;
  constexpr bool JOINT = SS::JOINT;
  constexpr int M = QJL ? D : 0;
  constexpr int NC = N * P / 32;
  constexpr int NW = NC + M / 32;
  constexpr int PSTRIDE = SS::PSTRIDE, QSTRIDE = SS::QSTRIDE;
  constexpr int NQT = QJL ? (M / 4) * QSTRIDE : 1;
  // table lookups per scheduling group: at most 32 table floats in flight (16
  // with coded values for 8 heads, whose accumulators take more registers)
  constexpr int PG_FLOATS = CODED_V && G >= 8 ? 16 : 32;
  constexpr int PG = kPairGroup * G <= PG_FLOATS ? kPairGroup : (PG_FLOATS / G > 0 ? PG_FLOATS / G : 1);
  constexpr int MERGE_FLOATS = VP::MERGE_FLOATS;
  constexpr int MAIN_FLOATS = SS::TABLE_FLOATS > MERGE_FLOATS ? SS::TABLE_FLOATS : MERGE_FLOATS;
  (void)BA;

  __shared__ __align__(16) float s_tab[MAIN_FLOATS];
  __shared__ __align__(16) float s_qt[NQT];
  __shared__ __align__(16) float s_p[WAVES][kWave][G];
  static_assert(CODED_V || sizeof(s_p[0]) >= MfmaPV<D, G, WAVES>::P_BYTES, "weight rows");
  // coded values: per-wavefront transposition blocks and the pair table
  constexpr int VW_WORDS = CODED_V ? CodedPV<D, G, WAVES, (VB > 0 ? VB : 2), QJL>::LDS_WORDS : 1;
  constexpr int VTAB = CODED_V ? (1 << (2 * VB - 1)) : 1;
  __shared__ __align__(16) uint32_t s_vw[WAVES][VW_WORDS];
  __shared__ __align__(16) float2 s_vtab[VTAB];
  constexpr int P16 = CODED_V ? CodedPV<D, G, WAVES, (VB > 0 ? VB : 2), QJL>::P16_BYTES : 16;
  __shared__ __align__(16) unsigned char s_p16[WAVES][P16];
  using FP = FusedPrep<D, BM, QJL, (FUSED ? G : 1), NT>;
  __shared__ __align__(16) unsigned char s_fused_raw[FUSED ? sizeof(FP) : 16];
  FP& fp = *reinterpret_cast<FP*>(s_fused_raw);

  const int tid = threadIdx.x;
  // grid (kv-head, sequence, split): split-major dispatch order, so that the
  // leading (larger) splits of every stream run first
  const int split = blockIdx.z;
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;
  const PrepLayout pl{D, N, A, M};
  const float* lv = a.codebook + size_t(h) * 2 * L;
  const float* prep0 = a.prep + (size_t(b) * a.n_q + size_t(h) * G) * pl.stride();

  const bool trailing = split >= a.n_lead && a.n_lead > 0;
  const int64_t t_begin = trailing ? int64_t(a.n_lead) * a.tokens_per_split +
                                         int64_t(split - a.n_lead) * a.tail_split
                                   : int64_t(split) * a.tokens_per_split;
  const int64_t t_end =
      min<int64_t>(t_begin + (trailing ? a.tail_split : a.tokens_per_split), a.n_tokens);
  const int64_t stream = b * a.n_kv + h;
  const uint8_t* cbase = codes + size_t(stream) * a.stream_bytes;
  // buffer ranges: the whole code stream, and this stream's V rows [0, t_end)
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cbase, static_cast<uint32_t>(a.stream_bytes));
  // values: this stream's fp16 rows [0, t_end), or its whole value-code stream
  const __amdgpu_buffer_rsrc_t vrs =
      CODED_V ? make_rsrc(a.codes_v + size_t(stream) * a.stream_bytes_v,
                          static_cast<uint32_t>(a.stream_bytes_v))
              : make_rsrc(V + size_t(stream) * a.capacity * D,
                          static_cast<uint32_t>((t_end + 31) / 32 * 32 * D * 2));
  const uint32_t nu_off = 4u * NW * static_cast<uint32_t>(a.capacity);
  const uint32_t row_bytes = 4u * static_cast<uint32_t>(a.capacity);

  VP sm;
  if constexpr (CODED_V) {
    sm.init(tid, a.capacity);
  } else {
    sm.init(tid);
  }
  const int lane = sm.lane, wave = sm.wave;

  // Per chunk of 64 tokens, every load of the chunk (code words, norms, V rows)
  // is issued at its start; V is consumed only after the score, so its latency
  // hides behind the table lookups.
  uint32_t cw[NW];
  uint16_t nu_bits = 0;  // fp16 residual norm, converted where it is used
  typename VP::VChunk vc;
  // lanes past the split end read neighbouring (or, past the stream, zero)
  // words; their scores are masked
  auto load_codes = [&](int64_t c) {
    const uint32_t t4 = static_cast<uint32_t>(c + lane) * 4u;
#pragma unroll
    for (int w = 0; w < NW; ++w) cw[w] = buf_load_b32(crs, t4 + w * row_bytes);
    if constexpr (QJL) nu_bits = buf_load_b16(crs, nu_off + t4 / 2);
  };

  // the preparation's own loads first, so that they do not queue behind the
  // first chunk (loads return in order)
  typename FP::Loads fl;
  if constexpr (FUSED) FP::load(fl, a, b, h, tid);
  float lvr[L];
#pragma unroll
  for (int r = 0; r < L; ++r) lvr[r] = lv[r];

  // Token ranges: either the workgroup's split is shared by its wavefronts in
  // interleaved chunks, or (wave_parts) every wavefront scans a contiguous
  // partition of it; either way the wavefronts are merged in the workgroup.
  int64_t c_first, c_end, c_step;
  if (a.wave_parts) {
    const int64_t tpw = a.tokens_per_split / WAVES;
    c_first = t_begin + int64_t(wave) * tpw;
    c_end = min<int64_t>(c_first + tpw, t_end);
    c_step = kWave;
  } else {
    c_first = t_begin + int64_t(wave) * kWave;
    c_end = t_end;
    c_step = NT;
  }
  // With the query prepared here (one workgroup per stream, a long prologue)
  // the first chunk's loads are issued before the tables are built; with the
  // split launch this measured slower (more registers live in the prologue).
  constexpr bool EARLY = FUSED;
  auto issue = [&](int64_t c0) {
    load_codes(c0);
    if constexpr (!LOGITS) {
      if constexpr (CODED_V) {
        sm.load_v(vc, c0, vrs);
      } else {
        sm.load_v(vc, c0, vrs, t_end);
      }
    }
  };
  // unconditional (a wavefront without tokens reads zeros or unused words
  // through the buffer ranges): a branch here would make the waits of the
  // preparation below cover these loads too
  if constexpr (EARLY) issue(c_first);
  if constexpr (FUSED) fp.run(fl, a, tid);

  // ---- tables: one thread per (pair, query head)
  {
    for (int ig = tid; ig < N * G; ig += NT) {
      const int i = ig / G, g = ig % G;
      float lt[A];
      if constexpr (FUSED) {
#pragma unroll
        for (int ac = 0; ac < A; ++ac) lt[ac] = fp.lut(g < (FUSED ? G : 1) ? g : 0, i, ac);
      } else {
        const float* lut = prep0 + size_t(g) * pl.stride() + pl.off_lut() + i * A;
#pragma unroll
        for (int ac = 0; ac < A; ++ac) lt[ac] = lut[ac];
      }
      if constexpr (JOINT) {
#pragma unroll
        for (int code = 0; code < NCODES; ++code)
          s_tab[i * PSTRIDE + code * G + g] = lvr[code & (L - 1)] * lt[code >> BM];
      } else {
#pragma unroll
        for (int ac = 0; ac < A; ++ac) s_tab[i * PSTRIDE + ac * G + g] = lt[ac];
      }
    }
    if constexpr (!JOINT) {
      if (tid < L) s_tab[N * PSTRIDE + tid] = lvr[tid];
    }
  }
  if constexpr (CODED_V) {
    // (level_v[rc] cos thetahat[ac], level_v[rc] sin thetahat[ac]) per joint code
    constexpr int LV = 1 << VB, AV = 1 << (VB - 1);
    for (int e = tid; e < LV * AV; e += NT) {
      const int rc = e & (LV - 1), ac = e >> VB;
      double sn, cs;
      sincospi(-1.0 + (2.0 * ac + 1.0) / double(AV), &sn, &cs);
      const double lvv = static_cast<double>(a.codebook_v[size_t(h) * 2 * LV + rc]);
      s_vtab[e] = make_float2(static_cast<float>(lvv * cs), static_cast<float>(lvv * sn));
    }
  }
  if constexpr (QJL) {
    const float kappa = 1.2533141373155003f / float(M);  // sqrt(pi/2) / m
    for (int kg = tid; kg < (M / 4) * G; kg += NT) {
      const int k = kg / G, g = kg % G;
      const float* sq = FUSED ? &fp.sq[g < (FUSED ? G : 1) ? g : 0][QJL && FUSED ? 4 * k : 0]
                              : prep0 + size_t(g) * pl.stride() + pl.off_sq() + 4 * k;
      const float q0 = sq[0], q1 = sq[1], q2 = sq[2], q3 = sq[3];
#pragma unroll
      for (int nib = 0; nib < 16; ++nib) {
        const float v = ((nib & 1) ? q0 : -q0) + ((nib & 2) ? q1 : -q1) + ((nib & 4) ? q2 : -q2) +
                        ((nib & 8) ? q3 : -q3);
        s_qt[k * QSTRIDE + nib * G + g] = kappa * v;
      }
    }
  }
  __syncthreads();

  for (int64_t c0 = c_first; c0 < c_end; c0 += c_step) {
    const int64_t t = c0 + lane;
    const bool valid = t < c_end;
    if (!EARLY || c0 != c_first) {
      // a wavefront requesting its chunk goes ahead of the ones computing:
      // the loads are in flight sooner (131k-token stream 68-70 -> 66 us)
      __builtin_amdgcn_s_setprio(2);
      issue(c0);
      __builtin_amdgcn_s_setprio(0);
    }

    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      // bound the work in flight (registers): the code words of each group of
      // PG pairs are pinned at the group's start, so neither their bit-field
      // extracts nor their table reads are hoisted above it
      if ((i % PG) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) pin_reg(s[g]);
#pragma unroll
        for (int w = (P * i) / 32; w <= (P * (i + PG) - 1) / 32 && w < NC; ++w) pin_reg(cw[w]);
      }
      const uint32_t code = code_at<P>(cw, i);
      float e[G];
      if constexpr (JOINT) {
        lds_fetch<G>(&s_tab[i * PSTRIDE + code * G], e);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] += e[g];
      } else {
        const float lvl = s_tab[N * PSTRIDE + (code & (L - 1))];
        lds_fetch<G>(&s_tab[i * PSTRIDE + (code >> BM) * G], e);
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
        if ((k % PG) == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) pin_reg(qs[g]);
          pin_reg(cw[NC + (k >> 3)]);
        }
        const uint32_t nib = (cw[NC + (k >> 3)] >> (4 * (k & 7))) & 15u;
        float e[G];
        lds_fetch<G>(&s_qt[k * QSTRIDE + nib * G], e);
#pragma unroll
        for (int g = 0; g < G; ++g) qs[g] += e[g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = fmaf(half_bits_to_float(nu_bits), qs[g], s[g]);
    }

    if constexpr (LOGITS) {
      if (valid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          a.logits[(size_t(b) * a.n_q + size_t(h) * G + g) * a.n_tokens + t] = s[g];
      }
    } else if constexpr (CODED_V) {
      sm.chunk(s, valid, a.scale_log2, vc, &s_p[wave][0][0], &s_vw[wave][0], s_vtab, c0, c_end,
               &s_p16[wave][0]);
    } else {
      sm.mask_v(vc, c0, t_end);
      sm.chunk(s, valid, a.scale_log2, vc, &s_p[wave][0][0]);
    }
  }
  if constexpr (CODED_V && !LOGITS) {
    // partial states only (the merge kernel applies S_v^T)
    const size_t row0 = size_t(b) * a.n_q + size_t(h) * G;
    __syncthreads();  // tables are dead; their LDS holds the cross-wave merge
    sm.finish(s_tab, tid, a.partial, row0, split, a.n_splits);
  } else if constexpr (!LOGITS) {
    const size_t row0 = size_t(b) * a.n_q + size_t(h) * G;
    __syncthreads();  // tables are dead; their LDS holds the cross-wave merge
    sm.finish(s_tab, tid, a.n_splits, split, a.out, a.partial, row0);
  }
}

}  // namespace

}  // namespace pgkq
