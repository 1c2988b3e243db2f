// PGKQ key encoder for gfx950.
//
// Steps (1)-(4) of the PGKQ pipeline (EdgeLLM-Nano paper page, "PGKQ
// pipeline"): randomized Hadamard transform, adjacent-pair polar coordinates,
// Lloyd-Max radius code and uniform-grid angle code, optional QJL residual
// sketch (sign bits of S_h eps~ plus an fp16 residual norm).
//
// A workgroup (4 wavefronts) walks a run of 64-key tiles of one (sequence,
// kv-head) stream:
//   * the key tile is staged in LDS with 16-byte coalesced loads, the channel
//     order and the transform's signs applied on the way;
//   * wavefront w transforms keys 16w..16w+15.  Key j sits on lanes j, j+16,
//     j+32 and j+48; lane row q (16 lanes) starts with channels
//     [q d/4, (q+1) d/4) of its key as float64.  The Walsh-Hadamard butterflies
//     over the low channel bits run in registers.  The two high channel bits
//     live in the lane row: their butterflies use the gfx950 row-swap permutes
//     (v_permlane16_swap / v_permlane32_swap) on two registers at a time, which
//     trade a register-index bit for the lane-row bit, so such a butterfly
//     costs one swap and one add per element and every polar pair stays in one
//     lane.  For fp16 keys every partial sum is exact in float64;
//   * a radius code is read from a per-head lookup table indexed by the high
//     word of x^2 + y^2 (a bucket holds at most one threshold, settled by one
//     exact 64-bit compare); an angle cell comes from exact sign and magnitude
//     comparisons;
//   * the residual eps~ is formed in float64 against a table of level x (cos,
//     sin) pre-multiplied by a per-head power of two, so its fp16 hi/lo parts
//     need no per-element rescaling (a key far outside that scale takes a
//     rescaled path); its norm stays float64 and is rounded once to fp16;
//   * the QJL projection U = S_h E^T runs on the matrix cores with fp16 hi/lo
//     parts of both operands (three products, fp32 accumulation).  S_h rows are
//     loaded as the A operand in an order that puts 16 consecutive sketch rows
//     of one key in one lane's accumulator, so a sign word takes one funnel
//     shift per bit;
//   * codes are packed per token in LDS (one byte per pair) and stored as one
//     coalesced 256-byte row segment per code word.
#include "device_common.hpp"

namespace pgkq {

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kTilesPerBlock = 16;
constexpr int kLutMax = 256;  // radius lookup entries, the two end buckets included

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, int ES>
struct EncodeSmem {
  static constexpr int RST = D * ES + 16;  // staged key row stride in bytes (bank spread)
  static constexpr int EST = D + 8;        // fp16 residual row stride in halves
  static constexpr int CST = D / 2 + 4;    // code row stride in bytes: one byte per pair,
                                           // an odd number of dwords
  static constexpr int NLD = D * ES / 64;  // 16-byte staging loads per thread per tile
};

__device__ __forceinline__ uint32_t pack_h2(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

template <int V>
struct Tag {
  static constexpr int value = V;
};

// f(Tag<I>) for I = B .. E - 1 (compile-time indices in an unrolled body)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Tag<B>{});
    static_for<B + 1, E>(f);
  }
}

// One Walsh-Hadamard butterfly level across lane rows.  Registers r and
// r | (1 << E) (bit E of r clear) are swapped between row pairs (lane bit 4:
// ROWS = 16, lane bit 5: ROWS = 32): afterwards the lower rows hold both
// operands of element r, the upper rows both operands of element r | 1 << E,
// so every lane forms the sum and the difference of one element.  The output
// keeps the sum in register r and the difference in register r | 1 << E: the
// lane-row bit and register bit E have exchanged the channel bits they stand
// for.  Without the transform only the exchange is done.
template <int ROWS, int E, bool TRANSFORM, int CPT>
__device__ __forceinline__ void row_butterfly(double (&x)[CPT]) {
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    if (r & (1 << E)) continue;
    const int r2 = r | (1 << E);
    uint32_t alo = __double2loint(x[r]), ahi = __double2hiint(x[r]);
    uint32_t blo = __double2loint(x[r2]), bhi = __double2hiint(x[r2]);
    if constexpr (ROWS == 16) {
      const auto lo = __builtin_amdgcn_permlane16_swap(alo, blo, false, false);
      const auto hi = __builtin_amdgcn_permlane16_swap(ahi, bhi, false, false);
      alo = lo[0]; blo = lo[1]; ahi = hi[0]; bhi = hi[1];
    } else {
      const auto lo = __builtin_amdgcn_permlane32_swap(alo, blo, false, false);
      const auto hi = __builtin_amdgcn_permlane32_swap(ahi, bhi, false, false);
      alo = lo[0]; blo = lo[1]; ahi = hi[0]; bhi = hi[1];
    }
    const double a = __hiloint2double(static_cast<int>(ahi), static_cast<int>(alo));
    const double b = __hiloint2double(static_cast<int>(bhi), static_cast<int>(blo));
    x[r] = TRANSFORM ? a + b : a;
    x[r2] = TRANSFORM ? a - b : b;
  }
}

// Mid-rise angle cell of (x, y) with 2^BA cells of width 2 pi / 2^BA from -pi,
// half-open [e_a, e_a+1) counter-clockwise; theta = pi counts as -pi and the
// zero vector as theta = 0.  Exact comparisons (b_angle <= 3: every edge is a
// multiple of pi/4).  Returned shifted into place above the radius code.
template <int BA, int SHIFT>
__device__ __forceinline__ uint32_t angle_bits(double x, double y) {
  // bitwise (not short-circuit) logic keeps the comparisons as lane masks
  const bool yp = y > 0.0, yn = y < 0.0, xn = x < 0.0;
  const bool a1 = yp | (!yn & !xn);  // theta in [0, pi)
  if constexpr (BA == 1) {
    return a1 ? (1u << SHIFT) : 0u;
  } else {
    const bool xp = x > 0.0;
    // the second quarter of that half-plane: x <= 0 above the x axis, x >= 0 below
    const bool a0 = (a1 & !xp & yp) | (!a1 & !xn);
    if constexpr (BA == 2) {
      return (a1 ? (2u << SHIFT) : 0u) | (a0 ? (1u << SHIFT) : 0u);
    } else {
      // upper half of the quadrant: |y| >= |x| in quadrants 0 and 2, |y| <= |x|
      // in quadrants 1 and 3; the zero vector stays in the lower half
      const bool ge = (fabs(y) >= fabs(x)) & (yp | yn);
      const bool le = fabs(y) <= fabs(x);
      const bool sub = (a0 & le) | (!a0 & ge);
      return (a1 ? (4u << SHIFT) : 0u) | (a0 ? (2u << SHIFT) : 0u) | (sub ? (1u << SHIFT) : 0u);
    }
  }
}

// v_med3_i32 with the lower bound wave-uniform (a scalar operand) and the upper
// bound in a vector register: one instruction for the clamp of a table index
__device__ __forceinline__ int clamp_med3(int v, int lo, int hi) {
  int r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(lo), "v"(hi));
  return r;
}

// ES = bytes per key element (2: fp16 keys, 4: fp32 keys); HT: randomized
// Hadamard transform on (else the identity, the "without Hadamard" ablation)
template <int D, int BM, bool QJL, int ES, bool HT>
__global__ void __launch_bounds__(kThreads, 2)
encode_kernel(EncodeArgs a, const float* __restrict__ S, const uint8_t* __restrict__ K,
              uint8_t* __restrict__ codes) {
  using SM = EncodeSmem<D, ES>;
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int P = BM + BA;
  constexpr int L = 1 << BM;
  constexpr int NC = N * P / 32;
  constexpr int M = QJL ? D : 0;
  constexpr int NSW = M / 32;
  constexpr int NW = NC + NSW;
  constexpr int CPT = D / 4;          // channels per lane in the transform phase
  constexpr int LB = CPT == 32 ? 5 : 4;  // log2(CPT)
  constexpr int RL = CPT / 8;         // pairs per contiguous run after the row butterflies
  constexpr int RST = SM::RST, EST = SM::EST, CST = SM::CST, NLD = SM::NLD;
  constexpr int EPL = 16 / ES;        // key elements per 16-byte load
  constexpr int KSTEPS = D / 16;      // MFMA contraction steps
  // D = 128: wave w owns sketch rows [32w, 32w+32) for both 32-key halves.
  // D = 64:  wave w owns rows [32 (w&1), +32) for keys [32 (w>>1), +32).
  constexpr int MT_PER_WAVE = D == 128 ? 2 : 1;
  constexpr bool USE_LUT = BM >= 3;   // at b_main = 2 three compares are cheaper
  static_assert(N % 32 == 0, "pairs must fill whole words");
  static_assert(CPT * ES % 16 == 0, "a lane's key slice is whole 16-byte vectors");
  static_assert(RL >= 2, "a run holds whole pairs");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;

  __shared__ __align__(16) uint4 s_lut[USE_LUT ? kLutMax : 1];
  __shared__ double2 s_LCS[QJL ? (1 << P) : 1];  // level x (cos, sin) x 2^E_h by joint code
  __shared__ int s_inv[D];
  __shared__ __align__(16) unsigned char s_key[kTile * RST];
  __shared__ __align__(16) _Float16 s_E[QJL ? 2 * kTile * EST : 1];
  __shared__ __align__(16) uint8_t s_code[kTile * CST];
  __shared__ uint16_t s_nu[kTile];
  __shared__ double s_T2s[16];  // sorted squared thresholds (+inf padded)
  __shared__ int s_meta[2];

  // ---- per-head metadata
  const float* cb = a.codebook + size_t(h) * 2 * L;
  const double tscale = HT ? double(D) : 1.0;  // X = sqrt(d) k~ under the transform
  // The radius code counts the thresholds below r.  A negative threshold is
  // below every radius, a NaN or +inf one below none; the others compare as
  // squares in the units of X (tscale T^2 is exact: a 24-bit significand
  // squared times a power of two).  Thread 0 sorts those squares into s_T2s
  // (padded with +inf), so that any table, ordered or not, is counted exactly.
  constexpr int NT = L - 1;                 // thresholds
  constexpr int NTP = NT < 4 ? 4 : (NT < 8 ? 8 : 16);  // padded to a power of two
  if (tid == 0) {
    int neg = 0, nv = 0;
    for (int i = 0; i < NT; ++i) {
      const double t = double(cb[L + i]);
      if (t < 0.0) {
        ++neg;
      } else if (t < __longlong_as_double(0x7FF0000000000000ll)) {
        const double t2 = tscale * t * t;
        int j = nv++;
        while (j > 0 && s_T2s[j - 1] > t2) { s_T2s[j] = s_T2s[j - 1]; --j; }
        s_T2s[j] = t2;
      }
    }
    for (int j = nv; j < NTP; ++j) s_T2s[j] = __longlong_as_double(0x7FF0000000000000ll);
    s_meta[0] = neg;
    s_meta[1] = nv;
  }
  __syncthreads();
  const int n_neg = __builtin_amdgcn_readfirstlane(s_meta[0]);
  const int n_valid = __builtin_amdgcn_readfirstlane(s_meta[1]);
  double T2r[NT];  // sorted; wave-uniform (scalar registers) where the chain uses them
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const double t2 = s_T2s[i];
    T2r[i] = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(t2)),
                              __builtin_amdgcn_readfirstlane(__double2loint(t2)));
  }
  // radius lookup over the sorted squares: bucket key = high word >> (20 - mb);
  // usable when they are distinct, fall in distinct buckets and span at most
  // kLutMax - 2 buckets
  int lut_shift = 0, lut_lo = 0, lut_hi = 0;
  bool lut_ok = false;
  if constexpr (USE_LUT) {
    bool sane = n_valid >= 1;
#pragma unroll
    for (int i = 1; i < NT; ++i) sane = sane && (i >= n_valid || T2r[i] > T2r[i - 1]);
    for (int mb = 2; sane && mb <= 12 && !lut_ok; ++mb) {
      const int sh = 20 - mb;
      bool distinct = true;
      int k1 = __double2hiint(T2r[0]) >> sh;
#pragma unroll
      for (int i = 1; i < NT; ++i) {
        if (i < n_valid) {
          const int ki = __double2hiint(T2r[i]) >> sh;
          distinct = distinct && ki > k1;
          k1 = ki;
        }
      }
      const int k0 = __double2hiint(T2r[0]) >> sh;
      if (distinct && k1 - k0 + 3 <= kLutMax) {
        lut_ok = true;
        lut_shift = sh;
        lut_lo = k0 - 1;   // every key below the first threshold's bucket
        lut_hi = k1 + 1;   // every key above the last threshold's bucket
      }
    }
    lut_ok = __builtin_amdgcn_readfirstlane(lut_ok ? 1 : 0) != 0;
    lut_shift = __builtin_amdgcn_readfirstlane(lut_shift);
    lut_lo = __builtin_amdgcn_readfirstlane(lut_lo);
    lut_hi = __builtin_amdgcn_readfirstlane(lut_hi);
    if (lut_ok) {
      // entry: the threshold square in the bucket (never exceeded if none) and
      // the count below the bucket; the first and last entries take every key
      // below / above the thresholds' buckets
      for (int e = tid; e <= lut_hi - lut_lo; e += kThreads) {
        const int key = lut_lo + e;
        uint32_t below = 0;
        uint64_t thr = ~0ull;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i < n_valid) {
            const int ki = __double2hiint(T2r[i]) >> lut_shift;
            below += (e == lut_hi - lut_lo || ki < key) ? 1u : 0u;
            if (ki == key && e != 0 && e != lut_hi - lut_lo)
              thr = static_cast<uint64_t>(__double_as_longlong(T2r[i]));
          }
        }
        if (e == 0) below = 0;
        s_lut[e] = make_uint4(static_cast<uint32_t>(thr), static_cast<uint32_t>(thr >> 32),
                              below + static_cast<uint32_t>(n_neg), 0u);
      }
    }
  }
  // lookup addressing: the entry of bucket key is lut_base[key] (the clamp bound
  // held in a vector register, so that the clamp is one three-operand median)
  const uint4* lut_base = s_lut - lut_lo;
  int lut_hi_v = lut_hi;
  asm volatile("" : "+v"(lut_hi_v));
  // per-head power of two for the residual: ||eps~|| is about d/2 levels of
  // 0.2 of the top level, brought near 2^7 (fp16 hi/lo parts then carry it to
  // 2^-22 relative without overflow)
  int eh = 0;
  {
    const double top = double(cb[L - 1]);
    if (top > 0.0 && top < 1e300) eh = 7 - ilogb(top * 0.2 * sqrt(double(N)));
    eh = __builtin_amdgcn_readfirstlane(min(60, max(-60, eh)));
  }
  if constexpr (QJL) {
    for (int e = tid; e < (1 << P); e += kThreads) {
      const int rc = e & (L - 1), ac = e >> BM;
      double sn, cs;
      sincospi(-1.0 + (2.0 * ac + 1.0) / double(1 << BA), &sn, &cs);
      const double lv = double(cb[rc]);
      s_LCS[e] = make_double2(ldexp(lv * cs, eh), ldexp(lv * sn, eh));
    }
  }
  // inverse of the channel order: input channel c' lands at position s_inv[c']
  for (int p = tid; p < D; p += kThreads) s_inv[a.perm ? int(a.perm[size_t(h) * D + p]) : p] = p;

  // ---- S_h as MFMA A operands (hi and lo), kept in registers for every tile.
  //      MFMA row i = 8 a + 4 hf + bb (the accumulator row of element r = 4 a + bb
  //      in lane half hf) is loaded with sketch row 16 hf + 4 a + bb of the
  //      wave's 32-row block, so lane l's accumulator holds sketch rows
  //      16 (l/32) + r, r = 0..15, of key l % 32
  const int nt = D == 128 ? wave : (wave & 1);
  const int mt0 = D == 128 ? 0 : (wave >> 1);
  half8 sah[QJL ? KSTEPS : 1], sal[QJL ? KSTEPS : 1];
  if constexpr (QJL) {
    const int i = lane & 31;
    const int srow_in_block = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const float* srow = S + (size_t(h) * M + 32 * nt + srow_in_block) * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const float4 u0 = *reinterpret_cast<const float4*>(srow + 16 * ks);
      const float4 u1 = *reinterpret_cast<const float4*>(srow + 16 * ks + 4);
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const _Float16 hi = static_cast<_Float16>(v[jj]);
        sah[ks][jj] = hi;
        sal[ks][jj] = static_cast<_Float16>(v[jj] - static_cast<float>(hi));  // difference exact
      }
    }
  }
  __syncthreads();

  // ---- staging map: this thread's 16-byte loads cover input channels
  //      [cin, cin + EPL) of key rows rin + (4096 / (D ES)) k; their positions
  //      in the reordered key and the sign flips of the transform
  const int cin = (tid * 16) % (D * ES) / ES;
  const int rin = (tid * 16) / (D * ES);
  constexpr int ROWS_PER_LOAD = 4096 / (D * ES);
  uint32_t dst[EPL];   // byte offset in s_key of element e in this thread's first row
  uint32_t flip = 0;   // bit e: negate element e
  const bool identity = a.perm == nullptr;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int pe = s_inv[cin + e];
    dst[e] = static_cast<uint32_t>(rin * RST + pe * ES);
    if (HT && a.signs[size_t(h) * D + pe] < 0) flip |= 1u << e;
  }
  u32x4 fmask;  // sign mask for the in-order (identity) staging path
  if constexpr (ES == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      fmask[w] = ((flip >> (2 * w)) & 1 ? 0x8000u : 0u) | ((flip >> (2 * w + 1)) & 1 ? 0x80000000u : 0u);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) fmask[w] = (flip >> w) & 1 ? 0x80000000u : 0u;
  }

  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  const int64_t tile0 = int64_t(blockIdx.x) * kTilesPerBlock;
  const int64_t tile1 = min<int64_t>(tile0 + kTilesPerBlock, n_tiles);
  const double inv_s = ldexp(HT ? 1.0 / sqrt(double(D)) : 1.0, eh);
  uint8_t* base = codes + (size_t(b) * a.n_kv + h) * a.stream_bytes;
  uint32_t* rows = reinterpret_cast<uint32_t*>(base);
  const __amdgpu_buffer_rsrc_t codes_rsrc = make_rsrc(base, static_cast<uint32_t>(a.stream_bytes));
  const uint8_t* kstream = K + (size_t(b) * a.n_kv + h) * a.n_tokens * size_t(D) * ES;

  // transform-phase lane roles: key kj of the tile, lane row q
  const int kj = 16 * wave + (lane & 15);
  const int q = lane >> 4;

  // The tile loop, once per radius-code mode: the mode is fixed per workgroup,
  // and two separate loops keep the register allocation of each to itself.
  auto run_tiles = [&](auto mode) {
    constexpr int MODE = decltype(mode)::value;
    u32x4 kr[NLD];
    auto load_tile = [&](int64_t tile) {
      const uint8_t* src = kstream + tile * kTile * size_t(D) * ES;
      const int valid_bytes = static_cast<int>(min<int64_t>(kTile, a.n_tokens - tile * kTile)) * D * ES;
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int off = tid * 16 + k * 4096;
        kr[k] = u32x4{0u, 0u, 0u, 0u};
        if (off < valid_bytes) kr[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
      }
    };
    auto stage = [&]() {
        // ---- stage the prefetched keys into LDS in the transform's channel order,
        //      signs applied; then request the next tile
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
          const u32x4 v = kr[k] ^ fmask;
          if (identity) {
            *reinterpret_cast<u32x4*>(s_key + (rin + ROWS_PER_LOAD * k) * RST + cin * ES) = v;
          } else {
            // scatter into the reordered positions; the row offset of load k is a
            // compile-time constant folded into the LDS instruction
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              unsigned char* pdst = s_key + dst[e] + ROWS_PER_LOAD * k * RST;
              if constexpr (ES == 2) {
                *reinterpret_cast<uint16_t*>(pdst) = static_cast<uint16_t>((e & 1) ? (v[e >> 1] >> 16) : v[e >> 1]);
              } else {
                *reinterpret_cast<uint32_t*>(pdst) = v[e];
              }
            }
          }
        }
    };
    // ---- QJL projection of a finished tile on the matrix cores: U = S_h E^T,
    //      lane l holds sketch rows 32 nt + 16 (l/32) + r of key 32 mt + l % 32.
    //      One group = the three hi/lo products of one contraction step of one
    //      32-key half; sign words by funnel shifts (bit r = 1 iff u >= 0),
    //      stored by the lanes that hold them.
    constexpr int NGRP = MT_PER_WAVE * KSTEPS;
    auto e_operands = [&](int g, half8& eh8, half8& el8) {
      const int key = 32 * (mt0 + g / KSTEPS) + (lane & 31);
      const int off = key * EST + 16 * (g % KSTEPS) + 8 * (lane >> 5);
      eh8 = *reinterpret_cast<const half8*>(s_E + off);
      el8 = *reinterpret_cast<const half8*>(s_E + kTile * EST + off);
    };
    auto sign_words = [&](const f32x16& acc, int mi, int64_t pt0, int pvalid) {
      const int key = 32 * (mt0 + mi) + (lane & 31);
      uint32_t neg = 0;  // bit r: u < 0 (the sign bit of the fp32 sum)
#pragma unroll
      for (int r = 15; r >= 0; --r) neg = __builtin_amdgcn_alignbit(neg, __float_as_uint(acc[r]), 31);
      const uint32_t upper = static_cast<uint32_t>(__shfl_xor(static_cast<int>(neg), 32));
      const bool ok = lane < 32 && key < pvalid;
      const uint32_t off = ok ? static_cast<uint32_t>(4 * ((NC + nt) * a.capacity + a.token_offset + pt0 + key))
                              : 0xFFFFFFFFu;
      buf_store_b32(codes_rsrc, off, ~(neg | (upper << 16)));
    };

    // Software pipeline over the workgroup's tiles, two barriers per tile:
    //   [transform of tile t (registers, s_code, s_nu), interleaved with the
    //    projection of tile t-1 from s_E]  barrier
    //   [residual split of tile t into s_E; code words of tile t stored;
    //    keys of tile t+1 staged into s_key]  barrier
    // so the matrix-core work of one tile overlaps the vector work of the next.
    if (tile0 < tile1) {
      load_tile(tile0);
      stage();
      if (tile0 + 1 < tile1) load_tile(tile0 + 1);
    }
    __syncthreads();
    for (int64_t tile = tile0; tile < tile1; ++tile) {
      const int64_t t0 = tile * kTile;
      const int nvalid = static_cast<int>(min<int64_t>(kTile, a.n_tokens - t0));

      // ---- transform phase: lane row q starts with channels [q CPT, q CPT + CPT)
      //      of key kj (reordered, signs flipped).  Its first part (conversion
      //      to float64 and the in-register butterflies) is cut into pieces that
      //      are issued between the matrix-core groups of the previous tile's
      //      projection, so that the two overlap.
      constexpr int NV = CPT * ES / 16;              // 16-byte LDS vectors per lane
      constexpr int NPIECE = NV + (HT ? 2 * LB : 0); // conversions, half butterfly levels
      u32x4 raw[NV];
      {
        const unsigned char* src = s_key + kj * RST + q * CPT * ES;
#pragma unroll
        for (int v = 0; v < NV; ++v) raw[v] = *reinterpret_cast<const u32x4*>(src + 16 * v);
      }
      double x[CPT];
      auto piece = [&](auto pc) {
        constexpr int c = decltype(pc)::value;
        if constexpr (c < NV) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (ES == 2) {
              x[c * 8 + 2 * w] = double(__half2float(__ushort_as_half(static_cast<uint16_t>(raw[c][w]))));
              x[c * 8 + 2 * w + 1] = double(__half2float(__ushort_as_half(static_cast<uint16_t>(raw[c][w] >> 16))));
            } else {
              x[c * 4 + w] = double(__uint_as_float(raw[c][w]));
            }
          }
        } else {
          // half of the butterflies of level (c - NV) / 2 (stride 2^level)
          constexpr int hh = 1 << ((c - NV) / 2);
          constexpr int half = (c - NV) % 2;
          int n = 0;
#pragma unroll
          for (int r = 0; r < CPT; ++r) {
            if ((r & hh) == 0) {
              if (n / (CPT / 4) == half) {
                const double u = x[r], w = x[r + hh];
                x[r] = u + w;
                x[r + hh] = u - w;
              }
              ++n;
            }
          }
        }
      };
      if constexpr (QJL) {
        // the projection of tile t - 1 (nothing to store before the first tile)
        const int64_t pt0 = (tile - 1) * kTile;
        const int pvalid = tile > tile0 ? static_cast<int>(min<int64_t>(kTile, a.n_tokens - pt0)) : 0;
        f32x16 acc = {};
        half8 eh8, el8, nh8, nl8;
        e_operands(0, eh8, el8);
        static_for<0, NGRP>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          constexpr int ks = g % KSTEPS;
          if constexpr (g + 1 < NGRP) e_operands(g + 1, nh8, nl8);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sah[ks], eh8, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sah[ks], el8, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sal[ks], eh8, acc, 0, 0, 0);
          static_for<(g * NPIECE) / NGRP, ((g + 1) * NPIECE) / NGRP>(piece);
          if constexpr (ks == KSTEPS - 1) {
            sign_words(acc, g / KSTEPS, pt0, pvalid);
            acc = f32x16{};
          }
          eh8 = nh8;
          el8 = nl8;
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
        static_for<0, NPIECE>(piece);
      }
      // the two high channel bits: lane-row butterflies.  Afterwards register s of
      // lane row q holds channel (s & (CPT/4 - 1)) | q << (LB - 2) | (s >> (LB - 2)) << LB,
      // so pairs stay in registers (2s, 2s+1) and register run k (2 RL registers)
      // is channels [8 RL k + 2 RL q, +2 RL): pairs [4 RL k + RL q, +RL)
      row_butterfly<16, LB - 2, HT>(x);
      row_butterfly<32, LB - 1, HT>(x);

      // ---- polar codes and residual.  The radius code: MODE 1 the bucket
      //      lookup, MODE 0 the compare chain (b_main = 2) or, for a table the
      //      lookup cannot bucket, a binary search of the sorted squares.
      double ss = 0.0;
      uint32_t run[4];
      // pairs in groups of four, each step for the whole group before the next
      // (the table reads of a group are in flight together)
      constexpr int GP = 4;
#pragma unroll
      for (int g = 0; g < CPT / 2; g += GP) {
        double r2[GP];
        uint32_t code[GP];
#pragma unroll
        for (int u = 0; u < GP; ++u) {
          const double xx = x[2 * (g + u)], yy = x[2 * (g + u) + 1];
          r2[u] = fma(xx, xx, yy * yy);
        }
        uint32_t rc[GP];
        if constexpr (MODE == 1) {
          uint4 e[GP];
#pragma unroll
          for (int u = 0; u < GP; ++u) {
            int key = static_cast<int>(static_cast<uint32_t>(__double2hiint(r2[u])) >> lut_shift);
            key = clamp_med3(key, lut_lo, lut_hi_v);
            e[u] = lut_base[key];
          }
#pragma unroll
          for (int u = 0; u < GP; ++u) {
            const uint64_t bits = static_cast<uint64_t>(__double_as_longlong(r2[u]));
            const uint64_t thr = (static_cast<uint64_t>(e[u].y) << 32) | e[u].x;
            rc[u] = e[u].z + (bits > thr ? 1u : 0u);
          }
        } else if constexpr (USE_LUT) {
#pragma unroll
          for (int u = 0; u < GP; ++u) {
            int pos = 0;
#pragma unroll
            for (int step = NTP / 2; step >= 1; step >>= 1)
              if (s_T2s[pos + step - 1] < r2[u]) pos += step;
            rc[u] = static_cast<uint32_t>(n_neg + pos);
          }
        } else {
#pragma unroll
          for (int u = 0; u < GP; ++u) {
            rc[u] = static_cast<uint32_t>(n_neg);
#pragma unroll
            for (int i = 0; i < NT; ++i) rc[u] += T2r[i] < r2[u] ? 1u : 0u;
          }
        }
#pragma unroll
        for (int u = 0; u < GP; ++u) {
          const int p = g + u;
          code[u] = rc[u] | angle_bits<BA, BM>(x[2 * p], x[2 * p + 1]);
          const int k = p / RL, i = p % RL;
          run[k] = i == 0 ? code[u] : (run[k] | (code[u] << (8 * i)));
        }
        if constexpr (QJL) {
          double2 lcs[GP];
#pragma unroll
          for (int u = 0; u < GP; ++u) lcs[u] = s_LCS[code[u]];
#pragma unroll
          for (int u = 0; u < GP; ++u) {
            const int p = g + u;
            const double ex = fma(x[2 * p], inv_s, -lcs[u].x);
            const double ey = fma(x[2 * p + 1], inv_s, -lcs[u].y);
            x[2 * p] = ex;
            x[2 * p + 1] = ey;
            ss = fma(ex, ex, ss);
            ss = fma(ey, ey, ss);
          }
        }
        sched_fence();
      }
      // runs of RL pair codes: pairs [4 RL k + RL q, +RL) of token kj
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint8_t* dstc = s_code + kj * CST + 4 * RL * k + RL * q;
        if constexpr (RL == 4) *reinterpret_cast<uint32_t*>(dstc) = run[k];
        else *reinterpret_cast<uint16_t*>(dstc) = static_cast<uint16_t>(run[k]);
      }

      if constexpr (QJL) {
        // the key's residual energy over its four lane rows (units 4^E_h)
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        if (q == 0) s_nu[kj] = f64_to_f16_rne_sat_nonneg(ldexp(sqrt(ss), -eh));
        // fp16 hi/lo parts of eps~ 2^E_h: exact to 2^-22 of ||eps~|| when the norm
        // lies in [1/2, 2^14]; a key outside takes its own power of two
        const bool in_range = ss >= 0.25 && ss <= 268435456.0;
        if (__ballot(!in_range) != 0) {
          // wave-uniform and rare: keys whose residual is far from the head's
          // scale are brought to ||eps~|| in [1, 2) by their own power of two
          int ek = 0;
          if (!in_range && ss > 0.0 && ss < __longlong_as_double(0x7FF0000000000000ll)) ek = -ilogb(sqrt(ss));
#pragma unroll
          for (int r = 0; r < CPT; ++r) x[r] = ldexp(x[r], ek);
        }
      }
      __syncthreads();

      if constexpr (QJL) {
        // lo = fp16(x - hi), the difference exact in fp32; the multiplier is -1
        // kept opaque so that the difference is formed by a mixed-precision FMA
        // straight from the fp16 hi part
        float neg1 = -1.0f;
        pin_reg(neg1);
        _Float16* Ehi = s_E + kj * EST;
        _Float16* Elo = s_E + kTile * EST + kj * EST;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hq[RL], lq[RL];
#pragma unroll
          for (int e = 0; e < RL; ++e) {
            const f32x2 xf = {static_cast<float>(x[2 * RL * k + 2 * e]),
                              static_cast<float>(x[2 * RL * k + 2 * e + 1])};
            const f16x2 hv = __builtin_convertvector(xf, f16x2);
            const f32x2 lf = {__builtin_fmaf(static_cast<float>(hv[0]), neg1, xf[0]),
                              __builtin_fmaf(static_cast<float>(hv[1]), neg1, xf[1])};
            hq[e] = pack_h2(hv);
            lq[e] = pack_h2(__builtin_convertvector(lf, f16x2));
          }
          const int c0 = 8 * RL * k + 2 * RL * q;  // first channel of run k
          if constexpr (RL == 4) {
            *reinterpret_cast<u32x4*>(Ehi + c0) = u32x4{hq[0], hq[1], hq[2], hq[3]};
            *reinterpret_cast<u32x4*>(Elo + c0) = u32x4{lq[0], lq[1], lq[2], lq[3]};
          } else {
            *reinterpret_cast<uint2*>(Ehi + c0) = make_uint2(hq[0], hq[1]);
            *reinterpret_cast<uint2*>(Elo + c0) = make_uint2(lq[0], lq[1]);
          }
        }
      }

      // ---- code words and residual norms: word w of token `lane` goes to row
      //      w, slot token_offset + t0 + lane (wavefront w % 4 builds it)
      const int64_t slot = a.token_offset + t0 + lane;
      const bool live = lane < nvalid;
      const uint32_t* crow = reinterpret_cast<const uint32_t*>(s_code + lane * CST);
#pragma unroll
      for (int w = 0; w < NC; ++w) {
        if ((w & 3) == wave) {
          uint32_t word = 0;
#pragma unroll
          for (int i = (32 * w) / P; i <= (32 * w + 31) / P && i < N; ++i) {
            const uint32_t code = (crow[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            const int o = P * i - 32 * w;
            word |= o >= 0 ? (code << o) : (code >> (-o));
          }
          if (live) __builtin_nontemporal_store(word, rows + size_t(w) * a.capacity + slot);
        }
      }
      if constexpr (QJL) {
        if (((NC + NSW) & 3) == wave && live) {
          uint16_t* nu = reinterpret_cast<uint16_t*>(base + size_t(4) * NW * a.capacity);
          __builtin_nontemporal_store(s_nu[lane], nu + slot);
        }
      }


      if (tile + 1 < tile1) {
        stage();
        if (tile + 2 < tile1) load_tile(tile + 2);
      }
      __syncthreads();
    }
    if constexpr (QJL) {
      // the projection of the last tile
      if (tile0 < tile1) {
        const int64_t pt0 = (tile1 - 1) * kTile;
        const int pvalid = static_cast<int>(min<int64_t>(kTile, a.n_tokens - pt0));
        static_for<0, MT_PER_WAVE>([&](auto mc) {
          constexpr int mi = decltype(mc)::value;
          f32x16 acc = {};
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            half8 eh8, el8;
            e_operands(mi * KSTEPS + ks, eh8, el8);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sah[ks], eh8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sah[ks], el8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sal[ks], eh8, acc, 0, 0, 0);
          }
          sign_words(acc, mi, pt0, pvalid);
        });
      }
    }
  };
  if (USE_LUT && lut_ok) run_tiles(Tag<1>{});
  else run_tiles(Tag<0>{});
}

template <int D, int BM, bool QJL, int ES>
void launch_encode_e(const EncodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.hadamard) {
    hipLaunchKernelGGL((encode_kernel<D, BM, QJL, ES, true>), grid, dim3(kThreads), 0, s, a, a.S,
                       static_cast<const uint8_t*>(a.K), a.codes);
  } else {
    hipLaunchKernelGGL((encode_kernel<D, BM, QJL, ES, false>), grid, dim3(kThreads), 0, s, a, a.S,
                       static_cast<const uint8_t*>(a.K), a.codes);
  }
}

template <int D, int BM, bool QJL>
hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t s) {
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  dim3 grid(static_cast<unsigned>((n_tiles + kTilesPerBlock - 1) / kTilesPerBlock),
            static_cast<unsigned>(a.n_kv), static_cast<unsigned>(a.n_seq));
  if (a.k_dtype == DT_F32) launch_encode_e<D, BM, QJL, 4>(a, grid, s);
  else launch_encode_e<D, BM, QJL, 2>(a, grid, s);
  return hipGetLastError();
}

template <int D>
hipError_t launch_encode_d(const Geometry& g, const EncodeArgs& a, hipStream_t s) {
  const bool q = g.m != 0;
  switch (g.bm) {
    case 2: return q ? launch_encode_t<D, 2, true>(a, s) : launch_encode_t<D, 2, false>(a, s);
    case 3: return q ? launch_encode_t<D, 3, true>(a, s) : launch_encode_t<D, 3, false>(a, s);
    case 4: return q ? launch_encode_t<D, 4, true>(a, s) : launch_encode_t<D, 4, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_encode(const Geometry& g, const EncodeArgs& a, hipStream_t s) {
  if (g.d == 64) return launch_encode_d<64>(g, a, s);
  if (g.d == 128) return launch_encode_d<128>(g, a, s);
  return hipErrorInvalidValue;
}

}  // namespace pgkq
