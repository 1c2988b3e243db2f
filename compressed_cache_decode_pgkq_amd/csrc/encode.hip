// PGKQ key encoder for gfx950.
//
// Steps (1)-(4) of the PGKQ pipeline (EdgeLLM-Nano paper page, "PGKQ
// pipeline"): randomized Hadamard transform, adjacent-pair polar coordinates,
// Lloyd-Max radius code and uniform-grid angle code, optional QJL residual
// sketch (sign bits of S_h eps~ plus an fp16 residual norm).
//
// A workgroup (4 wavefronts) walks a run of 64-key tiles of one (sequence,
// kv-head) stream:
//   * the key tile is staged in LDS with 16-byte coalesced loads;
//   * each key is spread over 4 adjacent lanes (d/4 channels each) as float64;
//     the Walsh-Hadamard butterflies run in registers for the low channel bits
//     and as DPP quad permutations for the two high bits.  For fp16 keys every
//     partial sum is exact in float64, so the radius and angle decisions are
//     taken on the exact transform (comparisons of x, y, |x|, |y| and of
//     x^2 + y^2 against d T_j^2);
//   * the residual eps~ and its norm stay in float64; the norm is rounded once
//     to fp16;
//   * the QJL projection U = E S_h^T (64 keys x m rows, contraction over d) runs
//     on the matrix cores: each operand is split into an fp16 high part and an
//     fp16 remainder (the residual row first scaled by a power of two, which
//     leaves every sign unchanged), and hi*hi + hi*lo + lo*hi accumulate in
//     fp32 (about 22 significant bits per product).  S_h is split once per
//     workgroup and kept in registers; each wavefront owns 32 sketch rows, so
//     one ballot over a 32x32 accumulator block yields the sign words of 32
//     keys;
//   * codes are packed per token in LDS and stored as one coalesced 256-byte
//     row segment per code word.
#include "device_common.hpp"

namespace pgkq {

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kTilesPerBlock = 16;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D, int ES>
struct EncodeSmem {
  static constexpr int RST = D * ES + 16;  // key row stride in bytes (bank spread)
  static constexpr int EST = D + 8;        // fp16 residual row stride in halves
  static constexpr int CST = D / 2 + 16;   // code row stride in bytes (16-byte aligned)
  static constexpr int NLD = D * ES / 64;  // 16-byte loads per thread per key tile
};

// x ~ hi + lo with fp16 parts: the fp32 rounding of x costs 2^-24 relative,
// the fp16 remainder about 2^-22; hi - xf is exact in fp32
__device__ __forceinline__ void split_f16(double x, _Float16& hi, _Float16& lo) {
  float xf = static_cast<float>(x);
  // keep the fp32 value: otherwise the two narrowings fold into one float64 ->
  // fp16 conversion, which the hardware lacks and which costs ~30 instructions
  pin_reg(xf);
  hi = static_cast<_Float16>(xf);
  lo = static_cast<_Float16>(xf - static_cast<float>(hi));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// split_f16 of x0 2^e and x1 2^e, returned as packed fp16 pairs.  The
// power-of-two scale is applied after the fp32 rounding (an exponent add at
// fp32 rate instead of a float64 product; equal unless x 2^e is below the fp32
// normal range, where both give fp16 parts of 0); the round-to-nearest-even
// conversions to fp16 take two elements per instruction.
__device__ __forceinline__ void split2_f16_scaled(double x0, double x1, int e, uint32_t& hi2, uint32_t& lo2) {
  float f0 = static_cast<float>(x0), f1 = static_cast<float>(x1);
  pin_reg(f0);
  pin_reg(f1);
  const f32x2 xf = {ldexpf(f0, e), ldexpf(f1, e)};
  const f16x2 h = __builtin_convertvector(xf, f16x2);
  const f32x2 l = xf - __builtin_convertvector(h, f32x2);  // exact
  hi2 = __builtin_bit_cast(uint32_t, h);
  lo2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(l, f16x2));
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// ES = bytes per key element (2: fp16 keys, 4: fp32 keys)
template <int D, int BM, bool QJL, int ES>
__global__ void __launch_bounds__(kThreads, 2)
encode_kernel(EncodeArgs a, const float* __restrict__ S, const uint8_t* __restrict__ K,
              uint8_t* __restrict__ codes) {
  using SM = EncodeSmem<D, ES>;
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int P = BM + BA;
  constexpr int L = 1 << BM;
  constexpr int A = 1 << BA;
  constexpr int NC = N * P / 32;
  constexpr int M = QJL ? D : 0;
  constexpr int NSW = M / 32;
  constexpr int NW = NC + NSW;
  constexpr int CPT = D / 4;          // channels per lane in the transform phase
  constexpr int RST = SM::RST, EST = SM::EST, CST = SM::CST, NLD = SM::NLD;
  constexpr int EPL = 16 / ES;        // key elements per 16-byte load
  constexpr int KSTEPS = D / 16;      // MFMA contraction steps
  // D = 128: wave w owns sketch rows [32w, 32w+32) for both 32-key halves.
  // D = 64:  wave w owns rows [32 (w&1), +32) for keys [32 (w>>1), +32).
  constexpr int MT_PER_WAVE = D == 128 ? 2 : 1;
  static_assert(N % 32 == 0, "pairs must fill whole words");
  static_assert(CPT * ES % 16 == 0, "a lane's key slice is whole 16-byte vectors");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;

  __shared__ double s_T2[L];
  __shared__ double2 s_LCS[L * A];  // level * (cos, sin) of each joint code: one 16-byte read
  __shared__ int s_inv[D];
  __shared__ __align__(16) unsigned char s_key[kTile * RST];
  __shared__ __align__(16) _Float16 s_E[2 * kTile * EST];
  __shared__ __align__(16) uint8_t s_code[kTile * CST];
  __shared__ uint32_t s_sw[kTile][NSW > 0 ? NSW : 1];
  __shared__ uint16_t s_nu[kTile];

  // ---- per-head metadata
  const float* cb = a.codebook + size_t(h) * 2 * L;
  const double tscale = a.hadamard ? double(D) : 1.0;  // X = sqrt(d) k~ under the transform
  for (int i = tid; i < L; i += kThreads) {
    if (i < L - 1) {
      const double t = double(cb[L + i]);
      s_T2[i] = tscale * t * t;  // exact: 24-bit significand squared, power-of-two factor
    } else {
      s_T2[i] = __longlong_as_double(0x7FF0000000000000ll);
    }
  }
  for (int e = tid; e < L * A; e += kThreads) {
    const int rc = e / A, ac = e % A;
    double sn, cs;
    sincospi(-1.0 + (2.0 * ac + 1.0) / double(A), &sn, &cs);
    const double lv = double(cb[rc]);
    s_LCS[e] = make_double2(lv * cs, lv * sn);
  }
  // inverse of the channel order: input channel c' lands at position s_inv[c']
  for (int p = tid; p < D; p += kThreads) s_inv[a.perm ? int(a.perm[size_t(h) * D + p]) : p] = p;

  // ---- S_h as MFMA B operands (hi and lo), kept in registers for every tile:
  //      lane holds S[row][16 ks + 8 (lane/32) + j], row = 32 nt + lane % 32
  const int nt = D == 128 ? wave : (wave & 1);
  const int mt0 = D == 128 ? 0 : (wave >> 1);
  half8 sbh[QJL ? KSTEPS : 1], sbl[QJL ? KSTEPS : 1];
  if constexpr (QJL) {
    const float* srow = S + (size_t(h) * M + 32 * nt + (lane & 31)) * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const float4 u0 = *reinterpret_cast<const float4*>(srow + 16 * ks);
      const float4 u1 = *reinterpret_cast<const float4*>(srow + 16 * ks + 4);
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        _Float16 hi, lo;
        split_f16(double(v[jj]), hi, lo);
        sbh[ks][jj] = hi;
        sbl[ks][jj] = lo;
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
    if (a.hadamard && a.signs[size_t(h) * D + pe] < 0) flip |= 1u << e;
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

  double T2r[L - 1];  // wave-uniform: kept in scalar registers
#pragma unroll
  for (int i = 0; i < L - 1; ++i) {
    const double t = s_T2[i];
    T2r[i] = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(t)),
                              __builtin_amdgcn_readfirstlane(__double2loint(t)));
  }
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  const int64_t tile0 = int64_t(blockIdx.x) * kTilesPerBlock;
  const int64_t tile1 = min<int64_t>(tile0 + kTilesPerBlock, n_tiles);
  const double inv_scale = a.hadamard ? 1.0 / sqrt(double(D)) : 1.0;
  uint8_t* base = codes + (size_t(b) * a.n_kv + h) * a.stream_bytes;
  uint32_t* rows = reinterpret_cast<uint32_t*>(base);
  const uint8_t* kstream = K + (size_t(b) * a.n_kv + h) * a.n_tokens * size_t(D) * ES;

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
  if (tile0 < tile1) load_tile(tile0);

  for (int64_t tile = tile0; tile < tile1; ++tile) {
    const int64_t t0 = tile * kTile;
    const int nvalid = static_cast<int>(min<int64_t>(kTile, a.n_tokens - t0));

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
    if (tile + 1 < tile1) load_tile(tile + 1);
    __syncthreads();

    // ---- transform phase: key j on lanes 4j..4j+3, quarter qt holds channels
    //      [qt*CPT, qt*CPT + CPT) of the reordered, sign-flipped key
    const int j = tid >> 2;
    const int qt = tid & 3;
    double x[CPT];
    {
      const unsigned char* src = s_key + j * RST + qt * CPT * ES;
#pragma unroll
      for (int v4 = 0; v4 < CPT * ES / 16; ++v4) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(src + 16 * v4);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (ES == 2) {
            x[v4 * 8 + 2 * w] = double(__half2float(__ushort_as_half(static_cast<uint16_t>(q[w]))));
            x[v4 * 8 + 2 * w + 1] = double(__half2float(__ushort_as_half(static_cast<uint16_t>(q[w] >> 16))));
          } else {
            x[v4 * 4 + w] = double(__uint_as_float(q[w]));
          }
        }
      }
    }

    if (a.hadamard) {
#pragma unroll
      for (int hh = 1; hh < CPT; hh <<= 1) {
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
          if ((r & hh) == 0) {
            const double u = x[r], w = x[r + hh];
            x[r] = u + w;
            x[r + hh] = u - w;
          }
        }
      }
      // the two high channel bits live in the lane index: partner value from
      // the DPP quad permutation, then x_new = partner +- x (exact either way)
      const double sg1 = (qt & 1) ? -1.0 : 1.0, sg2 = (qt & 2) ? -1.0 : 1.0;
#pragma unroll
      for (int r = 0; r < CPT; ++r) x[r] = fma(x[r], sg1, quad_xor<1>(x[r]));
#pragma unroll
      for (int r = 0; r < CPT; ++r) x[r] = fma(x[r], sg2, quad_xor<2>(x[r]));
    }

    // ---- polar codes, residual
    double ss = 0.0, mx = 0.0;
    uint32_t cpack[CPT / 8];
#pragma unroll
    for (int p = 0; p < CPT / 2; ++p) {
      const double xx = x[2 * p], yy = x[2 * p + 1];
      const double r2 = xx * xx + yy * yy;
      int rc = 0;
#pragma unroll
      for (int i = 0; i < L - 1; ++i) rc += (T2r[i] < r2) ? 1 : 0;
      const int ac = octant_cell(xx, yy) >> (3 - BA);
      const uint32_t code = static_cast<uint32_t>(rc | (ac << BM));
      if ((p & 3) == 0) cpack[p >> 2] = code;
      else cpack[p >> 2] |= code << (8 * (p & 3));
      if constexpr (QJL) {
        const double2 lcs = s_LCS[rc * A + ac];
        const double ex = xx * inv_scale - lcs.x;
        const double ey = yy * inv_scale - lcs.y;
        x[2 * p] = ex;
        x[2 * p + 1] = ey;
        ss += ex * ex + ey * ey;
        mx = fmax(mx, fmax(fabs(ex), fabs(ey)));
      }
    }
    // pairs [qt*CPT/2, +CPT/2) of key j
#pragma unroll
    for (int v = 0; v < CPT / 32; ++v) {
      u32x4 q = {cpack[4 * v], cpack[4 * v + 1], cpack[4 * v + 2], cpack[4 * v + 3]};
      *reinterpret_cast<u32x4*>(s_code + j * CST + qt * (CPT / 2) + 16 * v) = q;
    }
    if constexpr (CPT / 2 == 8) {  // d = 64: 8 codes per lane
      *reinterpret_cast<uint2*>(s_code + j * CST + qt * 8) = make_uint2(cpack[0], cpack[1]);
    }

    if constexpr (QJL) {
      const double s1 = ss + quad_xor<1>(ss);
      const double s2 = s1 + quad_xor<2>(s1);
      if (qt == 0) s_nu[j] = f64_to_f16_rne_sat_nonneg(sqrt(s2));
      // power-of-two scale that brings the largest residual entry of the key
      // to [1, 2): exact, and no sign changes
      double m1 = fmax(mx, quad_xor<1>(mx));
      m1 = fmax(m1, quad_xor<2>(m1));
      const int sexp = m1 > 0.0 ? -ilogb(m1) : 0;
      _Float16* Ehi = s_E + j * EST + qt * CPT;
      _Float16* Elo = s_E + kTile * EST + j * EST + qt * CPT;
#pragma unroll
      for (int v = 0; v < CPT / 8; ++v) {
        uint32_t hq[4], lq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split2_f16_scaled(x[8 * v + 2 * e], x[8 * v + 2 * e + 1], sexp, hq[e], lq[e]);
        *reinterpret_cast<u32x4*>(Ehi + 8 * v) = u32x4{hq[0], hq[1], hq[2], hq[3]};
        *reinterpret_cast<u32x4*>(Elo + 8 * v) = u32x4{lq[0], lq[1], lq[2], lq[3]};
      }
    }
    __syncthreads();

    // ---- QJL projection on the matrix cores; sign words from ballots
    if constexpr (QJL) {
      const _Float16* Ehi = s_E;
      const _Float16* Elo = s_E + kTile * EST;
#pragma unroll
      for (int mi = 0; mi < MT_PER_WAVE; ++mi) {
        const int mt = mt0 + mi;
        const int key = 32 * mt + (lane & 31);
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const int off = key * EST + 16 * ks + 8 * (lane >> 5);
          const half8 ah = *reinterpret_cast<const half8*>(Ehi + off);
          const half8 al = *reinterpret_cast<const half8*>(Elo + off);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, sbh[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, sbl[ks], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, sbh[ks], acc, 0, 0, 0);
        }
        // accumulator element r of lane l: key 8 (r/4) + 4 (l/32) + r%4 of the
        // 32-key half, sketch row 32 nt + l%32
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint64_t bal = __ballot(acc[r] >= 0.0f);
          if (lane == 0) {
            const int ka = 32 * mt + 8 * (r >> 2) + (r & 3);
            s_sw[ka][nt] = static_cast<uint32_t>(bal);
            s_sw[ka + 4][nt] = static_cast<uint32_t>(bal >> 32);
          }
        }
      }
      __syncthreads();
    }

    // ---- pack and store: word w of token `lane` goes to row w, slot token_offset + t0 + lane
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
#pragma unroll
      for (int w = 0; w < NSW; ++w) {
        if (((NC + w) & 3) == wave && live)
          __builtin_nontemporal_store(s_sw[lane][w], rows + size_t(NC + w) * a.capacity + slot);
      }
      if (((NC + NSW) & 3) == wave && live) {
        uint16_t* nu = reinterpret_cast<uint16_t*>(base + size_t(4) * NW * a.capacity);
        __builtin_nontemporal_store(s_nu[lane], nu + slot);
      }
    }
  }
}

template <int D, int BM, bool QJL>
hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t s) {
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  dim3 grid(static_cast<unsigned>((n_tiles + kTilesPerBlock - 1) / kTilesPerBlock),
            static_cast<unsigned>(a.n_kv), static_cast<unsigned>(a.n_seq));
  if (a.k_dtype == DT_F32) {
    hipLaunchKernelGGL((encode_kernel<D, BM, QJL, 4>), grid, dim3(kThreads), 0, s, a, a.S,
                       static_cast<const uint8_t*>(a.K), a.codes);
  } else {
    hipLaunchKernelGGL((encode_kernel<D, BM, QJL, 2>), grid, dim3(kThreads), 0, s, a, a.S,
                       static_cast<const uint8_t*>(a.K), a.codes);
  }
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
