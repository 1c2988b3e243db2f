// PGKQ key encoder for gfx950.
//
// Steps (1)-(4) of the PGKQ pipeline (EdgeLLM-Nano paper page, "PGKQ
// pipeline"): randomized Hadamard transform, adjacent-pair polar coordinates,
// Lloyd-Max radius code and uniform-grid angle code, optional QJL residual
// sketch (sign bits of S_h eps~ plus an fp16 residual norm).
//
// One workgroup (4 wavefronts) encodes a tile of 64 keys of one (sequence,
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
//   * the QJL projection runs lane-per-key: each wavefront owns a quarter of the
//     m sketch rows, so the S_h addresses are wave-uniform and every S value
//     read serves 64 keys; accumulation is fp32;
//   * codes are packed per token in LDS and stored as one coalesced 256-byte
//     row segment per code word.
#include "device_common.hpp"

namespace pgkq {

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

template <int D>
struct EncodeSmem {
  static constexpr int EST = D + 4;  // fp32 residual row stride (bank spread)
  static constexpr int kRawBytes = kTile * D * 4 > kTile * EST * 4 ? kTile * D * 4 : kTile * EST * 4;
};

template <int D, int BM, bool QJL>
__global__ void __launch_bounds__(kThreads)
encode_kernel(EncodeArgs a, const float* __restrict__ S, const uint8_t* __restrict__ K,
              uint8_t* __restrict__ codes) {
  constexpr int N = D / 2;
  constexpr int BA = BM - 1;
  constexpr int P = BM + BA;
  constexpr int L = 1 << BM;
  constexpr int A = 1 << BA;
  constexpr int NC = N * P / 32;
  constexpr int M = QJL ? D : 0;
  constexpr int NSW = M / 32;
  constexpr int NW = NC + NSW;
  constexpr int CPT = D / 4;            // channels per lane in the transform phase
  constexpr int RPT = QJL ? M / 4 : 1;  // sketch rows per lane in the projection
  constexpr int EST = EncodeSmem<D>::EST;
  static_assert(N % 32 == 0, "pairs must fill whole words");

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int64_t t0 = int64_t(blockIdx.x) * kTile;
  const int nvalid = static_cast<int>(min<int64_t>(kTile, a.n_tokens - t0));
  const int esize = a.k_dtype == DT_F32 ? 4 : 2;

  __shared__ double s_T2[L];
  __shared__ double s_LC[L * A];
  __shared__ double s_LS[L * A];
  __shared__ int s_perm[D];
  __shared__ double s_sign[D];
  __shared__ __align__(16) unsigned char s_raw[EncodeSmem<D>::kRawBytes];
  __shared__ uint8_t s_code[kTile][N + 4];
  __shared__ uint32_t s_sw[kTile][NSW > 0 ? NSW : 1];
  __shared__ uint16_t s_nu[kTile];

  // ---- per-head metadata
  const float* cb = a.codebook + size_t(h) * 2 * L;
  const double tscale = a.hadamard ? double(D) : 1.0;  // X = sqrt(d) k~ under the transform
  for (int i = tid; i < L; i += kThreads) {
    if (i < L - 1) {
      double t = double(cb[L + i]);
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
    s_LC[e] = lv * cs;
    s_LS[e] = lv * sn;
  }
  for (int c = tid; c < D; c += kThreads) {
    s_perm[c] = a.perm ? int(a.perm[size_t(h) * D + c]) : c;
    s_sign[c] = double(a.signs[size_t(h) * D + c]);
  }

  // ---- key tile -> LDS (16-byte coalesced loads; rows past n_tokens are zero)
  {
    const size_t row_bytes = size_t(D) * esize;
    const uint8_t* src = K + ((size_t(b) * a.n_kv + h) * a.n_tokens + t0) * row_bytes;
    const int tile_bytes = kTile * D * esize;
    const int valid_bytes = nvalid * D * esize;
    for (int off = tid * 16; off < tile_bytes; off += kThreads * 16) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (off < valid_bytes) v = *reinterpret_cast<const uint4*>(src + off);
      *reinterpret_cast<uint4*>(s_raw + off) = v;
    }
  }
  __syncthreads();

  // ---- transform phase: key j on lanes 4j..4j+3, lane quarter qt holds channels
  //      [qt*CPT, qt*CPT + CPT) of the reordered key
  const int j = tid >> 2;
  const int qt = tid & 3;
  double x[CPT];
#pragma unroll
  for (int r = 0; r < CPT; ++r) {
    const int c = qt * CPT + r;
    const int src = s_perm[c];
    double v;
    if (esize == 4) {
      v = double(reinterpret_cast<const float*>(s_raw)[j * D + src]);
    } else {
      v = double(__half2float(reinterpret_cast<const __half*>(s_raw)[j * D + src]));
    }
    x[r] = a.hadamard ? v * s_sign[c] : v;
  }
  __syncthreads();  // the raw tile region is reused for the residual below

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
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const double p = quad_xor<1>(x[r]);
      x[r] = (qt & 1) ? (p - x[r]) : (x[r] + p);
    }
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const double p = quad_xor<2>(x[r]);
      x[r] = (qt & 2) ? (p - x[r]) : (x[r] + p);
    }
  }

  // ---- polar codes, residual
  double T2r[L - 1];
#pragma unroll
  for (int i = 0; i < L - 1; ++i) T2r[i] = s_T2[i];
  const double inv_scale = a.hadamard ? 1.0 / sqrt(double(D)) : 1.0;
  double ss = 0.0;
#pragma unroll
  for (int p = 0; p < CPT / 2; ++p) {
    const double xx = x[2 * p], yy = x[2 * p + 1];
    const double r2 = xx * xx + yy * yy;
    int rc = 0;
#pragma unroll
    for (int i = 0; i < L - 1; ++i) rc += (T2r[i] < r2) ? 1 : 0;
    const int ac = octant_cell(xx, yy) >> (3 - BA);
    s_code[j][qt * (CPT / 2) + p] = static_cast<uint8_t>(rc | (ac << BM));
    if constexpr (QJL) {
      const double ex = xx * inv_scale - s_LC[rc * A + ac];
      const double ey = yy * inv_scale - s_LS[rc * A + ac];
      x[2 * p] = ex;
      x[2 * p + 1] = ey;
      ss += ex * ex + ey * ey;
    }
  }

  if constexpr (QJL) {
    double s1 = ss + quad_xor<1>(ss);
    double s2 = s1 + quad_xor<2>(s1);
    if (qt == 0) s_nu[j] = f64_to_f16_rne_sat(sqrt(s2));
    float* E = reinterpret_cast<float*>(s_raw);
#pragma unroll
    for (int r = 0; r < CPT; ++r) E[j * EST + qt * CPT + r] = static_cast<float>(x[r]);
  }
  __syncthreads();

  // ---- QJL projection: lane = key, wavefront = quarter of the sketch rows
  if constexpr (QJL) {
    const int jk = tid & 63;
    const int rq = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float* E = reinterpret_cast<const float*>(s_raw) + jk * EST;
    const float* Sr = S + (size_t(h) * M + size_t(rq) * RPT) * D;
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc[r] = 0.0f;
#pragma unroll 2
    for (int c = 0; c < D; c += 4) {
      const float4 e = *reinterpret_cast<const float4*>(E + c);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const float4 s4 = *reinterpret_cast<const float4*>(Sr + size_t(r) * D + c);
        float t = acc[r];
        t = fmaf(s4.x, e.x, t);
        t = fmaf(s4.y, e.y, t);
        t = fmaf(s4.z, e.z, t);
        t = fmaf(s4.w, e.w, t);
        acc[r] = t;
      }
    }
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) bits |= (acc[r] >= 0.0f ? 1u : 0u) << r;
    if (RPT == 32) {
      s_sw[jk][rq] = bits;
    } else {
      reinterpret_cast<uint16_t*>(&s_sw[jk][0])[rq] = static_cast<uint16_t>(bits);
    }
  }
  __syncthreads();

  // ---- pack and store: word w of token j goes to row w, slot token_offset + t0 + j
  const int lane = tid & 63;
  const int wave = tid >> 6;
  uint8_t* base = codes + (size_t(b) * a.n_kv + h) * a.stream_bytes;
  uint32_t* rows = reinterpret_cast<uint32_t*>(base);
  const int64_t slot = a.token_offset + t0 + lane;
  const bool live = lane < nvalid;
#pragma unroll
  for (int w = 0; w < NC; ++w) {
    if ((w & 3) == wave) {
      uint32_t word = 0;
#pragma unroll
      for (int i = (32 * w) / P; i <= (32 * w + 31) / P && i < N; ++i) {
        const uint32_t code = s_code[lane][i];
        const int o = P * i - 32 * w;
        word |= o >= 0 ? (code << o) : (code >> (-o));
      }
      if (live) rows[size_t(w) * a.capacity + slot] = word;
    }
  }
  if constexpr (QJL) {
#pragma unroll
    for (int w = 0; w < NSW; ++w) {
      if (((NC + w) & 3) == wave && live) rows[size_t(NC + w) * a.capacity + slot] = s_sw[lane][w];
    }
    if (((NC + NSW) & 3) == wave && live) {
      uint16_t* nu = reinterpret_cast<uint16_t*>(base + size_t(4) * NW * a.capacity);
      nu[slot] = s_nu[lane];
    }
  }
}

template <int D, int BM, bool QJL>
hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((a.n_tokens + kTile - 1) / kTile), static_cast<unsigned>(a.n_kv),
            static_cast<unsigned>(a.n_seq));
  hipLaunchKernelGGL((encode_kernel<D, BM, QJL>), grid, dim3(kThreads), 0, s, a, a.S,
                     static_cast<const uint8_t*>(a.K), a.codes);
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
