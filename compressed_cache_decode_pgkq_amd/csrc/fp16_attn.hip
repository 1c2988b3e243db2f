// FP16-cache decode attention for gfx950: the uncompressed comparator the
// EdgeLLM-Nano page measures fidelity against (its "FP16 wrapper" cache).
//
// Same split / online-softmax skeleton as the PGKQ scan, but the keys are read
// exactly like the values: a 16-lane group (8 at d = 64) holds one 256-byte key
// row, lane k the 8 channels [8k, 8k + 8), so every load instruction reads
// whole rows.  The lane's slice of the G query heads stays in registers for the
// whole scan.  Each lane forms the partial dot products of its 8 channels for
// the rows of the chunk; the partials of a row are then summed across its lane
// group by a reduce-scatter butterfly: at each level a lane keeps one half of
// its rows, sends the other half to a partner lane (DPP: xor 1, xor 2, the
// half-row mirror, the 8-lane rotation) and adds what it receives.  After the
// last level lane k holds the full scores of one row, which feed the shared
// softmax and the matrix-core P.V tail (values in 32-token tiles).  Queries are
// applied as a log2-domain softmax scale.
#include <type_traits>

#include "mfma_pv.hpp"

namespace pgkq {

namespace {

// f(integral_constant<int, I>) for I = B .. E - 1, so that array indices derived
// from I are compile-time constants however large the unrolled body grows
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// number of trailing one bits of i, at most cap
constexpr int trailing_ones(int i, int cap) { return (cap > 0 && (i & 1)) ? 1 + trailing_ones(i >> 1, cap - 1) : 0; }

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// DPP exchanges inside a 16-lane row: partner masks 1, 2, 7 (half-row mirror)
// and 8 (rotation by 8); linearly independent over GF(2)^4.
template <int LEVEL>
__device__ __forceinline__ float dpp_partner(float v) {
  constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x128;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true));
}

// Row kept at each level: the dual basis of the partner masks (1, 2, 7, 8):
// f0 = k0 ^ k2, f1 = k1 ^ k2, f2 = k2, f3 = k3 (bit j of the lane index k).
__device__ __forceinline__ int keep_bits(int k) {
  const int k0 = k & 1, k1 = (k >> 1) & 1, k2 = (k >> 2) & 1, k3 = (k >> 3) & 1;
  return (k0 ^ k2) | ((k1 ^ k2) << 1) | (k2 << 2) | (k3 << 3);
}

// Two wavefronts per SIMD for every shape: with 8 query heads at d = 128 (64
// query and 64 accumulator registers per lane) the 256-register budget still
// holds them without spilling, and the second wavefront hides the key loads.
template <int D, int G>
constexpr int fp16_min_waves() { return 2; }

template <int D, int G, bool WAVE_PARTS>
__global__ void __launch_bounds__(kThreads, (fp16_min_waves<D, G>()))
fp16_scan_kernel(Fp16DecodeArgs a, const __half* __restrict__ K, const __half* __restrict__ V) {
  using SM = MfmaPV<D, G, kWaves>;
  constexpr int LPT = D / 8;            // lanes per key row
  constexpr int TPI = kWave / LPT;      // key rows per wavefront load
  constexpr int NIT = kWave / TPI;      // rows per lane group per chunk (16 or 8)
  constexpr int LEVELS = NIT == 16 ? 4 : 3;
  __shared__ __align__(16) float s_merge[SM::MERGE_FLOATS];
  __shared__ __align__(16) float s_p[kWaves][kWave][G];
  static_assert(sizeof(s_p[0]) >= MfmaPV<D, G, kWaves>::P_BYTES, "weight rows");

  const int tid = threadIdx.x;
  // grid (kv-head, sequence, split): split-major, leading (larger) splits first
  const int split = blockIdx.z;
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;

  SM sm;
  sm.init(tid);
  const int wave = sm.wave, k = sm.lane % LPT, slot = sm.lane / LPT;

  // this lane's 8 channels of every query head of the group
  float qr[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      qr[g][j] = load_f(a.q, a.q_dtype, (size_t(b) * a.n_q + size_t(h) * G + g) * D + 8 * k + j);

  const int kb = keep_bits(k);
  const int my_row = kb & (NIT - 1);          // row of the chunk this lane ends up scoring
  const int prow = my_row * TPI + slot;       // its token index within the chunk

  const bool trailing = split >= a.n_lead && a.n_lead > 0;
  const int64_t t_begin = trailing ? int64_t(a.n_lead) * a.tokens_per_split +
                                         int64_t(split - a.n_lead) * a.tail_split
                                   : int64_t(split) * a.tokens_per_split;
  const int64_t t_end =
      min<int64_t>(t_begin + (trailing ? a.tail_split : a.tokens_per_split), a.n_tokens);
  const int64_t stream = b * a.n_kv + h;
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(K + size_t(stream) * a.capacity * D, static_cast<uint32_t>(t_end * D * 2));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + size_t(stream) * a.capacity * D,
                                               static_cast<uint32_t>((t_end + 31) / 32 * 32 * D * 2));

  int64_t c_first, c_end, c_step;
  if constexpr (WAVE_PARTS) {
    const int64_t tpw = a.tokens_per_split / kWaves;
    c_first = t_begin + int64_t(wave) * tpw;
    c_end = min<int64_t>(c_first + tpw, t_end);
    c_step = kWave;
  } else {
    c_first = t_begin + int64_t(wave) * kWave;
    c_end = t_end;
    c_step = kThreads;
  }
  for (int64_t c0 = c_first; c0 < c_end; c0 += c_step) {
    // key rows: same layout as the value rows.  With 8 query heads at d = 128
    // the key rows come in two halves and the value rows are requested after
    // the scores (registers).
    constexpr bool kSplitK = G * D > 512;
    constexpr int KPARTS = kSplitK ? 2 : 1;
    constexpr int KROWS = NIT / KPARTS;
    const uint32_t kbase = static_cast<uint32_t>(c0 + slot) * (D * 2) + k * 16;
    typename SM::VChunk vc;
    u32x4 kr[KROWS];
#pragma unroll
    for (int r = 0; r < KROWS; ++r) kr[r] = buf_load_b128(krs, kbase + r * TPI * D * 2);
    if constexpr (!kSplitK) sm.load_v(vc, c0, vrs, t_end);

    // partial dot products of row `it` (8 channels), reduced level by level as
    // soon as both halves of a level exist: at most LEVELS + 1 live per head
    float part[G][LEVELS + 1];
    float s[G];
    static_for<0, NIT>([&](auto itc) {
      constexpr int it = decltype(itc)::value;
      if constexpr (kSplitK && it == KROWS) {
        sched_fence();
#pragma unroll
        for (int r = 0; r < KROWS; ++r)
          kr[r] = buf_load_b128(krs, kbase + (KROWS + r) * TPI * D * 2);
      }
      __half2 hk[4];
      __builtin_memcpy(hk, &kr[it % KROWS], sizeof(hk));
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 f = __half22float2(hk[j]);
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = fmaf(f.y, qr[g][2 * j + 1], fmaf(f.x, qr[g][2 * j], dot[g]));
      }
      // carry the new leaf up the tree: level L combines when bit L of it
      // completes a pair of blocks, i.e. for the trailing one bits of it
      constexpr int TOP = trailing_ones(it, LEVELS);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float v = dot[g];
        static_for<0, TOP>([&](auto lc) {
          constexpr int L = decltype(lc)::value;
          const bool keep_hi = (kb >> L) & 1;
          const float lo = part[g][L], hi = v;
          const float keep = keep_hi ? hi : lo;
          const float send = keep_hi ? lo : hi;
          v = keep + dpp_partner<L>(send);
        });
        if constexpr (TOP < LEVELS) {
          part[g][TOP] = v;
        } else {
          s[g] = v;
        }
      }
    });
    if constexpr (kSplitK) {
      sched_fence();  // keep the value loads behind the key registers' last use
      sm.load_v(vc, c0, vrs, t_end);
    }
    const bool valid = c0 + prow < c_end;
    sm.mask_v(vc, c0, t_end);
    sm.chunk(s, valid, a.scale_log2, vc, &s_p[wave][0][0], prow);
  }
  const size_t row0 = size_t(b) * a.n_q + size_t(h) * G;
  __syncthreads();
  sm.finish(s_merge, tid, a.n_splits, split, a.out, a.partial, row0);
}

template <int D, int G>
hipError_t fp16_t(const Fp16DecodeArgs& a, hipStream_t s) {
  dim3 grid(unsigned(a.n_kv), unsigned(a.n_seq), unsigned(a.n_splits));
  if (a.wave_parts) {
    hipLaunchKernelGGL((fp16_scan_kernel<D, G, true>), grid, dim3(kThreads), 0, s, a, as_half(a.K), as_half(a.V));
  } else {
    hipLaunchKernelGGL((fp16_scan_kernel<D, G, false>), grid, dim3(kThreads), 0, s, a, as_half(a.K), as_half(a.V));
  }
  return hipGetLastError();
}

template <int D>
hipError_t fp16_g(const Fp16DecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 1: return fp16_t<D, 1>(a, s);
    case 2: return fp16_t<D, 2>(a, s);
    case 4: return fp16_t<D, 4>(a, s);
    case 8: return fp16_t<D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fp16_decode(const Fp16DecodeArgs& a, hipStream_t s) {
  if (a.d == 64) return fp16_g<64>(a, s);
  if (a.d == 128) return fp16_g<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pgkq
