// Per-token asymmetric round-to-nearest (RTN) key cache for gfx950: the
// simpler baseline the EdgeLLM-Nano page compares PGKQ with ("Comparison to
// simpler baselines": K at INT3 / INT4 with an FP16 scale and zero-point per
// key vector, V in FP16; 3.50 / 4.50 bits per element at d = 64).
//
// Record of one token (d b / 8 + 4 bytes): the d b-bit codes as one bit
// stream (code c at bits [b c, b c + b), LSB first) in d b / 32 uint32 words,
// then one uint32 holding the fp16 scale (low half) and the fp16 zero-point
// (high half).  Word w of token t sits at byte 4 (w capacity + t) of its
// stream, so a wavefront reading one word of 64 consecutive tokens reads 256
// contiguous bytes.
//
// Kernels:
//   rtn_encode      thread = token: min / max of the key, fp16 zero-point and
//                   scale, codes decided in float64, packed words stored
//                   coalesced across the wavefront;
//   rtn_query_prep  per (sequence, kv-head): the G query heads as fp32 [c][g]
//                   and their channel sums, so that
//                   logit = zp * sum_c q_c + scale * sum_c q_c code_c;
//   rtn_scan        the decode scan in the split skeleton of the PGKQ scan:
//                   lane = token for the score, the query read through the
//                   scalar cache (wave-uniform), then the shared online softmax
//                   and the matrix-core P.V tail over the value cache in
//                   32-token tiles.
#include "mfma_pv.hpp"

namespace pgkq {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

typedef __attribute__((address_space(4))) const float const_float;

// A pointer into the constant address space: loads through it with a
// wave-uniform address become scalar loads.  The asm ties the pointer to the
// current program point, so loads through it are issued after this line: the
// score loop takes a fresh pointer per code word, which keeps the query values
// in flight to one word's worth of SGPRs (all of them would not fit).
__device__ __forceinline__ const const_float* uniform_rows(const float* p) {
  const const_float* c = (const const_float*)(p);
  asm volatile("" : "+s"(c)::"memory");
  return c;
}

// ------------------------------------------------------------------ encode

template <int D, int BITS, int ES>
__global__ void __launch_bounds__(kThreads) rtn_encode_kernel(RtnEncodeArgs a) {
  constexpr int NC = D * BITS / 32;
  constexpr int QMAX = (1 << BITS) - 1;
  constexpr int NL = D * ES / 16;  // 16-byte loads per key row
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= a.n_tokens) return;
  const int64_t stream = int64_t(blockIdx.z) * a.n_kv + blockIdx.y;
  const uint8_t* row =
      static_cast<const uint8_t*>(a.K) + (stream * a.n_tokens + t) * int64_t(D) * ES;
  float k[D];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + i);
    if constexpr (ES == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        k[8 * i + 2 * j] = half_bits_to_float(static_cast<uint16_t>(raw[j] & 0xFFFFu));
        k[8 * i + 2 * j + 1] = half_bits_to_float(static_cast<uint16_t>(raw[j] >> 16));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) k[4 * i + j] = __uint_as_float(raw[j]);
    }
  }
  float mn = k[0], mx = k[0];
#pragma unroll
  for (int c = 1; c < D; ++c) {
    mn = fminf(mn, k[c]);
    mx = fmaxf(mx, k[c]);
  }
  // +0.0 turns a -0 extreme into +0 (min / max of signed zeros are otherwise
  // unordered); both are exact fp32 values rounded once to fp16
  const __half lo_h = __float2half_rn(mn + 0.0f);
  const __half hi_h = __float2half_rn(mx + 0.0f);
  const double zp = static_cast<double>(__half2float(lo_h));
  const double range = static_cast<double>(__half2float(hi_h)) - zp;  // exact, >= 0
  uint16_t sbits = f64_to_f16_rne_sat_nonneg(range / QMAX);
  if ((sbits & 0x7FFFu) == 0) sbits = 0x3C00u;  // zero range: scale 1
  const double sc = static_cast<double>(half_bits_to_float(sbits));

  uint32_t words[NC];
#pragma unroll
  for (int w = 0; w < NC; ++w) words[w] = 0u;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    // nearest code, ties to even, clamped to [0, 2^b - 1]
    double x = rint((static_cast<double>(k[c]) - zp) / sc);
    x = fmin(fmax(x, 0.0), static_cast<double>(QMAX));
    const uint32_t code = static_cast<uint32_t>(x);
    const int off = BITS * c, w = off >> 5, s = off & 31;
    words[w] |= code << s;
    if (s + BITS > 32) words[w + 1] |= code >> (32 - s);
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + size_t(stream) * a.stream_bytes) +
                  (a.token_offset + t);
#pragma unroll
  for (int w = 0; w < NC; ++w) __builtin_nontemporal_store(words[w], dst + size_t(w) * a.capacity);
  const uint32_t zbits = __half_as_ushort(lo_h);
  __builtin_nontemporal_store(static_cast<uint32_t>(sbits) | (zbits << 16),
                              dst + size_t(NC) * a.capacity);
}

// ------------------------------------------------------------------ query prep

template <int D>
__global__ void __launch_bounds__(D) rtn_query_prep_kernel(RtnDecodeArgs a) {
  const int c = threadIdx.x;
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int G = a.group;
  __shared__ float s_q[8][D];
  float* out = a.prep + (size_t(b) * a.n_kv + h) * rtn_prep_stride(D, G);
  for (int g = 0; g < G; ++g) {
    const float v = load_f(a.q, a.q_dtype, (size_t(b) * a.n_q + size_t(h) * G + g) * D + c);
    out[c * G + g] = v;
    s_q[g][c] = v;
  }
  __syncthreads();
  if (c < G) {
    double s = 0.0;
    for (int k = 0; k < D; ++k) s += static_cast<double>(s_q[c][k]);
    out[D * G + c] = static_cast<float>(s);
  }
}

// ------------------------------------------------------------------ scan

// sum_c q[c][g] * code_c over the D codes of one token (lane), the query read
// through scalar loads.  INT4: the nibbles of a word are split into the even
// and odd bytes and converted with the byte-to-float instructions.
// Every 8 channels the accumulators, the code words in use and the query
// pointer are pinned: the scheduler then cannot run one head's whole chain
// first (which would keep every query value of that head live in SGPRs) nor
// convert all codes up front (VGPRs).
template <int D, int BITS, int G>
__device__ __forceinline__ void rtn_dot(uint32_t (&cw)[D * BITS / 32 + 1], const float* qrow,
                                        float (&acc)[G]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < D / 8; ++w) {
#pragma unroll
      for (int g = 0; g < G; ++g) pin_reg(acc[g]);
      pin_reg(cw[w]);
      const const_float* qs = uniform_rows(qrow);
      const uint32_t lo = cw[w] & 0x0F0F0F0Fu;
      const uint32_t hi = (cw[w] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float c0 = static_cast<float>((lo >> (8 * j)) & 0xFFu);
        const float c1 = static_cast<float>((hi >> (8 * j)) & 0xFFu);
        const int ch = 8 * w + 2 * j;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g] = fmaf(c0, qs[ch * G + g], acc[g]);
          acc[g] = fmaf(c1, qs[(ch + 1) * G + g], acc[g]);
        }
      }
    }
  } else {
    const const_float* qs = nullptr;
#pragma unroll
    for (int ch = 0; ch < D; ++ch) {
      const int off = BITS * ch, w = off >> 5, s = off & 31;
      if (ch % 8 == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) pin_reg(acc[g]);
#pragma unroll
        for (int k = w; k <= (BITS * (ch + 8) - 1) / 32 && k < D * BITS / 32; ++k) pin_reg(cw[k]);
        qs = uniform_rows(qrow);
      }
      constexpr uint32_t mask = (1u << BITS) - 1u;
      const uint32_t code = (s + BITS <= 32) ? (cw[w] >> s) & mask
                                             : __builtin_amdgcn_alignbit(cw[w + 1], cw[w], s) & mask;
      const float cf = static_cast<float>(code);
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fmaf(cf, qs[ch * G + g], acc[g]);
    }
  }
}

template <int D, int BITS, int G, bool LOGITS>
__global__ void __launch_bounds__(kThreads, 2)
rtn_scan_kernel(RtnDecodeArgs a, const uint8_t* __restrict__ codes, const __half* __restrict__ V) {
  constexpr int NC = D * BITS / 32;
  constexpr int NW = NC + 1;
  constexpr int MERGE_FLOATS = MfmaPV<D, G, kWaves>::MERGE_FLOATS;
  __shared__ __align__(16) float s_merge[MERGE_FLOATS];
  __shared__ __align__(16) float s_p[kWaves][kWave][G];
  static_assert(sizeof(s_p[0]) >= MfmaPV<D, G, kWaves>::P_BYTES, "weight rows");

  const int tid = threadIdx.x;
  // grid (kv-head, sequence, split): split-major, leading (larger) splits first
  const int split = blockIdx.z;
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;
  const float* qrow = a.prep + (size_t(b) * a.n_kv + h) * rtn_prep_stride(D, G);

  const bool trailing = split >= a.n_lead && a.n_lead > 0;
  const int64_t t_begin = trailing ? int64_t(a.n_lead) * a.tokens_per_split +
                                         int64_t(split - a.n_lead) * a.tail_split
                                   : int64_t(split) * a.tokens_per_split;
  const int64_t t_end =
      min<int64_t>(t_begin + (trailing ? a.tail_split : a.tokens_per_split), a.n_tokens);
  const int64_t stream = b * a.n_kv + h;
  const __amdgpu_buffer_rsrc_t crs =
      make_rsrc(codes + size_t(stream) * a.stream_bytes, static_cast<uint32_t>(a.stream_bytes));
  const __amdgpu_buffer_rsrc_t vrs =
      make_rsrc(V + size_t(stream) * a.capacity * D, static_cast<uint32_t>((t_end + 31) / 32 * 32 * D * 2));
  const uint32_t row_bytes = 4u * static_cast<uint32_t>(a.capacity);

  MfmaPV<D, G, kWaves> sm;
  sm.init(tid);
  const int lane = sm.lane, wave = sm.wave;

  int64_t c_first, c_end, c_step;
  if (a.wave_parts) {
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
    const int64_t t = c0 + lane;
    const bool valid = t < c_end;
    // lanes past the split end read neighbouring (or, past the stream, zero)
    // words; their scores are masked
    uint32_t cw[NW];
    const uint32_t t4 = static_cast<uint32_t>(t) * 4u;
#pragma unroll
    for (int w = 0; w < NW; ++w) cw[w] = buf_load_b32(crs, t4 + w * row_bytes);
    typename MfmaPV<D, G, kWaves>::VChunk vc;
    if constexpr (!LOGITS) sm.load_v(vc, c0, vrs, t_end);

    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    rtn_dot<D, BITS, G>(cw, qrow, acc);
    const const_float* qs = uniform_rows(qrow);
    const float scale = half_bits_to_float(static_cast<uint16_t>(cw[NC] & 0xFFFFu));
    const float zp = half_bits_to_float(static_cast<uint16_t>(cw[NC] >> 16));
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = fmaf(zp, qs[D * G + g], scale * acc[g]);

    if constexpr (LOGITS) {
      if (valid) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          a.logits[(size_t(b) * a.n_q + size_t(h) * G + g) * a.n_tokens + t] = s[g];
      }
    } else {
      sm.mask_v(vc, c0, t_end);
      sm.chunk(s, valid, a.scale_log2, vc, &s_p[wave][0][0]);
    }
  }
  if constexpr (!LOGITS) {
    const size_t row0 = size_t(b) * a.n_q + size_t(h) * G;
    __syncthreads();
    sm.finish(s_merge, tid, a.n_splits, split, a.out, a.partial, row0);
  }
}

// ------------------------------------------------------------------ dispatch

template <int D, int BITS>
hipError_t encode_t(const RtnEncodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned((a.n_tokens + kThreads - 1) / kThreads), unsigned(a.n_kv),
                  unsigned(a.n_seq));
  if (a.k_dtype == DT_F32) {
    hipLaunchKernelGGL((rtn_encode_kernel<D, BITS, 4>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((rtn_encode_kernel<D, BITS, 2>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D, int BITS, int G>
hipError_t scan_t(const RtnDecodeArgs& a, bool lm, hipStream_t s) {
  const dim3 grid(unsigned(a.n_kv), unsigned(a.n_seq), unsigned(a.n_splits));
  if (lm) {
    hipLaunchKernelGGL((rtn_scan_kernel<D, BITS, G, true>), grid, dim3(kThreads), 0, s, a, a.codes,
                       as_half(a.V));
  } else {
    hipLaunchKernelGGL((rtn_scan_kernel<D, BITS, G, false>), grid, dim3(kThreads), 0, s, a,
                       a.codes, as_half(a.V));
  }
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t scan_g(const RtnDecodeArgs& a, bool lm, hipStream_t s) {
  switch (a.group) {
    case 1: return scan_t<D, BITS, 1>(a, lm, s);
    case 2: return scan_t<D, BITS, 2>(a, lm, s);
    case 4: return scan_t<D, BITS, 4>(a, lm, s);
    case 8: return scan_t<D, BITS, 8>(a, lm, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t scan_b(const RtnDecodeArgs& a, bool lm, hipStream_t s) {
  if (a.bits == 3) return scan_g<D, 3>(a, lm, s);
  if (a.bits == 4) return scan_g<D, 4>(a, lm, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rtn_encode(const RtnEncodeArgs& a, hipStream_t s) {
  if (a.d == 64) return a.bits == 3 ? encode_t<64, 3>(a, s) : encode_t<64, 4>(a, s);
  if (a.d == 128) return a.bits == 3 ? encode_t<128, 3>(a, s) : encode_t<128, 4>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rtn_query_prep(const RtnDecodeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.n_kv), unsigned(a.n_seq));
  if (a.d == 64) {
    hipLaunchKernelGGL(rtn_query_prep_kernel<64>, grid, dim3(64), 0, s, a);
  } else if (a.d == 128) {
    hipLaunchKernelGGL(rtn_query_prep_kernel<128>, grid, dim3(128), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rtn_scan(const RtnDecodeArgs& a, bool logits_mode, hipStream_t s) {
  if (a.d == 64) return scan_b<64>(a, logits_mode, s);
  if (a.d == 128) return scan_b<128>(a, logits_mode, s);
  return hipErrorInvalidValue;
}

}  // namespace pgkq
