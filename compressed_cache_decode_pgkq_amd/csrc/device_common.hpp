// Device helpers shared by the PGKQ kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgkq_internal.hpp"

namespace pgkq {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer access: a 128-bit resource (base, byte size) and 32-bit offsets
// in a VGPR.  Reads at offsets at or beyond the size return zero (the buffer
// unit's range check), so tail rows need no clamping.  The cache-kind bits
// request non-temporal (streaming) loads: the cache is read once.
constexpr int kLoadStream = 2;  // CDNA3/4 cache policy: NT
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kLoadStream));
}
__device__ __forceinline__ uint32_t buf_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kLoadStream));
}
__device__ __forceinline__ uint16_t buf_load_b16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, kLoadStream));
}
__device__ __forceinline__ uint8_t buf_load_b8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return static_cast<uint8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, static_cast<int>(off), 0, kLoadStream));
}

// 32-bit store through a buffer resource: an offset at or beyond the range is
// dropped by the buffer unit, so a lane stores or not without a branch.
__device__ __forceinline__ void buf_store_b32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(off), 0, kLoadStream);
}

// Compiler-only fence: emits no instruction, but no memory access is moved
// across it and it closes a scheduling region.  Used to keep the scheduler
// from hoisting every LDS table read of a long unrolled loop (register
// pressure).
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// Ties a register value to the current program point (emits nothing): work
// derived from it cannot be hoisted above this line.
__device__ __forceinline__ void pin_reg(uint32_t& v) { asm volatile("" : "+v"(v)::"memory"); }
__device__ __forceinline__ void pin_reg(float& v) { asm volatile("" : "+v"(v)::"memory"); }
__device__ __forceinline__ void pin_reg(double& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float load_f(const void* p, int dtype, int64_t i) {
  if (dtype == DT_F32) return static_cast<const float*>(p)[i];
  if (dtype == DT_F16) return __half2float(static_cast<const __half*>(p)[i]);
  // bf16: the upper half of an fp32
  uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
  return __uint_as_float(u);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// fp64 -> fp16 bits, round to nearest (ties to even), values beyond the fp16
// range saturate to 65504.  Written on the bit pattern so that exactly one
// rounding happens (no detour through fp32).  Only non-negative inputs occur
// (residual norms); the sign is carried anyway.
__device__ __forceinline__ uint16_t f64_to_f16_rne_sat(double x) {
  uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
  uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull) {  // inf or nan
    return mag == 0x7FF0000000000000ull ? static_cast<uint16_t>(sign | 0x7BFFu)
                                        : static_cast<uint16_t>(sign | 0x7E00u);
  }
  int e = static_cast<int>(mag >> 52);  // biased fp64 exponent
  uint64_t m = mag & 0x000FFFFFFFFFFFFFull;
  int eh = e - 1023 + 15;               // biased fp16 exponent
  if (eh >= 31) return static_cast<uint16_t>(sign | 0x7BFFu);
  uint64_t full;   // significand with the implicit bit
  int shift;       // bits to drop from the 53-bit significand
  if (e == 0) return sign;  // fp64 subnormal: far below the fp16 range
  full = m | 0x0010000000000000ull;
  if (eh >= 1) {
    shift = 42;  // keep 11 significant bits
  } else {
    shift = 42 + (1 - eh);  // fp16 subnormal
    if (shift > 63) return sign;
  }
  uint64_t kept = full >> shift;
  uint64_t rem = full & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (kept & 1))) kept += 1;
  uint32_t out;
  if (eh >= 1) {
    // kept in [2^10, 2^11]; a carry to 2^11 bumps the exponent
    uint32_t ee = static_cast<uint32_t>(eh);
    if (kept == (1ull << 11)) { kept = 1ull << 10; ee += 1; }
    if (ee >= 31) return static_cast<uint16_t>(sign | 0x7BFFu);
    out = (ee << 10) | static_cast<uint32_t>(kept & 0x3FFu);
  } else {
    // subnormal result; a carry into 2^10 yields the smallest normal naturally
    out = static_cast<uint32_t>(kept);
  }
  return static_cast<uint16_t>(sign | out);
}

// Wave-uniform maximum: DPP reductions inside each row of 16 lanes, then the
// four row results through readlane (no LDS traffic).
__device__ __forceinline__ float wave_max_uniform(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// 2^x with the hardware approximation (inputs are <= 0 here; results below the
// smallest normal flush to zero, which a softmax weight may do).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// double exchanged with the lane whose index differs in bit `mask` (1 or 2):
// DPP quad permutation, no LDS traffic.
template <int MASK>
__device__ __forceinline__ double quad_xor(double v) {
  static_assert(MASK == 1 || MASK == 2, "quad permutation only");
  constexpr int ctrl = (MASK == 1) ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  int lo = __double2loint(v), hi = __double2hiint(v);
  lo = __builtin_amdgcn_mov_dpp(lo, ctrl, 0xF, 0xF, true);
  hi = __builtin_amdgcn_mov_dpp(hi, ctrl, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

template <int MASK>
__device__ __forceinline__ float quad_xor_f(float v) {
  static_assert(MASK == 1 || MASK == 2, "quad permutation only");
  constexpr int ctrl = (MASK == 1) ? 0xB1 : 0x4E;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, true));
}

// Cell of the mid-rise angle grid with 8 cells of width pi/4 starting at -pi,
// decided by exact comparisons: the cell holding direction (x, y) when cells
// are half-open [e_a, e_{a+1}) counter-clockwise, theta = pi counted as -pi
// (cell 0), and the zero vector taken as theta = 0 (cell 4).  Coarser grids
// are prefixes: cell_b = cell_3 >> (3 - b).
// Written branch-free on the comparison bits.
__device__ __forceinline__ int octant_cell(double x, double y) {
  const int ypos = y > 0.0, yzero = y == 0.0, xneg = x < 0.0, xzero = x == 0.0;
  const int hi = ypos | (yzero & (xneg ^ 1));             // theta in [0, pi)
  const int q_hi = (xneg | xzero) & ypos;                  // [pi/2, pi)
  const int q_lo = xneg ^ 1;                               // [-pi/2, 0)
  const int quarter = hi ? q_hi : q_lo;
  const double ax = fabs(x), ay = fabs(y);
  const int le = ay <= ax, ge = ay >= ax;
  const int sub = (quarter ? le : ge) & ((xzero & yzero) ^ 1);  // zero vector: theta = 0
  return (hi << 2) | (quarter << 1) | sub;
}

// fp64 -> fp16 bits (nearest, ties to even; beyond range saturates to 65504)
// for non-negative x: round to fp32 with round-to-odd (truncate, then set the
// last bit if anything was dropped), then round that to fp16.  With 13 spare
// bits in the fp32 significand the second rounding equals a single direct
// rounding of x.
__device__ __forceinline__ uint16_t f64_to_f16_rne_sat_nonneg(double x) {
  float f = static_cast<float>(x);                       // nearest
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  u -= (back > x) ? 1u : 0u;                             // now truncated toward zero
  u |= (static_cast<double>(__uint_as_float(u)) != x) ? 1u : 0u;  // sticky bit
  f = __uint_as_float(u);
  f = fminf(f, 65504.0f);                                // saturate (65504 is exact)
  return __half_as_ushort(__float2half_rn(f));
}

// G consecutive floats of LDS (vector reads for G = 2, 4, 8).
template <int G>
__device__ __forceinline__ void lds_fetch(const float* p, float (&v)[G]) {
  if constexpr (G == 1) {
    v[0] = p[0];
  } else if constexpr (G == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
#pragma unroll
    for (int k = 0; k < G; k += 4) {
      const float4 t = *reinterpret_cast<const float4*>(p + k);
      v[k] = t.x;
      v[k + 1] = t.y;
      v[k + 2] = t.z;
      v[k + 3] = t.w;
    }
  }
}

// Orders the LDS accesses of one wavefront around this point (wave-private
// LDS rows written by some lanes and read by others).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pgkq
