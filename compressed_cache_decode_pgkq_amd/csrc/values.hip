// Conversion between fp16 value rows ([token][channel]) and the value cache in
// 32-token tiles read by the decode kernels (the B-operand order of the
// matrix-core weighted sum; layout in mfma_pv.hpp).
//
// One thread per (stream, 8 tokens, channel): the 8 tokens of one channel are
// 16 contiguous bytes of the cache, and consecutive threads take consecutive
// channels, so both the row side (one 2-byte element per token row, a whole
// row per thread group) and the cache side (16-byte pieces) are coalesced.
#include "mfma_pv.hpp"

namespace pgkq {

namespace {

constexpr int kValuesThreads = 256;

__global__ void __launch_bounds__(kValuesThreads)
values_kernel(ValuesArgs a) {
  const int64_t groups = (a.slot_offset + a.n_tokens + 7) / 8 - a.slot_offset / 8;
  const int64_t idx = int64_t(blockIdx.x) * kValuesThreads + threadIdx.x;
  if (idx >= groups * a.d) return;
  const int c = static_cast<int>(idx % a.d);
  const int64_t t8 = (a.slot_offset / 8 + idx / a.d) * 8;  // first slot of the 8
  const int64_t lo = a.slot_offset, hi = a.slot_offset + a.n_tokens;  // slots of the rows
  const uint16_t* src = reinterpret_cast<const uint16_t*>(a.src);
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.dst);
  for (int64_t stream = blockIdx.y; stream < a.n_streams; stream += gridDim.y) {
    const size_t cache0 = size_t(stream) * a.capacity * a.d + vtile_index(t8, c, a.d);
    const size_t rows0 = size_t(stream) * a.n_tokens * a.d + c;
    if (!a.unpack) {
      if (t8 >= lo && t8 + 8 <= hi) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = uint32_t(src[rows0 + size_t(t8 + 2 * j - lo) * a.d]) |
                 (uint32_t(src[rows0 + size_t(t8 + 2 * j + 1 - lo) * a.d]) << 16);
        *reinterpret_cast<u32x4*>(dst + cache0) = u32x4{w[0], w[1], w[2], w[3]};
      } else {  // a partial group: slots outside the rows keep their contents
        for (int j = 0; j < 8; ++j)
          if (t8 + j >= lo && t8 + j < hi) dst[cache0 + j] = src[rows0 + size_t(t8 + j - lo) * a.d];
      }
    } else {
      for (int j = 0; j < 8; ++j)
        if (t8 + j >= lo && t8 + j < hi) dst[rows0 + size_t(t8 + j - lo) * a.d] = src[cache0 + j];
    }
  }
}

}  // namespace

hipError_t launch_values(const ValuesArgs& a, hipStream_t s) {
  const int64_t groups = (a.slot_offset + a.n_tokens + 7) / 8 - a.slot_offset / 8;
  const int64_t per_stream = groups * a.d;
  const dim3 grid(unsigned((per_stream + kValuesThreads - 1) / kValuesThreads),
                  unsigned(a.n_streams < 65535 ? a.n_streams : 65535));
  hipLaunchKernelGGL(values_kernel, grid, dim3(kValuesThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pgkq
