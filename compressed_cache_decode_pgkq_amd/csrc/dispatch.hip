// Device layer of the PGKQ library: the dev_* calls of host_iface.hpp mapped
// onto the kernel launches, plus the pieces of the C ABI that use the HIP
// runtime directly (event records, the output fill of an empty decode, the
// built-in workspace of the allocation-free decode, the read probe).
#include <algorithm>
#include <mutex>

#include "device_common.hpp"
#include "pgkq.h"
#include "pgkq_internal.hpp"

namespace pgkq {

namespace {

int code(hipError_t e) { return static_cast<int>(e); }
hipStream_t hs(void* s) { return static_cast<hipStream_t>(s); }

__global__ void zero_fill_kernel(float* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

// Built-in workspace of pgkq_decode_attn_noalloc: a static device array, one
// copy per GPU (each holds it until the process ends).  Host code never uses
// the array's name as an address: its device address on each GPU is looked up
// once, with that GPU current, and kept in `ptr`.
static_assert(PGKQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[PGKQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchAddresses {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
ScratchAddresses g_scratch;

// Read probe: every workgroup reads one contiguous slice with 16-byte
// non-temporal buffer loads (the load path of the decode scans), kReadUnroll
// loads in flight per lane, and folds the words with XOR; the workgroup's fold
// is published with one atomic XOR, so no load can be dropped.  Offsets at or
// past the slice end read zero (the buffer range check), which XOR ignores.
// About two workgroups per CU: measured on the 1.32 GB decode cache, 4096
// workgroups each publishing per wavefront spent a quarter of the time in
// atomics on the one result word; 512 publishing once reach 6.9 TB/s.
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr uint32_t kReadStep = kReadThreads * 16 * kReadUnroll;  // bytes per iteration
constexpr uint64_t kReadSlices = 512;

__global__ void __launch_bounds__(kReadThreads)
stream_read_kernel(const uint8_t* __restrict__ src, uint64_t bytes, uint64_t slice,
                   uint32_t* xor_out) {
  __shared__ uint32_t s_fold[kReadThreads / kWave];
  const uint64_t begin = uint64_t(blockIdx.x) * slice;
  const uint32_t len = static_cast<uint32_t>(min(slice, bytes - begin));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + begin, len);
  uint32_t acc = 0;
  for (uint32_t off = threadIdx.x * 16u; off < len; off += kReadStep) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = buf_load_b128(rs, off + u * kReadThreads * 16u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o));
  if ((threadIdx.x & (kWave - 1)) == 0) s_fold[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / kWave; ++w) f ^= s_fold[w];
    atomicXor(xor_out, f);
  }
}

}  // namespace

int dev_calibrate(const CalibArgs& a, void* s) { return code(launch_calibrate(a, hs(s))); }
int dev_encode(const Geometry& g, const EncodeArgs& a, void* s) { return code(launch_encode(g, a, hs(s))); }
int dev_query_prep(const Geometry& g, const DecodeArgs& a, void* s) {
  return code(launch_query_prep(g, a, hs(s)));
}
int dev_decode_scan(const Geometry& g, const DecodeArgs& a, bool logits_mode, void* s) {
  return code(launch_decode_scan(g, a, logits_mode, hs(s)));
}
int dev_kv_decode_scan(const Geometry& g, const DecodeArgs& a, void* s) {
  return code(launch_kv_decode_scan(g, a, hs(s)));
}
int dev_kv_merge(const DecodeArgs& a, int d, int n_parts, void* s) {
  return code(launch_kv_merge(a, d, n_parts, hs(s)));
}
int dev_partial_merge(int d, int64_t n_seq, int64_t n_q, int n_splits, const float* partial,
                      float* out, void* s) {
  return code(launch_partial_merge(d, n_seq, n_q, n_splits, partial, out, hs(s)));
}
int dev_fp16_decode(const Fp16DecodeArgs& a, void* s) { return code(launch_fp16_decode(a, hs(s))); }
int dev_rtn_encode(const RtnEncodeArgs& a, void* s) { return code(launch_rtn_encode(a, hs(s))); }
int dev_rtn_query_prep(const RtnDecodeArgs& a, void* s) { return code(launch_rtn_query_prep(a, hs(s))); }
int dev_rtn_scan(const RtnDecodeArgs& a, bool logits_mode, void* s) {
  return code(launch_rtn_scan(a, logits_mode, hs(s)));
}
int dev_values(const ValuesArgs& a, void* s) { return code(launch_values(a, hs(s))); }

int dev_zero_fill(float* p, size_t n, void* s) {
  if (n == 0) return 0;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, hs(s), p, n);
  return code(hipGetLastError());
}

int dev_record_event(void* event, void* s) {
  return code(hipEventRecord(static_cast<hipEvent_t>(event), hs(s)));
}

int dev_stream_read(const void* src, uint64_t bytes, uint32_t* xor_out, void* s) {
  if (bytes == 0) return 0;
  // about kReadSlices slices of whole 32 KiB iterations (at least one)
  uint64_t slice = (bytes + kReadSlices - 1) / kReadSlices;
  slice = (slice + kReadStep - 1) / kReadStep * kReadStep;
  const uint64_t blocks = (bytes + slice - 1) / slice;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kReadThreads), 0,
                     hs(s), static_cast<const uint8_t*>(src), bytes, slice, xor_out);
  return code(hipGetLastError());
}

int dev_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return code(e);
  if (dev < 0 || dev >= kMaxDevices) return kDevTooManyDevices;
  std::lock_guard<std::mutex> lock(g_scratch.mu);
  if (!g_scratch.ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return code(e);
    if (!ptr) return code(hipErrorInvalidSymbol);
    g_scratch.ptr[dev] = ptr;
  }
  *out = g_scratch.ptr[dev];
  return 0;
}

}  // namespace pgkq
