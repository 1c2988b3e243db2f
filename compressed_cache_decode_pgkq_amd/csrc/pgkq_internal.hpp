// Internal interface between the device layer (dispatch.hip) and the kernel
// translation units.  Not installed; the public interface is pgkq.h.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "host_iface.hpp"

namespace pgkq {

// the fp16 bit patterns of the argument blocks, typed for the kernels
inline const __half* as_half(const uint16_t* p) {
  return reinterpret_cast<const __half*>(p);
}

hipError_t launch_values(const ValuesArgs& a, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s);
hipError_t launch_encode(const Geometry& g, const EncodeArgs& a, hipStream_t s);
hipError_t launch_query_prep(const Geometry& g, const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_scan(const Geometry& g, const DecodeArgs& a, bool logits_mode,
                              hipStream_t s);
hipError_t launch_kv_decode_scan(const Geometry& g, const DecodeArgs& a, hipStream_t s);
hipError_t launch_kv_merge(const DecodeArgs& a, int d, int n_parts, hipStream_t s);
hipError_t launch_partial_merge(int d, int64_t n_seq, int64_t n_q, int n_splits,
                                const float* partial, float* out, hipStream_t s);
hipError_t launch_fp16_decode(const Fp16DecodeArgs& a, hipStream_t s);
hipError_t launch_rtn_encode(const RtnEncodeArgs& a, hipStream_t s);
hipError_t launch_rtn_query_prep(const RtnDecodeArgs& a, hipStream_t s);
hipError_t launch_rtn_scan(const RtnDecodeArgs& a, bool logits_mode, hipStream_t s);

}  // namespace pgkq
