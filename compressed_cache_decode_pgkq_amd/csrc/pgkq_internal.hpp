// Internal interface between the C-ABI host layer (pgkq_host.cpp) and the
// kernel translation units.  Not installed; the public interface is pgkq.h.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pgkq {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

struct Geometry {
  int d;        // head_dim
  int bm;       // radius bits
  int ba;       // angle bits
  int m;        // QJL sketch size (0 = off)
  int hadamard; // 1 = randomized Hadamard, 0 = identity
  int P() const { return bm + ba; }
  int n() const { return d / 2; }
  int code_words() const { return n() * P() / 32; }
  int words() const { return code_words() + m / 32; }
  size_t record_bytes() const { return size_t(4) * words() + (m ? 2 : 0); }
};

struct EncodeArgs {
  const void* K;
  int k_dtype;
  int hadamard;
  int64_t n_seq, n_kv, n_tokens, capacity, token_offset;
  const int8_t* signs;
  const uint16_t* perm;  // may be null
  const float* codebook; // [n_kv][2L]
  const float* S;        // [n_kv][m][d] or null
  uint8_t* codes;
  size_t stream_bytes;   // capacity * record_bytes
};

struct CalibArgs {
  const void* K;
  int k_dtype;
  int d;
  int64_t n_seq, n_kv, n_tokens;
  int64_t rows_per_chunk;
  int64_t chunks_per_seq;  // token chunks per (sequence, kv-head) stream
  int64_t n_chunks;        // chunks per kv-head = n_seq * chunks_per_seq
  double* partial;  // [n_kv][n_chunks][d]
  double* sumsq;    // [n_kv][d]
  uint16_t* perm;   // [n_kv][d] or null
  float* codebook;  // [n_kv][2L]
  int reorder;
  int L;
  double base_levels[16];
  double base_thresholds[16];
};

// Query preparation output per (sequence, query head), floats:
//   [ q~ (d) | angle LUT (n * A) | S q~ (m) | pad to a multiple of 4 ]
struct PrepLayout {
  int d, n, A, m;
  __host__ __device__ int off_lut() const { return d; }
  __host__ __device__ int off_sq() const { return d + n * A; }
  __host__ __device__ int stride() const { return ((d + n * A + m) + 3) & ~3; }
};

struct DecodeArgs {
  const void* q;
  int q_dtype;
  int hadamard;
  int64_t n_seq, n_q, n_kv, n_tokens, capacity;
  int group;            // n_q / n_kv
  const int8_t* signs;
  const uint16_t* perm;
  const float* codebook;
  const float* S;
  const uint8_t* codes;
  size_t stream_bytes;
  const __half* V;
  float* out;           // final output (n_splits == 1) or null
  float* logits;        // logits mode output or null
  float* prep;          // workspace: query prep
  float* partial;       // workspace: partial states [n_seq][n_q][n_splits][d + 4]
  int n_splits;         // workgroups per (sequence, kv-head)
  int64_t tokens_per_split;
  int wave_parts;       // 1: each wavefront scans a contiguous partition of the split
  int fused_prep;       // 1: the scan prepares the query itself (one workgroup per stream)
  float scale_log2;     // softmax scale * log2(e)
  // decode step: before the scan, the query-prep launch encodes k_new (one key
  // per stream) into slot append_slot of `codes_w` and copies v_new into the
  // same slot of `V_w` (append_slot < 0: no append)
  int64_t append_slot;
  const void* k_new;
  int k_dtype;
  const __half* v_new;
  uint8_t* codes_w;
  __half* V_w;
  // PGKQ-KV: values coded by the key encoder without the transform
  int bm_v;                 // 0: fp16 values in V
  const uint8_t* codes_v;
  size_t stream_bytes_v;
  const float* codebook_v;  // [n_kv][2 L_v]
  const float* S_v;         // [n_kv][d][d] or null
};

struct Fp16DecodeArgs {
  const void* q;
  int q_dtype;
  int d;
  int64_t n_seq, n_q, n_kv, n_tokens, capacity;
  int group;
  const __half* K;
  const __half* V;
  float* out;
  float* partial;
  int n_splits;
  int64_t tokens_per_split;
  int wave_parts;       // 1: each wavefront scans a contiguous partition of the split
  float scale_log2;
};

// Per-token asymmetric RTN key cache (the INT3 / INT4 control).
struct RtnEncodeArgs {
  const void* K;
  int k_dtype;
  int d, bits;
  int64_t n_seq, n_kv, n_tokens, capacity, token_offset;
  uint8_t* codes;
  size_t stream_bytes;   // capacity * record bytes
};

// RTN query preparation per (sequence, kv-head), floats:
//   [ q[c][g] for c < d, g < G | sum_c q[c][g] for g < G | pad to 4 ]
__host__ __device__ inline int rtn_prep_stride(int d, int G) { return (d * G + G + 3) & ~3; }

struct RtnDecodeArgs {
  const void* q;
  int q_dtype;
  int d, bits;
  int64_t n_seq, n_q, n_kv, n_tokens, capacity;
  int group;
  const uint8_t* codes;
  size_t stream_bytes;
  const __half* V;
  float* out;
  float* logits;
  float* prep;          // workspace: [n_seq][n_kv][rtn_prep_stride]
  float* partial;       // workspace: partial states
  int n_splits;
  int64_t tokens_per_split;
  int wave_parts;
  float scale_log2;
};

// fp16 value rows <-> the 32-token-tile value cache
struct ValuesArgs {
  const __half* src;
  __half* dst;
  int64_t n_streams;
  int64_t n_tokens;
  int64_t capacity;
  int64_t slot_offset;
  int d;
  bool unpack;  // false: rows -> cache, true: cache -> rows
};

hipError_t launch_values(const ValuesArgs& a, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s);
hipError_t launch_encode(const Geometry& g, const EncodeArgs& a, hipStream_t s);
// largest query-head group for which the scan can prepare the query itself
constexpr int kFusedPrepMaxGroup = 2;

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
