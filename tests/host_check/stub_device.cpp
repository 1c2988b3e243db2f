// Stand-in device layer for the host-only build of the C-ABI layer (abi.cpp):
// every dev_* call checks the argument block it is handed and records the
// call, but launches nothing.  Linked with abi.cpp under the address and
// undefined-behaviour sanitizers, it lets the CPU tests drive the library's
// validation and planning code (every error path of the ABI tests) with no
// GPU.  Test infrastructure only: the product library links dispatch.hip.
#include <cstdio>
#include <cstdlib>

#include "host_iface.hpp"

namespace {

int g_calls = 0;
unsigned char g_scratch_stand_in[256];

void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "host-check device layer: %s\n", what);
    std::abort();
  }
}

void check_decode(const pgkq::Geometry& g, const pgkq::DecodeArgs& a) {
  require(a.n_tokens >= 1 && a.n_tokens <= a.capacity, "decode: tokens within capacity");
  require(a.stream_bytes == size_t(a.capacity) * g.record_bytes(), "decode: stream bytes");
  require(a.n_splits >= 1 && a.tokens_per_split >= 64, "decode: split plan");
  require(int64_t(a.n_splits) * a.tokens_per_split >= a.n_tokens, "decode: splits cover the tokens");
  if (a.n_lead > 0) {  // front-loaded sizes: they cover the tokens and no split is empty
    const int64_t lead = int64_t(a.n_lead) * a.tokens_per_split;
    require(a.n_lead < a.n_splits && a.tail_split >= 64 && a.tokens_per_split >= a.tail_split,
            "decode: front-loaded sizes");
    require(lead + int64_t(a.n_splits - a.n_lead) * a.tail_split >= a.n_tokens,
            "decode: front-loaded splits cover the tokens");
    require(lead + int64_t(a.n_splits - a.n_lead - 1) * a.tail_split < a.n_tokens,
            "decode: every front-loaded split holds a token");
  }
  require(a.n_splits <= 65535, "decode: splits fit the grid");
  require(a.group * a.n_kv == a.n_q, "decode: query-head groups");
  require(a.prep && a.partial && a.codes && a.signs && a.codebook, "decode: pointers");
}

}  // namespace

namespace pgkq {

int dev_calibrate(const CalibArgs& a, void*) {
  require(a.n_chunks == a.n_seq * a.chunks_per_seq, "calibrate: chunk count");
  ++g_calls;
  return 0;
}
int dev_encode(const Geometry& g, const EncodeArgs& a, void*) {
  require(a.n_tokens >= 1 && a.token_offset + a.n_tokens <= a.capacity, "encode: slots");
  require(a.stream_bytes == size_t(a.capacity) * g.record_bytes(), "encode: stream bytes");
  ++g_calls;
  return 0;
}
int dev_query_prep(const Geometry& g, const DecodeArgs& a, void*) {
  check_decode(g, a);
  ++g_calls;
  return 0;
}
int dev_decode_scan(const Geometry& g, const DecodeArgs& a, bool, void*) {
  check_decode(g, a);
  ++g_calls;
  return 0;
}
int dev_kv_decode_scan(const Geometry& g, const DecodeArgs& a, void*) {
  check_decode(g, a);
  ++g_calls;
  return 0;
}
int dev_kv_merge(const DecodeArgs&, int, int n_parts, void*) {
  require(n_parts >= 1, "kv merge: partials");
  ++g_calls;
  return 0;
}
int dev_partial_merge(int, int64_t, int64_t, int n_splits, const float* partial, float* out, void*) {
  require(n_splits > 1 && partial && out, "merge: partials");
  ++g_calls;
  return 0;
}
int dev_fp16_decode(const Fp16DecodeArgs& a, void*) {
  require(int64_t(a.n_splits) * a.tokens_per_split >= a.n_tokens, "fp16 decode: split plan");
  ++g_calls;
  return 0;
}
int dev_rtn_encode(const RtnEncodeArgs& a, void*) {
  require(a.token_offset + a.n_tokens <= a.capacity, "rtn encode: slots");
  ++g_calls;
  return 0;
}
int dev_rtn_query_prep(const RtnDecodeArgs& a, void*) {
  require(a.prep && a.n_tokens >= 1, "rtn prep");
  ++g_calls;
  return 0;
}
int dev_rtn_scan(const RtnDecodeArgs& a, bool, void*) {
  require(int64_t(a.n_splits) * a.tokens_per_split >= a.n_tokens, "rtn scan: split plan");
  ++g_calls;
  return 0;
}
int dev_values(const ValuesArgs& a, void*) {
  require(a.slot_offset + a.n_tokens <= a.capacity, "values: slots");
  ++g_calls;
  return 0;
}
int dev_zero_fill(float* p, size_t n, void*) {
  require(p && n > 0, "zero fill");
  ++g_calls;
  return 0;
}
int dev_record_event(void* event, void*) {
  require(event != nullptr, "event");
  return 0;
}
int dev_stream_read(const void* src, uint64_t bytes, uint32_t* xor_out, void*) {
  require(src && xor_out && bytes % 16 == 0, "stream read");
  ++g_calls;
  return 0;
}
int dev_scratch(void** out) {
  *out = g_scratch_stand_in;
  return 0;
}

}  // namespace pgkq

extern "C" int pgkq_hostcheck_calls(void) { return g_calls; }
