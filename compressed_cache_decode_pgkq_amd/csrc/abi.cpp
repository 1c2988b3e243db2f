// C-ABI layer of the PGKQ library: argument validation, workspace sizing,
// split selection and the calls into the device layer, plus the host-side
// Lloyd-Max codebook for the Beta radius prior.  See include/pgkq.h for the
// contract.  Plain C++ (no HIP headers): every device action goes through the
// dev_* functions of host_iface.hpp.
#include "pgkq.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "host_iface.hpp"

namespace {

using pgkq::Geometry;

constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kCalibRows = 2048;  // token rows per calibration workgroup

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pgkq_status check_params(const pgkq_params* p, Geometry* g) {
  if (!p) return PGKQ_ERR_NULL;
  if (p->head_dim != 64 && p->head_dim != 128) return PGKQ_ERR_UNSUPPORTED;
  if (p->b_main < 2 || p->b_main > 4) return PGKQ_ERR_UNSUPPORTED;
  if (p->b_angle != p->b_main - 1) return PGKQ_ERR_UNSUPPORTED;
  if (p->qjl_m != 0 && p->qjl_m != p->head_dim) return PGKQ_ERR_UNSUPPORTED;
  if (p->hadamard != 0 && p->hadamard != 1) return PGKQ_ERR_UNSUPPORTED;
  if (g) *g = Geometry{p->head_dim, p->b_main, p->b_angle, p->qjl_m, p->hadamard};
  return PGKQ_OK;
}

pgkq_status check_dtype(pgkq_dtype t, bool allow_bf16) {
  if (t == PGKQ_F32 || t == PGKQ_F16) return PGKQ_OK;
  if (t == PGKQ_BF16 && allow_bf16) return PGKQ_OK;
  return PGKQ_ERR_UNSUPPORTED;
}

pgkq_status check_streams(int64_t n_seq, int64_t n_kv) {
  if (n_seq < 1 || n_kv < 1) return PGKQ_ERR_SHAPE;
  if (n_seq > kMaxGridYZ || n_kv > kMaxGridYZ) return PGKQ_ERR_SHAPE;
  return PGKQ_OK;
}

pgkq_status check_group(int64_t n_q, int64_t n_kv, int* group) {
  if (n_q < 1 || n_q % n_kv != 0) return PGKQ_ERR_SHAPE;
  const int64_t g = n_q / n_kv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PGKQ_ERR_UNSUPPORTED;
  if (n_q > kMaxGridYZ) return PGKQ_ERR_SHAPE;
  *group = static_cast<int>(g);
  return PGKQ_OK;
}

pgkq_status map_dev(int e) { return e == 0 ? PGKQ_OK : PGKQ_ERR_HIP; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The scans address one stream's codes and value rows through buffer
// resources with 32-bit byte ranges and offsets.
constexpr size_t kMaxStreamBytes = 0xFFFFFFF0u;
// fp16 value caches are stored in 32-token tiles: their capacity is a
// multiple of the tile.
constexpr int64_t kValueTile = 32;

bool fits_buffer(int64_t capacity, size_t record_bytes, int d) {
  return size_t(capacity) * record_bytes <= kMaxStreamBytes &&
         size_t(capacity) * size_t(d) * 2 <= kMaxStreamBytes;
}

struct Splits {
  int n;             // workgroups per (sequence, kv-head)
  int64_t tokens_per;  // tokens per workgroup
  int wave_parts;    // 1: one partition per wavefront (merged in the workgroup)
  int partials() const { return n; }
};

constexpr int kScanWaves = 4;

// Partitions of the token axis per (sequence, kv-head).  Automatic: with many
// streams, workgroup splits of at least 512 tokens whose wavefronts interleave
// 64-token chunks, about 1024 workgroups in total: two rounds of the 512 that
// are resident at once (2 per CU), which measured faster than one round (a
// long tail) or four (more table builds); with few long streams (fewer than
// 64), one partition per wavefront, about 2048 in total.
// A requested count is honoured as the number of partial states merged per
// query head; when its partitions are short (at most 1024 tokens) each
// workgroup runs four consecutive partitions, one per wavefront, sharing one
// build of the lookup tables.  A split holds at most kMaxSplitTokens tokens
// (more splits are used when the request would give longer ones): a lane then
// adds at most 1024 weights and 1024 weighted rows into its fp32 state, so a
// long run of equal terms, whose rounding errors all have the same sign,
// stays inside the output tolerance (over 16 777 184 identical tokens one
// split drifted by 1.1e-2, splits of 2^20 tokens by 1.2e-3).
constexpr int64_t kMaxSplitTokens = int64_t(1) << 18;

Splits choose_splits(int64_t n_units, int64_t n_tokens, int32_t requested,
                     bool allow_wave_parts = true) {
  if (requested == 0 && allow_wave_parts && n_units < 64) {
    requested = static_cast<int32_t>(
        std::min<int64_t>((2048 + n_units - 1) / n_units, std::max<int64_t>(1, n_tokens / 256)));
  }
  if (allow_wave_parts && requested >= 2 * kScanWaves) {
    int64_t tpw = (n_tokens + requested - 1) / requested;
    tpw = std::max<int64_t>(64, round_up(static_cast<size_t>(tpw), 64));
    if (tpw <= 1024) {
      const int64_t tps = kScanWaves * tpw;
      const int64_t ns = std::max<int64_t>(1, (n_tokens + tps - 1) / tps);
      return Splits{static_cast<int>(ns), tps, 1};
    }
  }
  int64_t ns = requested > 0 ? requested : (1024 + n_units - 1) / n_units;
  const int64_t min_tokens = requested > 0 ? 64 : 512;
  const int64_t max_ns = std::max<int64_t>(1, (n_tokens + min_tokens - 1) / min_tokens);
  ns = std::min<int64_t>(std::max<int64_t>(ns, 1), max_ns);
  int64_t tps = (n_tokens + ns - 1) / ns;
  tps = std::max<int64_t>(64, round_up(static_cast<size_t>(tps), 64));
  tps = std::min<int64_t>(tps, kMaxSplitTokens);
  ns = std::max<int64_t>(1, (n_tokens + tps - 1) / tps);
  return Splits{static_cast<int>(std::min<int64_t>(ns, 0x7FFFFFFF)), tps, 0};
}

// Front-loaded split sizes for the scans whose workgroups interleave over one
// split: with the grid ordered split-major (all streams' split 0 first), the
// first half of the split indices runs in the first rounds of resident
// workgroups and the second half last.  Giving the leading splits three times
// the tokens of the trailing ones leaves short workgroups for the end, where
// the workgroups that the memory system served slowest would otherwise hold
// the kernel open (32k-token GQA decode, 8 splits: scan 214.7-215.0 ->
// 208.9-210.3 us, whole call 224-225 -> 218.6-219.6 us).  Sizes stay
// multiples of 64 tokens and every split keeps at least one token; otherwise
// the splits stay uniform.
struct SplitSizes {
  int n_lead = 0;
  int64_t lead = 0, tail = 0;
};
SplitSizes front_load(const Splits& sp, int64_t n_tokens) {
  SplitSizes z;
  if (sp.wave_parts || sp.n < 2) return z;
  const int nl = sp.n / 2, nt = sp.n - nl;
  int64_t tail = (n_tokens + (3 * nl + nt) - 1) / (3 * nl + nt);
  tail = static_cast<int64_t>(round_up(static_cast<size_t>(tail), 64));
  const int64_t lead = 3 * tail;
  if (int64_t(nl) * lead + int64_t(nt - 1) * tail >= n_tokens) return z;  // a split would be empty
  if (lead > kMaxSplitTokens) return z;
  z.n_lead = nl;
  z.lead = lead;
  z.tail = tail;
  return z;
}

// Decode workspace: query prep | split partials, each region 256-byte aligned.
size_t decode_ws(const Geometry& g, int64_t n_seq, int64_t n_q, const Splits& sp) {
  const pgkq::PrepLayout pl{g.d, g.n(), 1 << g.ba, g.m};
  size_t bytes = round_up(size_t(n_seq) * n_q * pl.stride() * sizeof(float), 256);
  if (sp.partials() > 1) bytes += round_up(size_t(n_seq) * n_q * sp.partials() * (g.d + 4) * sizeof(float), 256);
  return bytes;
}

size_t fp16_ws(int d, int64_t n_seq, int64_t n_q, const Splits& sp) {
  if (sp.partials() <= 1) return 0;
  return round_up(size_t(n_seq) * n_q * sp.partials() * (d + 4) * sizeof(float), 256);
}

// ---------------------------------------------------------------- RTN control

pgkq_status check_rtn(int32_t head_dim, int32_t bits) {
  if (head_dim != 64 && head_dim != 128) return PGKQ_ERR_UNSUPPORTED;
  if (bits != 3 && bits != 4) return PGKQ_ERR_UNSUPPORTED;
  return PGKQ_OK;
}

size_t rtn_record(int d, int bits) { return size_t(d) * bits / 8 + 4; }

size_t rtn_ws(int d, int group, int64_t n_seq, int64_t n_q, int64_t n_kv, const Splits& sp) {
  size_t bytes = round_up(size_t(n_seq) * n_kv * pgkq::rtn_prep_stride(d, group) * sizeof(float), 256);
  if (sp.partials() > 1) bytes += round_up(size_t(n_seq) * n_q * sp.partials() * (d + 4) * sizeof(float), 256);
  return bytes;
}

// ---------------------------------------------------------------- Lloyd-Max

// Gauss-Legendre nodes and weights on [-1, 1] (Newton iteration on P_N).
void gauss_legendre(int N, std::vector<double>& x, std::vector<double>& w) {
  x.assign(N, 0.0);
  w.assign(N, 0.0);
  const double pi = 3.14159265358979323846;
  for (int i = 0; i < N; ++i) {
    double z = std::cos(pi * (i + 0.75) / (N + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = 0.0;
      for (int j = 1; j <= N; ++j) {
        const double p2 = p1;
        p1 = p0;
        p0 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p2) / j;
      }
      dp = N * (z * p0 - p1) / (z * z - 1.0);
      const double dz = p0 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-16) break;
    }
    x[i] = z;
    w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

// rho = (r/||k||) sqrt(n), n = d/2 pairs: F(rho) = 1 - (1 - rho^2/n)^(n-1);
// rho f(rho) = (2 (n-1)/n) rho^2 (1 - rho^2/n)^(n-2) is a polynomial of degree
// 2n - 2, so an (n + 4)-point Gauss-Legendre rule integrates it exactly.
struct BetaPrior {
  int n;
  std::vector<double> gx, gw;
  explicit BetaPrior(int n_) : n(n_) { gauss_legendre(n + 4, gx, gw); }
  double cdf(double rho) const {
    double u = rho * rho / n;
    if (u >= 1.0) return 1.0;
    return -std::expm1((n - 1) * std::log1p(-u));
  }
  double quantile(double p) const {
    const double u = -std::expm1(std::log1p(-p) / (n - 1));
    return std::sqrt(n * u);
  }
  double moment(double a, double b) const {
    const double half = 0.5 * (b - a), mid = 0.5 * (a + b);
    double s = 0.0;
    for (size_t i = 0; i < gx.size(); ++i) {
      const double r = mid + half * gx[i];
      const double u = 1.0 - r * r / n;
      s += gw[i] * r * r * std::pow(u, n - 2);
    }
    return half * s * (2.0 * (n - 1) / n);
  }
};

pgkq_status lloyd_max(int head_dim, int b_main, double* levels, double* thresholds) {
  const int n = head_dim / 2;
  const int L = 1 << b_main;
  BetaPrior pr(n);
  const double top = std::sqrt(double(n));
  std::vector<double> c(L), e(L + 1), cn(L);
  for (int j = 0; j < L; ++j) c[j] = pr.quantile((j + 0.5) / L);
  bool done = false;
  for (int it = 0; it < 200000 && !done; ++it) {
    e[0] = 0.0;
    e[L] = top;
    for (int j = 1; j < L; ++j) e[j] = 0.5 * (c[j - 1] + c[j]);
    double moved = 0.0;
    for (int j = 0; j < L; ++j) {
      const double P = pr.cdf(e[j + 1]) - pr.cdf(e[j]);
      cn[j] = pr.moment(e[j], e[j + 1]) / P;
      moved = std::max(moved, std::fabs(cn[j] - c[j]));
    }
    c = cn;
    done = moved < 1e-13;
  }
  if (!done) return PGKQ_ERR_UNSUPPORTED;
  for (int j = 0; j < L; ++j) levels[j] = c[j];
  for (int j = 0; j + 1 < L; ++j) thresholds[j] = 0.5 * (c[j] + c[j + 1]);
  return PGKQ_OK;
}

// Lloyd-Max on an empirical sample (the PGKQ-KV' refit).  The sample is
// sorted once; a cell is then a contiguous run of it: with thresholds t_j, the
// samples coded j (#{t : t < x} = j) are those with t_{j-1} < x <= t_j, whose
// end index is the upper bound of t_j.  Cell sums are compensated (Neumaier),
// so a level is its cell's mean to a few ulps whatever the cell size.
double cell_mean(const double* x, int64_t lo, int64_t hi) {
  double s = 0.0, comp = 0.0;
  for (int64_t i = lo; i < hi; ++i) {
    const double t = s + x[i];
    comp += std::fabs(s) >= std::fabs(x[i]) ? (s - t) + x[i] : (x[i] - t) + s;
    s = t;
  }
  return (s + comp) / double(hi - lo);
}

pgkq_status lloyd_max_samples(const double* samples, int64_t n, int b_main, double* levels,
                              double* thresholds) {
  const int L = 1 << b_main;
  std::vector<double> x(samples, samples + n);
  std::sort(x.begin(), x.end());
  std::vector<double> c(L), t(L - 1);
  std::vector<int64_t> end(L), prev_end(L, -1);
  for (int j = 0; j < L; ++j) c[j] = x[static_cast<int64_t>((j + 0.5) * double(n) / L)];
  bool done = false;
  for (int it = 0; it < 100000 && !done; ++it) {
    for (int j = 0; j + 1 < L; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
    for (int j = 0; j + 1 < L; ++j)
      end[j] = std::upper_bound(x.begin(), x.end(), t[j]) - x.begin();
    end[L - 1] = n;
    if (end == prev_end) {
      done = true;
      break;
    }
    int64_t lo = 0;
    for (int j = 0; j < L; ++j) {
      if (end[j] > lo) c[j] = cell_mean(x.data(), lo, end[j]);
      lo = std::max(lo, end[j]);
    }
    prev_end = end;
  }
  if (!done) return PGKQ_ERR_UNSUPPORTED;
  for (int j = 0; j < L; ++j) levels[j] = c[j];
  for (int j = 0; j + 1 < L; ++j) thresholds[j] = 0.5 * (c[j] + c[j + 1]);
  return PGKQ_OK;
}

struct TableCache {
  std::mutex mu;
  bool have[2][5] = {};
  double lv[2][5][16];
  double th[2][5][16];
};
TableCache g_tables;

pgkq_status unit_table(int d, int bm, double* lv, double* th) {
  const int di = d == 64 ? 0 : 1;
  std::lock_guard<std::mutex> lock(g_tables.mu);
  if (!g_tables.have[di][bm]) {
    pgkq_status st = lloyd_max(d, bm, g_tables.lv[di][bm], g_tables.th[di][bm]);
    if (st != PGKQ_OK) return st;
    g_tables.have[di][bm] = true;
  }
  std::memcpy(lv, g_tables.lv[di][bm], sizeof(double) * 16);
  std::memcpy(th, g_tables.th[di][bm], sizeof(double) * 16);
  return PGKQ_OK;
}

// Device address of the built-in workspace of pgkq_decode_attn_noalloc on the
// current device (looked up once per device by the device layer).
pgkq_status scratch_address(void** out) {
  const int e = pgkq::dev_scratch(out);
  if (e == pgkq::kDevTooManyDevices) return PGKQ_ERR_UNSUPPORTED;
  return e == 0 && *out ? PGKQ_OK : PGKQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char* pgkq_status_string(pgkq_status s) {
  switch (s) {
    case PGKQ_OK: return "ok";
    case PGKQ_ERR_NULL: return "null pointer";
    case PGKQ_ERR_SHAPE: return "invalid shape";
    case PGKQ_ERR_UNSUPPORTED: return "unsupported parameters";
    case PGKQ_ERR_ALIGN: return "misaligned pointer";
    case PGKQ_ERR_WORKSPACE: return "workspace too small";
    case PGKQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* pgkq_version(void) { return "pgkq-mi355x 0.1 (gfx950)"; }

pgkq_status pgkq_stream_read(const void* src, uint64_t bytes, uint32_t* xor_out, void* stream) {
  if (bytes == 0) return PGKQ_OK;
  if (!src || !xor_out) return PGKQ_ERR_NULL;
  if (bytes % 16 || bytes > (uint64_t(1) << 39)) return PGKQ_ERR_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(xor_out) & 3u)) return PGKQ_ERR_ALIGN;
  return map_dev(pgkq::dev_stream_read(src, bytes, xor_out, stream));
}

size_t pgkq_record_bytes(const pgkq_params* p) {
  Geometry g;
  if (check_params(p, &g) != PGKQ_OK) return 0;
  return g.record_bytes();
}

size_t pgkq_codes_bytes(const pgkq_params* p, int64_t n_streams, int64_t capacity) {
  const size_t rb = pgkq_record_bytes(p);
  if (rb == 0 || n_streams < 0 || capacity < 0) return 0;
  return rb * size_t(n_streams) * size_t(capacity);
}

pgkq_status pgkq_lloyd_max_beta(int32_t head_dim, int32_t b_main, double* levels_host,
                                double* thresholds_host) {
  if (!levels_host || !thresholds_host) return PGKQ_ERR_NULL;
  if (head_dim < 4 || head_dim > 4096 || (head_dim & 1)) return PGKQ_ERR_UNSUPPORTED;
  if (b_main < 1 || b_main > 8) return PGKQ_ERR_UNSUPPORTED;
  try {
    return lloyd_max(head_dim, b_main, levels_host, thresholds_host);
  } catch (...) {
    return PGKQ_ERR_HIP;
  }
}

pgkq_status pgkq_lloyd_max_empirical(const double* samples_host, int64_t n_samples,
                                     int32_t b_main, double* levels_host,
                                     double* thresholds_host) {
  if (!samples_host || !levels_host || !thresholds_host) return PGKQ_ERR_NULL;
  if (b_main < 1 || b_main > 8) return PGKQ_ERR_UNSUPPORTED;
  if (n_samples < (int64_t(1) << b_main)) return PGKQ_ERR_SHAPE;
  for (int64_t i = 0; i < n_samples; ++i)
    if (!std::isfinite(samples_host[i])) return PGKQ_ERR_UNSUPPORTED;
  try {
    return lloyd_max_samples(samples_host, n_samples, b_main, levels_host, thresholds_host);
  } catch (...) {
    return PGKQ_ERR_HIP;
  }
}

size_t pgkq_calibrate_workspace_bytes(const pgkq_params* p, int64_t n_seq, int64_t n_kv,
                                      int64_t n_tokens) {
  Geometry g;
  if (check_params(p, &g) != PGKQ_OK || n_seq < 1 || n_kv < 1 || n_tokens < 1) return 0;
  const int64_t chunks = n_seq * ((n_tokens + kCalibRows - 1) / kCalibRows);
  return round_up(size_t(n_kv) * chunks * g.d * sizeof(double), 256);
}

pgkq_status pgkq_calibrate(const pgkq_params* p, const void* K, pgkq_dtype k_dtype, int64_t n_seq,
                           int64_t n_kv, int64_t n_tokens, int32_t reorder, double* sumsq,
                           uint16_t* perm, float* codebook, void* workspace, size_t workspace_bytes,
                           void* stream) {
  Geometry g;
  pgkq_status st = check_params(p, &g);
  if (st != PGKQ_OK) return st;
  if (!K || !sumsq || !codebook || !workspace) return PGKQ_ERR_NULL;
  if (reorder && !perm) return PGKQ_ERR_NULL;
  if ((st = check_dtype(k_dtype, false)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  if (n_tokens < 1) return PGKQ_ERR_SHAPE;
  if (!aligned16(K) || !aligned16(sumsq) || !aligned16(codebook) || !aligned16(workspace) ||
      (perm && !aligned16(perm)))
    return PGKQ_ERR_ALIGN;
  const size_t need = pgkq_calibrate_workspace_bytes(p, n_seq, n_kv, n_tokens);
  if (workspace_bytes < need) return PGKQ_ERR_WORKSPACE;
  pgkq::CalibArgs a{};
  a.K = K;
  a.k_dtype = static_cast<int>(k_dtype);
  a.d = g.d;
  a.n_seq = n_seq;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.rows_per_chunk = kCalibRows;
  a.chunks_per_seq = (n_tokens + kCalibRows - 1) / kCalibRows;
  a.n_chunks = n_seq * a.chunks_per_seq;
  if (a.chunks_per_seq > 0x7FFFFFFF) return PGKQ_ERR_SHAPE;
  a.partial = static_cast<double*>(workspace);
  a.sumsq = sumsq;
  a.perm = perm;
  a.codebook = codebook;
  a.reorder = reorder ? 1 : 0;
  a.L = 1 << g.bm;
  st = unit_table(g.d, g.bm, a.base_levels, a.base_thresholds);
  if (st != PGKQ_OK) return st;
  return map_dev(pgkq::dev_calibrate(a, stream));
}

pgkq_status pgkq_encode(const pgkq_params* p, const void* K, pgkq_dtype k_dtype, int64_t n_seq,
                        int64_t n_kv, int64_t n_tokens, const int8_t* signs, const uint16_t* perm,
                        const float* codebook, const float* S, void* codes, int64_t capacity,
                        int64_t token_offset, void* stream) {
  Geometry g;
  pgkq_status st = check_params(p, &g);
  if (st != PGKQ_OK) return st;
  if (!K || !signs || !codebook || !codes) return PGKQ_ERR_NULL;
  if (g.m && !S) return PGKQ_ERR_NULL;
  if ((st = check_dtype(k_dtype, false)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  if (n_tokens < 0 || token_offset < 0 || capacity < 1) return PGKQ_ERR_SHAPE;
  if (token_offset + n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (g.m && (capacity & 1)) return PGKQ_ERR_SHAPE;  // keeps every stream 4-byte aligned
  if ((n_tokens + 63) / 64 > 0x7FFFFFFF) return PGKQ_ERR_SHAPE;
  if (!fits_buffer(capacity, g.record_bytes(), 0)) return PGKQ_ERR_SHAPE;
  if (!aligned16(K) || !aligned16(signs) || !aligned16(codebook) || !aligned16(codes) ||
      (perm && !aligned16(perm)) || (S && !aligned16(S)))
    return PGKQ_ERR_ALIGN;
  if (n_tokens == 0) return PGKQ_OK;
  pgkq::EncodeArgs a{};
  a.K = K;
  a.k_dtype = static_cast<int>(k_dtype);
  a.hadamard = g.hadamard;
  a.n_seq = n_seq;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.token_offset = token_offset;
  a.signs = signs;
  a.perm = perm;
  a.codebook = codebook;
  a.S = g.m ? S : nullptr;
  a.codes = static_cast<uint8_t*>(codes);
  a.stream_bytes = size_t(capacity) * g.record_bytes();
  return map_dev(pgkq::dev_encode(g, a, stream));
}

size_t pgkq_decode_workspace_bytes(const pgkq_params* p, int64_t n_seq, int64_t n_q, int64_t n_kv,
                                   int64_t n_tokens, const pgkq_launch_opts* opts) {
  Geometry g;
  if (check_params(p, &g) != PGKQ_OK || n_seq < 1 || n_q < 1 || n_kv < 1 || n_tokens < 0) return 0;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  return decode_ws(g, n_seq, n_q, sp);
}

// The new token of a decode step (pgkq_decode_step): appended at slot `slot`.
struct StepIn {
  const void* k_new;
  pgkq_dtype k_dtype;
  const void* v_new;
  int64_t slot;
};

static pgkq_status decode_common(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                                 int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                 int64_t capacity, const int8_t* signs, const uint16_t* perm,
                                 const float* codebook, const float* S, const void* codes,
                                 const void* V, float* out, float* logits, float softmax_scale,
                                 const pgkq_launch_opts* opts, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 const StepIn* step = nullptr, bool builtin_scratch = false) {
  Geometry g;
  pgkq_status st = check_params(p, &g);
  if (st != PGKQ_OK) return st;
  // the static scratch stands in for the workspace; its address is taken only
  // once every argument has been validated
  if (builtin_scratch) workspace_bytes = PGKQ_NOALLOC_SCRATCH_BYTES;
  if (step) {
    if (!step->k_new || !step->v_new) return PGKQ_ERR_NULL;
    if ((st = check_dtype(step->k_dtype, false)) != PGKQ_OK) return st;
    if (!aligned16(step->k_new) || !aligned16(step->v_new)) return PGKQ_ERR_ALIGN;
    if (step->slot < 0 || step->slot + 1 != n_tokens) return PGKQ_ERR_SHAPE;
  }
  const bool logits_mode = logits != nullptr;
  if (!q || !signs || !codebook || !codes || (!workspace && !builtin_scratch)) return PGKQ_ERR_NULL;
  if (!logits_mode && (!V || !out)) return PGKQ_ERR_NULL;
  if (g.m && !S) return PGKQ_ERR_NULL;
  if ((st = check_dtype(q_dtype, true)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  int group = 0;
  if ((st = check_group(n_q, n_kv, &group)) != PGKQ_OK) return st;
  if (n_tokens < 0 || capacity < 1 || n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (g.m && (capacity & 1)) return PGKQ_ERR_SHAPE;
  if (!logits_mode && capacity % kValueTile) return PGKQ_ERR_SHAPE;
  // the logit hook reads no value rows: only its code stream has to fit
  if (!fits_buffer(capacity, g.record_bytes(), logits_mode ? 0 : g.d)) return PGKQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(signs) || !aligned16(codebook) || !aligned16(codes) ||
      (!builtin_scratch && !aligned16(workspace)) || (perm && !aligned16(perm)) || (S && !aligned16(S)) ||
      (V && !aligned16(V)) || (out && !aligned16(out)) || (logits && !aligned16(logits)))
    return PGKQ_ERR_ALIGN;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  if (sp.n > kMaxGridYZ) return PGKQ_ERR_SHAPE;  // splits are a grid dimension
  if (workspace_bytes < decode_ws(g, n_seq, n_q, sp)) return PGKQ_ERR_WORKSPACE;
  if (builtin_scratch && (st = scratch_address(&workspace)) != PGKQ_OK) return st;
  void* s = stream;
  if (n_tokens == 0) {
    if (logits_mode) return PGKQ_OK;
    return map_dev(pgkq::dev_zero_fill(out, size_t(n_seq) * n_q * g.d, s));
  }
  const pgkq::PrepLayout pl{g.d, g.n(), 1 << g.ba, g.m};
  pgkq::DecodeArgs a{};
  a.q = q;
  a.q_dtype = static_cast<int>(q_dtype);
  a.hadamard = g.hadamard;
  a.n_seq = n_seq;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.group = group;
  a.signs = signs;
  a.perm = perm;
  a.codebook = codebook;
  a.S = g.m ? S : nullptr;
  a.codes = static_cast<const uint8_t*>(codes);
  a.stream_bytes = size_t(capacity) * g.record_bytes();
  a.V = static_cast<const uint16_t*>(V);
  a.out = out;
  a.logits = logits;
  a.prep = static_cast<float*>(workspace);
  a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       round_up(size_t(n_seq) * n_q * pl.stride() * 4, 256));
  a.n_splits = sp.n;
  a.tokens_per_split = sp.tokens_per;
  a.wave_parts = sp.wave_parts;
  {
    const SplitSizes fl = front_load(sp, n_tokens);
    if (fl.n_lead > 0) {
      a.n_lead = fl.n_lead;
      a.tokens_per_split = fl.lead;
      a.tail_split = fl.tail;
    }
  }
  // one workgroup per stream: the scan prepares the query itself (no extra
  // launch, nothing repeated); a decode step keeps the separate launch, which
  // also appends the new token
  a.fused_prep = (sp.n == 1 && !sp.wave_parts && !step && group <= pgkq::kFusedPrepMaxGroup) ? 1 : 0;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(g.d));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.append_slot = -1;
  if (step) {
    // the preparation launch holds n_q + n_kv grid rows
    if (n_q + n_kv > kMaxGridYZ) return PGKQ_ERR_SHAPE;
    a.append_slot = step->slot;
    a.k_new = step->k_new;
    a.k_dtype = static_cast<int>(step->k_dtype);
    a.v_new = static_cast<const uint16_t*>(step->v_new);
    a.codes_w = static_cast<uint8_t*>(const_cast<void*>(codes));
    a.V_w = static_cast<uint16_t*>(const_cast<void*>(V));
  }
  int e = 0;
  if (!a.fused_prep) {
    e = pgkq::dev_query_prep(g, a, s);
    if (e != 0) return PGKQ_ERR_HIP;
  }
  if (opts && opts->scan_start) {
    if (pgkq::dev_record_event(opts->scan_start, s) != 0)
      return PGKQ_ERR_HIP;
  }
  e = pgkq::dev_decode_scan(g, a, logits_mode, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_stop) {
    if (pgkq::dev_record_event(opts->scan_stop, s) != 0)
      return PGKQ_ERR_HIP;
  }
  if (!logits_mode && sp.partials() > 1) {
    e = pgkq::dev_partial_merge(g.d, n_seq, n_q, sp.partials(), a.partial, out, s);
    if (e != 0) return PGKQ_ERR_HIP;
  }
  return PGKQ_OK;
}

pgkq_status pgkq_decode_attn(const pgkq_params* p, const void* q, pgkq_dtype q_dtype, int64_t n_seq,
                             int64_t n_q, int64_t n_kv, int64_t n_tokens, int64_t capacity,
                             const int8_t* signs, const uint16_t* perm, const float* codebook,
                             const float* S, const void* codes, const void* V, float* out,
                             float softmax_scale, const pgkq_launch_opts* opts, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!out) return PGKQ_ERR_NULL;
  return decode_common(p, q, q_dtype, n_seq, n_q, n_kv, n_tokens, capacity, signs, perm, codebook,
                       S, codes, V, out, nullptr, softmax_scale, opts, workspace, workspace_bytes,
                       stream);
}

pgkq_status pgkq_decode_attn_noalloc(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                                     int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                     int64_t capacity, const int8_t* signs, const uint16_t* perm,
                                     const float* codebook, const float* S, const void* codes,
                                     const void* V, float* out, float softmax_scale,
                                     const pgkq_launch_opts* opts, void* stream) {
  if (!out) return PGKQ_ERR_NULL;
  return decode_common(p, q, q_dtype, n_seq, n_q, n_kv, n_tokens, capacity, signs, perm, codebook,
                       S, codes, V, out, nullptr, softmax_scale, opts, nullptr, 0, stream, nullptr,
                       true);
}

pgkq_status pgkq_decode_step(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                             const void* k_new, pgkq_dtype k_dtype, const void* v_new,
                             int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_cached,
                             int64_t capacity, const int8_t* signs, const uint16_t* perm,
                             const float* codebook, const float* S, void* codes, void* V,
                             float* out, float softmax_scale, const pgkq_launch_opts* opts,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !codes || !V) return PGKQ_ERR_NULL;
  if (n_cached < 0 || n_cached >= capacity) return PGKQ_ERR_SHAPE;
  const StepIn step{k_new, k_dtype, v_new, n_cached};
  return decode_common(p, q, q_dtype, n_seq, n_q, n_kv, n_cached + 1, capacity, signs, perm,
                       codebook, S, codes, V, out, nullptr, softmax_scale, opts, workspace,
                       workspace_bytes, stream, &step);
}

// ---------------------------------------------------------------- PGKQ-KV

static pgkq_status check_kv(const pgkq_params* pk, const pgkq_params* pv, Geometry* gk,
                            Geometry* gv) {
  pgkq_status st = check_params(pk, gk);
  if (st != PGKQ_OK) return st;
  if ((st = check_params(pv, gv)) != PGKQ_OK) return st;
  if (gv->d != gk->d || gv->hadamard != 0) return PGKQ_ERR_UNSUPPORTED;
  if ((gv->m != 0) != (gk->m != 0)) return PGKQ_ERR_UNSUPPORTED;
  const int k = gk->bm, v = gv->bm;
  const bool pair_ok = (k == v) || (v == 2 && (k == 3 || k == 4));
  return pair_ok ? PGKQ_OK : PGKQ_ERR_UNSUPPORTED;
}

static size_t kv_ws(const Geometry& gk, int64_t n_seq, int64_t n_q, const Splits& sp) {
  const pgkq::PrepLayout pl{gk.d, gk.n(), 1 << gk.ba, gk.m};
  return round_up(size_t(n_seq) * n_q * pl.stride() * sizeof(float), 256) +
         round_up(size_t(n_seq) * n_q * sp.partials() * (2 * gk.d + 4) * sizeof(float), 256);
}

size_t pgkq_kv_decode_workspace_bytes(const pgkq_params* pk, const pgkq_params* pv, int64_t n_seq,
                                      int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                      const pgkq_launch_opts* opts) {
  Geometry gk, gv;
  if (check_kv(pk, pv, &gk, &gv) != PGKQ_OK || n_seq < 1 || n_q < 1 || n_kv < 1 || n_tokens < 0)
    return 0;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  return kv_ws(gk, n_seq, n_q, sp);
}

pgkq_status pgkq_kv_decode_attn(const pgkq_params* pk, const pgkq_params* pv, const void* q,
                                pgkq_dtype q_dtype, int64_t n_seq, int64_t n_q, int64_t n_kv,
                                int64_t n_tokens, int64_t capacity, const int8_t* signs,
                                const uint16_t* perm, const float* codebook_k, const float* S_k,
                                const void* codes_k, const float* codebook_v, const float* S_v,
                                const void* codes_v, float* out, float softmax_scale,
                                const pgkq_launch_opts* opts, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Geometry g, gv;
  pgkq_status st = check_kv(pk, pv, &g, &gv);
  if (st != PGKQ_OK) return st;
  if (!q || !signs || !codebook_k || !codes_k || !codebook_v || !codes_v || !out || !workspace)
    return PGKQ_ERR_NULL;
  if (g.m && (!S_k || !S_v)) return PGKQ_ERR_NULL;
  if ((st = check_dtype(q_dtype, true)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  int group = 0;
  if ((st = check_group(n_q, n_kv, &group)) != PGKQ_OK) return st;
  if (n_tokens < 0 || capacity < 1 || n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (g.m && (capacity & 1)) return PGKQ_ERR_SHAPE;
  if (!fits_buffer(capacity, std::max(g.record_bytes(), gv.record_bytes()), 0))
    return PGKQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(signs) || !aligned16(codebook_k) || !aligned16(codes_k) ||
      !aligned16(codebook_v) || !aligned16(codes_v) || !aligned16(out) || !aligned16(workspace) ||
      (perm && !aligned16(perm)) || (S_k && !aligned16(S_k)) || (S_v && !aligned16(S_v)))
    return PGKQ_ERR_ALIGN;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  if (sp.n > kMaxGridYZ) return PGKQ_ERR_SHAPE;  // splits are a grid dimension
  if (workspace_bytes < kv_ws(g, n_seq, n_q, sp)) return PGKQ_ERR_WORKSPACE;
  void* s = stream;
  if (n_tokens == 0) return map_dev(pgkq::dev_zero_fill(out, size_t(n_seq) * n_q * g.d, s));
  const pgkq::PrepLayout pl{g.d, g.n(), 1 << g.ba, g.m};
  pgkq::DecodeArgs a{};
  a.q = q;
  a.q_dtype = static_cast<int>(q_dtype);
  a.hadamard = g.hadamard;
  a.n_seq = n_seq;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.group = group;
  a.signs = signs;
  a.perm = perm;
  a.codebook = codebook_k;
  a.S = g.m ? S_k : nullptr;
  a.codes = static_cast<const uint8_t*>(codes_k);
  a.stream_bytes = size_t(capacity) * g.record_bytes();
  a.out = out;
  a.prep = static_cast<float*>(workspace);
  a.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       round_up(size_t(n_seq) * n_q * pl.stride() * 4, 256));
  a.n_splits = sp.n;
  a.tokens_per_split = sp.tokens_per;
  a.wave_parts = sp.wave_parts;
  {
    const SplitSizes fl = front_load(sp, n_tokens);
    if (fl.n_lead > 0) {
      a.n_lead = fl.n_lead;
      a.tokens_per_split = fl.lead;
      a.tail_split = fl.tail;
    }
  }
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(g.d));
  a.scale_log2 = scale * 1.4426950408889634f;
  a.append_slot = -1;
  a.bm_v = gv.bm;
  a.codes_v = static_cast<const uint8_t*>(codes_v);
  a.stream_bytes_v = size_t(capacity) * gv.record_bytes();
  a.codebook_v = codebook_v;
  a.S_v = gv.m ? S_v : nullptr;
  int e = pgkq::dev_query_prep(g, a, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_start) {
    if (pgkq::dev_record_event(opts->scan_start, s) != 0)
      return PGKQ_ERR_HIP;
  }
  e = pgkq::dev_kv_decode_scan(g, a, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_stop) {
    if (pgkq::dev_record_event(opts->scan_stop, s) != 0)
      return PGKQ_ERR_HIP;
  }
  return map_dev(pgkq::dev_kv_merge(a, g.d, sp.partials(), s));
}

pgkq_status pgkq_estimate_logits(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                                 int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                 int64_t capacity, const int8_t* signs, const uint16_t* perm,
                                 const float* codebook, const float* S, const void* codes,
                                 float* logits, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!logits) return PGKQ_ERR_NULL;
  return decode_common(p, q, q_dtype, n_seq, n_q, n_kv, n_tokens, capacity, signs, perm, codebook,
                       S, codes, nullptr, nullptr, logits, 0.f, nullptr, workspace,
                       workspace_bytes, stream);
}

size_t pgkq_fp16_decode_workspace_bytes(int32_t head_dim, int64_t n_seq, int64_t n_q,
                                        int64_t n_kv, int64_t n_tokens,
                                        const pgkq_launch_opts* opts) {
  if ((head_dim != 64 && head_dim != 128) || n_seq < 1 || n_q < 1 || n_kv < 1 || n_tokens < 0)
    return 0;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  return fp16_ws(head_dim, n_seq, n_q, sp);
}

static pgkq_status values_common(const void* src, void* dst, int64_t n_streams, int64_t n_tokens,
                                 int32_t head_dim, int64_t capacity, int64_t slot_offset,
                                 bool unpack, void* stream) {
  if (head_dim < 16 || head_dim > 1024 || head_dim % 16) return PGKQ_ERR_UNSUPPORTED;
  if (n_streams < 0 || n_tokens < 0 || slot_offset < 0 || capacity < 0) return PGKQ_ERR_SHAPE;
  if (capacity % kValueTile || slot_offset + n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (size_t(capacity) * size_t(head_dim) * 2 > kMaxStreamBytes) return PGKQ_ERR_SHAPE;
  if (n_streams == 0 || n_tokens == 0) return PGKQ_OK;  // nothing to move
  if (!src || !dst) return PGKQ_ERR_NULL;
  if (!aligned16(unpack ? src : dst) || (reinterpret_cast<uintptr_t>(unpack ? dst : src) & 1u))
    return PGKQ_ERR_ALIGN;
  pgkq::ValuesArgs a{};
  a.src = static_cast<const uint16_t*>(src);
  a.dst = static_cast<uint16_t*>(dst);
  a.n_streams = n_streams;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.slot_offset = slot_offset;
  a.d = head_dim;
  a.unpack = unpack;
  return map_dev(pgkq::dev_values(a, stream));
}

pgkq_status pgkq_pack_values(const void* rows, int64_t n_streams, int64_t n_tokens, int32_t head_dim,
                             void* cache, int64_t capacity, int64_t slot_offset, void* stream) {
  return values_common(rows, cache, n_streams, n_tokens, head_dim, capacity, slot_offset, false,
                       stream);
}

pgkq_status pgkq_unpack_values(const void* cache, int64_t n_streams, int64_t capacity,
                               int32_t head_dim, int64_t slot_offset, int64_t n_tokens, void* rows,
                               void* stream) {
  return values_common(cache, rows, n_streams, n_tokens, head_dim, capacity, slot_offset, true,
                       stream);
}

pgkq_status pgkq_fp16_decode_attn(const void* q, pgkq_dtype q_dtype, int64_t n_seq, int64_t n_q,
                                  int64_t n_kv, int64_t n_tokens, int64_t capacity,
                                  int32_t head_dim, const void* K16, const void* V16, float* out,
                                  float softmax_scale, const pgkq_launch_opts* opts,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (head_dim != 64 && head_dim != 128) return PGKQ_ERR_UNSUPPORTED;
  if (!q || !K16 || !V16 || !out) return PGKQ_ERR_NULL;
  pgkq_status st;
  if ((st = check_dtype(q_dtype, true)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  int group = 0;
  if ((st = check_group(n_q, n_kv, &group)) != PGKQ_OK) return st;
  if (n_tokens < 0 || capacity < 1 || n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (capacity % kValueTile) return PGKQ_ERR_SHAPE;
  if (!fits_buffer(capacity, 0, head_dim)) return PGKQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(K16) || !aligned16(V16) || !aligned16(out) ||
      (workspace && !aligned16(workspace)))
    return PGKQ_ERR_ALIGN;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  if (sp.n > kMaxGridYZ) return PGKQ_ERR_SHAPE;  // splits are a grid dimension
  const size_t need = fp16_ws(head_dim, n_seq, n_q, sp);
  if (need && (!workspace || workspace_bytes < need)) return PGKQ_ERR_WORKSPACE;
  void* s = stream;
  if (n_tokens == 0) return map_dev(pgkq::dev_zero_fill(out, size_t(n_seq) * n_q * head_dim, s));
  pgkq::Fp16DecodeArgs a{};
  a.q = q;
  a.q_dtype = static_cast<int>(q_dtype);
  a.d = head_dim;
  a.n_seq = n_seq;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.group = group;
  a.K = static_cast<const uint16_t*>(K16);
  a.V = static_cast<const uint16_t*>(V16);
  a.out = out;
  a.partial = static_cast<float*>(workspace);
  a.n_splits = sp.n;
  a.tokens_per_split = sp.tokens_per;
  a.wave_parts = sp.wave_parts;
  {
    const SplitSizes fl = front_load(sp, n_tokens);
    if (fl.n_lead > 0) {
      a.n_lead = fl.n_lead;
      a.tokens_per_split = fl.lead;
      a.tail_split = fl.tail;
    }
  }
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
  a.scale_log2 = scale * 1.4426950408889634f;
  if (opts && opts->scan_start) {
    if (pgkq::dev_record_event(opts->scan_start, s) != 0)
      return PGKQ_ERR_HIP;
  }
  int e = pgkq::dev_fp16_decode(a, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_stop) {
    if (pgkq::dev_record_event(opts->scan_stop, s) != 0)
      return PGKQ_ERR_HIP;
  }
  if (sp.partials() > 1)
    return map_dev(pgkq::dev_partial_merge(head_dim, n_seq, n_q, sp.partials(), a.partial, out, s));
  return PGKQ_OK;
}

size_t pgkq_rtn_record_bytes(int32_t head_dim, int32_t bits) {
  if (check_rtn(head_dim, bits) != PGKQ_OK) return 0;
  return rtn_record(head_dim, bits);
}

pgkq_status pgkq_rtn_encode(int32_t head_dim, int32_t bits, const void* K, pgkq_dtype k_dtype,
                            int64_t n_seq, int64_t n_kv, int64_t n_tokens, void* codes,
                            int64_t capacity, int64_t token_offset, void* stream) {
  pgkq_status st = check_rtn(head_dim, bits);
  if (st != PGKQ_OK) return st;
  if (!K || !codes) return PGKQ_ERR_NULL;
  if ((st = check_dtype(k_dtype, false)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  if (n_tokens < 0 || token_offset < 0 || capacity < 1) return PGKQ_ERR_SHAPE;
  if (token_offset + n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if ((n_tokens + 255) / 256 > 0x7FFFFFFF) return PGKQ_ERR_SHAPE;
  if (!aligned16(K) || !aligned16(codes)) return PGKQ_ERR_ALIGN;
  if (n_tokens == 0) return PGKQ_OK;
  pgkq::RtnEncodeArgs a{};
  a.K = K;
  a.k_dtype = static_cast<int>(k_dtype);
  a.d = head_dim;
  a.bits = bits;
  a.n_seq = n_seq;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.token_offset = token_offset;
  a.codes = static_cast<uint8_t*>(codes);
  a.stream_bytes = size_t(capacity) * rtn_record(head_dim, bits);
  return map_dev(pgkq::dev_rtn_encode(a, stream));
}

size_t pgkq_rtn_decode_workspace_bytes(int32_t head_dim, int64_t n_seq, int64_t n_q, int64_t n_kv,
                                       int64_t n_tokens, const pgkq_launch_opts* opts) {
  if ((head_dim != 64 && head_dim != 128) || n_seq < 1 || n_q < 1 || n_kv < 1 || n_tokens < 0)
    return 0;
  int group = 0;
  if (check_group(n_q, n_kv, &group) != PGKQ_OK) return 0;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  return rtn_ws(head_dim, group, n_seq, n_q, n_kv, sp);
}

static pgkq_status rtn_decode_common(int32_t head_dim, int32_t bits, const void* q,
                                     pgkq_dtype q_dtype, int64_t n_seq, int64_t n_q, int64_t n_kv,
                                     int64_t n_tokens, int64_t capacity, const void* codes,
                                     const void* V, float* out, float* logits, float softmax_scale,
                                     const pgkq_launch_opts* opts, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  pgkq_status st = check_rtn(head_dim, bits);
  if (st != PGKQ_OK) return st;
  const bool logits_mode = logits != nullptr;
  if (!q || !codes || !workspace) return PGKQ_ERR_NULL;
  if (!logits_mode && (!V || !out)) return PGKQ_ERR_NULL;
  if ((st = check_dtype(q_dtype, true)) != PGKQ_OK) return st;
  if ((st = check_streams(n_seq, n_kv)) != PGKQ_OK) return st;
  int group = 0;
  if ((st = check_group(n_q, n_kv, &group)) != PGKQ_OK) return st;
  if (n_tokens < 0 || capacity < 1 || n_tokens > capacity) return PGKQ_ERR_SHAPE;
  if (!logits_mode && capacity % kValueTile) return PGKQ_ERR_SHAPE;
  if (!fits_buffer(capacity, rtn_record(head_dim, bits), head_dim)) return PGKQ_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(codes) || !aligned16(workspace) || (V && !aligned16(V)) ||
      (out && !aligned16(out)) || (logits && !aligned16(logits)))
    return PGKQ_ERR_ALIGN;
  const Splits sp = choose_splits(n_seq * n_kv, std::max<int64_t>(n_tokens, 1),
                                  opts ? opts->n_splits : 0);
  if (sp.n > kMaxGridYZ) return PGKQ_ERR_SHAPE;  // splits are a grid dimension
  if (workspace_bytes < rtn_ws(head_dim, group, n_seq, n_q, n_kv, sp)) return PGKQ_ERR_WORKSPACE;
  void* s = stream;
  if (n_tokens == 0) {
    if (logits_mode) return PGKQ_OK;
    return map_dev(pgkq::dev_zero_fill(out, size_t(n_seq) * n_q * head_dim, s));
  }
  pgkq::RtnDecodeArgs a{};
  a.q = q;
  a.q_dtype = static_cast<int>(q_dtype);
  a.d = head_dim;
  a.bits = bits;
  a.n_seq = n_seq;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.n_tokens = n_tokens;
  a.capacity = capacity;
  a.group = group;
  a.codes = static_cast<const uint8_t*>(codes);
  a.stream_bytes = size_t(capacity) * rtn_record(head_dim, bits);
  a.V = static_cast<const uint16_t*>(V);
  a.out = out;
  a.logits = logits;
  a.prep = static_cast<float*>(workspace);
  a.partial = reinterpret_cast<float*>(
      static_cast<char*>(workspace) +
      round_up(size_t(n_seq) * n_kv * pgkq::rtn_prep_stride(head_dim, group) * 4, 256));
  a.n_splits = sp.n;
  a.tokens_per_split = sp.tokens_per;
  a.wave_parts = sp.wave_parts;
  {
    const SplitSizes fl = front_load(sp, n_tokens);
    if (fl.n_lead > 0) {
      a.n_lead = fl.n_lead;
      a.tokens_per_split = fl.lead;
      a.tail_split = fl.tail;
    }
  }
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt(float(head_dim));
  a.scale_log2 = scale * 1.4426950408889634f;
  int e = pgkq::dev_rtn_query_prep(a, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_start) {
    if (pgkq::dev_record_event(opts->scan_start, s) != 0)
      return PGKQ_ERR_HIP;
  }
  e = pgkq::dev_rtn_scan(a, logits_mode, s);
  if (e != 0) return PGKQ_ERR_HIP;
  if (opts && opts->scan_stop) {
    if (pgkq::dev_record_event(opts->scan_stop, s) != 0)
      return PGKQ_ERR_HIP;
  }
  if (!logits_mode && sp.partials() > 1) {
    e = pgkq::dev_partial_merge(head_dim, n_seq, n_q, sp.partials(), a.partial, out, s);
    if (e != 0) return PGKQ_ERR_HIP;
  }
  return PGKQ_OK;
}

pgkq_status pgkq_rtn_decode_attn(int32_t head_dim, int32_t bits, const void* q, pgkq_dtype q_dtype,
                                 int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                 int64_t capacity, const void* codes, const void* V, float* out,
                                 float softmax_scale, const pgkq_launch_opts* opts,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!out) return PGKQ_ERR_NULL;
  return rtn_decode_common(head_dim, bits, q, q_dtype, n_seq, n_q, n_kv, n_tokens, capacity, codes,
                           V, out, nullptr, softmax_scale, opts, workspace, workspace_bytes, stream);
}

pgkq_status pgkq_rtn_logits(int32_t head_dim, int32_t bits, const void* q, pgkq_dtype q_dtype,
                            int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                            int64_t capacity, const void* codes, float* logits, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!logits) return PGKQ_ERR_NULL;
  return rtn_decode_common(head_dim, bits, q, q_dtype, n_seq, n_q, n_kv, n_tokens, capacity, codes,
                           nullptr, nullptr, logits, 0.f, nullptr, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"
