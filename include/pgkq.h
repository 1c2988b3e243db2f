/*
 * pgkq.h - C ABI of the PGKQ compressed-key cache library for AMD Instinct
 * MI355X (gfx950).
 *
 * PGKQ (polar-guided key-cache quantization) is described on the EdgeLLM-Nano
 * paper page (signal-papers read view of arXiv 2610.14475), paragraph "PGKQ
 * pipeline" and the codebook paragraph after it, with the record size fixed by
 * the "Bit budget" paragraph.  Per key vector k of one (layer, kv-head):
 *   (0) optional channel reorder by decreasing l2 norm, high/low interleaved;
 *   (1) randomized Hadamard transform k~ = H (signs * k[perm]) / sqrt(d);
 *   (2) adjacent pairs (k~[2i], k~[2i+1]) -> polar radius r_i and angle theta_i;
 *   (3) r_i -> b_main-bit Lloyd-Max code (Beta prior), theta_i -> b_angle-bit
 *       code on a uniform mid-rise grid over [-pi, pi], b_angle = b_main - 1;
 *   (4) optional QJL residual: signs of S_h (k~ - k~hat) (m = head_dim bits)
 *       plus one fp16 residual norm.
 * Decode never rebuilds the keys: logits come from per-query lookup tables over
 * the codes plus the QJL correction, then softmax and the FP16-V weighted sum.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers unless the argument says "host".
 *    The caller owns all memory; the library allocates no device memory and
 *    keeps no device state between calls.  Its only state is a host-side
 *    cache of the unit Lloyd-Max tables (a function of head_dim and b_main
 *    alone, filled on first use under a mutex), so calls are thread-safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; results are valid after the stream syncs.
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error the function returns a non-zero pgkq_status and enqueues nothing.
 *    A HIP launch error maps to PGKQ_ERR_HIP.  No C++ exception crosses this ABI.
 *  - Device pointers must be 16-byte aligned.
 *  - One stream's codes and one stream's value rows (capacity * d * 2 bytes)
 *    must each stay under 4 GiB (the scans use 32-bit buffer offsets);
 *    larger capacities are rejected with PGKQ_ERR_SHAPE.
 *  - n_tokens == 0 is a valid no-op (outputs untouched, except that decode
 *    attention writes zeros to `out` because an empty softmax has no weights).
 *  - fp16 value caches ("V" below) are stored in 32-TOKEN TILES, the operand
 *    order of the matrix-core weighted sum: stream (b, h) holds `capacity`
 *    slots (capacity a multiple of 32, else PGKQ_ERR_SHAPE), and element
 *    (t, c) of it sits at half-word
 *      (t/32) 32 d + ((c/16) 4 + (t%32)/8) 128 + (c%16) 8 + t%8
 *    (16 contiguous bytes hold 8 consecutive tokens of one channel).  Streams
 *    lie back to back in [n_seq][n_kv] order, capacity * d half-words each.
 *    pgkq_pack_values / pgkq_unpack_values convert from / to plain rows.  Slots
 *    at or beyond n_tokens may hold any bits; they are never weighted.
 *
 * Code layout of one (sequence, kv-head) stream with room for `capacity` tokens
 * (exactly pgkq_record_bytes() bytes per token slot):
 *    P = b_main + b_angle bits per pair; joint code c_i = rc_i | (ac_i << b_main);
 *    per token a code stream of (d/2) P bits, c_i at bits [P i, P i + P), LSB
 *      first, in NC = (d/2) P / 32 uint32 words (bit q in word q/32, bit q%32);
 *    then, with QJL, m/32 sign words (bit j of the sketch in word j/32, bit j%32);
 *    word w of token t is stored at byte 4 (w capacity + t) of the stream;
 *    with QJL a row of `capacity` fp16 residual norms follows the words.
 *  Streams are stored back to back in [n_seq][n_kv] order, capacity * record
 *  bytes each.
 *
 * Per-kv-head inputs, shared by all sequences:
 *    signs    [n_kv][d]     int8, +1 / -1 (Rademacher vector of the transform)
 *    perm     [n_kv][d]     uint16 channel order of step (0), or NULL = identity
 *    codebook [n_kv][2L]    fp32, L = 2^b_main: L radius levels (ascending),
 *                           L-1 thresholds (a radius r gets code #{j : T_j < r}),
 *                           one unused pad; absolute radius units
 *    S        [n_kv][m][d]  fp32 QJL projection, NULL iff qjl_m == 0
 */
#ifndef PGKQ_H
#define PGKQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pgkq_status {
  PGKQ_OK = 0,
  PGKQ_ERR_NULL = 1,        /* a required pointer is NULL                       */
  PGKQ_ERR_SHAPE = 2,       /* a size is negative, inconsistent or out of range */
  PGKQ_ERR_UNSUPPORTED = 3, /* parameter combination the library does not build */
  PGKQ_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned          */
  PGKQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  PGKQ_ERR_HIP = 6          /* the HIP runtime reported an error                */
} pgkq_status;

typedef enum pgkq_dtype { PGKQ_F32 = 0, PGKQ_F16 = 1, PGKQ_BF16 = 2 } pgkq_dtype;

typedef struct pgkq_params {
  int32_t head_dim; /* d: 64 or 128                                              */
  int32_t b_main;   /* radius code bits: 2, 3 or 4                              */
  int32_t b_angle;  /* angle code bits: must equal b_main - 1                   */
  int32_t qjl_m;    /* QJL sketch size: 0 (off) or head_dim                     */
  int32_t hadamard; /* 1: randomized Hadamard transform; 0: identity transform  */
                    /*    (the "without Hadamard" ablation)                     */
} pgkq_params;

/* Optional launch settings; a NULL pointer means all defaults. */
typedef struct pgkq_launch_opts {
  int32_t n_splits;  /* token splits per (sequence, kv-head); 0 = automatic      */
  void* scan_start;  /* hipEvent_t recorded just before the token-scan kernel    */
  void* scan_stop;   /* hipEvent_t recorded just after it (both NULL = none)    */
} pgkq_launch_opts;

/* Human-readable name of a status code (static string). */
const char* pgkq_status_string(pgkq_status s);

/* Library version string (static). */
const char* pgkq_version(void);

/* Bytes of one token slot of one stream (30 at d=64, b_main=3, QJL m=64; the
 * record size of the "Bit budget" paragraph).  0 if the parameters are invalid. */
size_t pgkq_record_bytes(const pgkq_params* p);

/* Bytes of a code buffer holding n_streams streams of `capacity` slots
 * (record bytes of the "Bit budget" paragraph times slots times streams). */
size_t pgkq_codes_bytes(const pgkq_params* p, int64_t n_streams, int64_t capacity);

/* Host routine.  Lloyd-Max quantizer of rho = (r / ||k||) sqrt(d/2) under the
 * Beta(1, d/2 - 1) prior of r^2 / ||k||^2 (the codebook paragraph after "PGKQ
 * pipeline": Lloyd-Max for the Beta prior, not refit on data).  Writes
 * 2^b_main ascending levels and 2^b_main - 1 midpoint thresholds into HOST
 * arrays, float64.  Iterates until no level moves by more than 1e-13. */
pgkq_status pgkq_lloyd_max_beta(int32_t head_dim, int32_t b_main, double* levels_host,
                                double* thresholds_host);

/* Host routine.  Lloyd-Max quantizer refit on a sample of rho values (the
 * empirical-refit variant PGKQ-KV' of the PGKQ-KV paragraphs: the codebook
 * fitted to a short activation capture instead of the Beta prior).  The sample
 * is rho = r sqrt(d/2) / s_h for the pairs of captured rows (r the pair radius,
 * s_h the head's radius scale), so the result is scaled into a codebook by
 * s_h / sqrt(d/2) exactly like the Beta table.
 *   samples_host [n_samples] float64, HOST memory, finite, not modified;
 *                n_samples >= 2^b_main (else PGKQ_ERR_SHAPE)
 *   levels_host  out [2^b_main] float64, ascending
 *   thresholds_host out [2^b_main - 1] float64, midpoints of adjacent levels
 * Start: the sorted sample at index floor((j + 1/2) n / 2^b_main).  Step:
 * thresholds at midpoints, every sample in the cell #{t_j < rho} (the encoder's
 * decision rule), each non-empty cell's level set to the cell's mean (an empty
 * cell keeps its level).  Stops at the fixed point where no sample changes
 * cell; PGKQ_ERR_UNSUPPORTED if none is reached in 100000 steps, if b_main is
 * outside 1..8 or a sample is not finite.  Deterministic; allocates host memory
 * for a sorted copy of the sample. */
pgkq_status pgkq_lloyd_max_empirical(const double* samples_host, int64_t n_samples,
                                     int32_t b_main, double* levels_host,
                                     double* thresholds_host);

/* Bytes of workspace pgkq_calibrate needs (per-chunk float64 channel sums of
 * the calibration keys that open the "PGKQ pipeline" paragraph). */
size_t pgkq_calibrate_workspace_bytes(const pgkq_params* p, int64_t n_seq, int64_t n_kv,
                                      int64_t n_tokens);

/* Calibration over the keys about to be encoded (step (0) and the radius scale;
 * the "PGKQ pipeline" starts from calibration keys):
 *   K        [n_seq][n_kv][n_tokens][d] keys, dtype k_dtype (F32 or F16)
 *   sumsq    out [n_kv][d] float64: per channel sum of k^2 over sequences and tokens
 *   perm     out [n_kv][d] uint16: if reorder, channels sorted by descending sum of
 *            squares (stable), interleaved [pi_0, pi_{d-1}, pi_1, pi_{d-2}, ...];
 *            else the identity.  May be NULL when reorder == 0.
 *   codebook out [n_kv][2L] fp32: the Lloyd-Max levels/thresholds times
 *            s_h / sqrt(d/2), s_h = sqrt(sum_c sumsq[h][c] / (n_seq n_tokens)),
 *            each product formed in float64 and rounded once to fp32.
 * n_tokens must be >= 1.  The result is deterministic (fixed summation order). */
pgkq_status pgkq_calibrate(const pgkq_params* p, const void* K, pgkq_dtype k_dtype,
                           int64_t n_seq, int64_t n_kv, int64_t n_tokens, int32_t reorder,
                           double* sumsq, uint16_t* perm, float* codebook, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Encode keys into the code buffer (steps (1)-(4) of the "PGKQ pipeline"
 * paragraph; record layout as above, sized by the "Bit budget" paragraph):
 *   K      [n_seq][n_kv][n_tokens][d], dtype k_dtype (F32 or F16)
 *   codes  [n_seq][n_kv] streams of `capacity` slots; tokens are written to slots
 *          [token_offset, token_offset + n_tokens) of every stream, other slots
 *          are left untouched (appending to a live cache).
 * Decisions (radius and angle codes, residual norm) are taken in float64 on the
 * exact transform of the key; the QJL projection is accumulated in fp32. */
pgkq_status pgkq_encode(const pgkq_params* p, const void* K, pgkq_dtype k_dtype, int64_t n_seq,
                        int64_t n_kv, int64_t n_tokens, const int8_t* signs, const uint16_t* perm,
                        const float* codebook, const float* S, void* codes, int64_t capacity,
                        int64_t token_offset, void* stream);

/* Bytes of workspace pgkq_decode_attn / pgkq_estimate_logits need: the
 * prepared queries (the Hadamard rotation of Q named in the throughput
 * paragraph, with their lookup tables) and the split partial states. */
size_t pgkq_decode_workspace_bytes(const pgkq_params* p, int64_t n_seq, int64_t n_q,
                                   int64_t n_kv, int64_t n_tokens, const pgkq_launch_opts* opts);

/* Decode attention over the compressed keys and fp16 values (the end of the
 * "PGKQ pipeline" paragraph: logits computed analytically from the codes,
 * never from a rebuilt K; "Bit budget": V stays FP16):
 *   q     [n_seq][n_q][d], dtype q_dtype (F32, F16 or BF16); query head hq reads
 *         kv-head hq / (n_q / n_kv); n_q / n_kv must be 1, 2, 4 or 8
 *   codes as written by pgkq_encode, tokens [0, n_tokens) of each stream
 *   V     fp16 value cache in 32-token tiles (n_seq * n_kv streams of
 *         `capacity` slots, see the conventions above)
 *   out   [n_seq][n_q][d] fp32 = sum_t softmax_t(scale * logit_t) V_t
 * The weighted sum runs on the matrix cores: each softmax weight p (at most
 * 1) is split into two fp16 parts, hi = fp16(2^15 p) and lo = fp16(2^15 p -
 * hi), both parts multiply the fp16 values exactly and the products
 * accumulate in fp32 (the weight is carried to about 2^-22 relative); the
 * denominator sums the fp32 weights themselves.
 *   softmax_scale <= 0 selects 1 / sqrt(d).
 * The logit of token t is
 *   sum_i level[rc_i] (q~[2i] cos thetahat[ac_i] + q~[2i+1] sin thetahat[ac_i])
 *   + sqrt(pi/2)/m * nu_t * sum_j (S_h q~)_j (2 bit_tj - 1),
 * with q~ the query through the kv-head's transform.  The token range is split
 * across workgroups (flash-decoding); partial states are merged with a
 * log-sum-exp merge.  The split sizes are the library's choice (splits that
 * run first are given more tokens than the last ones, and no split holds more
 * than 2^18 tokens: a smaller requested count is raised to keep the fp32
 * accumulation of one split short); a plan with more than 65535 splits
 * returns PGKQ_ERR_SHAPE.  Workspace: pgkq_decode_workspace_bytes(). */
pgkq_status pgkq_decode_attn(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                             int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                             int64_t capacity, const int8_t* signs, const uint16_t* perm,
                             const float* codebook, const float* S, const void* codes,
                             const void* V, float* out, float softmax_scale,
                             const pgkq_launch_opts* opts, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Decode attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * pgkq_decode_attn without the workspace arguments.  The library's own scratch
 * of PGKQ_NOALLOC_SCRATCH_BYTES (8 MiB) serves as the workspace: a static
 * device array, one copy per GPU, held until the process ends; its address on
 * the current device is looked up on the first call there (the stream must
 * belong to the current device).  A call whose pgkq_decode_workspace_bytes()
 * exceeds the scratch returns PGKQ_ERR_WORKSPACE before anything is enqueued
 * (the 32k-token GQA cache of 16 x 32 query heads at 8 splits needs 3.2 MiB).
 * Every call on one GPU uses the same scratch and leaves its contents there:
 * calls that overlap on one GPU (other streams or threads) race.  Nothing in
 * the scratch needs to start at zero.  Same validation, kernels and results
 * as pgkq_decode_attn; allocates nothing. */
#define PGKQ_NOALLOC_SCRATCH_BYTES (8u << 20)
pgkq_status pgkq_decode_attn_noalloc(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                                     int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                     int64_t capacity, const int8_t* signs, const uint16_t* perm,
                                     const float* codebook, const float* S, const void* codes,
                                     const void* V, float* out, float softmax_scale,
                                     const pgkq_launch_opts* opts, void* stream);

/* One decode step of a live cache: append the new token, then attend over it
 * (the decode loop of the Table III paragraph: each generated token's key is
 * coded into the cache before the next logits are taken).
 * Encodes k_new [n_seq][n_kv][d] (k_dtype F32 or F16; steps (1)-(4), one key per
 * stream) into slot n_cached of every stream of `codes`, copies v_new
 * [n_seq][n_kv][d] fp16 into slot n_cached of the tiled V, then computes decode attention
 * over tokens [0, n_cached] exactly as pgkq_decode_attn with n_tokens =
 * n_cached + 1.  The append runs inside the query-preparation launch (no
 * extra kernel); its decisions are taken in float64 on the unnormalized
 * transform and its QJL projection is accumulated in float64.  Requires
 * 0 <= n_cached < capacity and n_q + n_kv <= 65535 (else PGKQ_ERR_SHAPE);
 * workspace as pgkq_decode_workspace_bytes() for n_cached + 1 tokens.  codes
 * and V are written (slot n_cached only). */
pgkq_status pgkq_decode_step(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                             const void* k_new, pgkq_dtype k_dtype, const void* v_new,
                             int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_cached,
                             int64_t capacity, const int8_t* signs, const uint16_t* perm,
                             const float* codebook, const float* S, void* codes, void* V,
                             float* out, float softmax_scale, const pgkq_launch_opts* opts,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The attention-logit hook of the throughput paragraph: raw logits (estimates
 * of <q, k_t>, no softmax scale) into logits [n_seq][n_q][n_tokens] fp32.  Same
 * device code as the score step of pgkq_decode_attn.  Workspace as for decode. */
pgkq_status pgkq_estimate_logits(const pgkq_params* p, const void* q, pgkq_dtype q_dtype,
                                 int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                 int64_t capacity, const int8_t* signs, const uint16_t* perm,
                                 const float* codebook, const float* S, const void* codes,
                                 float* logits, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Write fp16 value rows into the 32-token-tile value cache (the FP16 V of the
 * "Bit budget" paragraph; layout in the conventions above):
 *   rows   [n_streams][n_tokens][head_dim] fp16, plain rows (2-byte aligned)
 *   cache  n_streams streams of `capacity` slots (16-byte aligned);
 *          slots [slot_offset, slot_offset + n_tokens) are written, every
 *          other slot keeps its contents.
 * head_dim a multiple of 16 up to 1024; capacity a multiple of 32;
 * slot_offset + n_tokens <= capacity.  n_streams or n_tokens == 0 is a no-op
 * (the pointers may then be NULL).  One kernel, no workspace. */
pgkq_status pgkq_pack_values(const void* rows, int64_t n_streams, int64_t n_tokens, int32_t head_dim,
                             void* cache, int64_t capacity, int64_t slot_offset, void* stream);

/* The inverse: slots [slot_offset, slot_offset + n_tokens) of every stream of
 * the tiled cache into rows [n_streams][n_tokens][head_dim]. */
pgkq_status pgkq_unpack_values(const void* cache, int64_t n_streams, int64_t capacity,
                               int32_t head_dim, int64_t slot_offset, int64_t n_tokens, void* rows,
                               void* stream);

/* Bytes of workspace pgkq_fp16_decode_attn needs (split partial states). */
size_t pgkq_fp16_decode_workspace_bytes(int32_t head_dim, int64_t n_seq, int64_t n_q,
                                        int64_t n_kv, int64_t n_tokens,
                                        const pgkq_launch_opts* opts);

/* Uncompressed comparator: decode attention on an fp16 key cache, the FP16
 * cache of the throughput paragraph (232.16 tok/s there) and the reference
 * of the fidelity deltas in the Table III paragraph.
 *   K16 [n_seq][n_kv][capacity][d] fp16 rows; V16 the fp16 value cache in
 *   32-token tiles (as for decode); q, out, scale as for decode. */
pgkq_status pgkq_fp16_decode_attn(const void* q, pgkq_dtype q_dtype, int64_t n_seq, int64_t n_q,
                                  int64_t n_kv, int64_t n_tokens, int64_t capacity,
                                  int32_t head_dim, const void* K16, const void* V16, float* out,
                                  float softmax_scale, const pgkq_launch_opts* opts,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * PGKQ-KV: values coded as well (EdgeLLM-Nano paper page, PGKQ-KV paragraphs:
 * PGKQ's polar codes, Lloyd-Max tables and QJL sketch applied to V, with the
 * Hadamard rotation disabled for V).
 *
 * The value cache is encoded with pgkq_encode itself, called on V with value
 * parameters pv (pv->hadamard = 0; signs are then ignored and perm must be
 * NULL) and the value table and projection (pgkq_calibrate on V gives the
 * table).  Its records have the key layout above.  The decoder forms
 * sum_t p_t V-hat_t with V-hat_t the reconstruction the codes define: per pair
 * level_v[rc] (cos thetahat[ac], sin thetahat[ac]), plus, with QJL,
 * sqrt(pi/2)/m * nu_t * S_v^T (2 bits_t - 1).
 * Supported (b_main of K, b_main of V): equal widths 2, 3, 4, or V at 2 with
 * K at 3 or 4; QJL on both or on neither; same head_dim.
 * ------------------------------------------------------------------------ */

/* Bytes of workspace pgkq_kv_decode_attn needs (0 if the parameters are invalid). */
size_t pgkq_kv_decode_workspace_bytes(const pgkq_params* pk, const pgkq_params* pv, int64_t n_seq,
                                      int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                      const pgkq_launch_opts* opts);

/* Decode attention over PGKQ key codes and PGKQ value codes:
 *   q, signs, perm, codebook_k, S_k, codes_k as for pgkq_decode_attn;
 *   codebook_v [n_kv][2 L_v] fp32, S_v [n_kv][d][d] fp32 (NULL without QJL),
 *   codes_v written by pgkq_encode(pv, V, ...) with the same capacity;
 *   out [n_seq][n_q][d] fp32. */
pgkq_status pgkq_kv_decode_attn(const pgkq_params* pk, const pgkq_params* pv, const void* q,
                                pgkq_dtype q_dtype, int64_t n_seq, int64_t n_q, int64_t n_kv,
                                int64_t n_tokens, int64_t capacity, const int8_t* signs,
                                const uint16_t* perm, const float* codebook_k, const float* S_k,
                                const void* codes_k, const float* codebook_v, const float* S_v,
                                const void* codes_v, float* out, float softmax_scale,
                                const pgkq_launch_opts* opts, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * RTN control: per-token asymmetric round-to-nearest keys (EdgeLLM-Nano paper
 * page, "Comparison to simpler baselines": K quantized per token to INT3 or
 * INT4 with an FP16 scale and zero-point per key vector, V in FP16).
 *
 * Per key vector k (d values): zp = fp16(min_c k_c), hi = fp16(max_c k_c)
 * (a -0 extreme counts as +0), scale = fp16((hi - zp) / (2^bits - 1)) rounded
 * once from float64 (a zero result gives scale 1), and
 *   code_c = clamp(nearest_even((k_c - zp) / scale), 0, 2^bits - 1)
 * decided in float64.  The logit of token t is sum_c q_c (zp_t + scale_t code_tc).
 * Keys must be finite and within the fp16 range.
 *
 * Record of one token slot: d*bits/8 + 4 bytes (36 / 28 at d = 64, i.e. 4.50 /
 * 3.50 bits per element): NC = d*bits/32 code words holding the codes as one
 * bit stream (code c at bits [bits*c, bits*c + bits), LSB first; bit q in word
 * q/32, bit q%32), then one word with the fp16 scale in its low half and the
 * fp16 zero-point in its high half.  Word w of token t is stored at byte
 * 4 (w capacity + t) of the stream; streams back to back in [n_seq][n_kv]
 * order.  head_dim 64 or 128, bits 3 or 4.
 * ------------------------------------------------------------------------ */

/* Bytes of one RTN token slot, 0 if (head_dim, bits) is unsupported. */
size_t pgkq_rtn_record_bytes(int32_t head_dim, int32_t bits);

/* Quantize K [n_seq][n_kv][n_tokens][d] (F32 or F16) into slots
 * [token_offset, token_offset + n_tokens) of every stream of `codes`
 * (n_seq * n_kv streams of `capacity` slots); other slots are untouched. */
pgkq_status pgkq_rtn_encode(int32_t head_dim, int32_t bits, const void* K, pgkq_dtype k_dtype,
                            int64_t n_seq, int64_t n_kv, int64_t n_tokens, void* codes,
                            int64_t capacity, int64_t token_offset, void* stream);

/* Bytes of workspace pgkq_rtn_decode_attn / pgkq_rtn_logits need (0 if the
 * shape is invalid). */
size_t pgkq_rtn_decode_workspace_bytes(int32_t head_dim, int64_t n_seq, int64_t n_q,
                                       int64_t n_kv, int64_t n_tokens,
                                       const pgkq_launch_opts* opts);

/* Decode attention over RTN keys and fp16 values; q, V, out, softmax_scale,
 * opts and the split / merge scheme as for pgkq_decode_attn. */
pgkq_status pgkq_rtn_decode_attn(int32_t head_dim, int32_t bits, const void* q, pgkq_dtype q_dtype,
                                 int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                                 int64_t capacity, const void* codes, const void* V, float* out,
                                 float softmax_scale, const pgkq_launch_opts* opts,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Raw RTN logits <q, k-hat_t> into logits [n_seq][n_q][n_tokens] fp32 (same
 * device code as the score step of pgkq_rtn_decode_attn). */
pgkq_status pgkq_rtn_logits(int32_t head_dim, int32_t bits, const void* q, pgkq_dtype q_dtype,
                            int64_t n_seq, int64_t n_q, int64_t n_kv, int64_t n_tokens,
                            int64_t capacity, const void* codes, float* logits, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Measurement utility (not a step of the method).  The decode scans are
 * judged against the HBM bandwidth; besides the vendor figure, this reads a
 * buffer the way they do (16-byte non-temporal buffer loads, one contiguous
 * slice per workgroup, about 512 workgroups) and nothing else, so its rate is
 * the read ceiling measured on the same device.
 * ------------------------------------------------------------------------ */

/* Read `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple of 16
 * and at most 2^39) and XOR every 32-bit word of them into *xor_out (device,
 * 4-byte aligned; the caller sets its initial value).  bytes == 0 is a no-op.
 * Errors: PGKQ_ERR_NULL, PGKQ_ERR_SHAPE, PGKQ_ERR_ALIGN, PGKQ_ERR_HIP. */
pgkq_status pgkq_stream_read(const void* src, uint64_t bytes, uint32_t* xor_out, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PGKQ_H */
