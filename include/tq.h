/*
 * tq.h - 4-bit paged KV cache (TQ4/4, TQ4/2 and MX-FP4) and decode attention
 * that reads the compressed cache, for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; every device pointer is a HIP device
 * address, every `stream` argument is a hipStream_t (NULL = the legacy default
 * stream).  Calls that take a stream are asynchronous on it; kernel faults
 * surface at the caller's next synchronisation, as for any HIP launch.
 * Functions return a tq_status; tq_last_error() gives a thread-local message
 * for the last failure.  No function throws.
 *
 * Pages the operations come from (cited by title and section):
 *   [TQ-AMD] "TurboQuant 在 AMD GPU 上把長上下文延遲壓下來" (ROCm TurboQuant in
 *            vLLM): section 2 "TQ4/4 是最穩的預設值" - 4-bit K and 4-bit V,
 *            K = rotation + LUT quantization, V = uniform quantization;
 *            section 4 "Walsh-Hadamard 比隨機 rotation 更實用" - the rotation
 *            is a Walsh-Hadamard transform; section 5 - no QJL at 4 bits.
 *   [UQ]     "UltraQuant：4-bit KV 快取加速長代理": section "方法怎麼做，白話講"
 *            - WHT rotation, K/V asymmetry, Lloyd-Max 16-entry table, and the
 *            FP4 path (FP8 queries, FP4 KV, UE8M0 group scales, scaled MFMA).
 *   [ST]     "StateTree-Representation：讓 LLM 壓縮後仍保留 BF16 精度": vLLM
 *            paged KV blocks of 16 tokens.
 *
 * ---------------------------------------------------------------------------
 * Formats.  D = head_dim, P = D/2, Q = D/8, G = D/32, token row t in [0,16)
 * of a block, t = 4r + tt.  A pool is [num_blocks][num_kv_heads][record];
 * a record holds one 16-token block of one kv-head.  A byte holds two 4-bit
 * codes: the even channel in the low nibble.  fp16 values are little-endian.
 * Sections follow each other in the order listed; the large ones start on
 * 128-byte boundaries of the record, and at D = 128 every record is padded
 * to whole 128-byte lines (unused bytes, never written or read), so that a
 * block's records are written as whole lines.
 *
 * TQ4/4 (format 0, D = 64 or 128).  Per (token, kv-head):
 *   key scale  s = fp16_RNE(sqrt(sum_i k_i^2 / D)) (exact; saturates at 65504)
 *   key codes  x = unnormalized fp32 Walsh-Hadamard butterflies of k (stage
 *              order h = 1, 2, ..., D/2; (a, b) -> (a + b, a - b)),
 *              w = fp32(fp32(1/s) * fp32(1/sqrt(D))), u_i = fp32(x_i * w)
 *              (u = 0 if s = 0), t_j = fp32((c_j + c_{j+1}) * 0.5) over the fp16
 *              table c, code_i = #{ j : u_i > t_j } (nearest entry, ties low).
 *              Dequantized keys stay rotated: k_hat_i = c[code_i] * s.
 *   values     per 32-channel group: sc = fp16_sat(fp32(fp32(max - min) / 15)),
 *              mn = fp16_sat(min), code = clamp(RNE(fp32(fp32(v - mn) *
 *              fp32(1/sc))), 0, 15) (0 if sc = 0); v_hat = code * sc + mn.
 *   record (2432 B at D = 128: 2336 B of sections and 96 B of padding;
 *   1184 B at D = 64):
 *     Kc  16*P B   pair p of token t at ((p / Q) * 16 + t) * Q + p % Q
 *     Vc  16*P B   pair p = 16*gp + j of token t at ((r*16 + j)*G + gp)*4 + tt
 *     Vm  64*G B   sc(t,gp) at 2*((r*G + gp)*8 + tt),
 *                  mn(t,gp) at 2*((r*G + gp)*8 + 4 + tt)
 *     Ks  32 B     fp16 s of token t at 2t
 *
 * TQ4/2 (format 2, D = 64 or 128; [TQ-AMD] section 2 names 2-bit variants as
 * feasible): keys as TQ4/4; values by the same per-group rule with 2-bit codes:
 *   sc = fp16_sat(fp32(fp32(max - min) / 3)), code = clamp(RNE(fp32(fp32(v -
 *   mn) * fp32(1/sc))), 0, 3); v_hat = code * sc + mn.
 *   record (1920 B at D = 128: 1824 B of sections and 96 B of padding;
 *   928 B at D = 64):
 *     Kc  16*P B   as TQ4/4
 *     Vc2 8*P B    channel 2p + par, p = 16*gp + j, of token t: byte
 *                  ((r*16 + j)*(G/2) + gp/2)*4 + tt, bits 4*(gp%2) + 2*par
 *     Vm  64*G B   as TQ4/4
 *     Ks  32 B     as TQ4/4
 *   Supported by every call: quantize-append, decode, multi-token and cascade
 *   attention.
 *
 * MX-FP4 (format 1, D = 128).  Per (token, kv-head), groups of 32 channels:
 *   keys are rotated first, y = fp32(x * fp32(1/sqrt(D))), an exactly zero y
 *   stored as +0; values are not rotated (their zeros keep their sign).
 *   X = clamp(floor(log2(amax)) - 2, -127, 127) (amax = 0 -> -127), stored as
 *   the byte X + 127; element code = e2m1_RNE(value / 2^X) saturating at +-6,
 *   sign bit = the value's sign bit.  Queries: rotated the same way, cast to
 *   FP8 e4m3 (OCP e4m3fn, RNE, saturating), unit scale.
 *   record (2176 B, whole 128-byte lines):
 *     Kc4 1024 B   e2m1 key codes, placed as Kc
 *     Vc4 1024 B   e2m1 value codes, placed as Vc
 *     Ks4 64 B     key exponent byte of (t, gp) at gp*16 + t
 *     Vs4 64 B     value exponent byte of (t, gp) at (r*G + gp)*4 + tt
 *
 * Paging: token n of a quantize call goes to slot s = slot_mapping[n], block
 * s / 16, row s % 16 of every kv-head; s < 0 skips the token.  Decode reads
 * token t of sequence b from block block_table[b * max_blocks + t / 16].
 * Several sequences may name the same block.  Query head h uses kv-head
 * h / (num_q_heads / num_kv_heads).
 * ---------------------------------------------------------------------------
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1,  /* a host-checked argument is out of range or NULL   */
  TQ_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim 96)      */
  TQ_ERR_OOM = 3,          /* device allocation failed                          */
  TQ_ERR_WORKSPACE = 4,    /* workspace smaller than tq_decode_workspace_bytes  */
  TQ_ERR_HIP = 5           /* a HIP runtime call failed (see tq_last_error)     */
} tq_status;

typedef enum tq_format { TQ_FORMAT_TQ4 = 0, TQ_FORMAT_MXFP4 = 1, TQ_FORMAT_TQ4V2 = 2 } tq_format;
typedef enum tq_out_dtype { TQ_OUT_F32 = 0, TQ_OUT_BF16 = 1 } tq_out_dtype;

typedef struct tq_cache_desc {
  int32_t format;          /* tq_format                                          */
  int32_t head_dim;        /* TQ4/4, TQ4/2: 64 or 128; MX-FP4: 128                */
  int32_t num_kv_heads;    /* 1 .. 65536                                          */
  int32_t block_size;      /* must be 16                                          */
  int64_t num_blocks;      /* >= 1                                                */
  const float *key_table;  /* TQ4 only: host pointer to 16 strictly ascending
                              finite values, or NULL for the 16-level Lloyd-Max
                              quantizer of N(0,1) ([UQ] "方法怎麼做，白話講").
                              Rounded to fp16 (RNE) when the cache is created.
                              Must be NULL for MX-FP4.                            */
} tq_cache_desc;

typedef struct tq_cache tq_cache;  /* opaque handle */

/* Bytes of one (block, kv-head) record, padding included (TQ4/4: 2432 at
 * D = 128, 1184 at D = 64; TQ4/2: 1920 / 928; MX-FP4: 2176; see above). */
tq_status tq_record_bytes(const tq_cache_desc *desc, size_t *bytes);

/* Bytes of the whole pool: num_blocks * num_kv_heads * record bytes. */
tq_status tq_pool_bytes(const tq_cache_desc *desc, size_t *bytes);

/* Create a cache handle: a paged pool of 16-token blocks ([ST]: vLLM paged KV
 * blocks of 16 tokens) holding the 4-bit records of the chosen format
 * ([TQ-AMD] section 2 for TQ4/4; [UQ] "方法怎麼做，白話講" for MX-FP4), and the
 * key table the coder uses.  `pool` is a caller-owned device buffer of at least
 * tq_pool_bytes bytes (its contents are kept), or NULL: then the library
 * allocates the pool and fills it with zeros.  The library always owns the
 * handle and a small device table buffer.  Synchronous.  Errors:
 * INVALID_ARG (bad descriptor, pool too small, key table not ascending or not
 * finite), UNSUPPORTED (head_dim / format combination, or a key table whose
 * midpoints are too close for the coder's bin table: adjacent midpoints more
 * than 1/200 of the table's midpoint range apart are always accepted), OOM,
 * HIP. */
tq_status tq_create_cache(const tq_cache_desc *desc, void *pool, size_t pool_bytes, tq_cache **out);

/* The pool's device address and size, and the fp16 key table in use (16 fp16
 * bit patterns; NULL to skip; zeros for MX-FP4). */
tq_status tq_cache_info(const tq_cache *cache, void **pool, size_t *pool_bytes, uint16_t *key_table_f16);

/* The default key table, derived on the host: the 16-level Lloyd-Max
 * quantizer of N(0,1) (fp64 fixed point of Lloyd's conditions), each level
 * rounded to fp16; written as fp16 bit patterns.  No GPU needed. */
tq_status tq_default_key_table(uint16_t out_f16[16]);

/* Quantize and append tokens ([TQ-AMD] section 2; [UQ] "方法怎麼做，白話講").
 * k, v: device bf16 [num_tokens][num_kv_heads][head_dim], contiguous.
 * slot_mapping: device int32 [num_tokens]; slot = block * 16 + row, < 0 skips.
 * Slots must be < num_blocks * 16 and distinct within one call (trusted, not
 * checked on the device).  num_tokens = 0 is a no-op.  Asynchronous.  The
 * kernel's work distribution follows from the sizes (the environment variable
 * TQ_QUANT_LOOP, "static", "balanced" or "balanced-pairs", overrides it for
 * tests); the records written do not depend on it. */
tq_status tq_quantize_append(tq_cache *cache, const void *k, const void *v, const int32_t *slot_mapping,
                             int64_t num_tokens, void *stream);

/* Workspace bytes that tq_decode_attention needs for these sizes (split-K
 * partials; 0 when one split covers max_context_len). */
tq_status tq_decode_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, size_t *bytes);

/* Decode attention over the compressed cache, one query token per sequence:
 *   out[b, h] = sum_{t < T_b} softmax_t(scale * <q~[b,h], k_hat_t>) v_hat_t
 * with q~ the rotated query (TQ4: H_D q; MX-FP4: its e4m3 code values) and
 * k_hat, v_hat the dequantized cache rows of kv-head h / g.  The keys are
 * compared in the rotated domain, which leaves q . k unchanged ([TQ-AMD]
 * section 4).  Split-K over the context with a log-sum-exp merge; the split
 * size follows from the sizes (the environment variable TQ_SPLIT_BLOCKS, 1 to
 * 512 blocks, overrides it for tests; multi-token attention reads it too, 1 to
 * 4096, capped at what the chosen kernel stages).
 * q: device bf16 [batch][num_q_heads][head_dim]; out: device fp32 or bf16
 * (out_dtype) of the same shape; block_table: device int32
 * [batch][max_blocks]; context_lens: device int32 [batch], each in
 * [0, max_context_len] with ceil(len/16) <= max_blocks (trusted); a zero
 * length gives a zero row.  num_q_heads must be num_kv_heads * g with
 * g in {1, 2, 4, 8}.  max_context_len is the host's bound, used to size the
 * split.  softmax_scale > 0 (e.g. 1/sqrt(head_dim)).  TQ4 formats: the
 * rotated query times softmax_scale * log2(e) / sqrt(head_dim) is carried as
 * two fp16 parts, so each of its elements must stay within 65504 (at
 * head_dim 128 with the default scale: query elements below 4.5e4; not
 * checked, the values are on the device).  workspace: device buffer
 * of at least tq_decode_workspace_bytes (may be NULL when that is 0).
 * Asynchronous. */
tq_status tq_decode_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                              const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                              int32_t batch, int32_t num_q_heads, int32_t max_context_len, float softmax_scale,
                              void *workspace, size_t workspace_bytes, void *stream);

/* tq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and result without a workspace.  The
 * split-K partials go to a fixed device scratch of the library, 32 MiB
 * (33554432 bytes) per GPU, held from the first call on that GPU until the
 * process ends; sizes whose tq_decode_workspace_bytes exceeds it return
 * TQ_ERR_WORKSPACE.  Nothing is allocated and nothing needs clearing: every
 * partial the merge reads is written by the same call first.  All calls on
 * one GPU share its scratch, so calls that overlap on one GPU (several
 * streams, several threads) race; serialise them.  Asynchronous. */
tq_status tq_decode_attention_noalloc(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                      const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      float softmax_scale, void *stream);

/* ---------------------------------------------------------------------------
 * Multi-token attention over the compressed cache (every format): chunked
 * prefill of new tokens, or the verification of several proposed tokens.  The time to
 * first token that the pages report ([TQ-AMD] section 1; [UQ] "它實際證明了
 * 什麼") comes from prefilling over the cache; the operation is the causal
 * reading of attention over the cached context:
 *   out[q_start[b] + i, h] = sum_{t < T_b - M_b + i + 1} softmax_t(scale *
 *                            <q~, k_hat_t>) v_hat_t,   i < M_b,
 * with M_b = q_start[b+1] - q_start[b] query tokens of sequence b, the last
 * M_b tokens of its context of T_b = context_lens[b] tokens (their keys and
 * values already appended), q~ = H_D q (MX-FP4: its e4m3 code values, as in
 * decode), kv-head h / g as in decode.
 * q: device bf16 [num_tokens][num_q_heads][head_dim]; out: device fp32 or
 * bf16 (out_dtype) of the same shape; q_start: device int32 [batch + 1],
 * nondecreasing, q_start[0] = 0, q_start[batch] = num_tokens, each M_b in
 * [1, max_query_len] (or 0: the sequence has no query token) and M_b <= T_b
 * <= max_context_len, ceil(T_b / 16) <= max_blocks (all trusted, not checked
 * on the device).  num_q_heads a multiple of num_kv_heads (any ratio).
 * Host-checked: max_query_len <= max_context_len, num_tokens <= batch *
 * max_query_len.  workspace: device buffer of at least
 * tq_multitoken_workspace_bytes (NULL allowed when that is 0).
 * Asynchronous. */
tq_status tq_multitoken_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                        int64_t num_tokens, int32_t max_query_len, int32_t max_context_len,
                                        size_t *bytes);
tq_status tq_multitoken_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                  const int32_t *q_start, int64_t num_tokens, int32_t max_query_len,
                                  const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                  int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                  float softmax_scale, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Shared-prefix (cascade) decode attention (every format).  The same result as
 * tq_decode_attention, computed so that blocks shared by several sequences
 * are read once: the pages' agentic workloads keep long prefixes resident and
 * shared between sessions ([TQ-AMD] spec table; [UQ] "它實際證明了什麼"), and
 * paged blocks are what the sequences share ([ST]).
 * A group is a set of sequences whose block tables agree on a block range
 * [lo, hi): for every row (member b, head h) the partial softmax state over
 * the group's 16 (hi - lo) tokens is computed once for the whole group (all
 * members' heads of a kv-head together, each shared block read once), the
 * state over the sequence's own tokens separately, and all are combined by
 * the log-sum-exp merge.  Groups nest: the groups a sequence is in cover its
 * first P_b blocks contiguously, from block 0, in order of depth (the group
 * at depth d covers the blocks after those of depth d - 1); its own part is
 * tokens 16 P_b .. T_b - 1.  A group is one unit of parallel work (its
 * blocks are walked by one work-group per kv-head and 16 / 32 / 64 / 128
 * member rows), so callers cut long shared ranges into chained groups of a few
 * dozen blocks.
 * Arguments as tq_decode_attention, plus (all device, trusted):
 *   seq_prefix_blocks  int32 [batch]: P_b (0 for a sequence in no group),
 *                      16 P_b <= context_lens[b]
 *   seq_depth          int32 [batch]: the number of groups sequence b is in
 *   group_start        int32 [num_groups + 1], group_seqs int32 [...]: group
 *                      i's members are group_seqs[group_start[i] ..
 *                      group_start[i+1]) (at most max_group_size); the
 *                      shared blocks are read through the first member's table
 *   group_blocks       int32 [num_groups][2]: lo, hi (hi - lo <= max_group_blocks)
 *   group_depth        int32 [num_groups]: the group's depth (< max_depth)
 *   host: num_groups >= 0; when > 0, max_group_size in [1, batch] and
 *   max_depth in [1, num_groups]; 16 * max_group_blocks <= max_context_len;
 *   max_group_blocks <= 4096, MX-FP4: <= 256 (TQ_ERR_UNSUPPORTED beyond: cut
 *   longer shared ranges into chained groups).
 * num_q_heads / num_kv_heads must be 1, 2, 4 or 8.  workspace: device buffer
 * of at least tq_cascade_workspace_bytes (always needed).  Asynchronous: the
 * shared-block pass runs on a second stream of the handle (created on first
 * use, default priority), forked from `stream` and joined back to it by events
 * before the merge, so the call is ordered on `stream` like the others; calls
 * on one handle from several streams at once are not supported. */
tq_status tq_cascade_workspace_bytes(const tq_cache *cache, int32_t batch, int32_t num_q_heads,
                                     int32_t max_context_len, int32_t num_groups, int32_t max_group_size,
                                     int32_t max_group_blocks, int32_t max_depth, size_t *bytes);
tq_status tq_cascade_decode_attention(tq_cache *cache, const void *q, void *out, int32_t out_dtype,
                                      const int32_t *block_table, int32_t max_blocks, const int32_t *context_lens,
                                      int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                      float softmax_scale, const int32_t *seq_prefix_blocks,
                                      const int32_t *seq_depth, const int32_t *group_start,
                                      const int32_t *group_seqs, const int32_t *group_blocks,
                                      const int32_t *group_depth, int32_t num_groups, int32_t max_group_size,
                                      int32_t max_group_blocks, int32_t max_depth, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Calibrated key tables ([UQ] "方法怎麼做，白話講": the 16-entry key table is
 * refit on captured activations, about 20 vectors per rotated layer, and used
 * only on the tenth of the layers with the highest per-element key MSE).
 *
 * For each layer l the samples are the unit coordinates u = y / s of the rows
 * k[l] whose scale s is nonzero, computed exactly as the TQ4/4 key coder does
 * (fp32, see "key codes" above).  Lloyd's iteration runs in fp64 from the
 * initial table c: cell(u) = #{ j : u > (c_j + c_{j+1}) / 2 }; c_j = mean of
 * cell j's samples (an empty cell keeps c_j; a zero mean is +0); it stops when
 * an update changes no entry or after max_iters updates.
 *
 * Per layer it also reports the per-element mean squared key error of the
 * layer's rows coded with the initial table and with the fitted fp16 table:
 * codes by the coder's fp32 rule, k_hat = c[code] * s, compared with the exact
 * rotation H_D k in fp64 (equal to the error in the key's own coordinates,
 * H_D being orthonormal); all rows * head_dim elements count.
 *
 * k: device bf16 [num_layers][rows][head_dim] (rows = calibration tokens x
 * kv-heads, any order).  head_dim 64 or 128; num_layers 0 .. 65535 (0 is a
 * no-op); rows 0 .. 2^30 / head_dim.  init_table: host, 16 finite values,
 * strictly ascending after fp16 rounding (RNE), or NULL for the default table.
 * max_iters 0 .. 1e6.  Outputs, all device:
 *   tables_f16  uint16 [num_layers][16]  fitted entries rounded to fp16 (RNE)
 *                                        (required; pass them to
 *                                        tq_create_cache, which checks them)
 *   levels      double [num_layers][16]  fitted entries in fp64, or NULL
 *   mse         double [num_layers][2]   (initial table, fitted table), or NULL
 *   updates     int32  [num_layers]      Lloyd updates performed, or NULL
 * workspace: device buffer of at least tq_calibrate_workspace_bytes.
 * Asynchronous. */
tq_status tq_calibrate_workspace_bytes(int32_t num_layers, int64_t rows, int32_t head_dim, size_t *bytes);
tq_status tq_calibrate_key_tables(const void *k, int32_t num_layers, int64_t rows, int32_t head_dim,
                                  const float *init_table, int32_t max_iters, uint16_t *tables_f16,
                                  double *levels, double *mse, int32_t *updates, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* The layers that get a fitted table ([UQ] "方法怎麼做，白話講": the tenth
 * with the highest MSE).  Host only: mse is a host array [num_layers] (no
 * NaN); layers are ranked by it, largest first, an equal value ranking the
 * lower index first; layer i is chosen (chosen[i] = 1, else 0) when its rank
 * r satisfies 100 * r < percent * num_layers.  percent 0 .. 100. */
tq_status tq_select_layers(const double *mse, int32_t num_layers, int32_t percent, uint8_t *chosen);

/* ---------------------------------------------------------------------------
 * Test-only: the dequantized records, as every attention call of this library
 * consumes them ([TQ-AMD] section 2: k_hat = c[code] * s in the rotated domain,
 * v_hat = code * sc + mn; [UQ] "方法怎麼做，白話講": k_hat, v_hat = e2m1 * 2^X).
 * For each of the n block ids (device int32 [n]) and every kv-head h, writes
 * token t's dequantized key and value rows:
 *   k_out, v_out: device fp32 [n][num_kv_heads][16][head_dim], keys in the
 *   rotated domain;
 *   TQ4/4 and TQ4/2: k = fp32(c[code] * s), v = fp32(code * sc + mn) (exact
 *   products, one rounding of the sum; the attention kernels carry code * sc
 *   as two exact fp16 parts and add mn * p separately).  In a block holding a
 *   value scale >= 4096 every scale of the block is applied as sc * 2^-7 (the
 *   probabilities as p * 2^7); this stays exact for scales >= 2^-7;
 *   MX-FP4: k = e2m1 * 2^X, v = e2m1 * 2^X (exact).
 * The records are read as they are: rows past a sequence's context hold
 * whatever the pool holds.  A block id outside [0, num_blocks) gives rows of
 * zeros.  n = 0 is a no-op; n * num_kv_heads < 2^31.  Asynchronous. */
tq_status tq_debug_dequantize(tq_cache *cache, const int32_t *block_ids, int32_t n, float *k_out, float *v_out,
                              void *stream);

/* Free the handle made by tq_create_cache (the paged cache of [ST] and
 * [TQ-AMD] section 2), NULL-safe.  Synchronises the device first; frees the
 * library-owned pool if the library allocated it. */
void tq_free(tq_cache *cache);

/* Static text of a status code. */
const char *tq_status_string(tq_status status);

/* Thread-local text of the last failure in this thread ("" if none). */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
