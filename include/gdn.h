/*
 * gdn.h -- C ABI of the Gated DeltaNet (GDN) token-mixer library for AMD
 * Instinct MI355X (gfx950).
 *
 * The calls that form the layer's data-parallel hot path:
 *
 *   gdn_build_conv_chunks       host: exact (sequence, 8-token chunk) list
 *   gdn_causal_conv1d_varlen    GPU: width-4 causal conv over packed prefill
 *   gdn_causal_conv1d_varlen_tiles
 *                               GPU: the same, 8- or 16-token programs
 *   gdn_causal_conv1d_update    GPU: single-token conv for decode
 *   gdn_fused_recurrent_decode  GPU: gated delta rule over packed tokens
 *   gdn_chunk_gated_delta_rule  GPU: the same rule over prefill tokens,
 *                               chunkwise on the matrix cores
 *   gdn_chunk_workspace_size    host: scratch bytes the chunkwise call needs
 *   gdn_fused_conv_decode       GPU: conv update + gated delta rule, one launch
 *   gdn_chunk_rule_and_fused_decode
 *                               GPU: the chunkwise rule on a step's prefill
 *                               tokens and the fused decode of its decode
 *                               rows, sharing one grid
 *
 * Conventions shared by every call
 * --------------------------------
 * - bf16 values travel as raw 16-bit patterns (gdn_bf16).  fp32 -> bf16
 *   rounding is round-to-nearest-even.  Arithmetic is fp32.
 * - Unless marked "host", a pointer is a device pointer (HBM of the current
 *   HIP device).  The caller owns every buffer, scratch workspaces included.
 *   The library never allocates or frees device memory and caches no caller
 *   pointers; its only global state is the static scratch of
 *   gdn_chunk_rule_and_fused_decode_noalloc (and that scratch's per-device
 *   address).  It may be called from several threads, each on its own
 *   buffers.
 * - GPU calls validate their arguments on the host, then enqueue kernels on
 *   `stream` (a hipStream_t; NULL = the default stream) and return without
 *   waiting.  A call that returns an error enqueued nothing.
 * - "Stride" arguments count elements, not bytes, between consecutive token
 *   rows.  Within a row, channels (or heads, then head elements) are packed.
 * - Vector-access contract: bf16 row pointers and strides are multiples of
 *   8 elements (16 bytes); fp32 state pointers are 16-byte aligned.
 * - Sequences are packed back to back.  query_start_loc[s] .. [s+1] is the
 *   token range of sequence s; it must be non-decreasing with
 *   query_start_loc[0] == 0 and query_start_loc[num_seqs] == num_tokens
 *   (device-side preconditions: not checked, but the kernels clamp every
 *   range to [0, num_tokens), so a malformed array gives wrong results,
 *   never an access outside the buffers).  state_indices[s] selects the
 *   state slot of sequence s; a negative index marks padding: that sequence
 *   is skipped, its outputs and every slot are left untouched.  An index at
 *   or past num_slots is skipped the same way (the kernels check it).  Slots
 *   used in one call must be distinct.
 *
 * Return values: GDN_OK or a negative gdn_status; gdn_last_error() then
 * describes the failure (thread-local, valid until the thread's next call).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gdn_bf16;

/* Tokens per conv program: one descriptor covers tokens
 * [qsl[seq] + 8*chunk, min(qsl[seq] + 8*chunk + 8, qsl[seq+1])). */
#define GDN_CONV_CHUNK_TOKENS 8
/* The only conv width the library implements. */
#define GDN_CONV_WIDTH 4

typedef struct gdn_conv_chunk {
    int32_t seq;    /* sequence index into query_start_loc */
    int32_t chunk;  /* 8-token chunk index within that sequence */
} gdn_conv_chunk;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID = -1,      /* NULL pointer, bad count, bad pair, aliasing */
    GDN_ERR_UNSUPPORTED = -2,  /* width != 4, misaligned, unsupported head dim */
    GDN_ERR_CAPACITY = -3,     /* descriptor buffer or workspace too small */
    GDN_ERR_HIP = -4           /* the HIP runtime reported an error */
} gdn_status;

/* Text of the last error on the calling thread ("" after a success). */
const char *gdn_last_error(void);

/*
 * gdn_build_conv_chunks -- host only, synchronous.
 *
 * Source: page "perf(gdn): dispatch exact causal-conv chunks", section "What
 * changed": the conv is dispatched as one program per exact (sequence,
 * 8-token chunk) pair; the list is built once per engine step, uploaded once
 * and reused by every GDN layer of the step.
 *
 * For s = 0 .. num_seqs-1 and c = 0 .. ceil(L_s / 8) - 1 (L_s =
 * qsl_host[s+1] - qsl_host[s]) appends {s, c}: sequences in order, chunks
 * ascending; empty sequences contribute nothing.
 *
 *   qsl_host   host, int32 [num_seqs + 1], non-decreasing (checked)
 *   out_host   host, gdn_conv_chunk [capacity]; may be NULL if capacity == 0
 *   n_out      host, receives the number of descriptors needed
 *
 * Errors: GDN_ERR_INVALID (NULL qsl_host/n_out, num_seqs < 0, capacity < 0,
 * decreasing qsl, count overflow); GDN_ERR_CAPACITY when the list does not
 * fit: *n_out then holds the required count and out_host[0 .. capacity) holds
 * the first descriptors.  Pass capacity 0 to query the count.
 */
int gdn_build_conv_chunks(const int32_t *qsl_host, int32_t num_seqs,
                          gdn_conv_chunk *out_host, int32_t capacity, int32_t *n_out);

/*
 * gdn_causal_conv1d_varlen -- depthwise causal conv1d over packed prefill
 * tokens, width 4, optional SiLU, per-sequence carried state.
 *
 * Sources: page "perf(gdn): dispatch exact causal-conv chunks", section "What
 * changed" (one program per exact chunk descriptor; the descriptor is
 * optional and its (buffer, count) pair is validated together, reviewer
 * comment on the same page); page "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT,
 * and VRAM gaps vs vLLM", section "Existing evidence" (width-4 conv).
 *
 * For each sequence s with slot = state_indices[s] >= 0, tokens [a, a+L):
 *   window e = h || x[a .. a+L), h = conv_state[slot] if has_initial_state[s]
 *             else 3 zero rows (oldest first)
 *   y[a+p][c] = act(bias[c] + sum_{j<4} weight[c][j] * e[p+j][c])
 *             (weight[c][3] multiplies the current token; act = SiLU if silu)
 *   conv_state[slot] <- e[L .. L+3)   (the three newest window rows)
 *
 *   x                 bf16 [num_tokens][x_stride], channels [0, channels)
 *   weight            bf16 [channels][4]
 *   bias              bf16 [channels], or NULL for no bias
 *   conv_state        bf16 [num_slots][3][channels], read and written in place
 *   query_start_loc   int32 [num_seqs + 1]
 *   state_indices     int32 [num_seqs]
 *   has_initial_state uint8 [num_seqs], or NULL (= every sequence has one)
 *   chunks, n_chunks  descriptors from gdn_build_conv_chunks on the same
 *                     query_start_loc, copied to the device: the only
 *                     dispatch, so required whenever num_tokens > 0.  Both
 *                     NULL/0 is valid only with num_tokens == 0 (the call
 *                     then enqueues nothing); exactly one of them set is an
 *                     error.  A descriptor whose seq is not in [0, num_seqs)
 *                     or whose chunk lies past its sequence is skipped.
 *   y                 bf16 [num_tokens][y_stride]; must not overlap x,
 *                     conv_state, weight or bias
 *
 * Errors: GDN_ERR_INVALID (required pointer NULL, negative count,
 * (chunks == NULL) != (n_chunks == 0), num_tokens > 0 without descriptors,
 * fewer than ceil(num_tokens / 8) or more than num_tokens descriptors,
 * stride < channels, y overlapping x, conv_state, weight or bias,
 * num_slots < 1); GDN_ERR_UNSUPPORTED (width != 4, channels % 8, strides or
 * pointers off the 16-byte contract); GDN_ERR_HIP (launch failure).
 */
int gdn_causal_conv1d_varlen(const gdn_bf16 *x, int64_t x_stride,
                             const gdn_bf16 *weight, const gdn_bf16 *bias,
                             gdn_bf16 *conv_state, int32_t num_slots,
                             const int32_t *query_start_loc,
                             const int32_t *state_indices,
                             const uint8_t *has_initial_state,
                             const gdn_conv_chunk *chunks, int32_t n_chunks,
                             gdn_bf16 *y, int64_t y_stride,
                             int32_t num_seqs, int32_t num_tokens, int32_t channels,
                             int32_t width, int32_t silu, void *stream);

/*
 * gdn_causal_conv1d_varlen_tiles -- gdn_causal_conv1d_varlen with a choice of
 * program size: each program takes descriptors_per_program consecutive
 * entries of the descriptor list (1: 8-token programs, exactly
 * gdn_causal_conv1d_varlen; 2: 16-token programs).  The descriptors stay the
 * exact 8-token ones; when a program's second descriptor continues its first
 * (same sequence, next chunk), its 3-row halo is the first's last rows, so a
 * 16-token program reads 19 rows where two 8-token programs read 22.
 * Results are bit-identical to gdn_causal_conv1d_varlen for every input.
 *
 * Sources: page "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs
 * vLLM", section "Existing evidence" (the multi-token tile arm of the conv);
 * page "perf(gdn): dispatch exact causal-conv chunks", section "What changed"
 * (exact 8-token descriptors).
 *
 * Arguments, layouts and errors as gdn_causal_conv1d_varlen, plus:
 *   descriptors_per_program  1 or 2, else GDN_ERR_UNSUPPORTED; with 2, x_stride
 *                            and y_stride must be at most 2^26 elements
 *                            (GDN_ERR_UNSUPPORTED otherwise)
 */
int gdn_causal_conv1d_varlen_tiles(const gdn_bf16 *x, int64_t x_stride,
                                   const gdn_bf16 *weight, const gdn_bf16 *bias,
                                   gdn_bf16 *conv_state, int32_t num_slots,
                                   const int32_t *query_start_loc,
                                   const int32_t *state_indices,
                                   const uint8_t *has_initial_state,
                                   const gdn_conv_chunk *chunks, int32_t n_chunks,
                                   gdn_bf16 *y, int64_t y_stride,
                                   int32_t num_seqs, int32_t num_tokens, int32_t channels,
                                   int32_t width, int32_t silu,
                                   int32_t descriptors_per_program, void *stream);

/*
 * gdn_causal_conv1d_update -- the same conv for one new token per sequence
 * (decode): row b uses slot state_indices[b] (negative: row skipped).
 *
 *   y[b][c] = act(bias[c] + sum_{j<3} weight[c][j] * conv_state[slot][j][c]
 *                 + weight[c][3] * x[b][c])
 *   conv_state[slot] <- (conv_state[slot][1], conv_state[slot][2], x[b])
 *
 * Identical arithmetic to gdn_causal_conv1d_varlen, so a sequence advanced
 * by this call gives bit-identical outputs to the varlen call on the whole
 * sequence.  Layouts as above with num_tokens = batch.
 *
 * Errors: as gdn_causal_conv1d_varlen (minus the descriptor pair).
 */
int gdn_causal_conv1d_update(const gdn_bf16 *x, int64_t x_stride,
                             const gdn_bf16 *weight, const gdn_bf16 *bias,
                             gdn_bf16 *conv_state, int32_t num_slots,
                             const int32_t *state_indices,
                             gdn_bf16 *y, int64_t y_stride,
                             int32_t batch, int32_t channels, int32_t width,
                             int32_t silu, void *stream);

/*
 * gdn_fused_recurrent_decode -- the gated delta rule, fused per (sequence,
 * v-head), token by token, over packed tokens (decode: one token each).
 *
 * Sources: the fused GDN decode with a register-resident state named on page
 * "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section
 * "Existing evidence"; the rule itself from Yang, Kautz, Hatamizadeh, "Gated
 * Delta Networks: Improving Mamba2 with Delta Rule" (ICLR 2025).
 *
 * For each sequence s with slot = state_indices[s] >= 0 and v-head h (q/k
 * head hk = h / (num_v_heads / num_k_heads)):
 *   S = has_initial_state[s] ? state[slot][h] : 0      (dv x dk, fp32)
 *   for each token t of s:
 *     qh, kh = q[t][hk], k[t][hk], each divided by sqrt(sum x^2 + 1e-6)
 *              when qk_l2norm != 0
 *     a = exp(g[t][h]),  b = beta[t][h]
 *     S = a * S * (I - b kh kh^T) + b v[t][h] kh^T
 *     o[t][h] = scale * S qh
 *   state[slot][h] = S
 *
 *   q, k     bf16, token t head j at q + t*q_stride + j*head_k_dim
 *   v        bf16, token t head h at v + t*v_stride + h*head_v_dim
 *            (q, k and v may be column views of one conv output row)
 *   g, beta  fp32 [num_tokens][num_v_heads]  (g = log decay)
 *   state    fp32 [num_slots][num_v_heads][head_v_dim][head_k_dim], in place;
 *            row i (one v channel) is contiguous along head_k_dim
 *   query_start_loc  int32 [num_seqs + 1], or NULL: one token per sequence
 *            (then num_tokens == num_seqs and token s belongs to sequence s)
 *   o        bf16, token t head h at o + t*o_stride + h*head_v_dim
 *
 * Launch shape: with query_start_loc == NULL the call is laid out for
 * bandwidth (every state row streamed once); with it, for per-token
 * latency.  Both shapes do identical per-token arithmetic, so splitting a
 * sequence across calls gives bit-identical results.
 *
 * Errors: GDN_ERR_INVALID (required pointer NULL, negative count,
 * num_v_heads % num_k_heads, strides too small, num_tokens != num_seqs
 * without query_start_loc, o overlapping q/k/v/g/beta/state); GDN_ERR_UNSUPPORTED
 * (head_k_dim not in {16, 32, 64, 128}, head_v_dim not a positive multiple
 * of 8 up to 256, alignment contract); GDN_ERR_HIP.
 */
int gdn_fused_recurrent_decode(const gdn_bf16 *q, int64_t q_stride,
                               const gdn_bf16 *k, int64_t k_stride,
                               const gdn_bf16 *v, int64_t v_stride,
                               const float *g, const float *beta,
                               float *state, int32_t num_slots,
                               const int32_t *query_start_loc,
                               const int32_t *state_indices,
                               const uint8_t *has_initial_state,
                               gdn_bf16 *o, int64_t o_stride,
                               int32_t num_seqs, int32_t num_tokens,
                               int32_t num_k_heads, int32_t num_v_heads,
                               int32_t head_k_dim, int32_t head_v_dim,
                               float scale, int32_t qk_l2norm, void *stream);

/*
 * gdn_chunk_gated_delta_rule -- the same gated delta rule as
 * gdn_fused_recurrent_decode over packed prefill tokens, evaluated chunk by
 * chunk (64 tokens) in the equivalent matrix form on the matrix cores.
 *
 * Sources: the rule from Yang, Kautz, Hatamizadeh, "Gated Delta Networks:
 * Improving Mamba2 with Delta Rule" (ICLR 2025); its chunkwise form follows
 * from unrolling the recurrence over a chunk: with u_t the per-token update
 * vector, (I + A) U = R for a unit lower-triangular A built from the chunk's
 * keys, gates and betas (the pages name the prefill GDN path only by its
 * test, page "Qwen3.5-4b BF16 optimization and correctness (sm_120)",
 * section "Evidence").
 *
 * Two kernels run on `stream`: one prepares, for every (64-token chunk,
 * v-head) in parallel, the parts that do not depend on the state (the
 * inverse of I + A, the masked decayed Q K^T, per-token factors) in
 * `workspace`; the second walks each sequence's chunks in order.
 *
 * Arguments, layouts, state semantics and errors are those of
 * gdn_fused_recurrent_decode, except:
 *   query_start_loc  required (int32 [num_seqs + 1])
 *   head_k_dim       must be 128
 *   head_v_dim       a positive multiple of 32 up to 256
 *   q/k/v/o_stride   below 2^24 elements (32-bit offsets within a chunk)
 *   workspace        device scratch owned by the caller, 256-byte aligned,
 *                    at least gdn_chunk_workspace_size(num_seqs, num_tokens,
 *                    num_k_heads, num_v_heads) bytes; its contents on entry
 *                    do not matter and are overwritten.  Calls that share a
 *                    workspace must not overlap in time.
 * Errors beyond those: GDN_ERR_INVALID (NULL workspace, or a workspace
 * whose first gdn_chunk_workspace_size bytes overlap q, k, v, g, beta,
 * state or o), GDN_ERR_UNSUPPORTED
 * (misaligned workspace, a token stride of 2^24 elements or more),
 * GDN_ERR_CAPACITY (workspace_bytes too small).
 * Results equal the per-token recurrence up to fp32 rounding (a different
 * association of the same sums); sequence lengths need not be multiples of
 * 64.  Splitting a sequence across calls moves the chunk boundaries, so it
 * changes results only within that rounding.
 */
size_t gdn_chunk_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                int32_t num_k_heads, int32_t num_v_heads);

int gdn_chunk_gated_delta_rule(const gdn_bf16 *q, int64_t q_stride,
                               const gdn_bf16 *k, int64_t k_stride,
                               const gdn_bf16 *v, int64_t v_stride,
                               const float *g, const float *beta,
                               float *state, int32_t num_slots,
                               const int32_t *query_start_loc,
                               const int32_t *state_indices,
                               const uint8_t *has_initial_state,
                               gdn_bf16 *o, int64_t o_stride,
                               int32_t num_seqs, int32_t num_tokens,
                               int32_t num_k_heads, int32_t num_v_heads,
                               int32_t head_k_dim, int32_t head_v_dim,
                               void *workspace, size_t workspace_bytes,
                               float scale, int32_t qk_l2norm, void *stream);

/*
 * gdn_fused_conv_decode -- one decode step of the whole mixer: the
 * single-token conv update of every channel fused with the gated delta rule
 * on its output, in one launch.
 *
 * Sources: the width-4 conv and the fused GDN decode of page "RTX 5070 Ti:
 * close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section "Existing
 * evidence"; the rule from Yang, Kautz, Hatamizadeh, "Gated Delta Networks"
 * (ICLR 2025).
 *
 * Equivalent, bit for bit, to
 *   gdn_causal_conv1d_update(x, ..., y_tmp, ...)      (y_tmp in bf16)
 *   gdn_fused_recurrent_decode(q = y_tmp[:, 0 : HK dk],
 *                              k = y_tmp[:, HK dk : 2 HK dk],
 *                              v = y_tmp[:, 2 HK dk :], ...)
 * where the conv row is laid out q | k | v (channels = 2 HK dk + HV dv) and
 * batch row b uses slot state_indices[b] in both pools (negative: skipped).
 * The conv output is written to y only when y is not NULL.
 *
 *   x            bf16 [batch][x_stride]
 *   conv_weight  bf16 [channels][4];  conv_bias bf16 [channels] or NULL
 *   conv_state   bf16 [num_conv_slots][3][channels], in place
 *   g, beta      fp32 [batch][num_v_heads]
 *   state        fp32 [num_slots][num_v_heads][head_v_dim][head_k_dim], in place
 *   o            bf16, row b head h at o + b*o_stride + h*head_v_dim
 *   y            bf16 [batch][y_stride] or NULL
 *
 * Errors: GDN_ERR_INVALID (required pointer NULL, negative batch, slot
 * counts < 1, num_v_heads % num_k_heads, strides too small, o or y
 * overlapping x, state or conv_state, o overlapping g or beta, y
 * overlapping o); GDN_ERR_UNSUPPORTED (head dims as for
 * gdn_fused_recurrent_decode, more than 8192 conv channels read by one q/k
 * head group, alignment contract); GDN_ERR_HIP.
 */
int gdn_fused_conv_decode(const gdn_bf16 *x, int64_t x_stride,
                          const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias,
                          gdn_bf16 *conv_state, int32_t num_conv_slots,
                          const float *g, const float *beta,
                          float *state, int32_t num_slots,
                          const int32_t *state_indices,
                          gdn_bf16 *o, int64_t o_stride,
                          gdn_bf16 *y, int64_t y_stride,
                          int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                          int32_t head_k_dim, int32_t head_v_dim, int32_t silu,
                          float scale, int32_t qk_l2norm, void *stream);

/*
 * gdn_chunk_rule_and_fused_decode -- the recurrence of one engine step that
 * holds both prefill tokens and decode rows (after the prefill tokens' conv):
 * gdn_chunk_gated_delta_rule on the prefill tokens and gdn_fused_conv_decode
 * on the decode rows, with the chunkwise form's serial scan and the decode
 * sharing one grid.
 *
 * Sources: the serving workload of page "RTX 5070 Ti: close Qwen3.5-4B
 * TTFT, TPOT, and VRAM gaps vs vLLM", section "Problem" (concurrency 32, a
 * 2048-token batch budget), whose engine steps batch decode rows with
 * chunked-prefill tokens; the two operations are those of the two calls
 * named above.
 *
 * Why one grid: the scan walks each sequence's chunks in order on one
 * workgroup per (sequence, v-head, 64 v rows) and leaves most CUs idle for
 * its whole run; the decode is bandwidth-bound and independent of it.  The
 * scan's workgroups are placed first, the decode units take the CUs left,
 * then each CU a scan workgroup releases.
 *
 * Arguments:
 *   q .. workspace_bytes  the prefill tokens, exactly as the same-named
 *                         arguments of gdn_chunk_gated_delta_rule
 *   dec_x .. silu         the decode rows, as the arguments x .. silu of
 *                         gdn_fused_conv_decode (dec_g, dec_beta,
 *                         dec_state_indices, dec_o, dec_y, dec_batch for its
 *                         g, beta, state_indices, o, y, batch)
 *   state .. qk_l2norm    shared by both: the layer's recurrent-state pool
 *                         and head shape
 * The two halves run concurrently: a state slot may be used by only one of
 * them (state_indices and dec_state_indices disjoint, apart from negative
 * entries; a device-side precondition, not checked).  Every result --
 * o, dec_o, dec_y, the state slots and conv_state -- is bit-identical to
 * calling gdn_chunk_gated_delta_rule and then gdn_fused_conv_decode (either
 * order) with the same arguments.  An empty half (num_seqs or num_tokens 0,
 * dec_batch 0) is skipped: its other arguments are not checked (pointers
 * may be NULL) and overlap nothing; the call with both empty enqueues
 * nothing.  Shapes the shared grid does not take
 * (head_v_dim not a multiple of 64) run the two operations as consecutive
 * launches on `stream`.
 *
 * Errors: every error of either call, with its arguments; GDN_ERR_INVALID
 * when what one half writes (o, the workspace; dec_o, dec_y, conv_state)
 * overlaps an operand of the other half (q, k, v, g, beta, o, workspace;
 * dec_x, conv_weight, conv_bias, conv_state, dec_g, dec_beta, dec_o, dec_y).
 */
int gdn_chunk_rule_and_fused_decode(
    /* prefill tokens */
    const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride,
    const gdn_bf16 *v, int64_t v_stride, const float *g, const float *beta,
    const int32_t *query_start_loc, const int32_t *state_indices,
    const uint8_t *has_initial_state, gdn_bf16 *o, int64_t o_stride,
    int32_t num_seqs, int32_t num_tokens, void *workspace, size_t workspace_bytes,
    /* decode rows */
    const gdn_bf16 *dec_x, int64_t dec_x_stride,
    const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias,
    gdn_bf16 *conv_state, int32_t num_conv_slots,
    const float *dec_g, const float *dec_beta, const int32_t *dec_state_indices,
    gdn_bf16 *dec_o, int64_t dec_o_stride, gdn_bf16 *dec_y, int64_t dec_y_stride,
    int32_t dec_batch, int32_t silu,
    /* both */
    float *state, int32_t num_slots, int32_t num_k_heads, int32_t num_v_heads,
    int32_t head_k_dim, int32_t head_v_dim, float scale, int32_t qk_l2norm,
    void *stream);

/* Bytes of the static device scratch gdn_chunk_rule_and_fused_decode_noalloc
 * uses as its chunk workspace (one copy per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * gdn_chunk_rule_and_fused_decode_noalloc -- gdn_chunk_rule_and_fused_decode
 * without the workspace arguments, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The chunk workspace is instead a static device array
 * of GDN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held
 * until the process ends.
 *
 * Arguments, results and errors are those of gdn_chunk_rule_and_fused_decode
 * (which it calls with that array as the workspace); results are
 * bit-identical to it.  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.  Its first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress) and keeps the
 * address.
 *
 * Limit: a prefill half whose gdn_chunk_workspace_size(num_seqs, num_tokens,
 * num_k_heads, num_v_heads) exceeds GDN_NOALLOC_SCRATCH_BYTES is refused
 * with GDN_ERR_CAPACITY (at 16 q/k and 32 v heads that is about 96 chunks of
 * 64 tokens, e.g. 2048 tokens in up to 64 sequences).
 *
 * Sharing: every call on one GPU uses that GPU's one array, which keeps what
 * the last call wrote (nothing in it needs to start cleared: each call
 * writes every record it reads).  Calls that overlap in time on one GPU --
 * on different streams or from different threads -- race on the array and
 * give wrong results; the caller must order them, e.g. on one stream.
 */
int gdn_chunk_rule_and_fused_decode_noalloc(
    /* prefill tokens */
    const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride,
    const gdn_bf16 *v, int64_t v_stride, const float *g, const float *beta,
    const int32_t *query_start_loc, const int32_t *state_indices,
    const uint8_t *has_initial_state, gdn_bf16 *o, int64_t o_stride,
    int32_t num_seqs, int32_t num_tokens,
    /* decode rows */
    const gdn_bf16 *dec_x, int64_t dec_x_stride,
    const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias,
    gdn_bf16 *conv_state, int32_t num_conv_slots,
    const float *dec_g, const float *dec_beta, const int32_t *dec_state_indices,
    gdn_bf16 *dec_o, int64_t dec_o_stride, gdn_bf16 *dec_y, int64_t dec_y_stride,
    int32_t dec_batch, int32_t silu,
    /* both */
    float *state, int32_t num_slots, int32_t num_k_heads, int32_t num_v_heads,
    int32_t head_k_dim, int32_t head_v_dim, float scale, int32_t qk_l2norm,
    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
