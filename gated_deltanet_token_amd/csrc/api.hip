// C-ABI entry points of libgdn: host-side argument validation, the chunk
// descriptor builder, and kernel launches on the caller's stream.  Every
// check runs before anything is enqueued; a failing call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

#define GDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return GDN_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// byte range of a strided row buffer [rows][stride] whose rows use `cols`
// elements of `elem` bytes
struct Span {
    uintptr_t lo, hi;
};
Span row_span(const void *p, int64_t rows, int64_t stride, int64_t cols, int64_t elem) {
    const uintptr_t lo = (uintptr_t)p;
    if (rows <= 0 || cols <= 0) return {lo, lo};
    return {lo, lo + (uintptr_t)(((rows - 1) * stride + cols) * elem)};
}
// empty ranges overlap nothing
bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int check_conv_common(const void *x, int64_t x_stride, const void *weight, const void *bias,
                      const void *conv_state, int32_t num_slots, const void *y, int64_t y_stride,
                      int32_t rows, int32_t channels, int32_t width) {
    if (!x || !weight || !conv_state || !y) return fail(GDN_ERR_INVALID, "x, weight, conv_state and y are required");
    if (rows < 0 || channels <= 0) return fail(GDN_ERR_INVALID, "negative token count or non-positive channels");
    if (num_slots < 1) return fail(GDN_ERR_INVALID, "num_slots must be >= 1");
    if (width != GDN_CONV_WIDTH) return fail(GDN_ERR_UNSUPPORTED, "conv width %d: only 4 is implemented", width);
    if (x_stride < channels || y_stride < channels) return fail(GDN_ERR_INVALID, "row stride smaller than channels");
    if (channels % 8 || x_stride % 8 || y_stride % 8)
        return fail(GDN_ERR_UNSUPPORTED, "channels and strides must be multiples of 8 elements");
    if (!aligned16(x) || !aligned16(y) || !aligned16(weight) || !aligned16(conv_state) ||
        (bias && !aligned16(bias)))
        return fail(GDN_ERR_UNSUPPORTED, "x, y, weight, bias and conv_state must be 16-byte aligned");
    const Span ys = row_span(y, rows, y_stride, channels, 2);
    if (overlap(row_span(x, rows, x_stride, channels, 2), ys)) return fail(GDN_ERR_INVALID, "y overlaps x");
    const Span cs = {(uintptr_t)conv_state, (uintptr_t)conv_state + (uintptr_t)num_slots * 3 * channels * 2};
    const Span ws = {(uintptr_t)weight, (uintptr_t)weight + (uintptr_t)channels * width * 2};
    const Span bs = {(uintptr_t)bias, bias ? (uintptr_t)bias + (uintptr_t)channels * 2 : (uintptr_t)bias};
    if (overlap(ys, cs) || overlap(ys, ws) || overlap(ys, bs))
        return fail(GDN_ERR_INVALID, "y overlaps conv_state, weight or bias");
    return ok();
}

}  // namespace

GDN_EXPORT const char *gdn_last_error(void) { return g_err; }

GDN_EXPORT int gdn_build_conv_chunks(const int32_t *qsl_host, int32_t num_seqs, gdn_conv_chunk *out_host,
                                     int32_t capacity, int32_t *n_out) {
    if (!qsl_host || !n_out) return fail(GDN_ERR_INVALID, "qsl_host and n_out are required");
    if (num_seqs < 0 || capacity < 0) return fail(GDN_ERR_INVALID, "negative num_seqs or capacity");
    if (capacity > 0 && !out_host) return fail(GDN_ERR_INVALID, "out_host is NULL with capacity > 0");
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t len = (int64_t)qsl_host[s + 1] - qsl_host[s];
        if (len < 0) return fail(GDN_ERR_INVALID, "query_start_loc decreases at sequence %d", s);
        const int64_t chunks = (len + GDN_CONV_CHUNK_TOKENS - 1) / GDN_CONV_CHUNK_TOKENS;
        for (int64_t c = 0; c < chunks; ++c, ++n) {
            if (n < capacity) out_host[n] = gdn_conv_chunk{s, (int32_t)c};
        }
        if (n > INT32_MAX) return fail(GDN_ERR_INVALID, "descriptor count overflows int32");
    }
    *n_out = (int32_t)n;
    if (n > capacity) return fail(GDN_ERR_CAPACITY, "%lld descriptors needed, capacity %d", (long long)n, capacity);
    return ok();
}

// validation shared by the varlen conv entry points; fills `a` and sets
// `launch` when there is work
static int conv_varlen_args(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *weight, const gdn_bf16 *bias,
                            gdn_bf16 *conv_state, int32_t num_slots, const int32_t *query_start_loc,
                            const int32_t *state_indices, const uint8_t *has_initial_state,
                            const gdn_conv_chunk *chunks, int32_t n_chunks, gdn_bf16 *y, int64_t y_stride,
                            int32_t num_seqs, int32_t num_tokens, int32_t channels, int32_t width, int32_t silu,
                            gdn::ConvVarlenArgs &a, bool &launch) {
    launch = false;
    int rc = check_conv_common(x, x_stride, weight, bias, conv_state, num_slots, y, y_stride, num_tokens,
                               channels, width);
    if (rc) return rc;
    if (num_seqs < 0 || n_chunks < 0) return fail(GDN_ERR_INVALID, "negative num_seqs or n_chunks");
    if ((chunks == nullptr) != (n_chunks == 0))
        return fail(GDN_ERR_INVALID, "chunks and n_chunks must be given together");
    // the descriptors are the only dispatch: a call with tokens needs them
    if (n_chunks == 0) {
        if (num_tokens > 0)
            return fail(GDN_ERR_INVALID, "%d tokens but no chunk descriptors (build them with gdn_build_conv_chunks)",
                        num_tokens);
        return ok();
    }
    if (!query_start_loc || !state_indices) return fail(GDN_ERR_INVALID, "query_start_loc and state_indices are required");
    if (num_seqs == 0 || num_tokens == 0) return fail(GDN_ERR_INVALID, "descriptors given for an empty batch");
    if ((int64_t)n_chunks > (int64_t)num_tokens)
        return fail(GDN_ERR_INVALID, "more descriptors (%d) than tokens (%d)", n_chunks, num_tokens);
    // each descriptor covers at most 8 tokens, so fewer than ceil(T / 8) of
    // them cannot cover the call's tokens
    const int64_t min_chunks = ((int64_t)num_tokens + GDN_CONV_CHUNK_TOKENS - 1) / GDN_CONV_CHUNK_TOKENS;
    if ((int64_t)n_chunks < min_chunks)
        return fail(GDN_ERR_INVALID, "%d descriptors cannot cover %d tokens (at least %lld needed)", n_chunks,
                    num_tokens, (long long)min_chunks);
    a = gdn::ConvVarlenArgs{x, x_stride, weight, bias, conv_state, query_start_loc, state_indices,
                            has_initial_state, chunks, n_chunks, y, y_stride, channels, silu,
                            num_seqs, num_slots, num_tokens};
    launch = true;
    return ok();
}

GDN_EXPORT int gdn_causal_conv1d_varlen(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *weight,
                                        const gdn_bf16 *bias, gdn_bf16 *conv_state, int32_t num_slots,
                                        const int32_t *query_start_loc, const int32_t *state_indices,
                                        const uint8_t *has_initial_state, const gdn_conv_chunk *chunks,
                                        int32_t n_chunks, gdn_bf16 *y, int64_t y_stride, int32_t num_seqs,
                                        int32_t num_tokens, int32_t channels, int32_t width, int32_t silu,
                                        void *stream) {
    gdn::ConvVarlenArgs a{};
    bool launch;
    const int rc = conv_varlen_args(x, x_stride, weight, bias, conv_state, num_slots, query_start_loc,
                                    state_indices, has_initial_state, chunks, n_chunks, y, y_stride, num_seqs,
                                    num_tokens, channels, width, silu, a, launch);
    if (rc || !launch) return rc;
    return hip_status(gdn::launch_conv_varlen(a, (hipStream_t)stream), "conv varlen launch");
}

GDN_EXPORT int gdn_causal_conv1d_varlen_tiles(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *weight,
                                              const gdn_bf16 *bias, gdn_bf16 *conv_state, int32_t num_slots,
                                              const int32_t *query_start_loc, const int32_t *state_indices,
                                              const uint8_t *has_initial_state, const gdn_conv_chunk *chunks,
                                              int32_t n_chunks, gdn_bf16 *y, int64_t y_stride, int32_t num_seqs,
                                              int32_t num_tokens, int32_t channels, int32_t width, int32_t silu,
                                              int32_t descriptors_per_program, void *stream) {
    if (descriptors_per_program != 1 && descriptors_per_program != 2)
        return fail(GDN_ERR_UNSUPPORTED, "descriptors_per_program %d: must be 1 or 2", descriptors_per_program);
    gdn::ConvVarlenArgs a{};
    bool launch;
    const int rc = conv_varlen_args(x, x_stride, weight, bias, conv_state, num_slots, query_start_loc,
                                    state_indices, has_initial_state, chunks, n_chunks, y, y_stride, num_seqs,
                                    num_tokens, channels, width, silu, a, launch);
    if (rc || !launch) return rc;
    // the 16-token programs address rows with 32-bit byte offsets
    if (descriptors_per_program == 2 && (x_stride > ((int64_t)1 << 26) || y_stride > ((int64_t)1 << 26)))
        return fail(GDN_ERR_UNSUPPORTED, "16-token programs need row strides up to 2^26 elements");
    a.descriptors_per_program = descriptors_per_program;
    return hip_status(gdn::launch_conv_varlen(a, (hipStream_t)stream), "conv varlen launch");
}

GDN_EXPORT int gdn_causal_conv1d_update(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *weight,
                                        const gdn_bf16 *bias, gdn_bf16 *conv_state, int32_t num_slots,
                                        const int32_t *state_indices, gdn_bf16 *y, int64_t y_stride,
                                        int32_t batch, int32_t channels, int32_t width, int32_t silu,
                                        void *stream) {
    int rc = check_conv_common(x, x_stride, weight, bias, conv_state, num_slots, y, y_stride, batch,
                               channels, width);
    if (rc) return rc;
    if (batch == 0) return ok();
    if (!state_indices) return fail(GDN_ERR_INVALID, "state_indices is required");
    gdn::ConvUpdateArgs a{x, x_stride, weight, bias, conv_state, state_indices, y, y_stride, batch, channels, silu,
                          num_slots};
    return hip_status(gdn::launch_conv_update(a, (hipStream_t)stream), "conv update launch");
}

namespace {

// shared validation of the two recurrence entry points; returns GDN_OK and
// fills `a` when the call is valid and non-empty, 1 when there is nothing to do
int check_recurrent(const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride, const gdn_bf16 *v,
                    int64_t v_stride, const float *g, const float *beta, float *state, int32_t num_slots,
                    const int32_t *query_start_loc, const int32_t *state_indices, const uint8_t *has_initial_state,
                    gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens, int32_t num_k_heads,
                    int32_t num_v_heads, int32_t head_k_dim, int32_t head_v_dim, float scale, int32_t qk_l2norm,
                    gdn::RecurrentArgs &a) {
    if (!q || !k || !v || !g || !beta || !state || !state_indices || !o)
        return fail(GDN_ERR_INVALID, "q, k, v, g, beta, state, state_indices and o are required");
    if (num_seqs < 0 || num_tokens < 0) return fail(GDN_ERR_INVALID, "negative num_seqs or num_tokens");
    if (num_slots < 1) return fail(GDN_ERR_INVALID, "num_slots must be >= 1");
    if (num_k_heads <= 0 || num_v_heads <= 0 || num_v_heads % num_k_heads)
        return fail(GDN_ERR_INVALID, "num_v_heads must be a positive multiple of num_k_heads");
    if (head_k_dim != 16 && head_k_dim != 32 && head_k_dim != 64 && head_k_dim != 128)
        return fail(GDN_ERR_UNSUPPORTED, "head_k_dim %d: supported 16, 32, 64, 128", head_k_dim);
    if (head_v_dim <= 0 || head_v_dim % 8 || head_v_dim > 256)
        return fail(GDN_ERR_UNSUPPORTED, "head_v_dim %d: must be a multiple of 8 up to 256", head_v_dim);
    const int64_t qk_w = (int64_t)num_k_heads * head_k_dim, v_w = (int64_t)num_v_heads * head_v_dim;
    if (q_stride < qk_w || k_stride < qk_w || v_stride < v_w || o_stride < v_w)
        return fail(GDN_ERR_INVALID, "a token stride is smaller than its row of heads");
    if (q_stride % 8 || k_stride % 8 || v_stride % 8 || o_stride % 8)
        return fail(GDN_ERR_UNSUPPORTED, "token strides must be multiples of 8 elements");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
        return fail(GDN_ERR_UNSUPPORTED, "q, k, v, o and state must be 16-byte aligned");
    if (!query_start_loc && num_tokens != num_seqs)
        return fail(GDN_ERR_INVALID, "without query_start_loc num_tokens must equal num_seqs");
    const Span os = row_span(o, num_tokens, o_stride, v_w, 2);
    const Span st = {(uintptr_t)state, (uintptr_t)state + (uintptr_t)num_slots * (uintptr_t)v_w * head_k_dim * 4};
    const Span gs = {(uintptr_t)g, (uintptr_t)g + (uintptr_t)num_tokens * num_v_heads * 4};
    const Span bs = {(uintptr_t)beta, (uintptr_t)beta + (uintptr_t)num_tokens * num_v_heads * 4};
    if (overlap(os, row_span(q, num_tokens, q_stride, qk_w, 2)) ||
        overlap(os, row_span(k, num_tokens, k_stride, qk_w, 2)) ||
        overlap(os, row_span(v, num_tokens, v_stride, v_w, 2)) || overlap(os, st) || overlap(os, gs) ||
        overlap(os, bs))
        return fail(GDN_ERR_INVALID, "o overlaps q, k, v, g, beta or state");
    if (num_seqs == 0 || num_tokens == 0) {
        ok();
        return 1;
    }
    a = gdn::RecurrentArgs{q, q_stride, k, k_stride, v, v_stride, g, beta, state, query_start_loc, state_indices,
                           has_initial_state, o, o_stride, num_seqs, num_k_heads, num_v_heads, head_k_dim,
                           head_v_dim, scale, qk_l2norm, num_slots, num_tokens};
    return GDN_OK;
}

}  // namespace

GDN_EXPORT int gdn_fused_recurrent_decode(const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride,
                                          const gdn_bf16 *v, int64_t v_stride, const float *g, const float *beta,
                                          float *state, int32_t num_slots, const int32_t *query_start_loc,
                                          const int32_t *state_indices, const uint8_t *has_initial_state,
                                          gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens,
                                          int32_t num_k_heads, int32_t num_v_heads, int32_t head_k_dim,
                                          int32_t head_v_dim, float scale, int32_t qk_l2norm, void *stream) {
    gdn::RecurrentArgs a;
    const int rc = check_recurrent(q, q_stride, k, k_stride, v, v_stride, g, beta, state, num_slots,
                                   query_start_loc, state_indices, has_initial_state, o, o_stride, num_seqs,
                                   num_tokens, num_k_heads, num_v_heads, head_k_dim, head_v_dim, scale, qk_l2norm, a);
    if (rc == 1) return GDN_OK;
    if (rc) return rc;
    return hip_status(gdn::launch_recurrent(a, (hipStream_t)stream), "recurrent launch");
}

GDN_EXPORT size_t gdn_chunk_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_k_heads,
                                           int32_t num_v_heads) {
    if (num_seqs < 0 || num_tokens < 0 || num_k_heads < 0 || num_v_heads < 0) return 0;
    return (size_t)gdn::chunk_workspace_bytes(num_seqs, num_tokens, num_k_heads, num_v_heads);
}

namespace {

// the chunkwise call's checks; 1 = nothing to do, with GDN_OK recorded
int check_chunk(const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride, const gdn_bf16 *v,
                int64_t v_stride, const float *g, const float *beta, float *state, int32_t num_slots,
                const int32_t *query_start_loc, const int32_t *state_indices, const uint8_t *has_initial_state,
                gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens, int32_t num_k_heads,
                int32_t num_v_heads, int32_t head_k_dim, int32_t head_v_dim, void *workspace,
                size_t workspace_bytes, float scale, int32_t qk_l2norm, gdn::RecurrentArgs &a) {
    if (!query_start_loc) return fail(GDN_ERR_INVALID, "query_start_loc is required");
    const int rc = check_recurrent(q, q_stride, k, k_stride, v, v_stride, g, beta, state, num_slots,
                                   query_start_loc, state_indices, has_initial_state, o, o_stride, num_seqs,
                                   num_tokens, num_k_heads, num_v_heads, head_k_dim, head_v_dim, scale, qk_l2norm, a);
    if (rc) return rc;
    if (head_k_dim != 128) return fail(GDN_ERR_UNSUPPORTED, "chunked form: head_k_dim must be 128");
    if (head_v_dim % 32) return fail(GDN_ERR_UNSUPPORTED, "chunked form: head_v_dim must be a multiple of 32");
    // the kernels address a 64-token chunk's rows with 32-bit byte offsets
    if (q_stride >= (1 << 24) || k_stride >= (1 << 24) || v_stride >= (1 << 24) || o_stride >= (1 << 24))
        return fail(GDN_ERR_UNSUPPORTED, "chunked form: token strides must be below 2^24 elements");
    const size_t need = (size_t)gdn::chunk_workspace_bytes(num_seqs, num_tokens, num_k_heads, num_v_heads);
    if (!workspace) return fail(GDN_ERR_INVALID, "workspace is required (%zu bytes)", need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(GDN_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(GDN_ERR_CAPACITY, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    // the kernels write the first `need` bytes of the workspace: they must not
    // be any operand's
    const Span ws = {(uintptr_t)workspace, (uintptr_t)workspace + need};
    const int64_t qk_w = (int64_t)num_k_heads * head_k_dim, v_w = (int64_t)num_v_heads * head_v_dim;
    const Span st = {(uintptr_t)state, (uintptr_t)state + (uintptr_t)num_slots * (uintptr_t)v_w * head_k_dim * 4};
    const Span gs = {(uintptr_t)g, (uintptr_t)g + (uintptr_t)num_tokens * num_v_heads * 4};
    const Span bs = {(uintptr_t)beta, (uintptr_t)beta + (uintptr_t)num_tokens * num_v_heads * 4};
    if (overlap(ws, row_span(q, num_tokens, q_stride, qk_w, 2)) || overlap(ws, row_span(k, num_tokens, k_stride, qk_w, 2)) ||
        overlap(ws, row_span(v, num_tokens, v_stride, v_w, 2)) || overlap(ws, row_span(o, num_tokens, o_stride, v_w, 2)) ||
        overlap(ws, st) || overlap(ws, gs) || overlap(ws, bs))
        return fail(GDN_ERR_INVALID, "workspace overlaps q, k, v, g, beta, state or o");
    return GDN_OK;
}

}  // namespace

GDN_EXPORT int gdn_chunk_gated_delta_rule(const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride,
                                          const gdn_bf16 *v, int64_t v_stride, const float *g, const float *beta,
                                          float *state, int32_t num_slots, const int32_t *query_start_loc,
                                          const int32_t *state_indices, const uint8_t *has_initial_state,
                                          gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens,
                                          int32_t num_k_heads, int32_t num_v_heads, int32_t head_k_dim,
                                          int32_t head_v_dim, void *workspace, size_t workspace_bytes,
                                          float scale, int32_t qk_l2norm, void *stream) {
    gdn::RecurrentArgs a;
    const int rc = check_chunk(q, q_stride, k, k_stride, v, v_stride, g, beta, state, num_slots, query_start_loc,
                               state_indices, has_initial_state, o, o_stride, num_seqs, num_tokens, num_k_heads,
                               num_v_heads, head_k_dim, head_v_dim, workspace, workspace_bytes, scale, qk_l2norm, a);
    if (rc == 1) return GDN_OK;
    if (rc) return rc;
    return hip_status(gdn::launch_chunk_recurrent(a, workspace, num_tokens, (hipStream_t)stream),
                      "chunk recurrent launch");
}

namespace {

// the fused decode call's checks; 1 = nothing to do, with GDN_OK recorded
int check_fused(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias,
                gdn_bf16 *conv_state, int32_t num_conv_slots, const float *g, const float *beta, float *state,
                int32_t num_slots, const int32_t *state_indices, gdn_bf16 *o, int64_t o_stride, gdn_bf16 *y,
                int64_t y_stride, int32_t batch, int32_t num_k_heads, int32_t num_v_heads, int32_t head_k_dim,
                int32_t head_v_dim, int32_t silu, float scale, int32_t qk_l2norm, gdn::FusedDecodeArgs &a) {
    if (!x || !conv_weight || !conv_state || !g || !beta || !state || !state_indices || !o)
        return fail(GDN_ERR_INVALID, "x, conv_weight, conv_state, g, beta, state, state_indices and o are required");
    if (batch < 0) return fail(GDN_ERR_INVALID, "negative batch");
    if (num_conv_slots < 1 || num_slots < 1) return fail(GDN_ERR_INVALID, "slot counts must be >= 1");
    if (num_k_heads <= 0 || num_v_heads <= 0 || num_v_heads % num_k_heads)
        return fail(GDN_ERR_INVALID, "num_v_heads must be a positive multiple of num_k_heads");
    if (head_k_dim != 16 && head_k_dim != 32 && head_k_dim != 64 && head_k_dim != 128)
        return fail(GDN_ERR_UNSUPPORTED, "head_k_dim %d: supported 16, 32, 64, 128", head_k_dim);
    if (head_v_dim <= 0 || head_v_dim % 8 || head_v_dim > 256)
        return fail(GDN_ERR_UNSUPPORTED, "head_v_dim %d: must be a multiple of 8 up to 256", head_v_dim);
    const int64_t grp = num_v_heads / num_k_heads;
    if (2 * head_k_dim + grp * head_v_dim > gdn::fused_max_group_channels())
        return fail(GDN_ERR_UNSUPPORTED, "a q/k head group reads more than %d conv channels",
                    gdn::fused_max_group_channels());
    const int64_t channels = 2 * (int64_t)num_k_heads * head_k_dim + (int64_t)num_v_heads * head_v_dim;
    const int64_t v_w = (int64_t)num_v_heads * head_v_dim;
    if (channels > INT32_MAX) return fail(GDN_ERR_INVALID, "channel count overflows int32");
    if (x_stride < channels || (y && y_stride < channels) || o_stride < v_w)
        return fail(GDN_ERR_INVALID, "a row stride is smaller than its row");
    if (x_stride % 8 || (y && y_stride % 8) || o_stride % 8)
        return fail(GDN_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
    if (!aligned16(x) || !aligned16(conv_weight) || (conv_bias && !aligned16(conv_bias)) || !aligned16(conv_state) ||
        !aligned16(state) || !aligned16(o) || (y && !aligned16(y)))
        return fail(GDN_ERR_UNSUPPORTED, "x, conv_weight, conv_bias, conv_state, state, o and y must be 16-byte aligned");
    const Span xs = row_span(x, batch, x_stride, channels, 2);
    const Span os = row_span(o, batch, o_stride, v_w, 2);
    const Span sts = {(uintptr_t)state,
                      (uintptr_t)state + (uintptr_t)num_slots * (uintptr_t)v_w * head_k_dim * 4};
    const Span css = {(uintptr_t)conv_state, (uintptr_t)conv_state + (uintptr_t)num_conv_slots * 3 * channels * 2};
    const Span gs = {(uintptr_t)g, (uintptr_t)g + (uintptr_t)batch * num_v_heads * 4};
    const Span bes = {(uintptr_t)beta, (uintptr_t)beta + (uintptr_t)batch * num_v_heads * 4};
    if (overlap(xs, os) || overlap(os, sts) || overlap(os, css) || overlap(os, gs) || overlap(os, bes))
        return fail(GDN_ERR_INVALID, "o overlaps x, state, conv_state, g or beta");
    if (y) {
        const Span ys = row_span(y, batch, y_stride, channels, 2);
        if (overlap(xs, ys) || overlap(os, ys) || overlap(ys, sts) || overlap(ys, css))
            return fail(GDN_ERR_INVALID, "y overlaps x, o, state or conv_state");
    }
    if (batch == 0) {
        ok();
        return 1;
    }
    a = gdn::FusedDecodeArgs{x, x_stride, conv_weight, conv_bias, conv_state, (int)channels, g, beta, state,
                             state_indices, o, o_stride, y, y_stride, batch, num_k_heads, num_v_heads, head_k_dim,
                             head_v_dim, scale, qk_l2norm, silu, num_slots, num_conv_slots};
    return GDN_OK;
}

}  // namespace

GDN_EXPORT int gdn_fused_conv_decode(const gdn_bf16 *x, int64_t x_stride, const gdn_bf16 *conv_weight,
                                     const gdn_bf16 *conv_bias, gdn_bf16 *conv_state, int32_t num_conv_slots,
                                     const float *g, const float *beta, float *state, int32_t num_slots,
                                     const int32_t *state_indices, gdn_bf16 *o, int64_t o_stride, gdn_bf16 *y,
                                     int64_t y_stride, int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                                     int32_t head_k_dim, int32_t head_v_dim, int32_t silu, float scale,
                                     int32_t qk_l2norm, void *stream) {
    gdn::FusedDecodeArgs a;
    const int rc = check_fused(x, x_stride, conv_weight, conv_bias, conv_state, num_conv_slots, g, beta, state,
                               num_slots, state_indices, o, o_stride, y, y_stride, batch, num_k_heads, num_v_heads,
                               head_k_dim, head_v_dim, silu, scale, qk_l2norm, a);
    if (rc == 1) return GDN_OK;
    if (rc) return rc;
    return hip_status(gdn::launch_fused_conv_decode(a, (hipStream_t)stream), "fused conv decode launch");
}

GDN_EXPORT int gdn_chunk_rule_and_fused_decode(
    const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride, const gdn_bf16 *v, int64_t v_stride,
    const float *g, const float *beta, const int32_t *query_start_loc, const int32_t *state_indices,
    const uint8_t *has_initial_state, gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens,
    void *workspace, size_t workspace_bytes, const gdn_bf16 *dec_x, int64_t dec_x_stride,
    const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias, gdn_bf16 *conv_state, int32_t num_conv_slots,
    const float *dec_g, const float *dec_beta, const int32_t *dec_state_indices, gdn_bf16 *dec_o,
    int64_t dec_o_stride, gdn_bf16 *dec_y, int64_t dec_y_stride, int32_t dec_batch, int32_t silu, float *state,
    int32_t num_slots, int32_t num_k_heads, int32_t num_v_heads, int32_t head_k_dim, int32_t head_v_dim,
    float scale, int32_t qk_l2norm, void *stream) {
    // an empty half is skipped unchecked (its pointers may be NULL)
    gdn::RecurrentArgs a;
    const int rc_c = num_seqs == 0 || num_tokens == 0
                         ? (num_seqs < 0 || num_tokens < 0 ? fail(GDN_ERR_INVALID, "negative num_seqs or num_tokens")
                                                           : 1)
                         : check_chunk(q, q_stride, k, k_stride, v, v_stride, g, beta, state, num_slots,
                                       query_start_loc, state_indices, has_initial_state, o, o_stride, num_seqs,
                                       num_tokens, num_k_heads, num_v_heads, head_k_dim, head_v_dim, workspace,
                                       workspace_bytes, scale, qk_l2norm, a);
    if (rc_c < 0) return rc_c;
    gdn::FusedDecodeArgs f;
    const int rc_f = dec_batch == 0
                         ? 1
                         : check_fused(dec_x, dec_x_stride, conv_weight, conv_bias, conv_state, num_conv_slots,
                                       dec_g, dec_beta, state, num_slots, dec_state_indices, dec_o, dec_o_stride,
                                       dec_y, dec_y_stride, dec_batch, num_k_heads, num_v_heads, head_k_dim,
                                       head_v_dim, silu, scale, qk_l2norm, f);
    if (rc_f < 0) return rc_f;
    ok();
    // the two halves run at the same time: what one writes must be none of
    // the other's operands (the shared state pool aside: its slots must be
    // distinct across both halves, a precondition not checked here)
    const int64_t qk_w = (int64_t)num_k_heads * head_k_dim, v_w = (int64_t)num_v_heads * head_v_dim;
    const int64_t channels = 2 * qk_w + v_w;
    const int64_t nt = rc_c == 1 ? 0 : num_tokens, nb = rc_f == 1 ? 0 : dec_batch;
    const Span p_in[] = {row_span(q, nt, q_stride, qk_w, 2), row_span(k, nt, k_stride, qk_w, 2),
                         row_span(v, nt, v_stride, v_w, 2),
                         {(uintptr_t)g, (uintptr_t)g + (uintptr_t)(nt * num_v_heads * 4)},
                         {(uintptr_t)beta, (uintptr_t)beta + (uintptr_t)(nt * num_v_heads * 4)}};
    const Span p_out[] = {row_span(o, nt, o_stride, v_w, 2),
                          {(uintptr_t)workspace,
                           (uintptr_t)workspace + (nt ? (uintptr_t)gdn::chunk_workspace_bytes(
                                                            num_seqs, num_tokens, num_k_heads, num_v_heads)
                                                      : 0)}};
    const Span d_in[] = {row_span(dec_x, nb, dec_x_stride, channels, 2),
                         {(uintptr_t)conv_weight, (uintptr_t)conv_weight + (uintptr_t)(nb ? channels * 4 * 2 : 0)},
                         {(uintptr_t)conv_bias,
                          (uintptr_t)conv_bias + (uintptr_t)(nb && conv_bias ? channels * 2 : 0)},
                         {(uintptr_t)dec_g, (uintptr_t)dec_g + (uintptr_t)(nb * num_v_heads * 4)},
                         {(uintptr_t)dec_beta, (uintptr_t)dec_beta + (uintptr_t)(nb * num_v_heads * 4)}};
    const Span d_out[] = {row_span(dec_o, nb, dec_o_stride, v_w, 2),
                          row_span(dec_y, dec_y ? nb : 0, dec_y_stride, channels, 2),
                          {(uintptr_t)conv_state,
                           (uintptr_t)conv_state + (uintptr_t)(nb ? (int64_t)num_conv_slots * 3 * channels * 2 : 0)}};
    for (const Span &w : p_out) {
        for (const Span &r : d_in)
            if (overlap(w, r)) return fail(GDN_ERR_INVALID, "a prefill output (o, workspace) overlaps a decode input");
        for (const Span &r : d_out)
            if (overlap(w, r)) return fail(GDN_ERR_INVALID, "a prefill output (o, workspace) overlaps a decode output");
    }
    for (const Span &w : d_out)
        for (const Span &r : p_in)
            if (overlap(w, r))
                return fail(GDN_ERR_INVALID, "a decode output (o, y, conv_state) overlaps a prefill input");
    if (rc_c == 1 && rc_f == 1) return GDN_OK;
    if (rc_c == 1) return hip_status(gdn::launch_fused_conv_decode(f, (hipStream_t)stream), "fused conv decode launch");
    if (rc_f == 1)
        return hip_status(gdn::launch_chunk_recurrent(a, workspace, num_tokens, (hipStream_t)stream),
                          "chunk recurrent launch");
    return hip_status(gdn::launch_chunk_and_decode(a, workspace, num_tokens, f, (hipStream_t)stream),
                      "chunk and decode launch");
}

// ---------------------------------------------------------------------------
// The mixed-step call without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).
// Its workspace is `scratch`, one static device array: every GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code the array's name only stands in for the symbol; the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
// ---------------------------------------------------------------------------
namespace {

static_assert(GDN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];      // device address of `scratch`, per device (set once)

// the current device's copy of `scratch`
int scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

GDN_EXPORT int gdn_chunk_rule_and_fused_decode_noalloc(
    const gdn_bf16 *q, int64_t q_stride, const gdn_bf16 *k, int64_t k_stride, const gdn_bf16 *v, int64_t v_stride,
    const float *g, const float *beta, const int32_t *query_start_loc, const int32_t *state_indices,
    const uint8_t *has_initial_state, gdn_bf16 *o, int64_t o_stride, int32_t num_seqs, int32_t num_tokens,
    const gdn_bf16 *dec_x, int64_t dec_x_stride, const gdn_bf16 *conv_weight, const gdn_bf16 *conv_bias,
    gdn_bf16 *conv_state, int32_t num_conv_slots, const float *dec_g, const float *dec_beta,
    const int32_t *dec_state_indices, gdn_bf16 *dec_o, int64_t dec_o_stride, gdn_bf16 *dec_y, int64_t dec_y_stride,
    int32_t dec_batch, int32_t silu, float *state, int32_t num_slots, int32_t num_k_heads, int32_t num_v_heads,
    int32_t head_k_dim, int32_t head_v_dim, float scale, int32_t qk_l2norm, void *stream) {
    void *ws = nullptr;
    if (num_seqs > 0 && num_tokens > 0 && num_k_heads > 0 && num_v_heads > 0) {
        const int64_t need = gdn::chunk_workspace_bytes(num_seqs, num_tokens, num_k_heads, num_v_heads);
        if (need > (int64_t)GDN_NOALLOC_SCRATCH_BYTES)
            return fail(GDN_ERR_CAPACITY,
                        "%d tokens in %d sequences need %lld bytes of chunk workspace; the static scratch holds %llu "
                        "(use gdn_chunk_rule_and_fused_decode with a workspace)",
                        num_tokens, num_seqs, (long long)need, (unsigned long long)GDN_NOALLOC_SCRATCH_BYTES);
        const int rc = scratch_on_current_device(&ws);
        if (rc) return rc;
    }
    return gdn_chunk_rule_and_fused_decode(
        q, q_stride, k, k_stride, v, v_stride, g, beta, query_start_loc, state_indices, has_initial_state, o,
        o_stride, num_seqs, num_tokens, ws, ws ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0, dec_x, dec_x_stride,
        conv_weight, conv_bias, conv_state, num_conv_slots, dec_g, dec_beta, dec_state_indices, dec_o, dec_o_stride,
        dec_y, dec_y_stride, dec_batch, silu, state, num_slots, num_k_heads, num_v_heads, head_k_dim, head_v_dim,
        scale, qk_l2norm, stream);
}
