/*
 * gdn_oracle.c -- plain, serial, double-precision CPU oracle for the Gated
 * DeltaNet token-mixer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the HIP library is
 * checked against; it is never part of the product path.  Only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Serial as compiled for the tests.  The OpenMP pragmas mark loops whose
 * iterations are independent (channels of the conv, (sequence, v-head)
 * pairs of the recurrence); built with -fopenmp for the benchmark's
 * multi-core CPU baseline they run those iterations on several threads,
 * each iteration doing exactly the same operations in the same order, so
 * both builds give bit-identical results.
 *
 * Every function reads bf16 inputs exactly (bf16 -> double is exact), does
 * all arithmetic in double, and returns double results unrounded, so the
 * comparison with the GPU measures the GPU's error alone.  The state pools
 * the oracle carries are double too, so a sequence split across calls gives
 * bit-identical results to one pass (the same operations in the same order).
 *
 * Sources:
 *  - chunk descriptors: page "perf(gdn): dispatch exact causal-conv chunks",
 *    section "What changed" (one program per exact (sequence, 8-token chunk)
 *    pair, built once per engine step), and the reviewer comment on that page
 *    (descriptor optional, the (buffer, count) pair validated together);
 *  - conv width 4: page "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM
 *    gaps vs vLLM", section "Existing evidence" (the K=4 causal-conv arm);
 *  - the gated delta rule: Yang, Kautz, Hatamizadeh, "Gated Delta Networks:
 *    Improving Mamba2 with Delta Rule" (ICLR 2025), the recurrent form
 *    S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t;
 *    the fused decode is named on page "RTX 5070 Ti: ...", section
 *    "Existing evidence" (register-resident fused decode).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - conv taps: cross-correlation with K-1 zeros / carried state on the left;
 *    w[c][K-1] multiplies the current token;
 *  - conv_state slot: the K-1 inputs preceding the next token, oldest first;
 *  - GQA: v-head h reads q/k head h / (HV/HK);
 *  - L2 norm: x / sqrt(sum x^2 + 1e-6);
 *  - alpha = exp(g) from a log-decay g; o uses the state after the update.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CHUNK_TOKENS 8

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * Chunk descriptors.  For every sequence s (length L = qsl[s+1] - qsl[s]) and
 * every chunk c = 0 .. ceil(L/8)-1, append the pair (s, c), sequences in
 * order, chunks ascending.  Pairs are written flat: out[2n] = s,
 * out[2n+1] = c.  Returns 0, or -3 when more than `capacity` pairs are
 * needed (then *n_out holds the count needed and nothing beyond capacity
 * is written); -1 for a NULL pointer or a decreasing qsl.
 */
int oracle_build_conv_chunks(const int32_t *qsl, int32_t num_seqs,
                             int32_t *out, int32_t capacity, int32_t *n_out)
{
    if (!qsl || !n_out || num_seqs < 0 || capacity < 0) return -1;
    if (capacity > 0 && !out) return -1;
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t len = (int64_t)qsl[s + 1] - qsl[s];
        if (len < 0) return -1;
        int64_t nchunks = (len + ORACLE_CHUNK_TOKENS - 1) / ORACLE_CHUNK_TOKENS;
        for (int64_t c = 0; c < nchunks; ++c) {
            if (n < capacity) {
                out[2 * n] = s;
                out[2 * n + 1] = (int32_t)c;
            }
            ++n;
        }
    }
    *n_out = (int32_t)n;
    return n > capacity ? -3 : 0;
}

/*
 * Varlen depthwise causal conv1d over packed tokens.
 *
 * For sequence s with tokens [a, a+L) of x and slot = state_indices[s]:
 *   e = h || x[a .. a+L)   (K-1+L rows), h = state[slot] if has_init else 0
 *   y[a+p][c] = act( bias[c] + sum_{j<K} w[c][j] * e[p+j][c] )
 *   state[slot][i][c] = e[L+i][c]   for i < K-1   (bit copies of bf16 inputs)
 * A negative slot or L == 0 leaves y and the slot untouched.
 *
 * x: bf16 bits, token t at x + t*x_stride, channel c contiguous.
 * w: bf16 bits [C][K]; bias: bf16 bits [C] or NULL (zero).
 * conv_state: bf16 bits [num_slots][K-1][C].
 * y: double, token t at y + t*y_stride.
 * has_init: NULL means every sequence has an initial state.
 */
void oracle_causal_conv1d_varlen(const uint16_t *x, int64_t x_stride,
                                 const uint16_t *w, const uint16_t *bias,
                                 uint16_t *conv_state, int32_t num_slots,
                                 const int32_t *qsl, const int32_t *state_indices,
                                 const uint8_t *has_init,
                                 double *y, int64_t y_stride,
                                 int32_t num_seqs, int32_t channels,
                                 int32_t width, int32_t apply_silu)
{
    (void)num_slots;
    const int32_t C = channels, K = width;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t a = qsl[s];
        const int64_t L = (int64_t)qsl[s + 1] - a;
        const int32_t slot = state_indices[s];
        if (slot < 0 || L <= 0) continue;
        const int init = has_init ? has_init[s] != 0 : 1;
        uint16_t *st = conv_state + (int64_t)slot * (K - 1) * C;
#pragma omp parallel
        {
        /* one channel's window, bf16 bits (one buffer per thread) */
        uint16_t *e = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(K - 1 + L));
#pragma omp for schedule(static)
        for (int32_t c = 0; c < C; ++c) {
            /* build the window for this channel: carried state, then inputs */
            for (int32_t i = 0; i < K - 1; ++i)
                e[i] = init ? st[(int64_t)i * C + c] : 0;
            for (int64_t p = 0; p < L; ++p)
                e[K - 1 + p] = x[(a + p) * x_stride + c];
            for (int64_t p = 0; p < L; ++p) {
                double z = bias ? bf16_bits_to_double(bias[c]) : 0.0;
                for (int32_t j = 0; j < K; ++j)
                    z += bf16_bits_to_double(w[(int64_t)c * K + j]) *
                         bf16_bits_to_double(e[p + j]);
                y[(a + p) * y_stride + c] = apply_silu ? silu(z) : z;
            }
            /* the last K-1 window entries become the carried state */
            for (int32_t i = 0; i < K - 1; ++i)
                st[(int64_t)i * C + c] = e[L + i];
        }
        free(e);
        }
    }
}

/*
 * Single-token conv update (decode).  Batch row b uses slot state_indices[b]
 * (negative: row skipped).  The slot holds the K-1 previous inputs, oldest
 * first; the output is the K-tap correlation of (slot rows, x[b]); then the
 * window moves one token: the oldest row drops out and x[b] becomes newest.
 */
void oracle_causal_conv1d_update(const uint16_t *x, int64_t x_stride,
                                 const uint16_t *w, const uint16_t *bias,
                                 uint16_t *conv_state, int32_t num_slots,
                                 const int32_t *state_indices,
                                 double *y, int64_t y_stride,
                                 int32_t batch, int32_t channels,
                                 int32_t width, int32_t apply_silu)
{
    (void)num_slots;
    const int32_t C = channels, K = width;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t slot = state_indices[b];
        if (slot < 0) continue;
        uint16_t *st = conv_state + (int64_t)slot * (K - 1) * C;
        const uint16_t *xb = x + (int64_t)b * x_stride;
#pragma omp parallel for schedule(static)
        for (int32_t c = 0; c < C; ++c) {
            double z = bias ? bf16_bits_to_double(bias[c]) : 0.0;
            for (int32_t j = 0; j < K - 1; ++j)
                z += bf16_bits_to_double(w[(int64_t)c * K + j]) *
                     bf16_bits_to_double(st[(int64_t)j * C + c]);
            z += bf16_bits_to_double(w[(int64_t)c * K + K - 1]) *
                 bf16_bits_to_double(xb[c]);
            y[(int64_t)b * y_stride + c] = apply_silu ? silu(z) : z;
            for (int32_t j = 0; j + 1 < K - 1; ++j)
                st[(int64_t)j * C + c] = st[(int64_t)(j + 1) * C + c];
            if (K > 1) st[(int64_t)(K - 2) * C + c] = xb[c];
        }
    }
}

/*
 * Gated delta rule over packed tokens (decode is the case L = 1).
 *
 * For every sequence s (tokens [qsl[s], qsl[s+1]), or token s alone when qsl
 * is NULL) with slot = state_indices[s] >= 0, and every v-head h with
 * q/k head hk = h / (HV/HK):
 *   S = has_init ? state[slot][h] : 0          (dv x dk, row = v channel)
 *   for each token t:
 *     qh = norm(q[t][hk]), kh = norm(k[t][hk])   (norm = identity if off)
 *     a = exp(g[t][h]), b = beta[t][h]
 *     S = a * S * (I - b kh kh^T) + b v[t][h] kh^T
 *     o[t][h] = scale * S qh
 *   state[slot][h] = S
 * The product S (I - b kh kh^T) is expanded as S - b (S kh) kh^T; this is
 * the same matrix, not a reformulation of the update.
 *
 * q/k: bf16 bits, token t head j at q + t*q_stride + j*dk; v likewise with
 * dv; g, beta: float [T][HV]; state: double [num_slots][HV][dv][dk];
 * o: double, token t head h at o + t*o_stride + h*dv.
 */
void oracle_gated_delta_rule(const uint16_t *q, int64_t q_stride,
                             const uint16_t *k, int64_t k_stride,
                             const uint16_t *v, int64_t v_stride,
                             const float *g, const float *beta,
                             double *state, int32_t num_slots,
                             const int32_t *qsl, const int32_t *state_indices,
                             const uint8_t *has_init,
                             double *o, int64_t o_stride,
                             int32_t num_seqs, int32_t num_k_heads,
                             int32_t num_v_heads, int32_t dk, int32_t dv,
                             double scale, int32_t qk_l2norm)
{
    (void)num_slots;
    const int32_t HV = num_v_heads, group = num_v_heads / num_k_heads;
#pragma omp parallel
    {
    /* per-thread scratch: the normalized q and k rows, and S k */
    double *qh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for collapse(2) schedule(dynamic)
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int32_t h = 0; h < HV; ++h) {
        const int64_t t0 = qsl ? qsl[s] : s;
        const int64_t t1 = qsl ? qsl[s + 1] : s + 1;
        const int32_t slot = state_indices[s];
        if (slot < 0 || t1 <= t0) continue;
        const int init = has_init ? has_init[s] != 0 : 1;
        {
            const int32_t hk = h / group;
            double *S = state + ((int64_t)slot * HV + h) * dv * dk;
            if (!init)
                for (int64_t i = 0; i < (int64_t)dv * dk; ++i) S[i] = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                const uint16_t *qt = q + t * q_stride + (int64_t)hk * dk;
                const uint16_t *kt = k + t * k_stride + (int64_t)hk * dk;
                const uint16_t *vt = v + t * v_stride + (int64_t)h * dv;
                double nq = 0.0, nk = 0.0;
                for (int32_t j = 0; j < dk; ++j) {
                    qh[j] = bf16_bits_to_double(qt[j]);
                    kh[j] = bf16_bits_to_double(kt[j]);
                    nq += qh[j] * qh[j];
                    nk += kh[j] * kh[j];
                }
                if (qk_l2norm) {
                    const double rq = 1.0 / sqrt(nq + 1e-6);
                    const double rk = 1.0 / sqrt(nk + 1e-6);
                    for (int32_t j = 0; j < dk; ++j) {
                        qh[j] *= rq;
                        kh[j] *= rk;
                    }
                }
                const double a = exp((double)g[t * HV + h]);
                const double b = (double)beta[t * HV + h];
                /* u = S kh */
                for (int32_t i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * kh[j];
                    u[i] = acc;
                }
                /* S = a (S - b u kh^T) + b v kh^T */
                for (int32_t i = 0; i < dv; ++i) {
                    const double vi = bf16_bits_to_double(vt[i]);
                    for (int32_t j = 0; j < dk; ++j) {
                        double *sij = &S[(int64_t)i * dk + j];
                        *sij = a * (*sij - b * u[i] * kh[j]) + b * vi * kh[j];
                    }
                }
                /* o = scale S qh */
                for (int32_t i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qh[j];
                    o[t * o_stride + (int64_t)h * dv + i] = scale * acc;
                }
            }
        }
        }
    }
    free(qh);
    free(kh);
    free(u);
    }
}

/*
 * Round doubles to bf16 bits, round-to-nearest-even (no NaN/Inf expected).
 * Used only where an oracle-only pipeline feeds a bf16 activation from one
 * step into the next (conv output -> recurrence), as the layer does.
 */
void oracle_round_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        /* double -> nearest bf16: scale to the bf16 exponent's ulp and round
         * half-to-even with rint (default rounding mode is to-nearest-even) */
        double d = in[i];
        if (d == 0.0) {
            out[i] = signbit(d) ? 0x8000u : 0u;
            continue;
        }
        int ex;
        frexp(d, &ex);                      /* |d| in [2^(ex-1), 2^ex) */
        if (ex < -125) ex = -125;           /* subnormal range keeps ulp 2^-133 */
        const double ulp = ldexp(1.0, ex - 8);
        const double r = rint(d / ulp) * ulp;
        const float f = (float)r;           /* exact: r has <= 8 significant bits */
        uint32_t ubits;
        memcpy(&ubits, &f, sizeof ubits);
        out[i] = (uint16_t)(ubits >> 16);
    }
}
