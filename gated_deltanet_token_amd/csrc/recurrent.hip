// Fused gated delta rule over packed tokens (decode = one token per
// sequence), gfx950.
//
// Rule: Yang, Kautz, Hatamizadeh, "Gated Delta Networks" (ICLR 2025),
// recurrent form S <- a S (I - b k k^T) + b v k^T, o = scale S q; the fused
// decode with a register-resident state is the design named on page "RTX
// 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section
// "Existing evidence".
//
// Work split.  The state of one (sequence, v-head) is dv rows of dk fp32,
// each row contiguous.  Rows are independent (both dot products run along
// dk), so a head splits across workgroups by row blocks with no cross-
// workgroup reduction.  A row lives in a group of G lanes (G = 8 for
// dk >= 32): lane j of the group holds the dk/G elements
// {32m + 4j + e | e < 4} for dk = 128 (float4 slices m = 0..3), so every
// load/store instruction of a wave moves whole 128-byte lines of 8
// neighbouring rows.  The state stays in VGPRs for the whole token loop and
// is read and written exactly once per call, with streaming (nontemporal)
// 16-byte accesses.
//
// Per token (gdr_math.h), with raw (unnormalised) q and k and rk, rq the
// inverse norms:
//   u = (S k) rk, p = (S q) rq           -- one pass over the old row
//   c = b (v - a u)
//   S = a S + (c rk) k                   == a S (I - b kh kh^T) + b v kh^T
//   o = scale (a p + c (k.q) rk rq)      == scale S_new qh
// Only the two row sums sit on the per-token dependency chain; the norms and
// k.q are reduced alongside.  Every group sum uses the same DPP tree, so the
// result does not depend on how rows are spread over waves or workgroups:
// the decode and the varlen launch shapes give bit-identical tokens.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdr_math.h"

namespace gdn {

template <int DK, int W, int R>
struct RecurrentShape {
    using L = RowLayout<DK>;
    static constexpr int kThreads = 64 * W;
    static constexpr int kRowsPerWave = L::RG * R;
    static constexpr int kRowsPerBlock = kRowsPerWave * W;
};

template <int M>
struct TokenIn {
    uint2 k[M];
    uint2 q[M];
};

// VARLEN only names the instantiation (decode and varlen launches show up as
// separate kernels in a profile); the code is the same.
template <int DK, int W, int R, bool VARLEN>
__global__ __launch_bounds__(64 * W) void recurrent_kernel(RecurrentArgs a, int n_rowblocks) {
    using L = RowLayout<DK>;
    using Sh = RecurrentShape<DK, W, R>;
    constexpr int G = L::G, E = L::E, M = L::M, RG = L::RG;

    const int rb = blockIdx.x % n_rowblocks;
    const int sh = blockIdx.x / n_rowblocks;
    const int h = sh % a.num_v_heads;
    const int s = sh / a.num_v_heads;
    const int slot = a.state_indices[s];
    if ((unsigned)slot >= (unsigned)a.num_slots) return;   // padding, or outside the pool
    int t_begin = s, t_end = s + 1;
    if (a.qsl) clamp_range(a.qsl[s], a.qsl[s + 1], a.num_tokens, t_begin, t_end);
    if (t_end <= t_begin) return;
    const int HV = a.num_v_heads;
    const int hk = h / (HV / a.num_k_heads);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane % G;
    const int gi = lane / G;

    int row[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = rb * Sh::kRowsPerBlock + wave * Sh::kRowsPerWave + r * RG + gi;
        valid[r] = row[r] < a.dv;
    }

    float *S_head = a.state + ((int64_t)slot * HV + h) * (int64_t)a.dv * DK;
    float S[R][E];
    const bool init = a.has_init == nullptr || a.has_init[s] != 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            f32x4 v4 = {0.f, 0.f, 0.f, 0.f};
            if (init && valid[r]) v4 = load_stream4(S_head + (int64_t)row[r] * DK + m * 4 * G + 4 * j);
            S[r][4 * m + 0] = v4.x;
            S[r][4 * m + 1] = v4.y;
            S[r][4 * m + 2] = v4.z;
            S[r][4 * m + 3] = v4.w;
        }
    }

    const uint16_t *qp = a.q + (int64_t)hk * DK + 4 * j;
    const uint16_t *kp = a.k + (int64_t)hk * DK + 4 * j;
    const uint16_t *vp = a.v + (int64_t)h * a.dv;
    uint16_t *op = a.o + (int64_t)h * a.dv;

    // inputs of the token being processed; the next token's are fetched
    // before the current token's arithmetic starts
    TokenIn<M> cur;
    uint16_t vcur[R];
    float gcur, bcur;
    auto fetch = [&](int t, TokenIn<M> &in, uint16_t *vv, float &gg, float &bb) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            in.k[m] = *reinterpret_cast<const uint2 *>(kp + (int64_t)t * a.k_stride + m * 4 * G);
            in.q[m] = *reinterpret_cast<const uint2 *>(qp + (int64_t)t * a.q_stride + m * 4 * G);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) vv[r] = valid[r] ? vp[(int64_t)t * a.v_stride + row[r]] : (uint16_t)0;
        gg = a.g[(int64_t)t * HV + h];
        bb = a.beta[(int64_t)t * HV + h];
    };
    fetch(t_begin, cur, vcur, gcur, bcur);

    for (int t = t_begin; t < t_end; ++t) {
        TokenIn<M> nxt;
        uint16_t vnxt[R];
        float gnxt = 0.f, bnxt = 0.f;
        if (t + 1 < t_end) fetch(t + 1, nxt, vnxt, gnxt, bnxt);

        float kf[E], qf[E];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            kf[4 * m + 0] = bf16_lo(cur.k[m].x);
            kf[4 * m + 1] = bf16_hi(cur.k[m].x);
            kf[4 * m + 2] = bf16_lo(cur.k[m].y);
            kf[4 * m + 3] = bf16_hi(cur.k[m].y);
            qf[4 * m + 0] = bf16_lo(cur.q[m].x);
            qf[4 * m + 1] = bf16_hi(cur.q[m].x);
            qf[4 * m + 2] = bf16_lo(cur.q[m].y);
            qf[4 * m + 3] = bf16_hi(cur.q[m].y);
        }
        const TokenFactors f = token_factors<G, E>(kf, qf, a.l2norm != 0);
        const float alpha = expf(gcur);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float out = row_step<G, E>(S[r], kf, qf, f, alpha, bcur, bf16_to_f32(vcur[r]), a.scale);
            if (j == 0 && valid[r]) op[(int64_t)t * a.o_stride + row[r]] = f32_to_bf16(out);
        }

        if (t + 1 < t_end) {
            cur = nxt;
#pragma unroll
            for (int r = 0; r < R; ++r) vcur[r] = vnxt[r];
            gcur = gnxt;
            bcur = bnxt;
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (!valid[r]) continue;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const f32x4 v4 = {S[r][4 * m + 0], S[r][4 * m + 1], S[r][4 * m + 2], S[r][4 * m + 3]};
            store_stream4(S_head + (int64_t)row[r] * DK + m * 4 * G + 4 * j, v4);
        }
    }
}

// Single-token decode (no query_start_loc): one workgroup per (sequence, q/k
// head) holding every state row of the v heads that share that q/k head, R
// rows per lane group per pass.  At 32 sequences with 16 q/k heads and
// 2 x 128 v rows per q/k head this is 512 workgroups that are all resident
// at once, each with one pass, so the whole state is in flight from the
// start (32 16-byte loads per lane at dk = 128).  Every load of a pass --
// the state rows first, then q and k, then each row's v, g and beta -- is
// issued before any arithmetic, so no input's latency is paid after the
// state has arrived.
// Stores go through buffer resources whose range ends at the group's last
// row: the stores of rows past the end (which read the last row again), and
// the o store of every lane but the first of its group, get an offset past
// the range and are dropped, so nothing sits behind a branch.  With
// has_initial_state the state is read through a buffer resource too, whose
// range is zero for a sequence without one (every load returns zeros).
// Measured at the 32-sequence decode: without the two load barriers 27.5 us,
// with them 24.4 us; buffer loads where global ones suffice cost 1.5 us.
constexpr int kGroupThreads = 256;
constexpr int kGroupRows = 8;

// The slot lookup's and the first state rows' arguments are also passed
// ahead of the struct: the first 14 dwords arrive preloaded in SGPRs, so the
// slot load does not wait for an argument load.
template <int DK, int R, bool HAS_INIT>
__global__ __launch_bounds__(kGroupThreads) void recurrent_group_kernel(const int32_t *state_indices, float *state,
                                                                        const uint8_t *has_init, int num_k_heads,
                                                                        int num_v_heads, int num_slots, int dv_,
                                                                        int n_blocks, RecurrentArgs a_in) {
    using L = RowLayout<DK>;
    constexpr int G = L::G, E = L::E, M = L::M;
    constexpr int RPP = kGroupThreads / G;                   // rows covered once per lane

    RecurrentArgs a = a_in;
    a.state_indices = state_indices;
    a.state = state;
    a.has_init = has_init;
    a.num_k_heads = num_k_heads;
    a.num_v_heads = num_v_heads;
    a.num_slots = num_slots;
    a.dv = dv_;
    const int HK = a.num_k_heads, HV = a.num_v_heads, grp = HV / HK;
    // XCD-contiguous order: each XCD takes a contiguous range of (sequence, q/k head)
    const int bid = xcd_contiguous(blockIdx.x, n_blocks);
    const int s = bid / HK;
    const int hk = bid - s * HK;
    const int slot = a.state_indices[s];
    if ((unsigned)slot >= (unsigned)a.num_slots) return;   // padding, or outside the pool
    const int tid = threadIdx.x;
    const int j = (tid & 63) % G;
    const int dv = a.dv, n_rows = grp * dv;
    // the group's v heads are adjacent, so its rows (and its o and v
    // elements) are contiguous ranges
    float *S_grp = a.state + ((int64_t)slot * HV + (int64_t)hk * grp) * (int64_t)dv * DK;
    uint16_t *o_grp = a.o + (int64_t)s * a.o_stride + (int64_t)hk * grp * dv;
    const uint16_t *v_grp = a.v + (int64_t)s * a.v_stride + (int64_t)hk * grp * dv;
    const float *g_grp = a.g + (int64_t)s * HV + hk * grp;
    const float *b_grp = a.beta + (int64_t)s * HV + hk * grp;
    const int s_range = n_rows * DK * 4, o_range = n_rows * 2;
    const bool init = !HAS_INIT || __builtin_amdgcn_readfirstlane(a.has_init[s]) != 0;
    const __amdgpu_buffer_rsrc_t ld_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(S_grp, (short)0, init ? s_range : 0, kBufferFlags);
    const __amdgpu_buffer_rsrc_t st_rsrc = __builtin_amdgcn_make_buffer_rsrc(S_grp, (short)0, s_range, kBufferFlags);
    const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(o_grp, (short)0, o_range, kBufferFlags);

    uint2 kraw[M], qraw[M];
    int row[R];
    u32x4 Sraw[R][M];
    uint16_t vraw[R];
    float graw[R], braw[R];
    auto load_pass = [&](int base) {
#pragma unroll
        for (int r = 0; r < R; ++r) row[r] = base + r * RPP + tid / G;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m)
                if constexpr (HAS_INIT)
                    Sraw[r][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                               ld_rsrc, (row[r] * DK + 4 * j + 4 * G * m) * 4, 0,
                                                               kBufferStream));
                else
                    Sraw[r][m] = __builtin_bit_cast(
                        u32x4, load_stream4(S_grp + (int64_t)min(row[r], n_rows - 1) * DK + 4 * j + 4 * G * m));
        // (neither the compiler nor the scheduler moves memory accesses
        // across an empty asm that clobbers memory)
        asm volatile("" ::: "memory");
        if (base == 0) {
            const uint16_t *qp = a.q + (int64_t)s * a.q_stride + (int64_t)hk * DK + 4 * j;
            const uint16_t *kp = a.k + (int64_t)s * a.k_stride + (int64_t)hk * DK + 4 * j;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                kraw[m] = *reinterpret_cast<const uint2 *>(kp + m * 4 * G);
                qraw[m] = *reinterpret_cast<const uint2 *>(qp + m * 4 * G);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(row[r], n_rows - 1);
            const int hh = rr / dv;                          // v head within the group
            vraw[r] = v_grp[rr];
            graw[r] = g_grp[hh];
            braw[r] = b_grp[hh];
        }
        // every load of the pass is issued before any arithmetic needs one
        // (the scheduler moves no instruction across a sched_barrier(0))
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    load_pass(0);

    float kf[E], qf[E];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        kf[4 * m + 0] = bf16_lo(kraw[m].x);
        kf[4 * m + 1] = bf16_hi(kraw[m].x);
        kf[4 * m + 2] = bf16_lo(kraw[m].y);
        kf[4 * m + 3] = bf16_hi(kraw[m].y);
        qf[4 * m + 0] = bf16_lo(qraw[m].x);
        qf[4 * m + 1] = bf16_hi(qraw[m].x);
        qf[4 * m + 2] = bf16_lo(qraw[m].y);
        qf[4 * m + 3] = bf16_hi(qraw[m].y);
    }
    const TokenFactors f = token_factors<G, E>(kf, qf, a.l2norm != 0);

    for (int base = 0; base < n_rows; base += R * RPP) {
        if (base > 0) load_pass(base);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float S[E];
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t u = Sraw[r][m][e];
                    S[4 * m + e] = __builtin_bit_cast(float, u);
                }
            const float out = row_step<G, E>(S, kf, qf, f, expf(graw[r]), braw[r], bf16_to_f32(vraw[r]), a.scale);
            const bool live = row[r] < n_rows;
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(out), o_rsrc, live && j == 0 ? 2 * row[r] : o_range, 0,
                                                  0);
            const int s_off = live ? (row[r] * DK + 4 * j) * 4 : s_range;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const u32x4 w = {__builtin_bit_cast(uint32_t, S[4 * m + 0]), __builtin_bit_cast(uint32_t, S[4 * m + 1]),
                                 __builtin_bit_cast(uint32_t, S[4 * m + 2]), __builtin_bit_cast(uint32_t, S[4 * m + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(w, st_rsrc, s_off + 16 * G * m, 0, kBufferStream);
            }
        }
    }
}

template <int DK, int W, int R, bool VARLEN>
static hipError_t launch_shape(const RecurrentArgs &a, hipStream_t stream) {
    using Sh = RecurrentShape<DK, W, R>;
    const int nrb = (a.dv + Sh::kRowsPerBlock - 1) / Sh::kRowsPerBlock;
    const long long blocks = (long long)a.num_seqs * a.num_v_heads * nrb;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((recurrent_kernel<DK, W, R, VARLEN>), dim3((unsigned)blocks), dim3(Sh::kThreads), 0,
                       stream, a, nrb);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_group(const RecurrentArgs &a, hipStream_t stream) {
    const long long blocks = (long long)a.num_seqs * a.num_k_heads;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // byte offsets within a group's rows are 32-bit
    if ((long long)(a.num_v_heads / a.num_k_heads) * a.dv * DK * 4 + 16 * DK > 0x7fffffffLL)
        return launch_shape<DK, 2, 1, false>(a, stream);
    if (a.has_init)
        hipLaunchKernelGGL((recurrent_group_kernel<DK, kGroupRows, true>), dim3((unsigned)blocks), dim3(kGroupThreads),
                           0, stream, a.state_indices, a.state, a.has_init, a.num_k_heads, a.num_v_heads, a.num_slots,
                           a.dv, (int)blocks, a);
    else
        hipLaunchKernelGGL((recurrent_group_kernel<DK, kGroupRows, false>), dim3((unsigned)blocks),
                           dim3(kGroupThreads), 0, stream, a.state_indices, a.state, a.has_init, a.num_k_heads,
                           a.num_v_heads, a.num_slots, a.dv, (int)blocks, a);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_dk(const RecurrentArgs &a, hipStream_t stream) {
    // Token loops: 2 waves x 8 rows per workgroup (dk >= 32), the fastest
    // row-block shape measured.  Per-row arithmetic is shape-independent, so
    // decode and varlen give identical tokens.
    if (a.qsl == nullptr) return launch_group<DK>(a, stream);
    return launch_shape<DK, 2, 1, true>(a, stream);
}

hipError_t launch_recurrent(const RecurrentArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_dk<16>(a, stream);
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
