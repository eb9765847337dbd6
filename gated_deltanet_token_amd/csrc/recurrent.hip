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
    if (slot < 0) return;
    const int t_begin = a.qsl ? a.qsl[s] : s;
    const int t_end = a.qsl ? a.qsl[s + 1] : s + 1;
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
static hipError_t launch_dk(const RecurrentArgs &a, hipStream_t stream) {
    // 2 waves x 8 rows per workgroup (dk >= 32): the fastest of the shapes
    // measured at the 32-sequence decode (many small workgroups keep more
    // state loads in flight than fewer large ones).  Per-row arithmetic is
    // shape-independent, so decode and varlen give identical tokens.
    if (a.qsl == nullptr) return launch_shape<DK, 2, 1, false>(a, stream);
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
