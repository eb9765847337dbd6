// One unit of the fused decode step -- (sequence, q/k head): the conv update
// of that head group's channels and the gated delta rule on its state rows
// -- as a device function, so that the decode kernel and the mixed-step
// kernel (chunk scan and decode in one grid) run the same code and give
// bit-identical results.
//
// One unit owns every conv channel its head group reads -- its q and k
// channels and the v channels of the v heads that share the q/k head -- and
// all state rows of those v heads.  So each conv_state channel has exactly
// one reader-writer (no race between reading the old window and writing the
// new one), and the conv output never leaves the workgroup: it is rounded
// to bf16 (as the two-call path stores it), kept in LDS and consumed by the
// recurrence.
#pragma once

#include "conv_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdr_math.h"

namespace gdn {

// 4 waves, 8 state rows per lane group: at the decode shape (2 v heads of
// 128 rows per q/k head) one pass covers the whole group, and the 512
// workgroups of a 32-sequence batch are all resident at once on 256 CUs.
constexpr int kFusedThreads = 256;
constexpr int kFusedRows = 8;                      // rows per lane group per pass
constexpr int kMaxGroupChannels = 8192;            // q + k + v channels of one head group

// LDS of a unit: the conv output of the group, (2 DK + (HV / HK) dv) bf16,
// then -- in the form that runs alone on its CU -- the decay and beta of each
// of its HV / HK v heads as fp32 (after rounding the bf16 count up to even)
__host__ __device__ constexpr int fused_unit_lds_bytes(int dk, int grp, int dv) {
    return ((2 * dk + grp * dv + 1) & ~1) * 2 + 2 * grp * 4;
}

// whether a group of n_rows state rows is exactly one pass of a unit
template <int DK>
__host__ __device__ constexpr bool fused_unit_full(int n_rows) {
    return n_rows == kFusedRows * (kFusedThreads / RowLayout<DK>::G);
}

// bid: the unit, b * num_k_heads + hk.  act: LDS of at least
// fused_unit_lds_bytes.  Called by all kFusedThreads threads of a workgroup.
//
// Two forms with the same arithmetic (bit-identical results):
//  * ALONE = false, for the decode kernel, where every CU holds two units
//    and the launch is bound by HBM bandwidth: the first pass of state
//    loads goes out right after the conv loads, and each row reads its v
//    head's decay and beta when it needs them.  (The conv arithmetic then
//    waits for the state loads too: they are conditional, and the compiler
//    waits for every outstanding load at the join.  Letting the conv go
//    ahead, so that rows are processed and stored as their loads arrive,
//    made the decode kernel 4-7% slower: the stores then mix with the
//    loads of the other units.)
//  * ALONE = true, for the mixed-step grid, where a unit runs alone on a CU
//    next to the scan and its latency is what counts; only for FULL groups
//    (fused_unit_full).  Load order: the decay and beta of the thread's v
//    head, its conv vector's window, input and taps, then the state rows --
//    all unconditional, so the conv waits only for its own loads (memory
//    loads complete in order) -- and the decays and betas reach the rows
//    through LDS, so no row waits for a global load of its own.  Against
//    the first form, the c32 mixed step's recurrence measured 68.4 -> 63.5 us.
template <int DK, int R, bool ALONE = false>
__device__ __forceinline__ void fused_decode_unit(const FusedDecodeArgs &a, int bid, uint16_t *act) {
    using L = RowLayout<DK>;
    constexpr int G = L::G, E = L::E, M = L::M;
    constexpr int ROWS_PER_PASS = kFusedThreads / G;          // rows covered once per lane

    const int HK = a.num_k_heads, HV = a.num_v_heads, grp = HV / HK;
    const int b = bid / HK;
    const int hk = bid - b * HK;
    const int slot = a.state_indices[b];
    // padding, or outside either pool (the row uses the same index in both)
    if ((unsigned)slot >= (unsigned)min(a.num_slots, a.num_conv_slots)) return;
    const int tid = threadIdx.x;
    const int dv = a.dv;
    const int nq = DK, nv = grp * dv;                         // channels: q and k DK each, v grp*dv
    const int n_vec = (2 * nq + nv) / kConvVec;
    const int j = (tid & 63) % G;
    const int n_rows = nv;

    // one pass of state rows: row r of this lane group, loaded as streaming
    // 16-byte vectors (each state element is read and written once); rows
    // past the group are not loaded and start at zero
    int row[R];
    bool valid[R];
    float S[R][E];
    auto load_rows = [&](int base) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            row[r] = base + r * ROWS_PER_PASS + tid / G;      // row within the group
            valid[r] = ALONE || row[r] < n_rows;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int h = hk * grp + row[r] / dv, i = row[r] % dv;
            const float *Sp = a.state + (((int64_t)slot * HV + h) * dv + i) * DK + 4 * j;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                f32x4 v4 = {0.f, 0.f, 0.f, 0.f};
                if (valid[r]) v4 = load_stream4(Sp + 4 * G * m);
                S[r][4 * m + 0] = v4.x;
                S[r][4 * m + 1] = v4.y;
                S[r][4 * m + 2] = v4.z;
                S[r][4 * m + 3] = v4.w;
            }
        }
    };

    // ---- conv update of the group's channels, one 8-channel vector per
    // thread and iteration.  The first pass of state loads is issued right
    // after the first vector's loads: it does not depend on the conv, so its
    // latency overlaps the conv arithmetic and the barrier.
    // (ALONE: one vector of the conv, from a clamped, always-valid channel)
    auto conv_vec = [&](int c, bool load_state) {
        const int lc = min(c, n_vec - 1) * kConvVec;          // channel within the group (q | k | v)
        int ch;                                               // channel within the conv row
        if (lc < nq) ch = hk * DK + lc;
        else if (lc < 2 * nq) ch = HK * DK + hk * DK + (lc - nq);
        else ch = 2 * HK * DK + hk * nv + (lc - 2 * nq);
        uint16_t *st = a.conv_state + (int64_t)slot * 3 * a.channels + ch;
        const uint4 s0 = *reinterpret_cast<const uint4 *>(st);
        const uint4 s1 = *reinterpret_cast<const uint4 *>(st + a.channels);
        const uint4 s2 = *reinterpret_cast<const uint4 *>(st + 2 * (int64_t)a.channels);
        const uint4 xv = *reinterpret_cast<const uint4 *>(a.x + (int64_t)b * a.x_stride + ch);
        ConvTaps taps;
        load_taps(taps, a.conv_weight, a.conv_bias, ch);
        if (load_state) {
            // keep the compiler from moving the conv loads below the state
            // loads, or into the branch below
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            load_rows(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        if (c < n_vec) {
            const uint4 out = conv_row(taps, s0, s1, s2, xv, a.silu != 0);
            *reinterpret_cast<uint4 *>(st) = s1;
            *reinterpret_cast<uint4 *>(st + a.channels) = s2;
            *reinterpret_cast<uint4 *>(st + 2 * (int64_t)a.channels) = xv;
            if (a.y) *reinterpret_cast<uint4 *>(a.y + (int64_t)b * a.y_stride + ch) = out;
            *reinterpret_cast<uint4 *>(&act[lc]) = out;
        }
    };
    // ALONE: decay and beta of v head min(tid, grp - 1) of the group; threads
    // t < grp publish theirs through LDS
    float *gates = reinterpret_cast<float *>(act + ((2 * nq + nv + 1) & ~1));
    if constexpr (ALONE) {
        const int gh = hk * grp + min(tid, grp - 1);
        const float g_own = a.g[(int64_t)b * HV + gh];
        const float b_own = a.beta[(int64_t)b * HV + gh];
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        conv_vec(tid, true);
        for (int c = tid + kFusedThreads; c < n_vec; c += kFusedThreads) conv_vec(c, false);
        if (tid < grp) {
            gates[tid] = expf(g_own);
            gates[grp + tid] = b_own;
        }
    } else {
        for (int c = tid; c < n_vec; c += kFusedThreads) {
            const int lc = c * kConvVec;                      // channel within the group (q | k | v)
            int ch;                                           // channel within the conv row
            if (lc < nq) ch = hk * DK + lc;
            else if (lc < 2 * nq) ch = HK * DK + hk * DK + (lc - nq);
            else ch = 2 * HK * DK + hk * nv + (lc - 2 * nq);
            uint16_t *st = a.conv_state + (int64_t)slot * 3 * a.channels + ch;
            const uint4 s0 = *reinterpret_cast<const uint4 *>(st);
            const uint4 s1 = *reinterpret_cast<const uint4 *>(st + a.channels);
            const uint4 s2 = *reinterpret_cast<const uint4 *>(st + 2 * (int64_t)a.channels);
            const uint4 xv = *reinterpret_cast<const uint4 *>(a.x + (int64_t)b * a.x_stride + ch);
            ConvTaps taps;
            load_taps(taps, a.conv_weight, a.conv_bias, ch);
            if (c == tid) load_rows(0);
            const uint4 out = conv_row(taps, s0, s1, s2, xv, a.silu != 0);
            *reinterpret_cast<uint4 *>(st) = s1;
            *reinterpret_cast<uint4 *>(st + a.channels) = s2;
            *reinterpret_cast<uint4 *>(st + 2 * (int64_t)a.channels) = xv;
            if (a.y) *reinterpret_cast<uint4 *>(a.y + (int64_t)b * a.y_stride + ch) = out;
            *reinterpret_cast<uint4 *>(&act[lc]) = out;
        }
        if (tid >= n_vec) load_rows(0);
    }
    __syncthreads();

    // ---- gated delta rule, one token, for the grp * dv rows of the group
    float kf[E], qf[E];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[4 * m + e] = bf16_to_f32(act[4 * G * m + 4 * j + e]);
            kf[4 * m + e] = bf16_to_f32(act[nq + 4 * G * m + 4 * j + e]);
        }
    const TokenFactors f = token_factors<G, E>(kf, qf, a.l2norm != 0);

    for (int base = 0; base < (ALONE ? 1 : n_rows); base += R * ROWS_PER_PASS) {
        if (base > 0) load_rows(base);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(row[r], n_rows - 1);
            const int h = hk * grp + rr / dv, i = rr % dv;
            const float alpha = ALONE ? gates[rr / dv] : expf(a.g[(int64_t)b * HV + h]);
            const float beta = ALONE ? gates[grp + rr / dv] : a.beta[(int64_t)b * HV + h];
            const float v = bf16_to_f32(act[2 * nq + rr]);
            const float out = row_step<G, E>(S[r], kf, qf, f, alpha, beta, v, a.scale);
            if (valid[r]) {
                if (j == 0) a.o[(int64_t)b * a.o_stride + (int64_t)h * dv + i] = f32_to_bf16(out);
                float *Sp = a.state + (((int64_t)slot * HV + h) * dv + i) * DK + 4 * j;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const f32x4 w = {S[r][4 * m + 0], S[r][4 * m + 1], S[r][4 * m + 2], S[r][4 * m + 3]};
                    store_stream4(Sp + 4 * G * m, w);
                }
            }
        }
    }
}

}  // namespace gdn
