// Chunkwise gated delta rule for prefill tokens on gfx950 MFMA.
//
// Rule: Yang, Kautz, Hatamizadeh, "Gated Delta Networks" (ICLR 2025).  The
// recurrent step S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T can be
// written S_t = a_t S_{t-1} + u_t k_t^T with u_t = b_t (v_t - a_t S_{t-1} k_t).
// Unrolled over a chunk of C tokens from the state S0 entering the chunk
// (L_t = sum of g over the chunk up to t, G_t = exp(L_t)):
//
//   (I + A) U = R,   A_ti = b_t exp(L_t - L_i) (kh_t . kh_i)       (i < t)
//                    R_t  = b_t v_t - b_t G_t (S0 kh_t)
//   o_t  = scale (G_t S0 qh_t + sum_{i<=t} exp(L_t - L_i) (qh_t . kh_i) u_i)
//   S_C  = G_C S0 + sum_i exp(L_C - L_i) u_i kh_i^T
//
// Two launches:
//  * prep (one workgroup per (chunk, v-head), all chunks in parallel): the
//    parts that do not depend on the state -- norms, cumulative decay,
//    T = (I + A)^-1, P_ti = scale exp(L_t - L_i)(qh_t . kh_i) (i <= t), K^T
//    -- written to the caller's workspace;
//  * scan (one workgroup per (sequence, v-head, 32 v rows), serial over the
//    sequence's chunks): [K;Q] S0^T, R, U = T R, o = S0 part + P U and
//    S_C = G_C S0 + U'^T K, with the state slice held in VGPRs in the MFMA
//    accumulator layout and the next chunk's inputs prefetched.
//
// Precision: products of raw bf16 inputs (K K^T, Q K^T) are exact in the
// bf16 MFMA with fp32 accumulation.  Every product with an fp32 operand (the
// state, T, P, U, R) splits that operand into hi + lo bf16 parts (16
// significant bits) and sums the partial products.  T is inverted in fp32
// (16 x 16 diagonal blocks by substitution, off-diagonal blocks with fp32
// MFMA).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CT = 64;          // tokens per chunk
constexpr int DKC = 128;        // head_k_dim
constexpr int DVB = 32;         // v rows per scan workgroup
constexpr int NTH = 256;        // 4 waves
constexpr int LDK = DKC + 8;    // padded LDS row (bf16) of a [*][128] tile
constexpr int LDT = CT + 8;     // padded LDS row (bf16) of a [*][64] tile
constexpr int LDF = CT + 4;     // padded LDS row (fp32) of a [64][64] tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
// per (chunk, v-head): T hi, T lo, P hi, P lo ([64][64] bf16 each, [t][i]),
// then per-token scalars
struct ChunkRec {
    __bf16 Thi[CT][CT], Tlo[CT][CT], Phi[CT][CT], Plo[CT][CT];
    float beta[CT];   // b_t
    float bgr[CT];    // b_t G_t rk_t          (R = b v - bgr (K S0^T))
    float sqg[CT];    // scale rq_t G_t        (o = sqg (Q S0^T) + P U)
    float u2f[CT];    // exp(L_C - L_t) rk_t   (S_C = G_C S0 + (u2f U)^T K)
    float gC[CT];     // G_C in [0]
};
static_assert(sizeof(ChunkRec) % 256 == 0, "record alignment");
// per (chunk, q/k head): K^T [d][t]
struct KtRec {
    __bf16 Kt[DKC][CT];
};

__device__ __forceinline__ int chunk_count(int len) { return (len + CT - 1) / CT; }

// ---------------------------------------------------------------------------
// MFMA helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag(const __bf16 *base, int ld, int r0, int k0, int lane) {
    // operand fragment of a 16 x 32 tile whose rows are r0..r0+15 and whose
    // contraction index runs along a row: lane holds row r0 + lane%16,
    // elements k0 + 8*(lane/16) .. +7
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split(float v, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// C += X Y for 16x16 fp32 tiles in LDS; four 16x16x4 fp32 MFMAs
__device__ __forceinline__ f32x4 mm16_f32(const float (*X)[LDF], int xr, int xc, const float (*Y)[LDF], int yr,
                                          int yc, f32x4 c, int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float a = X[xr + (lane & 15)][xc + (lane >> 4) + 4 * s];
        const float b = Y[yr + (lane >> 4) + 4 * s][yc + (lane & 15)];
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    return c;
}

__device__ __forceinline__ void put16(float (*Z)[LDF], int zr, int zc, const f32x4 &c, float sgn, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Z[zr + 4 * (lane >> 4) + i][zc + (lane & 15)] = sgn * c[i];
}

// ---------------------------------------------------------------------------
// prep: one workgroup per (chunk, v-head)
// ---------------------------------------------------------------------------
struct PrepSmem {
    __bf16 K[CT][LDK];
    __bf16 Q[CT][LDK];
    float A[CT][LDF];
    float Tf[CT][LDF];
    float lam[CT], rk[CT], rq[CT], beta[CT];
};

__global__ __launch_bounds__(NTH) void chunk_prep_kernel(RecurrentArgs a, ChunkRec *recs, KtRec *kts,
                                                        int max_chunks) {
    __shared__ PrepSmem sm;
    const int HV = a.num_v_heads;
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int h = work % HV;
    const int gch = work / HV;                  // global chunk index
    // locate (sequence, chunk within it)
    int s = -1, j = 0;
    {
        int c = 0;
        for (int q = 0; q < a.num_seqs; ++q) {
            const int nc = chunk_count(a.qsl[q + 1] - a.qsl[q]);
            if (gch < c + nc) {
                s = q;
                j = gch - c;
                break;
            }
            c += nc;
        }
    }
    if (s < 0 || a.state_indices[s] < 0) return;
    const int t0 = a.qsl[s] + CT * j;
    const int n = min(CT, a.qsl[s + 1] - t0);
    const int grp = HV / a.num_k_heads;
    const int hk = h / grp;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    ChunkRec *rec = recs + (int64_t)gch * HV + h;

    // ---- stage 0: k/q rows, norms, cumulative decay, K^T
    {
        const int tok = tid >> 2, part = tid & 3;
        uint4 kv[4], qv[4];
        if (tok < n) {
            const uint4 *kp = reinterpret_cast<const uint4 *>(a.k + (int64_t)(t0 + tok) * a.k_stride + hk * DKC +
                                                              32 * part);
            const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (int64_t)(t0 + tok) * a.q_stride + hk * DKC +
                                                              32 * part);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                kv[m] = kp[m];
                qv[m] = qp[m];
            }
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) kv[m] = qv[m] = make_uint4(0, 0, 0, 0);
        }
        float skk = 0.f, sqq = 0.f;
        const bool write_kt = (h % grp) == 0;
        __bf16 *ktg = &kts[(int64_t)gch * a.num_k_heads + hk].Kt[0][0];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *reinterpret_cast<uint4 *>(&sm.K[tok][32 * part + 8 * m]) = kv[m];
            *reinterpret_cast<uint4 *>(&sm.Q[tok][32 * part + 8 * m]) = qv[m];
            float kf[8], qf[8];
            unpack8(kv[m], kf);
            unpack8(qv[m], qf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                skk = __builtin_fmaf(kf[e], kf[e], skk);
                sqq = __builtin_fmaf(qf[e], qf[e], sqq);
                if (write_kt) ktg[(32 * part + 8 * m + e) * CT + tok] = (__bf16)kf[e];
            }
        }
        skk = group_sum<4>(skk);
        sqq = group_sum<4>(sqq);
        if (part == 0) {
            sm.rk[tok] = a.l2norm ? rsqrtf(skk + 1e-6f) : 1.f;
            sm.rq[tok] = a.l2norm ? rsqrtf(sqq + 1e-6f) : 1.f;
        }
        if (w == 0) {
            // padded tokens: g = 0 and beta = 0 make them exact no-ops
            float gg = lane < n ? a.g[(int64_t)(t0 + lane) * HV + h] : 0.f;
            const float bb = lane < n ? a.beta[(int64_t)(t0 + lane) * HV + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gg, off, 64);
                if (lane >= off) gg += up;
            }
            sm.lam[lane] = gg;
            sm.beta[lane] = bb;
        }
    }
    __syncthreads();

    // per-token scalars for the scan
    if (w == 0) {
        const int t = lane;
        const float lam = sm.lam[t], lamC = sm.lam[CT - 1];
        const float G = expf(lam), rk = sm.rk[t];
        rec->beta[t] = sm.beta[t];
        rec->bgr[t] = sm.beta[t] * G * rk;
        rec->sqg[t] = a.scale * sm.rq[t] * G;
        rec->u2f[t] = expf(lamC - lam) * rk;
        rec->gC[t] = expf(lamC);
    }

    // ---- stage 1: K K^T -> A (fp32, LDS), Q K^T -> P (hi/lo, workspace)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ii = 16 * c + lr;
        if (c > w) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * lq + i;
                rec->Phi[t][ii] = (__bf16)0.f;
                rec->Plo[t][ii] = (__bf16)0.f;
            }
            continue;
        }
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DKC / 32; ++ks) {
            const bf16x8 ak = frag(&sm.K[0][0], LDK, 16 * w, 32 * ks, lane);
            const bf16x8 aq = frag(&sm.Q[0][0], LDK, 16 * w, 32 * ks, lane);
            const bf16x8 bk = frag(&sm.K[0][0], LDK, 16 * c, 32 * ks, lane);
            kk = mma(ak, bk, kk);
            qk = mma(aq, bk, qk);
        }
        const float lam_i = sm.lam[ii], rk_i = sm.rk[ii];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * w + 4 * lq + i;
            const float decay = ii <= t ? expf(sm.lam[t] - lam_i) : 0.f;
            sm.A[t][ii] = ii < t ? sm.beta[t] * sm.rk[t] * rk_i * decay * kk[i] : 0.f;
            __bf16 hi, lo;
            split(ii <= t ? a.scale * sm.rq[t] * rk_i * decay * qk[i] : 0.f, hi, lo);
            rec->Phi[t][ii] = hi;
            rec->Plo[t][ii] = lo;
        }
    }
    __syncthreads();

    // ---- stage 2: T = (I + A)^-1
    {
        float(*Tf)[LDF] = sm.Tf;
        float(*Am)[LDF] = sm.A;
        if (lane < 16) {
            // diagonal block w by forward substitution; lane j owns column j
            float xcol[16];
            const int b0 = 16 * w;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = t == lane ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < t; ++i) acc = __builtin_fmaf(-Am[b0 + t][b0 + i], xcol[i], acc);
                xcol[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Tf[b0 + t][b0 + lane] = xcol[t];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c <= w) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) Tf[16 * w + 4 * lq + i][16 * c + lr] = 0.f;
        }
        __syncthreads();
        // T_bc = -T_bb (sum_{c<=m<b} A_bm T_mc); wave c walks down column
        // block c, so every input is its own earlier result or a diagonal block
        const int c = w;
        for (int b = c + 1; b < 4 && w < 3; ++b) {
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            for (int mm = c; mm < b; ++mm) m = mm16_f32(Am, 16 * b, 16 * mm, Tf, 16 * mm, 16 * c, m, lane);
            put16(Tf, 16 * b, 16 * c, m, 1.f, lane);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16_f32(Tf, 16 * b, 16 * b, Tf, 16 * b, 16 * c, t, lane);
            put16(Tf, 16 * b, 16 * c, t, -1.f, lane);
        }
        __syncthreads();
        // hi/lo to the workspace, 8 consecutive entries per lane
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = tid + NTH * e;          // 512 groups of 8
            const int t = idx >> 3, i0 = (idx & 7) * 8;
            bf16x8 hv, lv;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __bf16 hi, lo;
                split(Tf[t][i0 + q], hi, lo);
                hv[q] = hi;
                lv[q] = lo;
            }
            *reinterpret_cast<bf16x8 *>(&rec->Thi[t][i0]) = hv;
            *reinterpret_cast<bf16x8 *>(&rec->Tlo[t][i0]) = lv;
        }
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, v-head, 32 v rows)
// ---------------------------------------------------------------------------
struct ScanSmem {
    __bf16 K[CT][LDK];
    __bf16 Q[CT][LDK];
    __bf16 Kt[DKC][LDT];
    __bf16 Shi[DVB][LDK], Slo[DVB][LDK];
    __bf16 Thi[CT][LDT], Tlo[CT][LDT];
    __bf16 Phi[CT][LDT], Plo[CT][LDT];
    __bf16 Rhi[DVB][LDT], Rlo[DVB][LDT];
    __bf16 Uhi[DVB][LDT], Ulo[DVB][LDT];
    __bf16 U2hi[DVB][LDT], U2lo[DVB][LDT];
    float beta[CT], bgr[CT], sqg[CT], u2f[CT], gC;
};

// one chunk's inputs in flight, in registers
struct ChunkIn {
    uint4 k[4], q[4];      // token tid/4, dims 32*(tid%4) ..
    uint4 kt[4];           // K^T row (tid*4 + m) / 8, segment (tid*4 + m) % 8
    uint4 t[4], p[4];      // T hi/lo, P hi/lo: 16-byte pieces tid + 256*m
    float sc;              // one per-token scalar
    float gc;              // G_C (thread 0)
    float v[2][4];         // v in the accumulator layout
};

__device__ __forceinline__ uint4 mask4(bool keep, const uint4 &v) {
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// Every load reads a valid address (rows past the chunk end re-read its last
// row) and padding is masked on values, so no load is predicated -- that
// keeps the in-flight chunk in registers.
__device__ __forceinline__ void fetch_chunk(ChunkIn &in, const RecurrentArgs &a, const ChunkRec *rec,
                                            const KtRec *kt, int t0, int n, int h, int hk, int vb, int tid) {
    const int tok = tid >> 2, part = tid & 3;
    const bool live = tok < n;
    const int row = t0 + min(tok, n - 1);
    const uint4 *kp = reinterpret_cast<const uint4 *>(a.k + (int64_t)row * a.k_stride + hk * DKC + 32 * part);
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (int64_t)row * a.q_stride + hk * DKC + 32 * part);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        in.k[m] = mask4(live, kp[m]);
        in.q[m] = mask4(live, qp[m]);
    }
    const uint4 *ktp = reinterpret_cast<const uint4 *>(&kt->Kt[0][0]);
    const uint4 *tp = reinterpret_cast<const uint4 *>(&rec->Thi[0][0]);   // Thi then Tlo
    const uint4 *pp = reinterpret_cast<const uint4 *>(&rec->Phi[0][0]);   // Phi then Plo
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        in.kt[m] = ktp[tid * 4 + m];
        in.t[m] = tp[tid + NTH * m];
        in.p[m] = pp[tid + NTH * m];
    }
    const float *scal = &rec->beta[0];
    in.sc = scal[tid];                            // beta, bgr, sqg, u2f: 4 x 64
    in.gc = rec->gC[0];
    const int lane = tid & 63, w = tid >> 6, lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = 16 * w + 4 * lq + i;
            const float vf = bf16_to_f32(a.v[(int64_t)(t0 + min(tt, n - 1)) * a.v_stride + (int64_t)h * a.dv +
                                             vb * DVB + 16 * rt + lr]);
            in.v[rt][i] = tt < n ? vf : 0.f;
        }
}

__device__ __forceinline__ void stage_chunk(ScanSmem &sm, const ChunkIn &in, int tid) {
    const int tok = tid >> 2, part = tid & 3;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        *reinterpret_cast<uint4 *>(&sm.K[tok][32 * part + 8 * m]) = in.k[m];
        *reinterpret_cast<uint4 *>(&sm.Q[tok][32 * part + 8 * m]) = in.q[m];
        const int e = tid * 4 + m;                 // K^T: 128 rows x 8 pieces
        *reinterpret_cast<uint4 *>(&sm.Kt[e >> 3][(e & 7) * 8]) = in.kt[m];
        const int f = tid + NTH * m;               // T/P: 2 x 64 rows x 8 pieces
        const int row = (f >> 3) & (CT - 1), col = (f & 7) * 8;
        if (f < CT * 8) {
            *reinterpret_cast<uint4 *>(&sm.Thi[row][col]) = in.t[m];
            *reinterpret_cast<uint4 *>(&sm.Phi[row][col]) = in.p[m];
        } else {
            *reinterpret_cast<uint4 *>(&sm.Tlo[row][col]) = in.t[m];
            *reinterpret_cast<uint4 *>(&sm.Plo[row][col]) = in.p[m];
        }
    }
    if (tid < 4 * CT) (&sm.beta[0])[tid] = in.sc;   // beta, bgr, sqg, u2f are contiguous
    if (tid == 0) sm.gC = in.gc;
}

__global__ __launch_bounds__(NTH) void chunk_scan_kernel(RecurrentArgs a, const ChunkRec *recs, const KtRec *kts,
                                                        int n_vblocks) {
    __shared__ ScanSmem sm;
    const int HV = a.num_v_heads;
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int vb = work % n_vblocks;
    const int sh = work / n_vblocks;
    const int h = sh % HV;
    const int s = sh / HV;
    const int slot = a.state_indices[s];
    if (slot < 0) return;
    const int t_begin = a.qsl[s];
    const int t_end = a.qsl[s + 1];
    if (t_end <= t_begin) return;
    const int hk = h / (HV / a.num_k_heads);
    int gch = 0;                                   // global index of this sequence's first chunk
    for (int q = 0; q < s; ++q) gch += chunk_count(a.qsl[q + 1] - a.qsl[q]);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // state slice in the accumulator layout: tile q = 2*rt + (dt - 2w),
    // element i -> row 16 rt + 4 lq + i, column 16 dt + lr
    float *S_g = a.state + ((int64_t)slot * HV + h) * (int64_t)a.dv * DKC + (int64_t)vb * DVB * DKC;
    f32x4 S[4];
    const bool init = a.has_init == nullptr || a.has_init[s] != 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rt = q >> 1, dt = 2 * w + (q & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[q][i] = init ? S_g[(16 * rt + 4 * lq + i) * DKC + 16 * dt + lr] : 0.f;
    }

    ChunkIn in;
    fetch_chunk(in, a, recs + (int64_t)gch * HV + h, kts + (int64_t)gch * a.num_k_heads + hk, t_begin,
                min(CT, t_end - t_begin), h, hk, vb, tid);

    for (int t0 = t_begin; t0 < t_end; t0 += CT, ++gch) {
        const int n = min(CT, t_end - t0);

        // ---- this chunk's inputs and the state entering it into LDS
        stage_chunk(sm, in, tid);
        float vv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[rt][i] = in.v[rt][i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rt = q >> 1, dt = 2 * w + (q & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __bf16 hi, lo;
                split(S[q][i], hi, lo);
                sm.Shi[16 * rt + 4 * lq + i][16 * dt + lr] = hi;
                sm.Slo[16 * rt + 4 * lq + i][16 * dt + lr] = lo;
            }
        }
        __syncthreads();
        // the next chunk's inputs travel while this one computes
        if (t0 + CT < t_end)
            fetch_chunk(in, a, recs + (int64_t)(gch + 1) * HV + h, kts + (int64_t)(gch + 1) * a.num_k_heads + hk,
                        t0 + CT, min(CT, t_end - t0 - CT), h, hk, vb, tid);

        // ---- R = b v - bgr (K S0^T) -> LDS;  o part = sqg (Q S0^T)
        f32x4 O[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 yk = {0.f, 0.f, 0.f, 0.f}, yq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DKC / 32; ++ks) {
                const bf16x8 ak = frag(&sm.K[0][0], LDK, 16 * w, 32 * ks, lane);
                const bf16x8 aq = frag(&sm.Q[0][0], LDK, 16 * w, 32 * ks, lane);
                const bf16x8 bh = frag(&sm.Shi[0][0], LDK, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Slo[0][0], LDK, 16 * rt, 32 * ks, lane);
                yk = mma(ak, bh, yk);
                yk = mma(ak, bl, yk);
                yq = mma(aq, bh, yq);
                yq = mma(aq, bl, yq);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * lq + i;
                const float r = sm.beta[t] * vv[rt][i] - sm.bgr[t] * yk[i];
                __bf16 hi, lo;
                split(r, hi, lo);
                sm.Rhi[16 * rt + lr][t] = hi;
                sm.Rlo[16 * rt + lr][t] = lo;
                O[rt][i] = sm.sqg[t] * yq[i];
            }
        }
        __syncthreads();

        // ---- U = T R (token tile w; T lower triangular) -> LDS, with U' = u2f U
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks > (w >> 1)) break;
                const bf16x8 ah = frag(&sm.Thi[0][0], LDT, 16 * w, 32 * ks, lane);
                const bf16x8 al = frag(&sm.Tlo[0][0], LDT, 16 * w, 32 * ks, lane);
                const bf16x8 bh = frag(&sm.Rhi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Rlo[0][0], LDT, 16 * rt, 32 * ks, lane);
                u = mma(ah, bh, u);
                u = mma(ah, bl, u);
                u = mma(al, bh, u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * lq + i;
                __bf16 hi, lo;
                split(u[i], hi, lo);
                sm.Uhi[16 * rt + lr][t] = hi;
                sm.Ulo[16 * rt + lr][t] = lo;
                split(sm.u2f[t] * u[i], hi, lo);
                sm.U2hi[16 * rt + lr][t] = hi;
                sm.U2lo[16 * rt + lr][t] = lo;
            }
        }
        __syncthreads();

        // ---- o = part + P U -> output;  S = G_C S + U'^T K
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 acc = O[rt];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks > (w >> 1)) break;
                const bf16x8 ah = frag(&sm.Phi[0][0], LDT, 16 * w, 32 * ks, lane);
                const bf16x8 al = frag(&sm.Plo[0][0], LDT, 16 * w, 32 * ks, lane);
                const bf16x8 bh = frag(&sm.Uhi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Ulo[0][0], LDT, 16 * rt, 32 * ks, lane);
                acc = mma(ah, bh, acc);
                acc = mma(ah, bl, acc);
                acc = mma(al, bh, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * lq + i;
                if (t < n)
                    a.o[(int64_t)(t0 + t) * a.o_stride + (int64_t)h * a.dv + vb * DVB + 16 * rt + lr] =
                        f32_to_bf16(acc[i]);
            }
        }
        const float gC = sm.gC;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rt = q >> 1, dt = 2 * w + (q & 1);
            f32x4 acc = S[q] * gC;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 ah = frag(&sm.U2hi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 al = frag(&sm.U2lo[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bk = frag(&sm.Kt[0][0], LDT, 16 * dt, 32 * ks, lane);
                acc = mma(ah, bk, acc);
                acc = mma(al, bk, acc);
            }
            S[q] = acc;
        }
        __syncthreads();
    }

#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rt = q >> 1, dt = 2 * w + (q & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) S_g[(16 * rt + 4 * lq + i) * DKC + 16 * dt + lr] = S[q][i];
    }
}

}  // namespace

int64_t chunk_max_chunks(int num_seqs, int num_tokens) {
    return (int64_t)(num_tokens + CT - 1) / CT + num_seqs;
}

int64_t chunk_workspace_bytes(int num_seqs, int num_tokens, int num_k_heads, int num_v_heads) {
    const int64_t mc = chunk_max_chunks(num_seqs, num_tokens);
    return mc * ((int64_t)num_v_heads * (int64_t)sizeof(ChunkRec) + (int64_t)num_k_heads * (int64_t)sizeof(KtRec));
}

hipError_t launch_chunk_recurrent(const RecurrentArgs &a, void *workspace, int num_tokens, hipStream_t stream) {
    const int64_t mc = chunk_max_chunks(a.num_seqs, num_tokens);
    ChunkRec *recs = reinterpret_cast<ChunkRec *>(workspace);
    KtRec *kts = reinterpret_cast<KtRec *>(reinterpret_cast<char *>(workspace) +
                                           mc * a.num_v_heads * (int64_t)sizeof(ChunkRec));
    const long long prep_blocks = mc * a.num_v_heads;
    const int nvb = a.dv / DVB;
    const long long scan_blocks = (long long)a.num_seqs * a.num_v_heads * nvb;
    if (scan_blocks == 0) return hipSuccess;
    if (prep_blocks > 0x7fffffffLL || scan_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)prep_blocks), dim3(NTH), 0, stream, a, recs, kts, (int)mc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_scan_kernel, dim3((unsigned)scan_blocks), dim3(NTH), 0, stream, a, recs, kts, nvb);
    return hipGetLastError();
}

}  // namespace gdn
