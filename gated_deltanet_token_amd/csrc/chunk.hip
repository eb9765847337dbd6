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
//    S_C^T = G_C S0^T + K^T U', with the state slice held transposed in VGPRs
//    in the MFMA accumulator layout (so every lane holds 4 consecutive dims
//    of a row and all LDS / global traffic is 8- or 16-byte vectors) and the
//    next chunk's inputs prefetched.
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
constexpr int NTH = 256;        // 4 waves
constexpr int LDK = DKC + 8;    // padded LDS row (bf16) of a [*][128] tile
constexpr int LDT = CT + 8;     // padded LDS row (bf16) of a [*][64] tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split(float v, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)v;
    lo = (__bf16)(v - (float)hi);
}

// four fp32 -> hi and lo bf16x4 (8-byte stores).  The same values as split()
// (hi = RNE(v), lo = RNE(v - hi)), converted two at a time with the packed
// conversion.
__device__ __forceinline__ void split4(const f32x4 &v, bf16x4 &hi, bf16x4 &lo) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const bf16x2v h01 = __builtin_convertvector((f32x2v){v[0], v[1]}, bf16x2v);
    const bf16x2v h23 = __builtin_convertvector((f32x2v){v[2], v[3]}, bf16x2v);
    const bf16x2v l01 = __builtin_convertvector((f32x2v){v[0] - (float)h01[0], v[1] - (float)h01[1]}, bf16x2v);
    const bf16x2v l23 = __builtin_convertvector((f32x2v){v[2] - (float)h23[0], v[3] - (float)h23[1]}, bf16x2v);
    hi = __builtin_shufflevector(h01, h23, 0, 1, 2, 3);
    lo = __builtin_shufflevector(l01, l23, 0, 1, 2, 3);
}

__device__ __forceinline__ void st4(__bf16 *p, const bf16x4 &v) { *reinterpret_cast<bf16x4 *>(p) = v; }

// Full-line workspace stores (T, K^T) and the final state are streaming
// (nontemporal): written once per launch, they leave no dirty lines behind
// for the next kernel to write back.  P is written in 32-byte pieces per
// row and stays on plain stores, which the L2 merges into whole lines.
__device__ __forceinline__ void st8_stream(__bf16 *p, const bf16x8 &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8 *>(p));
}

// A 64 x 64 lower-triangular fp32 matrix in LDS as its ten 16 x 16 blocks
// (b, c), b >= c, block index b (b + 1) / 2 + c; rows padded to 20 floats
constexpr int LDB = 20;
constexpr int NBLK = 10;
__device__ __forceinline__ constexpr int blk(int b, int c) { return b * (b + 1) / 2 + c; }
typedef float Blk[16][LDB];

// C += X Y for two 16 x 16 fp32 blocks; four 16x16x4 fp32 MFMAs
__device__ __forceinline__ f32x4 mm16(const Blk &X, const Blk &Y, f32x4 c, int lane) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float a = X[lane & 15][(lane >> 4) + 4 * s];
        const float b = Y[(lane >> 4) + 4 * s][lane & 15];
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    return c;
}

__device__ __forceinline__ void put16(Blk &Z, const f32x4 &c, float sgn, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Z[4 * (lane >> 4) + i][lane & 15] = sgn * c[i];
}

// ---------------------------------------------------------------------------
// where a global chunk index lands in the packed sequences
// ---------------------------------------------------------------------------
// Every lane of a wave reads one sequence's bounds at once (64 sequences per
// round trip) instead of walking the sequences one load after another.

// the sequence s holding packed chunk `gch` and the chunk's index j in it
// (s = -1 past the last chunk); called by every lane of the wave
__device__ __forceinline__ void locate_chunk(const int32_t *qsl, int num_seqs, int gch, int &s_out, int &j_out) {
    const int lane = threadIdx.x & 63;
    int before = 0;
    s_out = -1;
    j_out = 0;
    for (int s0 = 0; s0 < num_seqs; s0 += 64) {
        const int q = s0 + lane;
        const int lo = qsl[min(q, num_seqs)], hi = qsl[min(q + 1, num_seqs)];
        int incl = q < num_seqs ? chunk_count(hi - lo) : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int up = __shfl_up(incl, off, 64);
            if (lane >= off) incl += up;
        }
        const int total = __shfl(incl, 63, 64);
        if (gch < before + total) {
            // lanes whose sequences end at or before the chunk come first
            const int ls = __popcll(__ballot(before + incl <= gch));
            const int excl = ls > 0 ? __shfl(incl, ls - 1, 64) : 0;
            s_out = s0 + ls;
            j_out = gch - before - excl;
            return;
        }
        before += total;
    }
}

// number of chunks of the sequences before s; called by every lane of the wave
__device__ __forceinline__ int chunks_before(const int32_t *qsl, int s) {
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int s0 = 0; s0 < s; s0 += 64) {
        const int q = s0 + lane;
        const int lo = qsl[min(q, s)], hi = qsl[min(q + 1, s)];
        int nc = q < s ? chunk_count(hi - lo) : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) nc += __shfl_xor(nc, off, 64);
        total += nc;
    }
    return total;
}

// ---------------------------------------------------------------------------
// prep: one workgroup per (chunk, v-head)
// ---------------------------------------------------------------------------
// 31 KB, so that five workgroups share a CU and a 2,048-token step's
// (chunk, v-head) grid runs in one round: the q rows are not staged (the
// MFMA reads its q fragments from L2), and T reuses the space of the k rows,
// which are dead once A and P are formed.
struct PrepSmem {
    union {
        __bf16 K[CT][LDK];   // stages 0-1: the chunk's k rows
        Blk T[NBLK];         // stage 2: T = (I + A)^-1
    } u;
    Blk A[NBLK];
    float lam[CT], rk[CT], rq[CT], beta[CT];
};

__global__ __launch_bounds__(NTH) void chunk_prep_kernel(RecurrentArgs a, ChunkRec *recs, KtRec *kts,
                                                        int max_chunks) {
    __shared__ PrepSmem sm;
    const int HV = a.num_v_heads;
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int h = work % HV;
    const int gch = work / HV;                  // global chunk index
    int s, j;                                   // (sequence, chunk within it)
    locate_chunk(a.qsl, a.num_seqs, gch, s, j);
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
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            *reinterpret_cast<uint4 *>(&sm.u.K[tok][32 * part + 8 * m]) = kv[m];
            float kf[8], qf[8];
            unpack8(kv[m], kf);
            unpack8(qv[m], qf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                skk = __builtin_fmaf(kf[e], kf[e], skk);
                sqq = __builtin_fmaf(qf[e], qf[e], sqq);
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
    // K^T for the scan (once per q/k head): lane pair per dim d, 32 tokens each
    if ((h % grp) == 0) {
        const int d = tid >> 1, half = tid & 1;
        bf16x8 col[4];
#pragma unroll
        for (int j = 0; j < 32; ++j) col[j >> 3][j & 7] = sm.u.K[32 * half + j][d];
        __bf16 *dst = &kts[(int64_t)gch * a.num_k_heads + hk].Kt[d][32 * half];
#pragma unroll
        for (int m = 0; m < 4; ++m) st8_stream(dst + 8 * m, col[m]);
    }

    // ---- stage 1: tiles (i-tile c, t-tile w) of K K^T and K Q^T, laid out
    // so each lane holds 4 consecutive i of one row t of A and of P:
    // A (fp32) into its LDS block, P (hi/lo) to the workspace with 8-byte stores
    {
        const int t = 16 * w + lr;
        const float lam_t = sm.lam[t], beta_t = sm.beta[t], rk_t = sm.rk[t], rq_t = sm.rq[t];
        // q rows of t-tile w as B operands, straight from L2 (zero past the chunk end)
        bf16x8 bq[DKC / 32];
        {
            const __bf16 *qrow = reinterpret_cast<const __bf16 *>(a.q) + (int64_t)(t0 + min(t, n - 1)) * a.q_stride +
                                 hk * DKC + 8 * lq;
#pragma unroll
            for (int ks = 0; ks < DKC / 32; ++ks) {
                const uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * ks);
                bq[ks] = __builtin_bit_cast(bf16x8, t < n ? v : make_uint4(0, 0, 0, 0));
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i0 = 16 * c + 4 * lq;
            if (c > w) {
                const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
                st4(&rec->Phi[t][i0], z);
                st4(&rec->Plo[t][i0], z);
                continue;
            }
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, kq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DKC / 32; ++ks) {
                const bf16x8 ai = frag(&sm.u.K[0][0], LDK, 16 * c, 32 * ks, lane);
                const bf16x8 bk = frag(&sm.u.K[0][0], LDK, 16 * w, 32 * ks, lane);
                kk = mma(ai, bk, kk);
                kq = mma(ai, bq[ks], kq);
            }
            f32x4 av, pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = i0 + e;
                const float decay = i <= t ? expf(lam_t - sm.lam[i]) : 0.f;
                av[e] = i < t ? beta_t * rk_t * sm.rk[i] * decay * kk[e] : 0.f;
                pv[e] = i <= t ? a.scale * rq_t * sm.rk[i] * decay * kq[e] : 0.f;
            }
            *reinterpret_cast<f32x4 *>(&sm.A[blk(w, c)][lr][4 * lq]) = av;
            bf16x4 ph, pl;
            split4(pv, ph, pl);
            st4(&rec->Phi[t][i0], ph);
            st4(&rec->Plo[t][i0], pl);
        }
    }
    __syncthreads();

    // ---- stage 2: T = (I + A)^-1, block by block (T overwrites the k rows)
    {
        if (lane < 16) {
            // diagonal block w by forward substitution; lane j owns column j
            const Blk &Ad = sm.A[blk(w, w)];
            float xcol[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = r == lane ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc = __builtin_fmaf(-Ad[r][i], xcol[i], acc);
                xcol[r] = acc;
            }
            Blk &Td = sm.u.T[blk(w, w)];
#pragma unroll
            for (int r = 0; r < 16; ++r) Td[r][lane] = xcol[r];
        }
        __syncthreads();
        // T_bc = -T_bb (sum_{c<=m<b} A_bm T_mc); wave c walks down column
        // block c, so every input is its own earlier result or a diagonal block
        const int c = w;
        for (int b = c + 1; b < 4 && w < 3; ++b) {
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            for (int mm = c; mm < b; ++mm) m = mm16(sm.A[blk(b, mm)], sm.u.T[blk(mm, c)], m, lane);
            put16(sm.u.T[blk(b, c)], m, 1.f, lane);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sm.u.T[blk(b, b)], sm.u.T[blk(b, c)], t, lane);
            put16(sm.u.T[blk(b, c)], t, -1.f, lane);
        }
        __syncthreads();
        // hi/lo to the workspace, 8 consecutive entries per lane (zero above
        // the diagonal blocks)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = tid + NTH * e;          // 512 groups of 8
            const int t = idx >> 3, i0 = (idx & 7) * 8;
            const int bt = t >> 4, bc = i0 >> 4;
            bf16x8 hv, lv;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __bf16 hi, lo;
                split(bc <= bt ? sm.u.T[blk(bt, min(bc, bt))][t & 15][(i0 & 15) + q] : 0.f, hi, lo);
                hv[q] = hi;
                lv[q] = lo;
            }
            st8_stream(&rec->Thi[t][i0], hv);
            st8_stream(&rec->Tlo[t][i0], lv);
        }
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, v-head, 32 v rows)
// ---------------------------------------------------------------------------
// Only data that crosses waves lives in LDS (the state entering the chunk
// and R, U, U'); every MFMA operand a wave owns (its K / Q / T / P rows, its
// K^T rows) is loaded straight from global memory / L2 into registers a
// chunk ahead of use, into the second of two register sets.  45 KB of LDS
// would let three workgroups share a CU; registers are capped at 256 per
// lane (two waves per SIMD), so two do, which keeps a 3-sequence prefill
// (384 workgroups) resident at once.
template <int DVB>
struct ScanSmem {
    __bf16 Shi[DVB][LDK], Slo[DVB][LDK];     // S0 [r][d]
    __bf16 Rhi[DVB][LDT], Rlo[DVB][LDT];     // R^T [r][t]
    __bf16 Uhi[DVB][LDT], Ulo[DVB][LDT];     // U^T [r][t]
    __bf16 U2hi[DVB][LDT], U2lo[DVB][LDT];   // U'^T [r][t]
};

// operand fragment straight from global memory (row-major, `ld` elements)
__device__ __forceinline__ bf16x8 gfrag(const __bf16 *base, int64_t ld, int row, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (int64_t)row * ld + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ uint4 mask4(bool keep, const uint4 &v) {
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

__device__ __forceinline__ bf16x8 maskf(bool keep, const bf16x8 &v) {
    return __builtin_bit_cast(bf16x8, mask4(keep, __builtin_bit_cast(uint4, v)));
}

// DVB v rows per workgroup (NRT = DVB / 16 row tiles per wave): 32 rows,
// two workgroups per CU; or 64 rows, one workgroup per CU, when 32-row
// workgroups would outnumber the CUs (a CU running two of them is what sets
// the pace; one 64-row workgroup shares each token tile's operand loads
// between twice the rows).
template <int DVB>
__global__ __launch_bounds__(NTH, DVB == 64 ? 1 : 2) void chunk_scan_kernel(RecurrentArgs a, const ChunkRec *recs,
                                                                            const KtRec *kts, int n_vblocks) {
    constexpr int NRT = DVB / 16;
    __shared__ ScanSmem<DVB> sm;
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
    int gch = chunks_before(a.qsl, s);             // global index of this sequence's first chunk

    // the wave index is uniform over the wave: as a scalar, the loops that
    // stop at it are scalar branches rather than exec-masked regions
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int kh_off = hk * DKC;
    const int o_col_bytes = 2 * (h * a.dv + vb * DVB);
    const __bf16 *kbase = reinterpret_cast<const __bf16 *>(a.k) + kh_off;
    const __bf16 *qbase = reinterpret_cast<const __bf16 *>(a.q) + kh_off;

    // the state slice, transposed, in the accumulator layout of S^T tiles
    // (d-tile dt, v-row tile rt): tile q = 2*rt + (dt - 2w); lane holds
    // S[16 rt + lr][16 dt + 4 lq .. +3] -- four consecutive dims of one row
    float *S_g = a.state + ((int64_t)slot * HV + h) * (int64_t)a.dv * DKC + (int64_t)vb * DVB * DKC;
    f32x4 S[2 * NRT];
    const bool init = a.has_init == nullptr || a.has_init[s] != 0;
#pragma unroll
    for (int q = 0; q < 2 * NRT; ++q) {
        const int rt = q >> 1, dt = 2 * w + (q & 1);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        S[q] = init ? load_stream4(&S_g[(16 * rt + lr) * DKC + 16 * dt + 4 * lq]) : z;
    }

    // per-lane operands of one chunk.  Two register sets alternate (the
    // chunk loop is unrolled by two), so the next chunk's loads land in the
    // other set and nothing has to wait for them before the next chunk.
    struct Ops {
        bf16x8 kf[4], qf[4];            // K, Q rows 16w + lr, dims 32 ks + 8 lq ..
        f32x4 sb, sbgr, ssqg, su2;      // factors of tokens 16w + 4lq + i
        float gc;                       // G_C (stored for every token; a per-lane load)
        uint16_t vraw[NRT][4];            // v of tokens 16w + 4lq + i, rows 16 rt + lr
        bf16x8 th[2], tl[2];            // T rows 16w + lr, cols 32 ks + 8 lq ..
        bf16x8 ph[2], pl[2];            // P rows 16w + lr
        bf16x8 ktf[2][2];               // K^T rows 16 (2w + j) + lr
    };
    auto load_y = [&](Ops &op, int c_t0, int c_n, const ChunkRec *rec) {
        const int row = c_t0 + min(16 * w + lr, c_n - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            op.kf[ks] = gfrag(kbase, a.k_stride, row, 32 * ks, lane);
            op.qf[ks] = gfrag(qbase, a.q_stride, row, 32 * ks, lane);
        }
        const int t4 = 16 * w + 4 * lq;
        op.sb = *reinterpret_cast<const f32x4 *>(&rec->beta[t4]);
        op.sbgr = *reinterpret_cast<const f32x4 *>(&rec->bgr[t4]);
        op.ssqg = *reinterpret_cast<const f32x4 *>(&rec->sqg[t4]);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                op.vraw[rt][i] = a.v[(int64_t)(c_t0 + min(t4 + i, c_n - 1)) * a.v_stride + (int64_t)h * a.dv +
                                     vb * DVB + 16 * rt + lr];
    };
    auto load_t = [&](Ops &op, const ChunkRec *rec) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            op.th[ks] = gfrag(&rec->Thi[0][0], CT, 16 * w + lr, 32 * ks, lane);
            op.tl[ks] = gfrag(&rec->Tlo[0][0], CT, 16 * w + lr, 32 * ks, lane);
        }
        op.su2 = *reinterpret_cast<const f32x4 *>(&rec->u2f[16 * w + 4 * lq]);
    };
    auto load_p = [&](Ops &op, const ChunkRec *rec, const KtRec *kt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            op.ph[ks] = gfrag(&rec->Phi[0][0], CT, 16 * w + lr, 32 * ks, lane);
            op.pl[ks] = gfrag(&rec->Plo[0][0], CT, 16 * w + lr, 32 * ks, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                op.ktf[j][ks] = gfrag(&kt->Kt[0][0], CT, 16 * (2 * w + j) + lr, 32 * ks, lane);
        }
        op.gc = rec->gC[16 * w + 4 * lq];
    };

    // one chunk: consumes `cur`, prefetches the next chunk into `nxt`
    auto chunk = [&](const Ops &cur, Ops &nxt, int t0, int gch_c) {
        const int n = min(CT, t_end - t0);
        // the next chunk's operands; the last chunk reloads its own (always
        // in bounds, and the loads stay unconditional: no branch for the
        // wait-count tracking to merge)
        const bool more = t0 + CT < t_end;
        const int t_next = more ? t0 + CT : t0;
        const int n_next = min(CT, t_end - t_next);
        const int g_next = more ? gch_c + 1 : gch_c;
        const ChunkRec *rec_next = recs + (int64_t)g_next * HV + h;
        const KtRec *kt_next = kts + (int64_t)g_next * a.num_k_heads + hk;

        // The chunk's o rows through a buffer resource that covers exactly
        // them: a padded token (t >= n) stores at the end of the range, where
        // the hardware range check drops it.  The stores then need no branch,
        // and no branch means no conservative wait for every load in flight
        // (this chunk's prefetch included) where the paths merge.
        const int o_row_bytes = 2 * (int)a.o_stride;
        const int o_range = n * o_row_bytes;
        const __amdgpu_buffer_rsrc_t o_rsrc =
            __builtin_amdgcn_make_buffer_rsrc(a.o + (int64_t)t0 * a.o_stride, (short)0, o_range, kBufferFlags);

        // ---- the state entering the chunk -> LDS (hi/lo)
#pragma unroll
        for (int q = 0; q < 2 * NRT; ++q) {
            const int rt = q >> 1, dt = 2 * w + (q & 1);
            bf16x4 hi, lo;
            split4(S[q], hi, lo);
            st4(&sm.Shi[16 * rt + lr][16 * dt + 4 * lq], hi);
            st4(&sm.Slo[16 * rt + lr][16 * dt + 4 * lq], lo);
        }
        __syncthreads();
        load_y(nxt, t_next, n_next, rec_next);     // next chunk's K, Q, v, factors

        // ---- R = b v - bgr (K S0^T) -> LDS;  o part = sqg (Q S0^T)
        const bool live = 16 * w + lr < n;
        f32x4 O[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4 yk = {0.f, 0.f, 0.f, 0.f}, yq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DKC / 32; ++ks) {
                const bf16x8 bh = frag(&sm.Shi[0][0], LDK, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Slo[0][0], LDK, 16 * rt, 32 * ks, lane);
                const bf16x8 ka = maskf(live, cur.kf[ks]), qa = maskf(live, cur.qf[ks]);
                yk = mma(ka, bh, yk);
                yq = mma(qa, bh, yq);
                yk = mma(ka, bl, yk);
                yq = mma(qa, bl, yq);
            }
            f32x4 r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vv = 16 * w + 4 * lq + i < n ? bf16_to_f32(cur.vraw[rt][i]) : 0.f;
                r[i] = cur.sb[i] * vv - cur.sbgr[i] * yk[i];
                O[rt][i] = cur.ssqg[i] * yq[i];
            }
            bf16x4 hi, lo;
            split4(r, hi, lo);
            st4(&sm.Rhi[16 * rt + lr][16 * w + 4 * lq], hi);
            st4(&sm.Rlo[16 * rt + lr][16 * w + 4 * lq], lo);
        }
        __syncthreads();
        load_t(nxt, rec_next);

        // ---- U = T R (token tile w; T lower triangular) -> LDS, with U' = u2f U
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks > (w >> 1)) break;
                const bf16x8 bh = frag(&sm.Rhi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Rlo[0][0], LDT, 16 * rt, 32 * ks, lane);
                u = mma(cur.th[ks], bh, u);
                u = mma(cur.th[ks], bl, u);
                u = mma(cur.tl[ks], bh, u);
            }
            f32x4 u2;
#pragma unroll
            for (int i = 0; i < 4; ++i) u2[i] = cur.su2[i] * u[i];
            bf16x4 hi, lo;
            split4(u, hi, lo);
            st4(&sm.Uhi[16 * rt + lr][16 * w + 4 * lq], hi);
            st4(&sm.Ulo[16 * rt + lr][16 * w + 4 * lq], lo);
            split4(u2, hi, lo);
            st4(&sm.U2hi[16 * rt + lr][16 * w + 4 * lq], hi);
            st4(&sm.U2lo[16 * rt + lr][16 * w + 4 * lq], lo);
        }
        __syncthreads();
        load_p(nxt, rec_next, kt_next);

        // ---- o = part + P U -> output;  S^T = G_C S^T + K^T U'
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            f32x4 acc = O[rt];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks > (w >> 1)) break;
                const bf16x8 bh = frag(&sm.Uhi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.Ulo[0][0], LDT, 16 * rt, 32 * ks, lane);
                acc = mma(cur.ph[ks], bh, acc);
                acc = mma(cur.ph[ks], bl, acc);
                acc = mma(cur.pl[ks], bh, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * w + 4 * lq + i;
                const int off = t < n ? (t * o_row_bytes + o_col_bytes + 2 * (16 * rt + lr)) : o_range;
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[i]), o_rsrc, off, 0, 0);
            }
        }
        const float g_c = cur.gc;
#pragma unroll
        for (int q = 0; q < 2 * NRT; ++q) {
            const int rt = q >> 1, j = q & 1;
            f32x4 acc = S[q] * g_c;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 bh = frag(&sm.U2hi[0][0], LDT, 16 * rt, 32 * ks, lane);
                const bf16x8 bl = frag(&sm.U2lo[0][0], LDT, 16 * rt, 32 * ks, lane);
                acc = mma(cur.ktf[j][ks], bh, acc);
                acc = mma(cur.ktf[j][ks], bl, acc);
            }
            S[q] = acc;
        }
        // no barrier: the next chunk writes S (read only before the second
        // barrier above), then R, U, U' only after barriers every wave passes
        // once it is done with this chunk
    };

    Ops A, B;
    {
        const ChunkRec *rec = recs + (int64_t)gch * HV + h;
        load_y(A, t_begin, min(CT, t_end - t_begin), rec);
        load_t(A, rec);
        load_p(A, rec, kts + (int64_t)gch * a.num_k_heads + hk);
    }
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * CT, gch += 2) {
        chunk(A, B, t0, gch);
        if (t0 + CT >= t_end) break;
        chunk(B, A, t0 + CT, gch + 1);
    }

#pragma unroll
    for (int q = 0; q < 2 * NRT; ++q) {
        const int rt = q >> 1, dt = 2 * w + (q & 1);
        store_stream4(&S_g[(16 * rt + lr) * DKC + 16 * dt + 4 * lq], S[q]);
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
    constexpr int kCUs = 256;
    const long long heads = (long long)a.num_seqs * a.num_v_heads;
    const bool wide = heads * (a.dv / 32) > kCUs && (a.dv % 64) == 0;
    const int nvb = a.dv / (wide ? 64 : 32);
    const long long scan_blocks = heads * nvb;
    if (scan_blocks == 0) return hipSuccess;
    if (prep_blocks > 0x7fffffffLL || scan_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)prep_blocks), dim3(NTH), 0, stream, a, recs, kts, (int)mc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wide)
        hipLaunchKernelGGL(chunk_scan_kernel<64>, dim3((unsigned)scan_blocks), dim3(NTH), 0, stream, a, recs, kts, nvb);
    else
        hipLaunchKernelGGL(chunk_scan_kernel<32>, dim3((unsigned)scan_blocks), dim3(NTH), 0, stream, a, recs, kts, nvb);
    return hipGetLastError();
}

}  // namespace gdn
