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
//  * prep (one workgroup per (chunk, one or two v-heads of a q/k head), all
//    chunks in parallel): the parts that do not depend on the state --
//    norms, cumulative decay, T = (I + A)^-1, P_ti = scale exp(L_t - L_i)
//    (qh_t . kh_i) (i <= t) -- written to the caller's workspace;
//  * scan (one workgroup per (sequence, v-head, 32 or 64 v rows), serial
//    over the sequence's chunks, each wave owning 16 v rows): [K;Q] S0^T,
//    R, U = T R, o = S0 part + P U and S_C^T = G_C S0^T + K^T U', with the
//    wave's state rows and every intermediate held in VGPRs in the MFMA
//    accumulator layout, the chunk's shared operands staged in LDS and the
//    next chunk's prefetched.
//
// Precision: products of raw bf16 inputs (K K^T, Q K^T) are exact in the
// bf16 MFMA with fp32 accumulation.  Every product with an fp32 operand (the
// state, T, P, U, R) splits that operand into hi + lo bf16 parts (16
// significant bits) and sums the partial products.  T is inverted in fp32
// (16 x 16 diagonal blocks by substitution, off-diagonal blocks with fp32
// MFMA).
#include "fused_unit.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CT = 64;          // tokens per chunk
constexpr int DKC = 128;        // head_k_dim
constexpr int NTH = 256;        // 4 waves
constexpr int LDK = DKC + 8;    // padded LDS row (bf16) of a [*][128] tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
// per (chunk, v-head): T hi, T lo, P hi, P lo -- lower triangular, so only
// their ten 16 x 16 blocks (b, c), b >= c, block index b (b + 1) / 2 + c,
// each [16][16] bf16 ([t][i]) -- then per-token scalars
constexpr int NBLK16 = 10;
struct ChunkRec {
    __bf16 TP[4][NBLK16][16][16];   // T hi, T lo, P hi, P lo
    float beta[CT];   // b_t
    float bgr[CT];    // b_t G_t rk_t          (R = b v - bgr (K S0^T))
    float sqg[CT];    // scale rq_t G_t        (o = sqg (Q S0^T) + P U)
    float u2f[CT];    // exp(L_C - L_t) rk_t   (S_C = G_C S0 + (u2f U)^T K)
    float gC[CT];     // G_C in [0]
};
static_assert(sizeof(ChunkRec) % 256 == 0, "record alignment");

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

// exp(x) as one hardware 2^x (v_exp_f32, about 1 ulp) of x log2(e): the
// rounding of the product adds a relative error of about |x| 2^-24 (below
// 1e-5 for every |x| < 100; beyond that the decay is below 1e-43 and flushes
// to zero).  The decays within a chunk use it; the library expf takes some
// ten instructions more per call.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// four fp32 -> hi and lo bf16x4 (8-byte stores): hi = RNE(v), lo =
// RNE(v - hi), converted two at a time with the packed conversion.
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

// Workspace stores are written through the L2 (sc1): the scan reads the
// records right after the prep, on the same XCD (both kernels order their
// work head-major), and finds them in its L2, while the end of the prep has
// no dirty lines to write back.  A relaxed device-scope atomic store is how
// HIP expresses such a store; it is an ordinary 8- or 4-byte vector store
// with the sc1 bit.  (Streaming stores for the records made the whole call
// 2-3% slower; plain ones left the prep's end writing back its records.)
// The scan's final state is streaming.
__device__ __forceinline__ void st4(__bf16 *p, const bf16x4 &v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f32(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// the sequence s holding packed chunk `gch`, the chunk's index j in it and
// the sequence's token range [lo, hi) (s = -1 past the last chunk); called
// by every lane of the wave
// (sequence bounds are clamped to [0, num_tokens) as everywhere in the
// library: a malformed query_start_loc gives wrong results, never an access
// outside the token rows or the workspace)
__device__ __forceinline__ void locate_chunk(const int32_t *qsl, int num_seqs, int num_tokens, int gch, int &s_out,
                                             int &j_out, int &lo_out, int &hi_out) {
    const int lane = threadIdx.x & 63;
    int before = 0;
    s_out = -1;
    j_out = 0;
    lo_out = hi_out = 0;
    for (int s0 = 0; s0 < num_seqs; s0 += 64) {
        const int q = s0 + lane;
        int lo, hi;
        clamp_range(qsl[min(q, num_seqs)], qsl[min(q + 1, num_seqs)], num_tokens, lo, hi);
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
            lo_out = __shfl(lo, ls, 64);
            hi_out = __shfl(hi, ls, 64);
            return;
        }
        before += total;
    }
}

// number of chunks of the sequences before s; called by every lane of the wave
__device__ __forceinline__ int chunks_before(const int32_t *qsl, int s, int num_tokens) {
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int s0 = 0; s0 < s; s0 += 64) {
        const int q = s0 + lane;
        int lo, hi;
        clamp_range(qsl[min(q, s)], qsl[min(q + 1, s)], num_tokens, lo, hi);
        int nc = q < s ? chunk_count(hi - lo) : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) nc += __shfl_xor(nc, off, 64);
        total += nc;
    }
    return total;
}

// ---------------------------------------------------------------------------
// prep: one workgroup per (chunk, VPW v-heads of one q/k head)
// ---------------------------------------------------------------------------
// The v-heads that share a q/k head share the chunk's k and q rows, their
// norms and the products K K^T and Q K^T; only the gates and betas -- so A,
// T and P -- are per v-head.  With two v-heads per workgroup (VPW = 2, an
// even number of v-heads per q/k head) eight waves form the shared part once
// and each v-head gets four waves for its inversion; the ten tiles of K K^T
// and Q K^T go round-robin over the waves (at most two per wave).  The q
// rows are not staged (the MFMA reads its q fragments from L2), and T reuses
// the space of the k rows, which are dead once A and P are formed: 53 KB at
// VPW = 2 (three workgroups per CU), 31 KB at VPW = 1 (five).
//
// A workgroup's work is one chain of dependent steps, and a 2,048-token
// step has only about two workgroups per CU, so the order below keeps that
// chain short: each wave issues the q loads of its first tile before
// anything else, the waves with one tile fewer take the gates and the
// per-token scalars, and every block of T goes to the workspace as soon as
// it is final instead of in a pass at the end.
template <int VPW>
struct PrepSmem {
    union {
        __bf16 K[CT][LDK];   // stages 0-1: the chunk's k rows
        Blk T[VPW][NBLK];    // stage 2: T = (I + A)^-1 per v-head
    } u;
    Blk A[VPW][NBLK];
    float rk[CT], rq[CT];
    float lam[VPW][CT], beta[VPW][CT];
};

// t-tile and i-tile of lower-triangular block b (b = bt (bt + 1) / 2 + bc)
__device__ __forceinline__ void tile_of(int b, int &bt, int &bc) {
    bt = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
    bc = b - bt * (bt + 1) / 2;
}

// the q rows of t-tile bt as MFMA B operands, straight from L2 (zero past
// the chunk end)
__device__ __forceinline__ void load_qfrag(bf16x8 (&bq)[DKC / 32], const RecurrentArgs &a, int t0, int n, int hk,
                                           int bt, int lr, int lq) {
    const int t = 16 * bt + lr;
    const __bf16 *qrow = reinterpret_cast<const __bf16 *>(a.q) + (int64_t)(t0 + min(t, n - 1)) * a.q_stride +
                         hk * DKC + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < DKC / 32; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4 *>(qrow + 32 * ks);
        bq[ks] = __builtin_bit_cast(bf16x8, t < n ? v : make_uint4(0, 0, 0, 0));
    }
}

// block bi of T (final, in LDS) to the record as hi and lo bf16, by one
// whole wave: lane l takes row l / 4, four consecutive columns.  The block
// was written by this same wave's lanes in another layout; the fences keep
// the compiler from moving the reads above those writes (a wave's LDS
// accesses complete in order).
__device__ __forceinline__ void store_tblock(const Blk &Tb, ChunkRec *rec, int bi, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int r = lane >> 2, c0 = 4 * (lane & 3);
    const f32x4 v = *reinterpret_cast<const f32x4 *>(&Tb[r][c0]);
    bf16x4 h, l;
    split4(v, h, l);
    st4(&rec->TP[0][bi][r][c0], h);
    st4(&rec->TP[1][bi][r][c0], l);
}

// Tile b of the prep's stage 1 by one wave, in two steps: the products
// (tile_products: its K K^T part KK and / or its Q K^T part KQ, with bq the
// q fragments of the tile's t-tile), then the element work (tile_elements:
// A of each v-head into LDS for KK, P of each v-head to the records for KQ).
// A wave with two tiles forms both tiles' products before the element work
// of either, so the second tile's LDS reads and products overlap the first
// tile's instead of following them.
template <int VPW, bool KK, bool KQ>
__device__ __forceinline__ void tile_products(PrepSmem<VPW> &sm, int b, const bf16x8 (&bq)[DKC / 32], int lane,
                                              f32x4 &kk, f32x4 &kq) {
    int bt, bc;
    tile_of(b, bt, bc);
    kk = kq = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DKC / 32; ++ks) {
        const bf16x8 ai = frag(&sm.u.K[0][0], LDK, 16 * bc, 32 * ks, lane);
        if (KK) {
            const bf16x8 bk = frag(&sm.u.K[0][0], LDK, 16 * bt, 32 * ks, lane);
            kk = mma(ai, bk, kk);
        }
        if (KQ) kq = mma(ai, bq[ks], kq);
    }
}

template <int VPW, bool KK, bool KQ>
__device__ __forceinline__ void tile_elements(PrepSmem<VPW> &sm, const RecurrentArgs &a, ChunkRec *rec0, int b,
                                              int lane, const f32x4 &kk, const f32x4 &kq) {
    const int lr = lane & 15, lq = lane >> 4;
    int bt, bc;
    tile_of(b, bt, bc);
    const int t = 16 * bt + lr, i0 = 16 * bc + 4 * lq;
    // Every value is computed for all 16 x 16 positions and the triangle is
    // kept by selects: with the LDS reads and the exponential under a
    // condition, the compiler branched around each element and waited for
    // each read on its own.  (Above the diagonal lam_t - lam_i may be
    // positive and its exponential large or infinite; the select drops it.)
    const float rk_t = sm.rk[t], rq_t = sm.rq[t];
    const f32x4 rk_i = *reinterpret_cast<const f32x4 *>(&sm.rk[i0]);
#pragma unroll
    for (int v = 0; v < VPW; ++v) {
        const float lam_t = sm.lam[v][t];
        const float fa = sm.beta[v][t] * rk_t, fp = a.scale * rq_t;
        const f32x4 lam_i = *reinterpret_cast<const f32x4 *>(&sm.lam[v][i0]);
        f32x4 av, pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = i0 + e;
            const float wi = rk_i[e] * exp_fast(lam_t - lam_i[e]);     // rk_i exp(L_t - L_i)
            av[e] = i < t ? fa * wi * kk[e] : 0.f;
            pv[e] = i <= t ? fp * wi * kq[e] : 0.f;
        }
        if (KK) *reinterpret_cast<f32x4 *>(&sm.A[v][b][lr][4 * lq]) = av;
        if (KQ) {
            bf16x4 ph, pl;
            split4(pv, ph, pl);
            st4(&rec0[v].TP[2][b][lr][4 * lq], ph);
            st4(&rec0[v].TP[3][b][lr][4 * lq], pl);
        }
    }
}

template <int VPW>
__global__ __launch_bounds__(NTH * VPW) void chunk_prep_kernel(const int32_t *qsl, const uint16_t *k,
                                                                 const uint16_t *q, int64_t k_stride,
                                                                 int64_t q_stride, int num_seqs, int num_tokens,
                                                                 int num_v_heads, int n_blocks,
                                                                 RecurrentArgs a_in, ChunkRec *recs) {
    // the chunk lookup's and the row loads' arguments, also passed ahead of
    // the struct: the first 14 dwords arrive preloaded in SGPRs
    RecurrentArgs a = a_in;
    a.qsl = qsl;
    a.k = k;
    a.q = q;
    a.k_stride = k_stride;
    a.q_stride = q_stride;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_v_heads = num_v_heads;
    constexpr int NT = NTH * VPW, NW = NT / 64;
    // Stage 1's work, the ten lower-triangular tiles of K K^T and Q K^T, is
    // spread so that no wave has two full tiles more than another: tiles
    // 0-7 whole, round-robin, and tiles 8 and 9 (both of t-tile 3) split
    // into their K K^T and Q K^T halves.  The Q K^T halves go to the waves
    // whose own tile is of t-tile 3 (their q fragments serve again), the
    // K K^T halves and the gates / per-token scalars to waves of the rest:
    //   VPW = 2: waves 2, 3 the K K^T halves, 6, 7 the Q K^T halves, 4, 5 the scalars
    //   VPW = 1: waves 0, 1 the K K^T halves, 2, 3 the Q K^T halves, 1 the scalars
    constexpr int GW = VPW == 2 ? 4 : 1;        // waves GW + v: gates and per-token scalars of v-head v
    constexpr int HKK = VPW == 2 ? 2 : 0;       // waves HKK, HKK + 1: the K K^T halves of tiles 8, 9
    constexpr int HKQ = VPW == 2 ? 6 : 2;       // waves HKQ, HKQ + 1: the Q K^T halves of tiles 8, 9
    __shared__ PrepSmem<VPW> sm;
    const int HV = a.num_v_heads, NP = HV / VPW;
    // head-pair-major, XCD-contiguous: an XCD prepares all chunks of a range
    // of v-heads, the heads whose scan workgroups it also runs, so the scan
    // finds the records in its own L2
    const int work = xcd_contiguous(blockIdx.x, n_blocks);
    const int mcg = n_blocks / NP;              // chunks the grid covers (an upper bound)
    const int h0 = (work / mcg) * VPW;          // the workgroup's first v-head
    const int gch = work % mcg;                 // global chunk index
    int s, j, lo, hi;                           // (sequence, chunk within it, its tokens)
    locate_chunk(a.qsl, a.num_seqs, a.num_tokens, gch, s, j, lo, hi);
    // (a padded sequence, state index < 0, is prepared too: its records are
    // never read, and the row loads need not wait for the index)
    if (s < 0) return;
    const int t0 = lo + CT * j;
    const int n = min(CT, hi - t0);
    const int grp = HV / a.num_k_heads;
    const int hk = h0 / grp;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // q of the wave's first tile (b = w), in flight during stage 0
    bf16x8 bq[DKC / 32];
    {
        int bt, bc;
        tile_of(w, bt, bc);
        load_qfrag(bq, a, t0, n, hk, bt, lr, lq);
    }

    // ---- stage 0: k/q rows and norms (first four waves); cumulative decay of
    // v-head v (wave GW + v)
    if (tid < NTH) {
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
    }
    if (w >= GW && w < GW + VPW) {
        // padded tokens: g = 0 and beta = 0 make them exact no-ops
        const int v = w - GW, h = h0 + v;
        float gg = lane < n ? a.g[(int64_t)(t0 + lane) * HV + h] : 0.f;
        const float bb = lane < n ? a.beta[(int64_t)(t0 + lane) * HV + h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(gg, off, 64);
            if (lane >= off) gg += up;
        }
        sm.lam[v][lane] = gg;
        sm.beta[v][lane] = bb;
    }
    __syncthreads();

    // per-token scalars for the scan (wave GW + v for v-head v)
    if (w >= GW && w < GW + VPW) {
        const int v = w - GW, t = lane;
        ChunkRec *rec = recs + (int64_t)gch * HV + h0 + v;
        const float lam = sm.lam[v][t], lamC = sm.lam[v][CT - 1];
        const float G = expf(lam), rk = sm.rk[t];
        st_f32(&rec->beta[t], sm.beta[v][t]);
        st_f32(&rec->bgr[t], sm.beta[v][t] * G * rk);
        st_f32(&rec->sqg[t], a.scale * sm.rq[t] * G);
        st_f32(&rec->u2f[t], expf(lamC - lam) * rk);
        st_f32(&rec->gC[t], expf(lamC));
    }
    // ---- stage 1: the lower-triangular tiles (t-tile bt, i-tile bc) of
    // K K^T and K Q^T, laid out so each lane holds 4 consecutive i of one row
    // t; per v-head, A (fp32) into its LDS block and P (hi/lo) to the
    // workspace with 8-byte stores.  A wave's next full tile's q loads go out
    // as soon as this tile's products have read its q.
    ChunkRec *rec0 = recs + (int64_t)gch * HV + h0;
    const bool half_kk = w == HKK || w == HKK + 1, half_kq = w == HKQ || w == HKQ + 1;
    auto tile = [&](int b) {
        f32x4 kk, kq, hk_, hq_;
        tile_products<VPW, true, true>(sm, b, bq, lane, kk, kq);
        // a half of tile 8 or 9 after the wave's last whole tile: its
        // products now, with this tile's (the Q K^T half uses the same q
        // fragments: this tile is of t-tile 3 too)
        const bool last = b + NW >= 8;
        if (last && half_kk) tile_products<VPW, true, false>(sm, 8 + (w - HKK), bq, lane, hk_, hq_);
        if (last && half_kq) tile_products<VPW, false, true>(sm, 8 + (w - HKQ), bq, lane, hk_, hq_);
        if (!last) {
            int nbt, nbc;
            tile_of(b + NW, nbt, nbc);
            load_qfrag(bq, a, t0, n, hk, nbt, lr, lq);
        }
        tile_elements<VPW, true, true>(sm, a, rec0, b, lane, kk, kq);
        if (last && half_kk) tile_elements<VPW, true, false>(sm, a, rec0, 8 + (w - HKK), lane, hk_, hq_);
        if (last && half_kq) tile_elements<VPW, false, true>(sm, a, rec0, 8 + (w - HKQ), lane, hk_, hq_);
    };
    // With eight waves each has exactly one whole tile, written without a
    // loop: a loop the compiler cannot prove runs makes it count the q
    // fragment loads as possibly outstanding after it, and it then waits for
    // every memory operation, this stage's record stores included, before
    // it reuses their registers.
    if constexpr (NW == 8) {
        tile(w);
    } else {
        for (int b = w; b < 8; b += NW) tile(b);
    }
    __syncthreads();

    // ---- stage 2: per v-head v (waves 4 v .. 4 v + 3), T = (I + A)^-1 block
    // by block (T overwrites the k rows)
    {
        const int v = w >> 2, wb = w & 3;
        ChunkRec *rec = recs + (int64_t)gch * HV + h0 + v;
        {
            // diagonal block wb by forward substitution on all 64 lanes: lane
            // (j, g) = (lane % 16, lane / 16) owns rows 4 g .. 4 g + 3 of
            // column j.  Row group p becomes final in phase p: its lanes take
            // the terms of their own group's earlier rows, then hand the four
            // final values to the later groups (an LDS permute), which take
            // the group's terms.  Every element gets the terms of rows
            // 0, 1, 2, ... in that order, each as one fused multiply-add:
            // the same operations as a sweep of one lane per column.
            const Blk &Ad = sm.A[v][blk(wb, wb)];
            const int j = lane & 15, g = lane >> 4;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = 4 * g + e == j ? 1.f : 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // this phase's coefficients of the lane's rows, A[4 g + e][4 p .. 4 p + 3]
                // (read whatever g is, so the reads need not wait for the permute)
                f32x4 ap[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ap[e] = *reinterpret_cast<const f32x4 *>(&Ad[4 * g + e][4 * p]);
                if (g == p) {
#pragma unroll
                    for (int e = 1; e < 4; ++e)
#pragma unroll
                        for (int f = 0; f < e; ++f) x[e] = __builtin_fmaf(-ap[e][f], x[f], x[e]);
                }
                if (p == 3) break;
                float xp[4];
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    xp[f] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (j + 16 * p),
                                                                                  __builtin_bit_cast(int, x[f])));
                if (g > p) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int f = 0; f < 4; ++f) x[e] = __builtin_fmaf(-ap[e][f], xp[f], x[e]);
                }
            }
            Blk &Td = sm.u.T[v][blk(wb, wb)];
#pragma unroll
            for (int e = 0; e < 4; ++e) Td[4 * g + e][j] = x[e];
        }
        __syncthreads();
        store_tblock(sm.u.T[v][blk(wb, wb)], rec, blk(wb, wb), lane);
        // The off-diagonal blocks as 2 x 2 block inverses of the 32 x 32
        // halves T1 = (T00, T10, T11) and T2 = (T22, T32, T33), then the
        // lower-left half -T2 A21 T1 (A21 = A20, A21, A30, A31):
        //   level 1: T10 = -T11 A10 T00 (wave 0), T32 = -T33 A32 T22 (wave 1);
        //            meanwhile waves 2 and 3 (b = 2, 3) form the parts of
        //            X_b0 = A_b0 T00 + A_b1 T10 and X_b1 = A_b1 T11 that need
        //            no level-1 block: A_b0 T00 and X_b1
        //   level 2: X_b0 += A_b1 T10 (waves 2, 3); X written over A21
        //   level 3: T20 = -T22 X20, T21 = -T22 X21, T30 = -(T32 X20 + T33 X30),
        //            T31 = -(T32 X21 + T33 X31), one block per wave
        // Every product is a 16 x 16 fp32 block product on the matrix cores,
        // each block's terms summed in the same order as a block-column walk;
        // the longest chain is five of them.
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};   // waves 2, 3: X_b0, X_b1
        if (wb < 2) {
            const int b = wb == 0 ? 1 : 3, c = b - 1;       // T10 or T32
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            m = mm16(sm.A[v][blk(b, c)], sm.u.T[v][blk(c, c)], m, lane);
            put16(sm.u.T[v][blk(b, c)], m, 1.f, lane);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sm.u.T[v][blk(b, b)], sm.u.T[v][blk(b, c)], t, lane);
            put16(sm.u.T[v][blk(b, c)], t, -1.f, lane);
            store_tblock(sm.u.T[v][blk(b, c)], rec, blk(b, c), lane);
        } else {
            x0 = mm16(sm.A[v][blk(wb, 0)], sm.u.T[v][blk(0, 0)], x0, lane);
            x1 = mm16(sm.A[v][blk(wb, 1)], sm.u.T[v][blk(1, 1)], x1, lane);
        }
        __syncthreads();                                     // T10 final
        if (wb >= 2) x0 = mm16(sm.A[v][blk(wb, 1)], sm.u.T[v][blk(1, 0)], x0, lane);
        __syncthreads();                                     // every A_b0, A_b1 read before any is overwritten
        if (wb >= 2) {
            put16(sm.A[v][blk(wb, 0)], x0, 1.f, lane);
            put16(sm.A[v][blk(wb, 1)], x1, 1.f, lane);
        }
        __syncthreads();
        const int xb = 2 + (wb >> 1), xc = wb & 1;          // this wave's block (xb, xc) of the lower-left half
        {
            // T_bc = -(T_b2 X_2c + T_b3 X_3c) (T_23 = 0)
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sm.u.T[v][blk(xb, 2)], sm.A[v][blk(2, xc)], t, lane);
            if (xb == 3) t = mm16(sm.u.T[v][blk(3, 3)], sm.A[v][blk(3, xc)], t, lane);
            put16(sm.u.T[v][blk(xb, xc)], t, -1.f, lane);
            store_tblock(sm.u.T[v][blk(xb, xc)], rec, blk(xb, xc), lane);
        }
    }
}
// ---------------------------------------------------------------------------
// scan, row-split form: one workgroup per (sequence, v-head, 16 NW v rows),
// wave w owning 16 v rows with the whole chain of a chunk in its registers
// ---------------------------------------------------------------------------
// Every product of a chunk is a product of an operand shared by the whole
// workgroup (K, Q, K^T, T, P: the chunk's, staged once in LDS) with a
// wave-private one (the wave's state rows, then R, U, U' of its rows):
//   Y_k = K S_w^T, Y_q = Q S_w^T         (64 tokens x 16 rows, over 128 dims)
//   R = b v - bgr Y_k,  U = T R,  o = sqg Y_q + P U,
//   S_w^T <- G_C S_w^T + K^T (u2f U)     (128 dims x 16 rows, over 64 tokens)
// The wave-private operand is always the B side, taken straight from the
// previous product's accumulators: an accumulator tile gives lane l the
// elements (4 (l / 16) + i, l % 16), i < 4, so two tiles stacked along the
// contraction index give lane l the contraction positions 4 (l / 16) + i and
// 16 + 4 (l / 16) + i of a 32-wide block.  The shared A side is read from LDS
// with the same positions (one 16-byte read per fragment, below), so no
// accumulator ever goes through LDS and no barrier separates the phases.
// The waves meet twice per chunk, to restage the next chunk's operands
// (prefetched into registers while the current chunk runs).
// Within every 32-column block of a staged A-side tile the columns are
// stored permuted, so that the eight columns a lane group g takes (4 g .. 4 g
// + 3 and 16 + 4 g .. 16 + 4 g + 3) sit side by side at 8 g .. 8 g + 7: a
// fragment is one aligned 16-byte read.  Column c of a block is stored at
// 8 ((c % 16) / 4) + 4 (c / 16) + c % 4; eight consecutive columns 8 h .. 8 h
// + 7 (h < 4) therefore land as two 4-column halves at pstart(8 h) and
// pstart(8 h) + 8.  Rows padded by 8 bf16 (16 bytes): eight consecutive rows
// of a 16-byte fragment read then fall on eight different 16-byte bank
// groups (row pitch = 16 mod 128 bytes).
constexpr int RLDK = DKC + 8;
constexpr int RLDT = CT + 8;
__device__ __forceinline__ int pstart(int c8) {       // c8: first column of 8, a multiple of 8
    return (c8 & ~31) + 16 * ((c8 >> 3) & 1) + 4 * ((c8 >> 4) & 1);
}
template <int NW>
struct RowScanSmem {
    alignas(16) __bf16 K[CT][RLDK];                  // [t][d]; also read transposed as K^T
    alignas(16) __bf16 Q[CT][RLDK];
    alignas(16) __bf16 Th[CT][RLDT];                 // [t][i]
    alignas(16) __bf16 Tl[CT][RLDT];
    alignas(16) __bf16 Ph[CT][RLDT];
    alignas(16) __bf16 Pl[CT][RLDT];
    // [t][r], this workgroup's rows.  The 64-row form's LDS (~82 KB) keeps one
    // workgroup per CU: with rows padded by 4 instead of 8 it fits in 80 KB,
    // and in the mixed-step grid decode units then share CUs with scan
    // workgroups, which made the grid ~3% slower (their memory traffic slows
    // the scan's operand fetches; a higher wave priority for the scan did not
    // help).
    alignas(16) __bf16 V[CT][16 * NW + 8];
    alignas(16) float sc[5][CT];                     // beta, bgr, sqg, u2f, G_C
};

// A-side fragment whose contraction positions follow two stacked
// accumulator tiles: element e of lane l is (row r0 + l % 16, column
// k0 + 4 (l / 16) + e) for e < 4 and column k0 + 16 + 4 (l / 16) + e - 4 for
// e >= 4 -- in the permuted block layout, the 8 elements from k0 + 8 (l / 16)
__device__ __forceinline__ bf16x8 afrag(const __bf16 *base, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// The same A-side fragment of K^T (rows d0 .. d0 + 15, contraction over the
// tokens t0 + 4 (l / 16) + e and t0 + 16 + 4 (l / 16) + e - 4), read straight
// from the staged K tile [t][d] with two gfx950 LDS transpose reads
// (ds_read_b64_tr_b16).  Within each group of 16 lanes such a read gives
// lane j, as its element e, element j % 4 of the 8-byte piece whose address
// lane 4 e + j / 4 of the group supplies (checked on the GPU with an
// in-bounds probe).  So lane 4 e + q of group g points at the four
// consecutive d0 + 4 q .. d0 + 4 q + 3 of token row t0 + 4 g + e; four
// consecutive columns stay contiguous in the permuted block layout.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 ktfrag(const __bf16 *K, int d0, int t0, int lane) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int d = d0 + 4 * q;                            // a multiple of 4
    const int col = (d & ~31) + 8 * ((d >> 2) & 3) + 4 * ((d >> 4) & 1);
    const __bf16 *p = K + (t0 + 4 * g + e) * RLDK + col;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + 16 * RLDK));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// B-side fragment (hi and lo bf16 parts) from two accumulator tiles stacked
// along the contraction index
__device__ __forceinline__ void bsplit(const f32x4 &x0, const f32x4 &x1, bf16x8 &hi, bf16x8 &lo) {
    bf16x4 h0, l0, h1, l1;
    split4(x0, h0, l0);
    split4(x1, h1, l1);
    hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int NW>
struct RowStage {
    static constexpr int NT = 64 * NW, DVB = 16 * NW;
    static constexpr int NK = CT * DKC / 8 / NT;          // K (and Q) vectors per thread
    static constexpr int NTP = 4 * NBLK16 * 32 / NT;      // 16-byte pieces of the T and P blocks per thread
    static constexpr int NV = CT * DVB / 8 / NT;          // v vectors per thread
    uint4 k[NK], q[NK];
    uint4 tp[NTP];
    uint4 v[NV];
    uint4 sc;                                          // threads < 80: 4 scalars of one of 5 arrays
};

// One scan workgroup's work: the 16 NW v rows from 16 NW vb of one
// (sequence s, v-head h), work = (h num_seqs + s) n_vblocks + vb, through that
// sequence's chunks (head-major, like the prep's order, so an XCD scans the
// v-heads whose records it prepared).  Called by all 64 NW threads of a workgroup; sm is the
// workgroup's LDS.  Each kernel inlines its own instance (TAG): with one
// instance shared by two kernels, hipcc 7.2 scheduled the scan kernel's loop
// with 26 more AGPR moves.
template <int NW, int TAG = 0>
__device__ __forceinline__ void scan_rows_unit(const RecurrentArgs &a, const ChunkRec *recs,
                                               int n_vblocks, int work, RowScanSmem<NW> &sm) {
    using St = RowStage<NW>;
    constexpr int NT = St::NT, DVB = St::DVB;
    const int HV = a.num_v_heads;
    const int vb = work % n_vblocks;
    const int sh = work / n_vblocks;
    const int s = sh % a.num_seqs;
    const int h = sh / a.num_seqs;
    const int slot = a.state_indices[s];
    if ((unsigned)slot >= (unsigned)a.num_slots) return;   // padding, or outside the pool
    int t_begin, t_end;
    clamp_range(a.qsl[s], a.qsl[s + 1], a.num_tokens, t_begin, t_end);
    if (t_end <= t_begin) return;
    const int hk = h / (HV / a.num_k_heads);
    const int gch0 = chunks_before(a.qsl, s, a.num_tokens);
    // the records of the sequence's chunks lie within the workspace (always,
    // for a well-formed query_start_loc)
    if (gch0 + chunk_count(t_end - t_begin) > (a.num_tokens + CT - 1) / CT + a.num_seqs) return;

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, g = lane >> 4;
    const int r0 = vb * DVB;                         // the workgroup's first v row
    const int rw = 16 * w + lr;                      // this lane's v row within the workgroup

    // the wave's state rows as the accumulator tiles of S_w^T: tile dt,
    // lane holds S[r0 + rw][16 dt + 4 g + i]
    float *S_g = a.state + (((int64_t)slot * HV + h) * a.dv + r0 + rw) * DKC + 4 * g;
    f32x4 S[8];
    const bool init = a.has_init == nullptr || a.has_init[s] != 0;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        S[dt] = init ? load_stream4(S_g + 16 * dt) : z;
    }

    // the operands of a chunk, global -> registers, in four parts issued at
    // the start of the four phases of the chunk before: all at once they
    // filled the memory pipeline and held the wave at the issue for ~2,000
    // cycles.  Rows past the chunk end read its last token again (finite
    // values, not zeroed): the prep gives a padded token beta = bgr = 0 and a
    // zero gate, so its R, U and U' are exactly zero, the K^T column it adds
    // to the state update (the repeated token's k) multiplies zeros, and its
    // Y rows, computed from the repeated token, are never used.
    auto fetch_kq = [&](St &st, int t0, int n) {
#pragma unroll
        for (int j = 0; j < St::NK; ++j) {
            const int idx = tid + NT * j, t = idx >> 4, c = (idx & 15) * 8;
            const int64_t row = t0 + min(t, n - 1);
            st.k[j] = *reinterpret_cast<const uint4 *>(a.k + row * a.k_stride + hk * DKC + c);
            st.q[j] = *reinterpret_cast<const uint4 *>(a.q + row * a.q_stride + hk * DKC + c);
        }
    };
    // T and P: the record's ten blocks of each of the four matrices are
    // 1280 consecutive 16-byte pieces
    auto fetch_t = [&](St &st, int gch) {
        const uint4 *src = reinterpret_cast<const uint4 *>(&recs[(int64_t)gch * HV + h].TP[0][0][0][0]);
#pragma unroll
        for (int j = 0; j < St::NTP; ++j) st.tp[j] = src[tid + NT * j];
    };
    auto fetch_pv = [&](St &st, int t0, int n, int gch) {
        const ChunkRec *rec = recs + (int64_t)gch * HV + h;
#pragma unroll
        for (int j = 0; j < St::NV; ++j) {
            const int idx = tid + NT * j, t = idx / (DVB / 8), c = (idx % (DVB / 8)) * 8;
            st.v[j] = *reinterpret_cast<const uint4 *>(a.v + (int64_t)(t0 + min(t, n - 1)) * a.v_stride +
                                                       (int64_t)h * a.dv + r0 + c);
        }
        // beta, bgr, sqg, u2f, G_C: 5 x 64 consecutive floats of the record
        st.sc = *reinterpret_cast<const uint4 *>(&rec->beta[0] + 4 * min(tid, 79));
    };
    // 8 consecutive columns c8 .. c8 + 7 of a row: two 4-column halves, 8
    // positions apart in the permuted block layout
    auto st16 = [](__bf16 *row, int c8, const uint4 &v) {
        __bf16 *p = row + pstart(c8);
        *reinterpret_cast<uint2 *>(p) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2 *>(p + 8) = make_uint2(v.z, v.w);
    };
    auto stage = [&](const St &st) {
#pragma unroll
        for (int j = 0; j < St::NK; ++j) {
            const int idx = tid + NT * j, t = idx >> 4, c = (idx & 15) * 8;
            st16(sm.K[t], c, st.k[j]);
            st16(sm.Q[t], c, st.q[j]);
        }
#pragma unroll
        for (int j = 0; j < St::NTP; ++j) {
            // piece p: matrix m, block (bt, bc), row r, half hf
            const int p = tid + NT * j, m = p / (NBLK16 * 32), q = p - m * (NBLK16 * 32);
            const int b = q >> 5, r = (q >> 1) & 15, hf = q & 1;
            const int bt = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3, bc = b - bt * (bt + 1) / 2;
            st16(&sm.Th[0][0] + m * (CT * RLDT) + (16 * bt + r) * RLDT, 16 * bc + 8 * hf, st.tp[j]);
        }
#pragma unroll
        for (int j = 0; j < St::NV; ++j) {
            const int idx = tid + NT * j, t = idx / (DVB / 8), c = (idx % (DVB / 8)) * 8;
            *reinterpret_cast<uint4 *>(&sm.V[t][c]) = st.v[j];
        }
        if (tid < 80) *reinterpret_cast<uint4 *>(&sm.sc[0][0] + 4 * tid) = st.sc;
    };

    const int o_col_bytes = 2 * (h * a.dv + r0 + rw);
    const int o_row_bytes = 2 * (int)a.o_stride;

    // the blocks above T's and P's diagonal blocks that the products read,
    // (0, 1) and (2, 3), are zero; the restaging never writes them
    for (int e = tid; e < 4 * 2 * 16 * 2; e += NT) {
        const int m = e >> 6, z = (e >> 5) & 1, r = (e >> 1) & 15, hf = e & 1;
        st16(&sm.Th[0][0] + m * (CT * RLDT) + (16 * (2 * z) + r) * RLDT, 16 * (2 * z + 1) + 8 * hf,
             make_uint4(0, 0, 0, 0));
    }
    St st;
    {
        const int n0 = min(CT, t_end - t_begin);
        fetch_kq(st, t_begin, n0);
        fetch_t(st, gch0);
        fetch_pv(st, t_begin, n0, gch0);
    }
    stage(st);
    __syncthreads();

    int gch = gch0;
    for (int t0 = t_begin; t0 < t_end; t0 += CT, ++gch) {
        const int n = min(CT, t_end - t0);
        // the next chunk's operands; the last chunk fetches its own again
        // (in bounds, and unconditional: a load behind a branch would make
        // the compiler wait for it where the paths merge, before this chunk)
        const bool more = t0 + CT < t_end;
        const int t_next = more ? t0 + CT : t0, n_next = min(CT, t_end - t_next);
        const int g_next = more ? gch + 1 : gch;
        fetch_kq(st, t_next, n_next);

        // ---- Y_k = K S_w^T, Y_q = Q S_w^T (token tiles tt)
        f32x4 yk[4], yq[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) yk[tt] = yq[tt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            bf16x8 bh, bl;
            bsplit(S[2 * kb], S[2 * kb + 1], bh, bl);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const bf16x8 ka = afrag(&sm.K[0][0], RLDK, 16 * tt, 32 * kb, lane);
                const bf16x8 qa = afrag(&sm.Q[0][0], RLDK, 16 * tt, 32 * kb, lane);
                yk[tt] = mma(ka, bh, yk[tt]);
                yq[tt] = mma(qa, bh, yq[tt]);
                yk[tt] = mma(ka, bl, yk[tt]);
                yq[tt] = mma(qa, bl, yq[tt]);
            }
        }
        // ---- R = b v - bgr Y_k; the o part sqg Y_q
        f32x4 R[4], O[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t4 = 16 * tt + 4 * g;
            const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sm.sc[0][t4]);
            const f32x4 bgr4 = *reinterpret_cast<const f32x4 *>(&sm.sc[1][t4]);
            const f32x4 sqg4 = *reinterpret_cast<const f32x4 *>(&sm.sc[2][t4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vv = bf16_to_f32(__builtin_bit_cast(uint16_t, sm.V[t4 + i][rw]));
                R[tt][i] = b4[i] * vv - bgr4[i] * yk[tt][i];
                O[tt][i] = sqg4[i] * yq[tt][i];
            }
        }
        // ---- U = T R (T lower triangular: token tile tt needs blocks ib <= tt / 2); U' = u2f U
        f32x4 U[4], U2[4];
        {
            bf16x8 rh[2], rl[2];
            bsplit(R[0], R[1], rh[0], rl[0]);
            bsplit(R[2], R[3], rh[1], rl[1]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ib = 0; ib <= tt / 2; ++ib) {
                    const bf16x8 th = afrag(&sm.Th[0][0], RLDT, 16 * tt, 32 * ib, lane);
                    const bf16x8 tl = afrag(&sm.Tl[0][0], RLDT, 16 * tt, 32 * ib, lane);
                    u = mma(th, rh[ib], u);
                    u = mma(th, rl[ib], u);
                    u = mma(tl, rh[ib], u);
                }
                U[tt] = u;
                const f32x4 u2f4 = *reinterpret_cast<const f32x4 *>(&sm.sc[3][16 * tt + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) U2[tt][i] = u2f4[i] * u[i];
            }
        }
        // ---- o = sqg Y_q + P U -> output (rows past the chunk end fall
        // outside the buffer range, so the hardware drops their stores)
        fetch_t(st, g_next);
        {
            const int o_range = n * o_row_bytes;
            const __amdgpu_buffer_rsrc_t o_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                a.o + (int64_t)t0 * a.o_stride, (short)0, o_range, kBufferFlags);
            bf16x8 uh[2], ul[2];
            bsplit(U[0], U[1], uh[0], ul[0]);
            bsplit(U[2], U[3], uh[1], ul[1]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 acc = O[tt];
#pragma unroll
                for (int ib = 0; ib <= tt / 2; ++ib) {
                    const bf16x8 ph = afrag(&sm.Ph[0][0], RLDT, 16 * tt, 32 * ib, lane);
                    const bf16x8 pl = afrag(&sm.Pl[0][0], RLDT, 16 * tt, 32 * ib, lane);
                    acc = mma(ph, uh[ib], acc);
                    acc = mma(ph, ul[ib], acc);
                    acc = mma(pl, uh[ib], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[i]), o_rsrc,
                                                          (16 * tt + 4 * g + i) * o_row_bytes + o_col_bytes, 0, 0);
            }
        }
        // ---- S_w^T = G_C S_w^T + K^T U'
        fetch_pv(st, t_next, n_next, g_next);
        {
            const float g_c = sm.sc[4][0];
            bf16x8 vh[2], vl[2];
            bsplit(U2[0], U2[1], vh[0], vl[0]);
            bsplit(U2[2], U2[3], vh[1], vl[1]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                f32x4 acc = S[dt] * g_c;
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const bf16x8 ka = ktfrag(&sm.K[0][0], 16 * dt, 32 * tb, lane);
                    acc = mma(ka, vh[tb], acc);
                    acc = mma(ka, vl[tb], acc);
                }
                S[dt] = acc;
            }
        }
        if (!more) break;
        __syncthreads();                 // every wave is done with this chunk's operands
        stage(st);
        __syncthreads();
    }

#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_stream4(S_g + 16 * dt, S[dt]);
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void chunk_scan_rows_kernel(RecurrentArgs a, const ChunkRec *recs,
                                                                     int n_vblocks) {
    __shared__ RowScanSmem<NW> sm;
    scan_rows_unit<NW>(a, recs, n_vblocks, xcd_contiguous(blockIdx.x, gridDim.x), sm);
}

// The scan and a batch of fused decode units (fused_unit.h) in one grid, for
// an engine step that holds both prefill chunks and decode rows.  Blocks
// [0, n_scan_pad) are scan workgroups (n_scan_pad: the scan's count rounded
// up to a multiple of the XCD count; the extra ones exit at once), the rest
// decode units.  Workgroups are dispatched in block order, so the scan --
// the step's long serial chain -- starts first on as many CUs as it has
// workgroups; the decode units fill the other CUs and then each CU a scan
// workgroup releases.  Each role runs its own kernel's code on its own
// operands, so results are bit-identical to the two launches.  The kernel
// has the scan's LDS and registers, so a CU holds one decode unit at a time
// where the decode kernel fits two.
constexpr int kMixedThreads = 256;
static_assert(kFusedThreads == kMixedThreads, "decode units and 64-row scan workgroups are both 4 waves");
static_assert(sizeof(RowScanSmem<4>) >= fused_unit_lds_bytes(0, kMaxGroupChannels / 8, 8),
              "a decode unit's conv output, decays and betas fit in the scan's LDS");

__global__ __launch_bounds__(kMixedThreads, 1) void chunk_scan_decode_kernel(RecurrentArgs a, const ChunkRec *recs,
                                                                           int n_vblocks,
                                                                           int n_scan, int n_scan_pad,
                                                                           FusedDecodeArgs f, int n_dec) {
    __shared__ RowScanSmem<4> sm;
    const int bid = blockIdx.x;
    if (bid < n_scan_pad) {
        if (bid < n_scan) scan_rows_unit<4, 1>(a, recs, n_vblocks, xcd_contiguous(bid, n_scan), sm);
    } else {
        // n_scan_pad is a multiple of the XCD count: bid - n_scan_pad stays on bid's XCD
        // a unit runs alone on its CU here: the latency form when the group is one full pass
        const int unit = xcd_contiguous(bid - n_scan_pad, n_dec);
        if (fused_unit_full<DKC>(f.num_v_heads / f.num_k_heads * f.dv))
            fused_decode_unit<DKC, kFusedRows, true>(f, unit, reinterpret_cast<uint16_t *>(&sm));
        else
            fused_decode_unit<DKC, kFusedRows, false>(f, unit, reinterpret_cast<uint16_t *>(&sm));
    }
}

}  // namespace

int64_t chunk_max_chunks(int num_seqs, int num_tokens) {
    return (int64_t)(num_tokens + CT - 1) / CT + num_seqs;
}

int64_t chunk_workspace_bytes(int num_seqs, int num_tokens, int num_k_heads, int num_v_heads) {
    const int64_t mc = chunk_max_chunks(num_seqs, num_tokens);
    (void)num_k_heads;
    return mc * (int64_t)num_v_heads * (int64_t)sizeof(ChunkRec);
}

namespace {

struct ChunkLaunch {
    ChunkRec *recs;
    long long prep_blocks, scan_blocks;
    int nvb;
    bool wide;
};

ChunkLaunch chunk_launch(const RecurrentArgs &a, void *workspace, int num_tokens) {
    ChunkLaunch c;
    const int64_t mc = chunk_max_chunks(a.num_seqs, num_tokens);
    c.recs = reinterpret_cast<ChunkRec *>(workspace);
    c.prep_blocks = mc * a.num_v_heads;
    // 64 v rows (four waves) per workgroup whenever head_v_dim allows: each
    // chunk's operands then serve twice the rows, which measured faster at
    // every prefill shape tried (one to three sequences, 500 to 2048 tokens),
    // even where 32-row workgroups would have used twice the CUs
    c.wide = (a.dv % 64) == 0;
    c.nvb = a.dv / (c.wide ? 64 : 32);
    c.scan_blocks = (long long)a.num_seqs * a.num_v_heads * c.nvb;
    return c;
}

hipError_t launch_prep(const RecurrentArgs &a, const ChunkLaunch &c, hipStream_t stream) {
    // two v-heads per prep workgroup whenever the v-heads of a q/k head pair up
    if ((a.num_v_heads / a.num_k_heads) % 2 == 0)
        hipLaunchKernelGGL(chunk_prep_kernel<2>, dim3((unsigned)(c.prep_blocks / 2)), dim3(2 * NTH), 0, stream, a.qsl,
                           a.k, a.q, a.k_stride, a.q_stride, a.num_seqs, a.num_tokens, a.num_v_heads,
                           (int)(c.prep_blocks / 2), a, c.recs);
    else
        hipLaunchKernelGGL(chunk_prep_kernel<1>, dim3((unsigned)c.prep_blocks), dim3(NTH), 0, stream, a.qsl, a.k, a.q,
                           a.k_stride, a.q_stride, a.num_seqs, a.num_tokens, a.num_v_heads, (int)c.prep_blocks, a,
                           c.recs);
    return hipGetLastError();
}

hipError_t launch_scan(const RecurrentArgs &a, const ChunkLaunch &c, hipStream_t stream) {
    if (c.wide)
        hipLaunchKernelGGL(chunk_scan_rows_kernel<4>, dim3((unsigned)c.scan_blocks), dim3(256), 0, stream, a, c.recs,
                           c.nvb);
    else
        hipLaunchKernelGGL(chunk_scan_rows_kernel<2>, dim3((unsigned)c.scan_blocks), dim3(128), 0, stream, a, c.recs,
                           c.nvb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_recurrent(const RecurrentArgs &a, void *workspace, int num_tokens, hipStream_t stream) {
    const ChunkLaunch c = chunk_launch(a, workspace, num_tokens);
    if (c.scan_blocks == 0) return hipSuccess;
    if (c.prep_blocks > 0x7fffffffLL || c.scan_blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e = launch_prep(a, c, stream);
    if (e != hipSuccess) return e;
    return launch_scan(a, c, stream);
}

hipError_t launch_chunk_and_decode(const RecurrentArgs &a, void *workspace, int num_tokens,
                                   const FusedDecodeArgs &f, hipStream_t stream) {
    const ChunkLaunch c = chunk_launch(a, workspace, num_tokens);
    const long long n_dec = (long long)f.batch * f.num_k_heads;
    if (c.scan_blocks == 0) return launch_fused_conv_decode(f, stream);
    if (n_dec == 0) return launch_chunk_recurrent(a, workspace, num_tokens, stream);
    const long long n_scan_pad = (c.scan_blocks + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (c.prep_blocks > 0x7fffffffLL || n_scan_pad + n_dec > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e = launch_prep(a, c, stream);
    if (e != hipSuccess) return e;
    // one grid where the scan runs in 64-row workgroups and the decode in
    // 128-wide rows; other shapes take the two launches
    if (!c.wide || f.dk != DKC) {
        e = launch_scan(a, c, stream);
        if (e != hipSuccess) return e;
        return launch_fused_conv_decode(f, stream);
    }
    hipLaunchKernelGGL(chunk_scan_decode_kernel, dim3((unsigned)(n_scan_pad + n_dec)), dim3(kMixedThreads), 0, stream,
                       a, c.recs, c.nvb, (int)c.scan_blocks, (int)n_scan_pad, f, (int)n_dec);
    return hipGetLastError();
}

}  // namespace gdn
