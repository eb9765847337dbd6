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
// so a chunk costs a handful of dense products (K K^T, Q K^T, [K;Q] S0^T,
// T R, P U, U^T K) plus the inverse T = (I + A)^-1 of a unit lower-triangular
// C x C matrix, instead of C dependent rank-1 steps.
//
// Work split: one workgroup (4 waves) per (sequence, v-head, block of 32 v
// rows); it walks its sequence chunk by chunk (C = 64) holding its 32 x 128
// slice of the fp32 state in VGPRs (the MFMA accumulator layout).  v rows are
// independent in every product, so blocks need no communication.  K/Q are
// shared by the 8 workgroups of one q/k head; the XCD-contiguous block order
// keeps them on one XCD's L2.
//
// Precision: products of raw bf16 inputs (K K^T, Q K^T) are exact in the
// bf16 MFMA with fp32 accumulation.  Every product with an fp32 operand (the
// state, T, P, U, R) splits that operand into hi + lo bf16 parts (16
// significant bits) and sums the partial products, so the state keeps close
// to fp32 accuracy.  The inverse T is computed in fp32 (diagonal 16 x 16
// blocks by substitution, off-diagonal blocks with fp32 MFMA).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CT = 64;          // tokens per chunk
constexpr int DKC = 128;        // head_k_dim
constexpr int DVB = 32;         // v rows per workgroup
constexpr int NTH = 256;        // 4 waves
constexpr int LDK = DKC + 8;    // padded row (bf16 elements) of a [*][128] tile
constexpr int LDT = CT + 8;     // padded row (bf16 elements) of a [*][64] tile
constexpr int LDF = CT + 4;     // padded row (fp32) of a [64][64] fp32 tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Smem {
    __bf16 K[CT][LDK];          // raw k rows of the chunk, [t][d]
    __bf16 Q[CT][LDK];          // raw q rows, [t][d]
    __bf16 Kt[DKC][LDT];        // k transposed, [d][t]
    __bf16 Shi[DVB][LDK];       // state slice S0 [r][d], hi part
    __bf16 Slo[DVB][LDK];       //                      lo part
    __bf16 Thi[CT][LDT];        // T = (I + A)^-1, [t][i]
    __bf16 Tlo[CT][LDT];
    __bf16 Phi[CT][LDT];        // P = scale exp(L_t - L_i) (qh_t . kh_i), i <= t
    __bf16 Plo[CT][LDT];
    __bf16 Rhi[DVB][LDT];       // R transposed, [r][t]
    __bf16 Rlo[DVB][LDT];
    union {
        struct {
            __bf16 Uhi[DVB][LDT];   // U transposed, [r][t]
            __bf16 Ulo[DVB][LDT];
            __bf16 U2hi[DVB][LDT];  // exp(L_C - L_t) rk_t U, transposed
            __bf16 U2lo[DVB][LDT];
        } u;
        float Tf[CT][LDF];          // fp32 T while it is being built
    } x;
    float A[CT][LDF];           // strictly lower A, fp32
    float lam[CT], gam[CT], beta[CT], rk[CT], rq[CT];
};

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

// fp32 16x16x16 product C += X Y with X = rows of an fp32 LDS tile at
// (xr, xc), Y = fp32 LDS tile at (yr, yc); four 16x16x4 fp32 MFMAs
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

// write a 16x16 C tile (MFMA accumulator layout) into an fp32 LDS tile
__device__ __forceinline__ void put16(float (*Z)[LDF], int zr, int zc, const f32x4 &c, float sgn, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Z[zr + 4 * (lane >> 4) + i][zc + (lane & 15)] = sgn * c[i];
}

__global__ __launch_bounds__(NTH) void chunk_gdr_kernel(RecurrentArgs a, int n_vblocks) {
    __shared__ Smem sm;

    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int vb = work % n_vblocks;
    const int sh = work / n_vblocks;
    const int h = sh % a.num_v_heads;
    const int s = sh / a.num_v_heads;
    const int slot = a.state_indices[s];
    if (slot < 0) return;
    const int t_begin = a.qsl[s];
    const int t_end = a.qsl[s + 1];
    if (t_end <= t_begin) return;
    const int HV = a.num_v_heads;
    const int hk = h / (HV / a.num_k_heads);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;          // wave: owns token tile w and state column tiles 2w, 2w+1
    const int lr = lane & 15;        // accumulator column within a tile
    const int lq = lane >> 4;        // accumulator row group within a tile

    // state slice in the accumulator layout: tile q = 2*rt + (dt - 2w),
    // element i -> row 16 rt + 4 lq + i, column 16 dt + lr
    float *S_g = a.state + ((int64_t)slot * HV + h) * (int64_t)a.dv * DKC + (int64_t)vb * DVB * DKC;
    f32x4 S[4];
    const bool init = a.has_init == nullptr || a.has_init[s] != 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rt = q >> 1, dt = 2 * w + (q & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[q][i] = init ? S_g[(16 * rt + 4 * lq + i) * DKC + 16 * dt + lr] : 0.f;
    }

    const float scale = a.scale;
    for (int t0 = t_begin; t0 < t_end; t0 += CT) {
        const int n = min(CT, t_end - t0);

        // ---- stage 0: chunk inputs into LDS, norms, cumulative decay
        {
            const int tok = tid >> 2, part = tid & 3;   // 4 lanes per token, 32 dims each
            uint4 kv[4], qv[4];
            if (tok < n) {
                const uint4 *kp = reinterpret_cast<const uint4 *>(a.k + (int64_t)(t0 + tok) * a.k_stride +
                                                                  hk * DKC + 32 * part);
                const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + (int64_t)(t0 + tok) * a.q_stride +
                                                                  hk * DKC + 32 * part);
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
                *reinterpret_cast<uint4 *>(&sm.K[tok][32 * part + 8 * m]) = kv[m];
                *reinterpret_cast<uint4 *>(&sm.Q[tok][32 * part + 8 * m]) = qv[m];
                float kf[8], qf[8];
                unpack8(kv[m], kf);
                unpack8(qv[m], qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    skk = __builtin_fmaf(kf[e], kf[e], skk);
                    sqq = __builtin_fmaf(qf[e], qf[e], sqq);
                    sm.Kt[32 * part + 8 * m + e][tok] = (__bf16)kf[e];
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
                sm.gam[lane] = expf(gg);
                sm.beta[lane] = bb;
            }
            // the state slice entering the chunk, split for the MFMA operand
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
        }
        // v values of this lane's accumulator tiles (token tile w, v-row tiles 0, 1)
        float vv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * w + 4 * lq + i;
                vv[rt][i] = tt < n ? bf16_to_f32(a.v[(int64_t)(t0 + tt) * a.v_stride + (int64_t)h * a.dv +
                                                     vb * DVB + 16 * rt + lr])
                                   : 0.f;
            }
        __syncthreads();

        // ---- stage 1: K K^T, Q K^T -> A, P;  [K;Q] S0^T -> R, the S0 part of O
        f32x4 O[2];
        {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c > w) break;
                f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DKC / 32; ++ks) {
                    const bf16x8 ak = frag(&sm.K[0][0], LDK, 16 * w, 32 * ks, lane);
                    const bf16x8 aq = frag(&sm.Q[0][0], LDK, 16 * w, 32 * ks, lane);
                    const bf16x8 bk = frag(&sm.K[0][0], LDK, 16 * c, 32 * ks, lane);
                    kk = mma(ak, bk, kk);
                    qk = mma(aq, bk, qk);
                }
                const int ii = 16 * c + lr;
                const float lam_i = sm.lam[ii], rk_i = sm.rk[ii];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * w + 4 * lq + i;
                    const float decay = ii <= t ? expf(sm.lam[t] - lam_i) : 0.f;
                    sm.A[t][ii] = ii < t ? sm.beta[t] * sm.rk[t] * rk_i * decay * kk[i] : 0.f;
                    __bf16 hi, lo;
                    split(ii <= t ? scale * sm.rq[t] * rk_i * decay * qk[i] : 0.f, hi, lo);
                    sm.Phi[t][ii] = hi;
                    sm.Plo[t][ii] = lo;
                }
            }
            // zero the strictly upper tiles of P (read by the triangular products)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c <= w) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.Phi[16 * w + 4 * lq + i][16 * c + lr] = (__bf16)0.f;
                    sm.Plo[16 * w + 4 * lq + i][16 * c + lr] = (__bf16)0.f;
                }
            }
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
                    const float bt = sm.beta[t];
                    const float r = bt * vv[rt][i] - bt * sm.gam[t] * sm.rk[t] * yk[i];
                    __bf16 hi, lo;
                    split(r, hi, lo);
                    sm.Rhi[16 * rt + lr][t] = hi;
                    sm.Rlo[16 * rt + lr][t] = lo;
                    O[rt][i] = scale * sm.rq[t] * sm.gam[t] * yq[i];
                }
            }
        }
        __syncthreads();

        // ---- stage 2: T = (I + A)^-1 in fp32
        {
            float(*Tf)[LDF] = sm.x.Tf;
            float(*Am)[LDF] = sm.A;
            // diagonal blocks: wave w inverts block w by forward substitution,
            // lane j < 16 owns column j
            if (lane < 16) {
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
            // blocks above the diagonal are zero
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c <= w) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) Tf[16 * w + 4 * lq + i][16 * c + lr] = 0.f;
            }
            __syncthreads();
            // off-diagonal blocks T_bc = -T_bb (sum_{c<=m<b} A_bm T_mc), by
            // distance from the diagonal; wave 0: (1,0) (2,0) (3,0),
            // wave 1: (2,1) (3,1), wave 2: (3,2).  Each block's inputs come
            // from its own wave or from the diagonal.
            const int c = w;
            for (int b = c + 1; b < 4 && w < 3; ++b) {
                f32x4 m = {0.f, 0.f, 0.f, 0.f};
                for (int mm = c; mm < b; ++mm) m = mm16_f32(Am, 16 * b, 16 * mm, Tf, 16 * mm, 16 * c, m, lane);
                put16(Tf, 16 * b, 16 * c, m, 1.f, lane);      // park M in the target block
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
                t = mm16_f32(Tf, 16 * b, 16 * b, Tf, 16 * b, 16 * c, t, lane);
                put16(Tf, 16 * b, 16 * c, t, -1.f, lane);
            }
            __syncthreads();
            // fp32 -> hi/lo bf16 operand copies
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int idx = tid + NTH * e;       // 4096 entries
                const int t = idx >> 6, i = idx & 63;
                __bf16 hi, lo;
                split(Tf[t][i], hi, lo);
                sm.Thi[t][i] = hi;
                sm.Tlo[t][i] = lo;
            }
        }
        __syncthreads();

        // ---- stage 3: U = T R  (token tile w; T lower triangular)
        {
            const float lamC = sm.lam[CT - 1];
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
                    sm.x.u.Uhi[16 * rt + lr][t] = hi;
                    sm.x.u.Ulo[16 * rt + lr][t] = lo;
                    split(expf(lamC - sm.lam[t]) * sm.rk[t] * u[i], hi, lo);
                    sm.x.u.U2hi[16 * rt + lr][t] = hi;
                    sm.x.u.U2lo[16 * rt + lr][t] = lo;
                }
            }
        }
        __syncthreads();

        // ---- stage 4: O += P U -> output;  S = G_C S + U2^T K
        {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                f32x4 acc = O[rt];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks > (w >> 1)) break;
                    const bf16x8 ah = frag(&sm.Phi[0][0], LDT, 16 * w, 32 * ks, lane);
                    const bf16x8 al = frag(&sm.Plo[0][0], LDT, 16 * w, 32 * ks, lane);
                    const bf16x8 bh = frag(&sm.x.u.Uhi[0][0], LDT, 16 * rt, 32 * ks, lane);
                    const bf16x8 bl = frag(&sm.x.u.Ulo[0][0], LDT, 16 * rt, 32 * ks, lane);
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
            const float gC = sm.gam[CT - 1];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rt = q >> 1, dt = 2 * w + (q & 1);
                f32x4 acc = S[q] * gC;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 ah = frag(&sm.x.u.U2hi[0][0], LDT, 16 * rt, 32 * ks, lane);
                    const bf16x8 al = frag(&sm.x.u.U2lo[0][0], LDT, 16 * rt, 32 * ks, lane);
                    const bf16x8 bk = frag(&sm.Kt[0][0], LDT, 16 * dt, 32 * ks, lane);
                    acc = mma(ah, bk, acc);
                    acc = mma(al, bk, acc);
                }
                S[q] = acc;
            }
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

hipError_t launch_chunk_recurrent(const RecurrentArgs &a, hipStream_t stream) {
    const int nvb = a.dv / DVB;
    const long long blocks = (long long)a.num_seqs * a.num_v_heads * nvb;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_gdr_kernel, dim3((unsigned)blocks), dim3(NTH), 0, stream, a, nvb);
    return hipGetLastError();
}

}  // namespace gdn
