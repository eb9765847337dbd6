// Per-token arithmetic of the token-by-token gated delta rule, shared by the
// fused decode kernels: one state row lives in a group of G lanes, lane j
// holding the E = dk/G elements {4G*m + 4j + e}.  Every multiply-add is an
// explicit fma and every group sum uses the same DPP tree, so any kernel
// built on these functions produces bit-identical tokens.
//
// Rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
// S <- a S (I - b kh kh^T) + b v kh^T, o = scale S qh, evaluated per row as
//   u = (S k) rk, p = (S q) rq, c = b (v - a u),
//   S = a S + (c rk) k,  o = scale (a p + c (k.q) rk rq).
#pragma once

#include "gdn_device.h"

namespace gdn {

template <int DK>
struct RowLayout {
    static constexpr int G = DK >= 32 ? 8 : 4;    // lanes per state row
    static constexpr int E = DK / G;              // fp32 elements per lane
    static constexpr int M = E / 4;               // float4 slices per lane
    static constexpr int RG = 64 / G;             // row groups per wave
    static_assert(E % 4 == 0 && E >= 4, "head_k_dim must be 16, 32, 64 or 128");
};

// q/k factors of one token, the same in every lane of a group
struct TokenFactors {
    float rk, rq, kq;   // inverse norms (1 without normalisation), (k.q) rk rq
};

template <int G, int E>
__device__ __forceinline__ TokenFactors token_factors(const float (&kf)[E], const float (&qf)[E], bool l2norm) {
    float skk = 0.f, sqq = 0.f, skq = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        skk = __builtin_fmaf(kf[e], kf[e], skk);
        sqq = __builtin_fmaf(qf[e], qf[e], sqq);
        skq = __builtin_fmaf(kf[e], qf[e], skq);
    }
    skk = group_sum<G>(skk);
    sqq = group_sum<G>(sqq);
    skq = group_sum<G>(skq);
    TokenFactors f;
    f.rk = l2norm ? rsqrtf(skk + 1e-6f) : 1.f;
    f.rq = l2norm ? rsqrtf(sqq + 1e-6f) : 1.f;
    f.kq = (skq * f.rk) * f.rq;
    return f;
}

// one token's update of one state row (this lane's E elements); returns o
template <int G, int E>
__device__ __forceinline__ float row_step(float (&S)[E], const float (&kf)[E], const float (&qf)[E],
                                          const TokenFactors &f, float alpha, float beta, float v, float scale) {
    float u = 0.f, p = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        u = __builtin_fmaf(S[e], kf[e], u);
        p = __builtin_fmaf(S[e], qf[e], p);
    }
    u = group_sum<G>(u) * f.rk;
    p = group_sum<G>(p) * f.rq;
    const float coef = beta * __builtin_fmaf(-alpha, u, v);
    const float ck = coef * f.rk;
#pragma unroll
    for (int e = 0; e < E; ++e) S[e] = __builtin_fmaf(ck, kf[e], alpha * S[e]);
    return scale * __builtin_fmaf(alpha, p, coef * f.kq);
}

}  // namespace gdn
