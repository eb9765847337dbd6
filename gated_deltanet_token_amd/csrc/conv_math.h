// Width-4 causal conv arithmetic shared by the conv kernels and the fused
// conv + recurrence decode: the same operations in the same order, so every
// path gives bit-identical conv outputs.
#pragma once

#include "gdn_device.h"

namespace gdn {

constexpr int kConvVec = 8;   // channels per lane (one 16-byte bf16 vector)

struct ConvTaps {
    float w[kConvVec][4];
    float b[kConvVec];
};

__device__ __forceinline__ void load_taps(ConvTaps &t, const uint16_t *weight, const uint16_t *bias,
                                          int c0) {
    // weight [C][4] bf16: 8 channels x 4 taps = 64 contiguous bytes
    const uint4 *wp = reinterpret_cast<const uint4 *>(weight + (int64_t)c0 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = wp[i];           // channels 2i and 2i+1
        t.w[2 * i][0] = bf16_lo(v.x);     t.w[2 * i][1] = bf16_hi(v.x);
        t.w[2 * i][2] = bf16_lo(v.y);     t.w[2 * i][3] = bf16_hi(v.y);
        t.w[2 * i + 1][0] = bf16_lo(v.z); t.w[2 * i + 1][1] = bf16_hi(v.z);
        t.w[2 * i + 1][2] = bf16_lo(v.w); t.w[2 * i + 1][3] = bf16_hi(v.w);
    }
    if (bias) {
        unpack8(*reinterpret_cast<const uint4 *>(bias + c0), t.b);
    } else {
#pragma unroll
        for (int c = 0; c < kConvVec; ++c) t.b[c] = 0.0f;
    }
}

__device__ __forceinline__ uint4 select4(bool c, const uint4 &a, const uint4 &b) {
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// One output row from four window rows (oldest first).  The accumulation
// order -- bias, then taps 0..3 with fused multiply-adds -- is the same in the
// varlen and the update kernels, so both give bit-identical results.
__device__ __forceinline__ uint4 conv_row(const ConvTaps &t, const uint4 &e0, const uint4 &e1,
                                          const uint4 &e2, const uint4 &e3, bool silu) {
    float f0[8], f1[8], f2[8], f3[8], out[8];
    unpack8(e0, f0); unpack8(e1, f1); unpack8(e2, f2); unpack8(e3, f3);
#pragma unroll
    for (int c = 0; c < kConvVec; ++c) {
        float acc = t.b[c];
        acc = __builtin_fmaf(t.w[c][0], f0[c], acc);
        acc = __builtin_fmaf(t.w[c][1], f1[c], acc);
        acc = __builtin_fmaf(t.w[c][2], f2[c], acc);
        acc = __builtin_fmaf(t.w[c][3], f3[c], acc);
        out[c] = silu ? silu_f32(acc) : acc;
    }
    return pack8(out);
}

}  // namespace gdn
