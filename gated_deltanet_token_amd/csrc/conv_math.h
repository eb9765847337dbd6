// Width-4 causal conv arithmetic shared by the conv kernels and the fused
// conv + recurrence decode: the same operations in the same order, so every
// path gives bit-identical conv outputs.
//
// Per channel the output is bias + w0 e0 + w1 e1 + w2 e2 + w3 e3 (e0 the
// oldest window row).  The sum runs on the gfx950 bf16 dot product
// (v_dot2_f32_bf16: two bf16 products added to an fp32 accumulator): the
// weights of a channel are already stored as the bf16 pairs (w0, w1) and
// (w2, w3), and one byte permute pairs a channel's value in two window rows.
// Products of bf16 values are exact in fp32, so this is the fp32 sum of the
// same terms, two at a time, without unpacking any operand.
#pragma once

#include "gdn_device.h"

namespace gdn {

constexpr int kConvVec = 8;   // channels per lane (one 16-byte bf16 vector)

struct ConvTaps {
    uint32_t w01[kConvVec];   // bf16 pair (tap 0, tap 1) of each channel
    uint32_t w23[kConvVec];   // bf16 pair (tap 2, tap 3)
    float b[kConvVec];
};

__device__ __forceinline__ void load_taps(ConvTaps &t, const uint16_t *weight, const uint16_t *bias,
                                          int c0) {
    // weight [C][4] bf16: 8 channels x 4 taps = 64 contiguous bytes
    const uint4 *wp = reinterpret_cast<const uint4 *>(weight + (int64_t)c0 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = wp[i];           // channels 2i and 2i+1
        t.w01[2 * i] = v.x;
        t.w23[2 * i] = v.y;
        t.w01[2 * i + 1] = v.z;
        t.w23[2 * i + 1] = v.w;
    }
    // Without a bias the load still reads a valid address (the weights) and
    // the value is zeroed: a load behind a branch would make the compiler
    // wait for it, and everything issued before it, at the join.
    const uint4 bv = *reinterpret_cast<const uint4 *>(bias ? bias + c0 : weight + c0);
    const uint32_t keep = bias ? ~0u : 0u;
    unpack8(make_uint4(bv.x & keep, bv.y & keep, bv.z & keep, bv.w & keep), t.b);
}

__device__ __forceinline__ uint4 select4(bool c, const uint4 &a, const uint4 &b) {
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// bf16 pair (older, newer) of the even / odd channel of two packed words
__device__ __forceinline__ uint32_t pair_even(uint32_t older, uint32_t newer) {
    return __builtin_amdgcn_perm(newer, older, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_odd(uint32_t older, uint32_t newer) {
    return __builtin_amdgcn_perm(newer, older, 0x07060302u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
// The same product into a new register: the three-operand encoding, so a
// bias shared by several output rows is not first copied into each row's
// accumulator (the compiler emits the two-operand form, whose accumulator is
// also its destination, plus a copy).
__device__ __forceinline__ float dot2_bf16_3op(uint32_t a, uint32_t b, float c) {
    float d;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// The 8 channels of two consecutive window rows as bf16 pairs (older, newer),
// channel c in p[c].  An output row uses the pairs of its window rows (0, 1)
// and (2, 3); a kernel that produces several rows builds each pair of
// neighbouring rows once.
struct RowPairs {
    uint32_t p[kConvVec];
};

__device__ __forceinline__ RowPairs row_pairs(const uint4 &older, const uint4 &newer) {
    RowPairs r;
    r.p[0] = pair_even(older.x, newer.x); r.p[1] = pair_odd(older.x, newer.x);
    r.p[2] = pair_even(older.y, newer.y); r.p[3] = pair_odd(older.y, newer.y);
    r.p[4] = pair_even(older.z, newer.z); r.p[5] = pair_odd(older.z, newer.z);
    r.p[6] = pair_even(older.w, newer.w); r.p[7] = pair_odd(older.w, newer.w);
    return r;
}

// One output row from the pairs of its window rows (0, 1) and (2, 3).  The
// accumulation order -- bias, then taps (0, 1), then taps (2, 3) -- is the
// same in every kernel, so all give bit-identical results.
__device__ __forceinline__ uint4 conv_pairs(const ConvTaps &t, const RowPairs &p01, const RowPairs &p23,
                                            bool silu) {
    float out[kConvVec];
#pragma unroll
    for (int c = 0; c < kConvVec; ++c) {
        float acc = dot2_bf16_3op(p01.p[c], t.w01[c], t.b[c]);
        acc = dot2_bf16(p23.p[c], t.w23[c], acc);
        out[c] = silu ? silu_f32(acc) : acc;
    }
    return pack8(out);
}

// One output row from four window rows (oldest first).
__device__ __forceinline__ uint4 conv_row(const ConvTaps &t, const uint4 &e0, const uint4 &e1,
                                          const uint4 &e2, const uint4 &e3, bool silu) {
    return conv_pairs(t, row_pairs(e0, e1), row_pairs(e2, e3), silu);
}

}  // namespace gdn
