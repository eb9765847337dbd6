// Width-4 depthwise causal conv1d for packed varlen prefill tokens and for
// single-token decode, gfx950.
//
// Dispatch follows page "perf(gdn): dispatch exact causal-conv chunks",
// section "What changed": one program per exact (sequence, 8-token chunk)
// descriptor.  Here a program is one workgroup per (descriptor, channel
// tile); each lane owns 8 channels (one 16-byte bf16 vector per token row),
// keeps the 3-row halo and its 8 token rows in VGPRs and slides the 4-tap
// window in registers.  The conv is depthwise, so no lane needs another
// lane's data: nothing is staged in LDS.
//
// Only the chunk-0 program of a sequence touches its conv_state slot: it
// reads the old rows as its halo and writes the new rows, taking them from x
// (read-only) or from the old rows it already holds.  No other program reads
// the slot, so the in-place update has no read/write race.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kConvVec = 8;                             // channels per lane
constexpr int kConvThreads = 256;                       // 4 waves
constexpr int kConvTile = kConvThreads * kConvVec;      // 2048 channels
constexpr int kChunk = 8;                               // tokens per descriptor

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

__global__ __launch_bounds__(kConvThreads) void conv_varlen_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride, const uint16_t *__restrict__ weight,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ conv_state,
    const int32_t *__restrict__ qsl, const int32_t *__restrict__ state_indices,
    const uint8_t *__restrict__ has_init, const gdn_conv_chunk *__restrict__ chunks, int n_chunks,
    uint16_t *__restrict__ y, int64_t y_stride, int channels, int silu) {
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int tile = work / n_chunks;
    const int ci = work - tile * n_chunks;
    const gdn_conv_chunk d = chunks[ci];
    const int slot = state_indices[d.seq];
    if (slot < 0) return;
    const int a = qsl[d.seq];
    const int end = qsl[d.seq + 1];
    const int t0 = a + d.chunk * kChunk;
    if (t0 >= end) return;
    const int n = min(kChunk, end - t0);
    const int c0 = tile * kConvTile + threadIdx.x * kConvVec;
    if (c0 >= channels) return;

    uint16_t *st = conv_state + (int64_t)slot * 3 * channels + c0;
    const uint4 zero = make_uint4(0, 0, 0, 0);

    // window rows: h[0..2] = halo (oldest first), r[0..n) = this chunk's tokens.
    // Every load reads a valid address (halo: the slot or the 3 preceding
    // rows of the same sequence; tokens past the chunk end re-read its last
    // row) and masking is done on values, so no load is predicated.
    uint4 h[3], r[kChunk];
    const bool first = d.chunk == 0;
    const bool zero_halo = first && has_init != nullptr && has_init[d.seq] == 0;
    const uint16_t *hp = first ? st : x + (int64_t)(t0 - 3) * x_stride + c0;
    const int64_t hstride = first ? (int64_t)channels : x_stride;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const uint4 v = *reinterpret_cast<const uint4 *>(hp + i * hstride);
        h[i] = select4(zero_halo, zero, v);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
        r[i] = *reinterpret_cast<const uint4 *>(x + (int64_t)(t0 + min(i, n - 1)) * x_stride + c0);

    ConvTaps taps;
    load_taps(taps, weight, bias, c0);

    const bool act = silu != 0;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        if (i < n) {
            const uint4 e0 = i >= 3 ? r[i - 3] : h[i];
            const uint4 e1 = i >= 2 ? r[i - 2] : h[i + 1];
            const uint4 e2 = i >= 1 ? r[i - 1] : h[2];
            const uint4 out = conv_row(taps, e0, e1, e2, r[i], act);
            *reinterpret_cast<uint4 *>(y + (int64_t)(t0 + i) * y_stride + c0) = out;
        }
    }

    if (first) {
        // new slot rows = window rows L, L+1, L+2 (window = halo || sequence)
        // (an always-valid load and value selects rather than a run-time
        // register index, which would push the window out to scratch memory)
        const int L = end - a;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int wi = L + i;          // window index; < 3 means an old halo row
            const uint4 fromx =
                *reinterpret_cast<const uint4 *>(x + (int64_t)(a + max(wi - 3, 0)) * x_stride + c0);
            const uint4 old = select4(wi == 0, h[0], select4(wi == 1, h[1], h[2]));
            const uint4 v = select4(wi >= 3, fromx, old);
            *reinterpret_cast<uint4 *>(st + (int64_t)i * channels) = v;
        }
    }
}

__global__ __launch_bounds__(kConvThreads) void conv_update_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride, const uint16_t *__restrict__ weight,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ conv_state,
    const int32_t *__restrict__ state_indices, uint16_t *__restrict__ y, int64_t y_stride,
    int channels, int n_tiles, int silu) {
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x - b * n_tiles;
    const int slot = state_indices[b];
    if (slot < 0) return;
    const int c0 = tile * kConvTile + threadIdx.x * kConvVec;
    if (c0 >= channels) return;
    uint16_t *st = conv_state + (int64_t)slot * 3 * channels + c0;
    const uint4 s0 = *reinterpret_cast<const uint4 *>(st);
    const uint4 s1 = *reinterpret_cast<const uint4 *>(st + channels);
    const uint4 s2 = *reinterpret_cast<const uint4 *>(st + 2 * (int64_t)channels);
    const uint4 xv = *reinterpret_cast<const uint4 *>(x + (int64_t)b * x_stride + c0);
    ConvTaps taps;
    load_taps(taps, weight, bias, c0);
    *reinterpret_cast<uint4 *>(y + (int64_t)b * y_stride + c0) = conv_row(taps, s0, s1, s2, xv, silu != 0);
    *reinterpret_cast<uint4 *>(st) = s1;
    *reinterpret_cast<uint4 *>(st + channels) = s2;
    *reinterpret_cast<uint4 *>(st + 2 * (int64_t)channels) = xv;
}

hipError_t launch_conv_varlen(const ConvVarlenArgs &a, hipStream_t stream) {
    const int n_tiles = (a.channels + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)a.n_chunks * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(conv_varlen_kernel, dim3((unsigned)blocks), dim3(kConvThreads), 0, stream,
                       a.x, a.x_stride, a.weight, a.bias, a.conv_state, a.qsl, a.state_indices,
                       a.has_init, a.chunks, a.n_chunks, a.y, a.y_stride, a.channels, a.silu);
    return hipGetLastError();
}

hipError_t launch_conv_update(const ConvUpdateArgs &a, hipStream_t stream) {
    const int n_tiles = (a.channels + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)a.batch * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(conv_update_kernel, dim3((unsigned)blocks), dim3(kConvThreads), 0, stream,
                       a.x, a.x_stride, a.weight, a.bias, a.conv_state, a.state_indices, a.y,
                       a.y_stride, a.channels, n_tiles, a.silu);
    return hipGetLastError();
}

}  // namespace gdn
