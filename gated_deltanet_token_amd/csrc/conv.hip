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
#include "conv_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kConvThreads = 256;                       // 4 waves
constexpr int kConvTile = kConvThreads * kConvVec;      // 2048 channels
constexpr int kChunk = 8;                               // tokens per descriptor

template <int THREADS, bool SILU, bool WT>
__global__ __launch_bounds__(THREADS) void conv_varlen_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride, const uint16_t *__restrict__ weight,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ conv_state,
    const int32_t *__restrict__ qsl, const int32_t *__restrict__ state_indices,
    const uint8_t *__restrict__ has_init, const gdn_conv_chunk *__restrict__ chunks,
    uint16_t *__restrict__ y, int64_t y_stride, int channels, int n_tiles, int num_seqs, int num_slots,
    int num_tokens) {
    constexpr int TILE = THREADS * kConvVec;
    // Chunk-major and XCD-contiguous: each XCD takes one contiguous range of
    // (descriptor, channel tile) items, so a chunk's halo rows are rows its
    // neighbouring chunk fetched into the same L2.
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int ci = work / n_tiles;
    const int tile = work - ci * n_tiles;
    const int c0 = tile * TILE + threadIdx.x * kConvVec;
    if (c0 >= channels) return;

    // The taps first: they do not depend on the descriptor, and the first
    // output row needs them, so its wait does not cover the row loads.
    ConvTaps taps;
    load_taps(taps, weight, bias, c0);

    // A descriptor naming no sequence of the call, and a slot index outside
    // the pool, are skipped like padding: nothing is read or written for them.
    const gdn_conv_chunk d = chunks[ci];
    const bool bad = (unsigned)d.seq >= (unsigned)num_seqs || d.chunk < 0;
    const int seq = bad ? 0 : d.seq;
    const int slot = state_indices[seq];
    if (bad || (unsigned)slot >= (unsigned)num_slots) return;
    int a, end;
    clamp_range(qsl[seq], qsl[seq + 1], num_tokens, a, end);
    if (d.chunk >= (end - a + kChunk - 1) / kChunk) return;
    const int t0 = a + d.chunk * kChunk;
    const int n = min(kChunk, end - t0);

    uint16_t *st = conv_state + (int64_t)slot * 3 * channels + c0;

    // window rows: h[0..2] = halo (oldest first), r[0..n) = this chunk's tokens.
    // Every load reads a valid address (halo: the slot or the 3 preceding
    // rows of the same sequence; tokens past the chunk end re-read its last
    // row) and masking is done on values, so no load is predicated.  A
    // sequence without an initial state zeroes its halo through a mask.
    uint4 h[3], r[kChunk];
    const bool first = d.chunk == 0;
    const uint16_t *hp = first ? st : x + (int64_t)(t0 - 3) * x_stride + c0;
    const int64_t hstride = first ? (int64_t)channels : x_stride;
#pragma unroll
    for (int i = 0; i < 3; ++i) h[i] = *reinterpret_cast<const uint4 *>(hp + i * hstride);
    // Rows 0-4 are read by this program only: streaming loads.  Rows 5-7
    // are also the next chunk's halo and stay on plain loads, so that the
    // neighbour finds them in L2.
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint16_t *p = x + (int64_t)(t0 + min(i, n - 1)) * x_stride + c0;
        r[i] = i < kChunk - 3 ? load_stream16(p) : *reinterpret_cast<const uint4 *>(p);
    }
    // (the flag is read unconditionally, from a valid byte, for the same reason as the bias)
    const uint8_t flag = *(has_init != nullptr ? has_init + seq : reinterpret_cast<const uint8_t *>(chunks + ci));
    const uint32_t keep = (first && has_init != nullptr && flag == 0) ? 0u : ~0u;
#pragma unroll
    for (int i = 0; i < 3; ++i) h[i] = make_uint4(h[i].x & keep, h[i].y & keep, h[i].z & keep, h[i].w & keep);

    // Output rows, written through the L2 (WT: a buffer resource over the
    // chunk's rows, whose range also drops the rows past the chunk end): the
    // prefill path reads them right away (the chunkwise rule's q, k and v)
    // and finds them in the caches, and the end of the kernel has no dirty
    // lines to write back.  (Plain stores when the row stride is too large
    // for 32-bit buffer offsets.)
    // Window row j is h[j] for j < 3, else r[j - 3]; pair j holds window
    // rows (j, j + 1) and serves output rows j and j - 2.
    RowPairs pr[kChunk + 2];
#pragma unroll
    for (int j = 0; j < kChunk + 2; ++j) {
        const uint4 &older = j < 3 ? h[j] : r[j - 3];
        const uint4 &newer = j + 1 < 3 ? h[j + 1] : r[j - 2];
        pr[j] = row_pairs(older, newer);
    }
    const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        y + (int64_t)t0 * y_stride, (short)0, WT ? n * (int)y_stride * 2 : 0, kBufferFlags);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint4 out = conv_pairs(taps, pr[i], pr[i + 2], SILU);
        if (WT) {
            const u32x4 o4 = {out.x, out.y, out.z, out.w};
            __builtin_amdgcn_raw_buffer_store_b128(o4, y_rsrc, (i * (int)y_stride + c0) * 2, 0, kBufferWriteThrough);
        } else if (i < n) {
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
    int channels, int n_tiles, int silu, int num_slots) {
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x - b * n_tiles;
    const int slot = state_indices[b];
    if ((unsigned)slot >= (unsigned)num_slots) return;     // padding, or outside the pool
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

template <int THREADS>
hipError_t launch_conv_varlen_t(const ConvVarlenArgs &a, hipStream_t stream) {
    constexpr int TILE = THREADS * kConvVec;
    const int n_tiles = (a.channels + TILE - 1) / TILE;
    const long long blocks = (long long)a.n_chunks * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // the write-through path addresses the chunk's 8 rows with 32-bit byte offsets
    const bool wt = a.y_stride <= ((int64_t)1 << 26);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(THREADS), 0, stream, a.x, a.x_stride, a.weight,
                           a.bias, a.conv_state, a.qsl, a.state_indices, a.has_init, a.chunks, a.y, a.y_stride,
                           a.channels, n_tiles, a.num_seqs, a.num_slots, a.num_tokens);
    };
    if (a.silu) {
        if (wt) go(conv_varlen_kernel<THREADS, true, true>);
        else go(conv_varlen_kernel<THREADS, true, false>);
    } else {
        if (wt) go(conv_varlen_kernel<THREADS, false, true>);
        else go(conv_varlen_kernel<THREADS, false, false>);
    }
    return hipGetLastError();
}

hipError_t launch_conv_varlen(const ConvVarlenArgs &a, hipStream_t stream) {
    return launch_conv_varlen_t<kConvThreads>(a, stream);
}

hipError_t launch_conv_update(const ConvUpdateArgs &a, hipStream_t stream) {
    const int n_tiles = (a.channels + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)a.batch * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(conv_update_kernel, dim3((unsigned)blocks), dim3(kConvThreads), 0, stream,
                       a.x, a.x_stride, a.weight, a.bias, a.conv_state, a.state_indices, a.y,
                       a.y_stride, a.channels, n_tiles, a.silu, a.num_slots);
    return hipGetLastError();
}

}  // namespace gdn
