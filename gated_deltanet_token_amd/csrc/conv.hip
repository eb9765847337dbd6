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

// The arguments of the descriptor chain come first: the first 14 dwords
// arrive preloaded in SGPRs, and the grid size is one of them (gridDim would
// be a load from the dispatch's hidden arguments).
template <int THREADS, bool SILU, bool WT>
__global__ __launch_bounds__(THREADS) void conv_varlen_kernel(
    const gdn_conv_chunk *__restrict__ chunks, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ state_indices, const uint16_t *__restrict__ weight, int n_tiles, int num_seqs,
    int num_slots, int num_tokens, int channels, int n_blocks,
    const uint16_t *__restrict__ bias, const uint16_t *__restrict__ x, int64_t x_stride,
    const uint8_t *__restrict__ has_init, uint16_t *__restrict__ conv_state,
    uint16_t *__restrict__ y, int64_t y_stride) {
    constexpr int TILE = THREADS * kConvVec;
    // Chunk-major and XCD-contiguous: each XCD takes one contiguous range of
    // (descriptor, channel tile) items, so a chunk's halo rows are rows its
    // neighbouring chunk fetched into the same L2.
    const int work = xcd_contiguous(blockIdx.x, n_blocks);
    const int ci = work / n_tiles;
    const int tile = work - ci * n_tiles;
    const int c0 = tile * TILE + threadIdx.x * kConvVec;
    const bool lane_ok = c0 < channels;

    // The taps first: they do not depend on the descriptor, and the first
    // output row needs them, so its wait does not cover the row loads.  (A
    // lane past the channel count reads channel 0's and exits below.)
    ConvTaps taps;
    load_taps(taps, weight, bias, lane_ok ? c0 : 0);

    // A descriptor naming no sequence of the call, a slot index outside the
    // pool, and a chunk past its sequence's end are skipped like padding:
    // nothing is read or written for them.  Every test is made in one exit,
    // after the slot and the bounds are fetched together (the tests combine
    // without short-circuit), so the row addresses wait for two dependent
    // round trips (descriptor, then slot and bounds) rather than one per test.
    const gdn_conv_chunk d = chunks[ci];
    const bool bad = (unsigned)d.seq >= (unsigned)num_seqs || d.chunk < 0;
    const int seq = bad ? 0 : d.seq;
    const int slot = state_indices[seq];
    const int lo_raw = qsl[seq], hi_raw = qsl[seq + 1];
    // (the slot and the bounds issued before either is waited for; every
    // argument used past the exit fetched before it, with the first ones,
    // rather than in a round trip of its own after it)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"s"(x), "s"(weight), "s"(bias), "s"(conv_state), "s"(y), "s"(has_init), "s"(x_stride),
                 "s"(y_stride), "s"(channels));
    int a, end;
    clamp_range(lo_raw, hi_raw, num_tokens, a, end);
    const bool skip = bad | ((unsigned)slot >= (unsigned)num_slots) | (d.chunk >= (end - a + kChunk - 1) / kChunk);
    if (!lane_ok | skip) return;
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

// ---------------------------------------------------------------------------
// 16-token programs (two consecutive descriptors per workgroup), page "RTX
// 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section
// "Existing evidence" (the multi-token tile arm), applied to the exact 8-token
// descriptors of page "perf(gdn): dispatch exact causal-conv chunks".  When
// the pair's second descriptor continues the first (same sequence, next
// chunk) its halo is the first's last three rows, already in registers: 19
// rows are read for 16 tokens instead of 22.  The arithmetic of each token is
// that of conv_varlen_kernel, so the results are bit-identical.
// ---------------------------------------------------------------------------

// one descriptor of a pair, resolved (ok: processed; a descriptor past the
// list, naming no sequence of the call, past its sequence's end, or whose
// slot lies outside the pool is skipped like padding)
struct ConvDesc {
    bool ok, first;
    int seq, chunk, slot, a, end, t0, n;
};

__device__ __forceinline__ ConvDesc conv_desc(const gdn_conv_chunk *chunks, int ci, int n_chunks,
                                              const int32_t *qsl, const int32_t *state_indices, int num_seqs,
                                              int num_slots, int num_tokens) {
    ConvDesc c;
    const gdn_conv_chunk d = chunks[min(ci, n_chunks - 1)];
    const bool bad = ci >= n_chunks || (unsigned)d.seq >= (unsigned)num_seqs || d.chunk < 0;
    c.seq = bad ? 0 : d.seq;
    c.chunk = d.chunk;
    c.slot = state_indices[c.seq];
    clamp_range(qsl[c.seq], qsl[c.seq + 1], num_tokens, c.a, c.end);
    c.ok = !bad && (unsigned)c.slot < (unsigned)num_slots && d.chunk < (c.end - c.a + kChunk - 1) / kChunk;
    c.first = c.ok && d.chunk == 0;
    c.t0 = c.ok ? c.a + d.chunk * kChunk : 0;       // a skipped one reads row 0 (the call has tokens)
    c.n = c.ok ? min(kChunk, c.end - c.t0) : 1;
    return c;
}

// outputs of one descriptor from its window (halo already masked), and for a
// sequence's chunk 0 its new slot rows; as in conv_varlen_kernel
template <bool SILU>
__device__ __forceinline__ void conv_emit(const ConvTaps &taps, const uint4 (&h)[3], const uint4 (&r)[kChunk],
                                          const ConvDesc &c, const uint16_t *x, int64_t x_stride,
                                          uint16_t *conv_state, int channels, uint16_t *y, int64_t y_stride,
                                          int c0) {
    if (!c.ok) return;
    RowPairs pr[kChunk + 2];
#pragma unroll
    for (int j = 0; j < kChunk + 2; ++j) {
        const uint4 &older = j < 3 ? h[j] : r[j - 3];
        const uint4 &newer = j + 1 < 3 ? h[j + 1] : r[j - 2];
        pr[j] = row_pairs(older, newer);
    }
    const __amdgpu_buffer_rsrc_t y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        y + (int64_t)c.t0 * y_stride, (short)0, c.n * (int)y_stride * 2, kBufferFlags);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint4 out = conv_pairs(taps, pr[i], pr[i + 2], SILU);
        const u32x4 o4 = {out.x, out.y, out.z, out.w};
        __builtin_amdgcn_raw_buffer_store_b128(o4, y_rsrc, (i * (int)y_stride + c0) * 2, 0, kBufferWriteThrough);
    }
    if (c.first) {
        uint16_t *st = conv_state + (int64_t)c.slot * 3 * channels + c0;
        const int L = c.end - c.a;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int wi = L + i;
            const uint4 fromx =
                *reinterpret_cast<const uint4 *>(x + (int64_t)(c.a + max(wi - 3, 0)) * x_stride + c0);
            const uint4 old = select4(wi == 0, h[0], select4(wi == 1, h[1], h[2]));
            *reinterpret_cast<uint4 *>(st + (int64_t)i * channels) = select4(wi >= 3, fromx, old);
        }
    }
}

// One workgroup per (descriptor pair, channel tile).  Every load reads a
// valid address (as in conv_varlen_kernel); the second descriptor's own halo
// goes through a buffer resource whose range is zero when the pair is
// contiguous, so that case reads nothing for it, without a branch.  Row and
// halo offsets are 32-bit: the launch requires strides up to 2^26.
template <int THREADS, bool SILU>
__global__ __launch_bounds__(THREADS) void conv_varlen16_kernel(
    const uint16_t *__restrict__ x, int64_t x_stride, const uint16_t *__restrict__ weight,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ conv_state,
    const int32_t *__restrict__ qsl, const int32_t *__restrict__ state_indices,
    const uint8_t *__restrict__ has_init, const gdn_conv_chunk *__restrict__ chunks, int n_chunks,
    uint16_t *__restrict__ y, int64_t y_stride, int channels, int n_tiles, int num_seqs, int num_slots,
    int num_tokens) {
    constexpr int TILE = THREADS * kConvVec;
    const int work = xcd_contiguous(blockIdx.x, gridDim.x);
    const int pair = work / n_tiles;
    const int tile = work - pair * n_tiles;
    const int c0 = tile * TILE + threadIdx.x * kConvVec;
    if (c0 >= channels) return;
    ConvTaps taps;
    load_taps(taps, weight, bias, c0);

    const ConvDesc d0 = conv_desc(chunks, 2 * pair, n_chunks, qsl, state_indices, num_seqs, num_slots, num_tokens);
    const ConvDesc d1 = conv_desc(chunks, 2 * pair + 1, n_chunks, qsl, state_indices, num_seqs, num_slots,
                                  num_tokens);
    const bool cont = d0.ok && d1.ok && d1.seq == d0.seq && d1.chunk == d0.chunk + 1;

    uint4 h0[3], r0[kChunk], g1[3], r1[kChunk];
    {
        const uint16_t *hp = d0.first ? conv_state + (int64_t)d0.slot * 3 * channels + c0
                                      : x + (int64_t)(d0.ok ? d0.t0 - 3 : 0) * x_stride + c0;
        const int64_t hs = d0.first ? (int64_t)channels : d0.ok ? x_stride : 0;
#pragma unroll
        for (int i = 0; i < 3; ++i) h0[i] = *reinterpret_cast<const uint4 *>(hp + i * hs);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint16_t *p = x + (int64_t)(d0.t0 + min(i, d0.n - 1)) * x_stride + c0;
        r0[i] = i < kChunk - 3 ? load_stream16(p) : *reinterpret_cast<const uint4 *>(p);
    }
    {
        // the second descriptor's own halo: the slot rows or its 3 preceding x rows
        const uint16_t *hb = d1.first ? conv_state + (int64_t)d1.slot * 3 * channels
                                      : x + (int64_t)(d1.ok ? d1.t0 - 3 : 0) * x_stride;
        const int hs = d1.first ? channels : (int)x_stride;
        const int range = (cont || !d1.ok) ? 0 : (2 * hs + channels) * 2;
        const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(hb), (short)0,
                                                                            range, kBufferFlags);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hr, (i * hs + c0) * 2,
                                                                                             0, 0));
            g1[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        const uint16_t *p = x + (int64_t)(d1.t0 + min(i, d1.n - 1)) * x_stride + c0;
        r1[i] = i < kChunk - 3 ? load_stream16(p) : *reinterpret_cast<const uint4 *>(p);
    }
    // has_initial_state, read unconditionally from valid bytes
    const uint8_t f0 = *(has_init != nullptr ? has_init + d0.seq : reinterpret_cast<const uint8_t *>(chunks));
    const uint8_t f1 = *(has_init != nullptr ? has_init + d1.seq : reinterpret_cast<const uint8_t *>(chunks));
    const uint32_t k0 = (d0.first && has_init != nullptr && f0 == 0) ? 0u : ~0u;
    const uint32_t k1 = (d1.first && has_init != nullptr && f1 == 0) ? 0u : ~0u;
    uint4 h1[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        h0[i] = make_uint4(h0[i].x & k0, h0[i].y & k0, h0[i].z & k0, h0[i].w & k0);
        const uint4 own = make_uint4(g1[i].x & k1, g1[i].y & k1, g1[i].z & k1, g1[i].w & k1);
        h1[i] = select4(cont, r0[kChunk - 3 + i], own);
    }
    conv_emit<SILU>(taps, h0, r0, d0, x, x_stride, conv_state, channels, y, y_stride, c0);
    conv_emit<SILU>(taps, h1, r1, d1, x, x_stride, conv_state, channels, y, y_stride, c0);
}

// (the slot lookup's and the window's arguments first: the first 14 dwords
// arrive preloaded in SGPRs)
__global__ __launch_bounds__(kConvThreads) void conv_update_kernel(
    const int32_t *__restrict__ state_indices, int n_tiles, int num_slots, uint16_t *__restrict__ conv_state,
    const uint16_t *__restrict__ x, int64_t x_stride, int channels, int silu,
    const uint16_t *__restrict__ weight, const uint16_t *__restrict__ bias, uint16_t *__restrict__ y,
    int64_t y_stride) {
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
        hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(THREADS), 0, stream, a.chunks, a.qsl,
                           a.state_indices, a.weight, n_tiles, a.num_seqs, a.num_slots, a.num_tokens, a.channels,
                           (int)blocks, a.bias, a.x, a.x_stride, a.has_init, a.conv_state, a.y, a.y_stride);
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
    if (a.descriptors_per_program == 1) return launch_conv_varlen_t<kConvThreads>(a, stream);
    // 16-token programs: one workgroup per (descriptor pair, channel tile)
    const int n_tiles = (a.channels + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)((a.n_chunks + 1) / 2) * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.silu)
        hipLaunchKernelGGL((conv_varlen16_kernel<kConvThreads, true>), dim3((unsigned)blocks), dim3(kConvThreads), 0,
                           stream, a.x, a.x_stride, a.weight, a.bias, a.conv_state, a.qsl, a.state_indices,
                           a.has_init, a.chunks, a.n_chunks, a.y, a.y_stride, a.channels, n_tiles, a.num_seqs,
                           a.num_slots, a.num_tokens);
    else
        hipLaunchKernelGGL((conv_varlen16_kernel<kConvThreads, false>), dim3((unsigned)blocks), dim3(kConvThreads), 0,
                           stream, a.x, a.x_stride, a.weight, a.bias, a.conv_state, a.qsl, a.state_indices,
                           a.has_init, a.chunks, a.n_chunks, a.y, a.y_stride, a.channels, n_tiles, a.num_seqs,
                           a.num_slots, a.num_tokens);
    return hipGetLastError();
}

hipError_t launch_conv_update(const ConvUpdateArgs &a, hipStream_t stream) {
    const int n_tiles = (a.channels + kConvTile - 1) / kConvTile;
    const long long blocks = (long long)a.batch * n_tiles;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(conv_update_kernel, dim3((unsigned)blocks), dim3(kConvThreads), 0, stream,
                       a.state_indices, n_tiles, a.num_slots, a.conv_state, a.x, a.x_stride, a.channels, a.silu,
                       a.weight, a.bias, a.y, a.y_stride);
    return hipGetLastError();
}

}  // namespace gdn
