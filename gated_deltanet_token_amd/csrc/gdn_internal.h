// Internal launch interface between the C-ABI entry points (api.hip) and the
// kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

struct ConvVarlenArgs {
    const uint16_t *x;
    int64_t x_stride;
    const uint16_t *weight;
    const uint16_t *bias;
    uint16_t *conv_state;
    const int32_t *qsl;
    const int32_t *state_indices;
    const uint8_t *has_init;
    const gdn_conv_chunk *chunks;
    int n_chunks;
    uint16_t *y;
    int64_t y_stride;
    int channels;
    int silu;
    int num_seqs;                // descriptors naming another sequence are skipped
    int num_slots;               // state indices at or past it are skipped
    int num_tokens;              // sequence ends are clamped to it
    int descriptors_per_program = 1;   // 1: 8-token programs; 2: 16-token programs
};

struct ConvUpdateArgs {
    const uint16_t *x;
    int64_t x_stride;
    const uint16_t *weight;
    const uint16_t *bias;
    uint16_t *conv_state;
    const int32_t *state_indices;
    uint16_t *y;
    int64_t y_stride;
    int batch;
    int channels;
    int silu;
    int num_slots;               // state indices at or past it are skipped
};

struct RecurrentArgs {
    const uint16_t *q;
    int64_t q_stride;
    const uint16_t *k;
    int64_t k_stride;
    const uint16_t *v;
    int64_t v_stride;
    const float *g;
    const float *beta;
    float *state;
    const int32_t *qsl;          // nullptr: one token per sequence
    const int32_t *state_indices;
    const uint8_t *has_init;     // nullptr: all have an initial state
    uint16_t *o;
    int64_t o_stride;
    int num_seqs;
    int num_k_heads;
    int num_v_heads;
    int dk;
    int dv;
    float scale;
    int l2norm;
    int num_slots;               // state indices at or past it are skipped
    int num_tokens;              // token ranges are clamped to [0, num_tokens)
};

struct FusedDecodeArgs {
    const uint16_t *x;           // [batch][x_stride]: q | k | v channels
    int64_t x_stride;
    const uint16_t *conv_weight;
    const uint16_t *conv_bias;
    uint16_t *conv_state;
    int channels;                // 2 HK dk + HV dv
    const float *g;
    const float *beta;
    float *state;
    const int32_t *state_indices;
    uint16_t *o;
    int64_t o_stride;
    uint16_t *y;                 // optional conv output
    int64_t y_stride;
    int batch;
    int num_k_heads;
    int num_v_heads;
    int dk;
    int dv;
    float scale;
    int l2norm;
    int silu;
    int num_slots;               // recurrent-state slots; indices at or past it are skipped
    int num_conv_slots;          // conv_state slots; likewise
};

hipError_t launch_conv_varlen(const ConvVarlenArgs &a, hipStream_t stream);
hipError_t launch_conv_update(const ConvUpdateArgs &a, hipStream_t stream);
hipError_t launch_recurrent(const RecurrentArgs &a, hipStream_t stream);
int fused_max_group_channels();
hipError_t launch_fused_conv_decode(const FusedDecodeArgs &a, hipStream_t stream);
// chunkwise form: workspace of chunk_workspace_bytes(...) bytes, 256-byte aligned
int64_t chunk_workspace_bytes(int num_seqs, int num_tokens, int num_k_heads, int num_v_heads);
hipError_t launch_chunk_recurrent(const RecurrentArgs &a, void *workspace, int num_tokens, hipStream_t stream);
// the chunkwise form and a fused decode batch on disjoint state slots, their
// last kernels sharing one grid
hipError_t launch_chunk_and_decode(const RecurrentArgs &a, void *workspace, int num_tokens,
                                   const FusedDecodeArgs &f, hipStream_t stream);

}  // namespace gdn
