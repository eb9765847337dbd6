// Decode step with the conv update fused into the gated delta rule, gfx950:
// one workgroup per (sequence, q/k head), each running one unit of
// fused_unit.h.
//
// Arithmetic is that of gdn_causal_conv1d_update followed by
// gdn_fused_recurrent_decode (conv_math.h, gdr_math.h), so the fused call
// is bit-identical to the two calls.  It saves a launch per decode step and
// the conv output's round trip through HBM.
#include "fused_unit.h"

namespace gdn {

namespace {

// The fields the unit's first fetches use (slot index, then the conv window
// and the state rows) are also passed ahead of the struct: the first 14
// dwords of the arguments arrive preloaded in SGPRs, so the slot load is
// issued without waiting for an argument load.  Measured in the engine
// trace: 24.1 -> 23.8 us per launch.
template <int DK, int R>
__global__ __launch_bounds__(kFusedThreads) void fused_conv_decode_kernel(
    const int32_t *state_indices, float *state, uint16_t *conv_state, const uint16_t *x, int num_k_heads,
    int num_slots, int num_conv_slots, int n_blocks, FusedDecodeArgs a_in) {
    extern __shared__ uint16_t act[];                         // conv output of this group: q | k | v
    FusedDecodeArgs a = a_in;
    a.state_indices = state_indices;
    a.state = state;
    a.conv_state = conv_state;
    a.x = x;
    a.num_k_heads = num_k_heads;
    a.num_slots = num_slots;
    a.num_conv_slots = num_conv_slots;
    // XCD-contiguous order: each XCD takes a contiguous range of (sequence, head group)
    fused_decode_unit<DK, R>(a, xcd_contiguous(blockIdx.x, n_blocks), act);
}

template <int DK>
hipError_t launch_dk(const FusedDecodeArgs &a, hipStream_t stream) {
    const long long blocks = (long long)a.batch * a.num_k_heads;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int grp = a.num_v_heads / a.num_k_heads;
    const size_t lds = (size_t)(2 * DK + grp * a.dv) * sizeof(uint16_t);
    hipLaunchKernelGGL((fused_conv_decode_kernel<DK, kFusedRows>), dim3((unsigned)blocks), dim3(kFusedThreads), lds, stream,
                       a.state_indices, a.state, a.conv_state, a.x, a.num_k_heads, a.num_slots, a.num_conv_slots,
                       (int)blocks, a);
    return hipGetLastError();
}

}  // namespace

int fused_max_group_channels() { return kMaxGroupChannels; }

hipError_t launch_fused_conv_decode(const FusedDecodeArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_dk<16>(a, stream);
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
