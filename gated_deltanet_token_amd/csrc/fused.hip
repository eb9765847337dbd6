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

template <int DK, int R>
__global__ __launch_bounds__(kFusedThreads) void fused_conv_decode_kernel(FusedDecodeArgs a) {
    extern __shared__ uint16_t act[];                         // conv output of this group: q | k | v
    // XCD-contiguous order: each XCD takes a contiguous range of (sequence, head group)
    fused_decode_unit<DK, R>(a, xcd_contiguous(blockIdx.x, gridDim.x), act);
}

template <int DK>
hipError_t launch_dk(const FusedDecodeArgs &a, hipStream_t stream) {
    const long long blocks = (long long)a.batch * a.num_k_heads;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int grp = a.num_v_heads / a.num_k_heads;
    const size_t lds = (size_t)(2 * DK + grp * a.dv) * sizeof(uint16_t);
    hipLaunchKernelGGL((fused_conv_decode_kernel<DK, kFusedRows>), dim3((unsigned)blocks), dim3(kFusedThreads), lds, stream,
                       a);
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
