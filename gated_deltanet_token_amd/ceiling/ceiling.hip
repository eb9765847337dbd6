// Reference kernels for the benchmark's measured bandwidth ceilings (not part
// of the GDN path): a plain streaming copy and a streaming in-place
// read-modify-write, 16 bytes per lane per access, 1, 4 or 16 accesses per
// lane (all loads of a lane issued before its stores; the best count differs
// with the access pattern and size, so the benchmark takes the fastest).  It
// times them on the same byte counts and buffers as the varlen conv (a copy
// of x into y) and the decode (its state traffic), so each kernel's fraction
// of what HBM allows for that access shape can be stated beside its fraction
// of the 8 TB/s peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CEIL_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int kPerLane>
__global__ __launch_bounds__(kThreads) void stream_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                        int64_t n) {
    const int64_t base = ((int64_t)blockIdx.x * kThreads * kPerLane) + threadIdx.x;
    u32x4 v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        v[i] = j < n ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        if (j < n) __builtin_nontemporal_store(v[i], dst + j);
    }
}

// x <- x + 0 on fp32 words: every byte read once and written once
template <int kPerLane>
__global__ __launch_bounds__(kThreads) void stream_rmw(u32x4 *__restrict__ buf, int64_t n) {
    const int64_t base = ((int64_t)blockIdx.x * kThreads * kPerLane) + threadIdx.x;
    u32x4 v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        v[i] = j < n ? __builtin_nontemporal_load(buf + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        if (j < n) {
            u32x4 w;
            for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, v[i][e]) + 0.0f);
            __builtin_nontemporal_store(w, buf + j);
        }
    }
}

int64_t blocks_for(int64_t n, int per_lane) { return (n + (int64_t)kThreads * per_lane - 1) / ((int64_t)kThreads * per_lane); }

template <int U>
void launch_copy(const void *src, void *dst, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL((stream_copy<U>), dim3((unsigned)blocks_for(n, U)), dim3(kThreads), 0, stream,
                       (const u32x4 *)src, (u32x4 *)dst, n);
}

template <int U>
void launch_rmw(void *buf, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL((stream_rmw<U>), dim3((unsigned)blocks_for(n, U)), dim3(kThreads), 0, stream, (u32x4 *)buf, n);
}

}  // namespace

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned) from src to
// dst on `stream`, per_lane (1, 4 or 16) 16-byte accesses per lane.  Returns
// 0, or -1 for bad arguments, -4 for a launch error.
CEIL_EXPORT int ceiling_stream_copy(const void *src, void *dst, int64_t bytes, int per_lane, void *stream) {
    if (!src || !dst || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    const int64_t n = bytes / 16;
    switch (per_lane) {
        case 1: launch_copy<1>(src, dst, n, (hipStream_t)stream); break;
        case 4: launch_copy<4>(src, dst, n, (hipStream_t)stream); break;
        case 16: launch_copy<16>(src, dst, n, (hipStream_t)stream); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Read and rewrite `bytes` of fp32 words in place (x + 0), per_lane as above.
CEIL_EXPORT int ceiling_stream_rmw(void *buf, int64_t bytes, int per_lane, void *stream) {
    if (!buf || bytes <= 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
    const int64_t n = bytes / 16;
    switch (per_lane) {
        case 1: launch_rmw<1>(buf, n, (hipStream_t)stream); break;
        case 4: launch_rmw<4>(buf, n, (hipStream_t)stream); break;
        case 16: launch_rmw<16>(buf, n, (hipStream_t)stream); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
