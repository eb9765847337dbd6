// Device-side helpers shared by the GDN kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 -> fp32 is a shift; fp32 -> bf16 uses the gfx950
// packed convert (round to nearest even).
// ---------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Streaming 16-byte fp32 access (nontemporal hint) for data that a launch
// reads once and writes once, such as the recurrent state: it is not kept in
// the caches for reuse that never comes.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 load_stream4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void store_stream4(float *p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

// streaming 16-byte access to 8 bf16 (a row slice read or written once)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint16_t *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// unpack 8 bf16 (one 16-byte vector) into fp32
__device__ __forceinline__ void unpack8(const uint4 &v, float *f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float *f) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

// ---------------------------------------------------------------------------
// Cross-lane sums inside aligned groups of 4 or 8 lanes with DPP.  Every lane
// of a group ends with the same, bit-identical total: each step adds a
// partner's value (x + y == y + x), and the partners pair up symmetrically.
// ---------------------------------------------------------------------------
enum : int {
    kDppQuadXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141,  // lane j <- lane 7-j within each 8 lanes
};

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
    return x + __builtin_bit_cast(float, y);
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 4 || G == 8, "group of 4 or 8 lanes");
    if constexpr (G == 8) x = dpp_add<kDppRowHalfMirror>(x);
    x = dpp_add<kDppQuadXor1>(x);
    x = dpp_add<kDppQuadXor2>(x);
    return x;
}

// ---------------------------------------------------------------------------
// A sequence's token range from query_start_loc, clamped to [0, num_tokens)
// with hi >= lo.  For a well-formed query_start_loc this is the identity; a
// malformed one gives wrong results but no access outside the token rows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void clamp_range(int lo_raw, int hi_raw, int num_tokens, int &lo, int &hi) {
    lo = min(max(lo_raw, 0), num_tokens);
    hi = min(max(hi_raw, lo), num_tokens);
}

// ---------------------------------------------------------------------------
// XCD-aware block order.  The dispatcher hands consecutive workgroup ids to
// the 8 XCDs in turn; this maps them so that each XCD receives one
// contiguous range of work items (neighbouring items share its L2).  A
// bijection on [0, n) for any n.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

// dword 3 of a raw (unstructured) buffer resource on gfx950.  A buffer access
// whose offset lies at or past the resource's byte range is dropped (store)
// or returns zero (load): masked accesses without a branch.
constexpr int kBufferFlags = 0x00020000;
// cache-policy operand of the buffer builtins for a streaming (nt) access
constexpr int kBufferStream = 2;
// cache-policy operand for a store written through the L2 (sc1, device
// scope): the line stays in the writing XCD's L2 for a reader there, and is
// not left dirty for the end of the kernel to write back
constexpr int kBufferWriteThrough = 16;

__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
    const int xcd = bid % kNumXcd;
    const int local = bid / kNumXcd;
    const int q = n / kNumXcd, r = n % kNumXcd;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + local;
}

}  // namespace gdn
