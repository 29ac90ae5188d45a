// dlrm_device.h -- device-side helpers shared by the gfx950 kernels of the
// DLRMv1 forward library: kernel-argument structs, lane-group reductions over
// DPP / ds_swizzle, and the closed-form decoding of a flat pair index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dlrm_mi355x.h"

namespace dlrm {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kBlock = 256;        // threads per block of the gather / interaction kernels

// Per-table pointers of one multi-table bag launch, passed by value in the
// kernel arguments (64 tables x 4 x 8 bytes = 2 KiB).  Indices and offsets
// are all int32 (idx32 != 0) or all int64.
struct TableArgs {
    const float* w[DLRM_MAX_TABLES];
    const void* idx[DLRM_MAX_TABLES];
    const void* off[DLRM_MAX_TABLES];
    int64_t nidx[DLRM_MAX_TABLES];
    int idx32;
};

typedef float floatx4 __attribute__((ext_vector_type(4)));

// A load through a pointer into global memory that the compiler cannot place
// by itself (pointers kept in per-lane-indexed kernel-argument arrays or in
// LDS): the cast makes it a global load, counted by vmcnt alone.  Through a
// generic pointer it would be a flat load, which the compiler must also wait
// for before every later LDS access.
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}

// Element k of an index or offset array of element type IT.  The hot loops
// take IT as a template argument, chosen once per phase: a width test at
// every load splits the loads into separate blocks, and the compiler then
// waits for each one before the next is issued.
template <typename IT>
__device__ __forceinline__ int64_t ld_idx(const void* base, int64_t k) {
    return (int64_t)ld_global<IT>(static_cast<const IT*>(base) + k);
}
// The same with the width a runtime value (off the hot loops).
__device__ __forceinline__ int64_t ld_index(const void* base, int64_t k, int idx32) {
    if (idx32) return ld_idx<int32_t>(base, k);
    return ld_idx<int64_t>(base, k);
}

// ---- lane-group sums ---------------------------------------------------------
// Sum of v over aligned groups of G lanes (G a power of two <= 64); every lane
// of a group receives the same, bitwise-identical total.  Within a 16-lane
// DPP row the butterfly uses quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_mirror; the 32-lane step uses ds_swizzle in
// bit-mask mode (xor 16) and the 64-lane step a cross-half permute.

__device__ __forceinline__ float dpp_quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_half_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_mirror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}
__device__ __forceinline__ float swizzle_xor16(float v) {
    // offset bits: and_mask = 0x1F, or_mask = 0, xor_mask = 0x10
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G must be a power of two <= 64");
    if constexpr (G >= 2) v += dpp_quad_xor1(v);
    if constexpr (G >= 4) v += dpp_quad_xor2(v);
    if constexpr (G >= 8) v += dpp_row_half_mirror(v);
    if constexpr (G >= 16) v += dpp_row_mirror(v);
    if constexpr (G >= 32) v += swizzle_xor16(v);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// ---- flat pair index ---------------------------------------------------------
// p = i(i-1)/2 + j with 0 <= j < i enumerates the strict lower triangle in
// row-major order.  i = floor((1 + sqrt(1 + 8p)) / 2) is first estimated in
// fp32, then corrected with exact integer comparisons so that rounding of the
// square root can never move a pair to a neighbouring row.
__device__ __forceinline__ void pair_from_flat(int p, int& i, int& j) {
    int r = (int)((1.0f + sqrtf((float)(8 * p + 1))) * 0.5f);
    while (r * (r - 1) / 2 > p) --r;
    while ((r + 1) * r / 2 <= p) ++r;
    i = r;
    j = p - r * (r - 1) / 2;
}

__device__ __forceinline__ float4 f4_add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float f4_dot(float4 a, float4 b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
    return acc;
}

}  // namespace dlrm
