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

// Element k of an index or offset array of the launch's width (a branch on a
// kernel argument, the same for every lane).
__device__ __forceinline__ int64_t ld_index(const void* base, int64_t k, int idx32) {
    if (idx32) return (int64_t) static_cast<const int32_t*>(base)[k];
    return static_cast<const int64_t*>(base)[k];
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
