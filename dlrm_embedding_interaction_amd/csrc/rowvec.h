// rowvec.h -- row access helpers shared by the gfx950 bag / interaction
// kernels: 16-byte (float4) or 4-byte element vectors, the lane-group shape
// that covers one embedding row, and the host-side dispatch over it.
#pragma once

#include "dlrm_device.h"

namespace dlrm {

template <int VEC> struct Vec;
template <> struct Vec<4> {
    using T = float4;
    static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ T load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    // a row of a table or of x in global memory (see ld_global)
    static __device__ __forceinline__ T gload(const float* p) {
        const floatx4 v = ld_global<floatx4>(p);
        return make_float4(v[0], v[1], v[2], v[3]);
    }
    static __device__ __forceinline__ void store(float* p, T v) { *reinterpret_cast<float4*>(p) = v; }
    static __device__ __forceinline__ T add(T a, T b) { return f4_add(a, b); }
    static __device__ __forceinline__ float dot(T a, T b, float acc) { return f4_dot(a, b, acc); }
    static __device__ __forceinline__ T fma(float w, T v, T acc) {
        return make_float4(fmaf(w, v.x, acc.x), fmaf(w, v.y, acc.y), fmaf(w, v.z, acc.z), fmaf(w, v.w, acc.w));
    }
    static __device__ __forceinline__ T max(T a, T b) {
        return make_float4(fmaxf(a.x, b.x), fmaxf(a.y, b.y), fmaxf(a.z, b.z), fmaxf(a.w, b.w));
    }
    static __device__ __forceinline__ T div(T a, float d) { return make_float4(a.x / d, a.y / d, a.z / d, a.w / d); }
    static __device__ __forceinline__ T splat(float v) { return make_float4(v, v, v, v); }
};
template <> struct Vec<1> {
    using T = float;
    static __device__ __forceinline__ T zero() { return 0.f; }
    static __device__ __forceinline__ T load(const float* p) { return *p; }
    static __device__ __forceinline__ T gload(const float* p) { return ld_global<float>(p); }
    static __device__ __forceinline__ void store(float* p, T v) { *p = v; }
    static __device__ __forceinline__ T add(T a, T b) { return a + b; }
    static __device__ __forceinline__ float dot(T a, T b, float acc) { return fmaf(a, b, acc); }
    static __device__ __forceinline__ T fma(float w, T v, T acc) { return fmaf(w, v, acc); }
    static __device__ __forceinline__ T max(T a, T b) { return fmaxf(a, b); }
    static __device__ __forceinline__ T div(T a, float d) { return a / d; }
    static __device__ __forceinline__ T splat(float v) { return v; }
};

// ---- host side ---------------------------------------------------------------

static inline int pow2_at_least(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Picks VEC, G, C for row length D and whether 16-byte access is allowed.
struct RowShape {
    int vec, g, c;
};
static inline RowShape row_shape(int D, bool aligned16) {
    RowShape r;
    r.vec = (aligned16 && D % 4 == 0) ? 4 : 1;
    const int units = D / r.vec;
    if (r.vec == 4) {
        r.g = units <= 64 ? pow2_at_least(units) : 64;
        r.c = (units + r.g - 1) / r.g;
        r.c = pow2_at_least(r.c);
    } else {
        r.g = 64;
        r.c = pow2_at_least((units + 63) / 64);
    }
    return r;
}

// Dispatch over (VEC, G, C) with a functor template F<VEC, G, C>.
#define DLRM_DISPATCH_ROW(rs, CALL)                                        \
    do {                                                                   \
        if ((rs).vec == 4) {                                               \
            switch ((rs).g * 16 + ((rs).c > 1 ? (rs).c : 0)) {             \
                case 1 * 16: { CALL(4, 1, 1); }                            \
                case 2 * 16: { CALL(4, 2, 1); }                            \
                case 4 * 16: { CALL(4, 4, 1); }                            \
                case 8 * 16: { CALL(4, 8, 1); }                            \
                case 16 * 16: { CALL(4, 16, 1); }                          \
                case 32 * 16: { CALL(4, 32, 1); }                          \
                case 64 * 16: { CALL(4, 64, 1); }                          \
                case 64 * 16 + 2: { CALL(4, 64, 2); }                      \
                case 64 * 16 + 4: { CALL(4, 64, 4); }                      \
                default: return hipErrorInvalidValue;                      \
            }                                                              \
        } else {                                                           \
            switch ((rs).c) {                                              \
                case 1: { CALL(1, 64, 1); }                                \
                case 2: { CALL(1, 64, 2); }                                \
                case 4: { CALL(1, 64, 4); }                                \
                case 8: { CALL(1, 64, 8); }                                \
                case 16: { CALL(1, 64, 16); }                              \
                default: return hipErrorInvalidValue;                      \
            }                                                              \
        }                                                                  \
    } while (0)

}  // namespace dlrm
