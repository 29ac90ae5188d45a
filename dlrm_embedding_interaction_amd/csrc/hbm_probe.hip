// hbm_probe.hip -- three measurement kernels that set the ceilings the
// forward's kernels are judged against on gfx950:
//
//  * read_stream_kernel: a plain sequential read of a large buffer, 16 bytes
//    per lane (global_load_dwordx4), 8 loads in flight per lane, blocks
//    striding over the whole buffer.  Its rate is the HBM read ceiling this
//    library can reach (the datasheet's 8 TB/s is the other bound).
//  * l2_stream_kernel: every block reads the same buffer, which then stays
//    in L2; one block per CU gives the rate at which a CU pulls L2-resident
//    data, the bound of the single-launch forward's weight stream.
//  * gather_rows_kernel: reads rows of `dim` floats picked by an index list,
//    one row per group of dim/4 lanes, 8 rows in flight per group, and adds
//    them up.  With uniform random indices over a table much larger than the
//    caches it is the ceiling for random-row embedding gathers, the access
//    pattern of the bag sums (a bag of one index is one row gather).
//
// No kernel here writes memory except one float per block, behind a test on
// the loaded data that never passes for finite sums of finite data, so the
// loads cannot be removed and the traffic counted is the reads alone.
#include "dlrm_device.h"
#include "dlrm_internal.h"

namespace dlrm {

namespace {

constexpr int kProbeUnroll = 8;
constexpr float kNever = -3.0e38f;  // a finite sum of finite table data never equals it exactly

__global__ __launch_bounds__(kBlock) void read_stream_kernel(const float4* __restrict__ src, int64_t n4,
                                                             float* __restrict__ sink) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t chunk = (int64_t)kBlock * kProbeUnroll;
    const int64_t stride = (int64_t)gridDim.x * chunk;
    int64_t i = (int64_t)blockIdx.x * chunk + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kBlock < n4; i += stride) {
        float4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * kBlock];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc = f4_add(acc, v[u]);
    }
    for (; i < n4; i += kBlock) acc = f4_add(acc, src[i]);
    const float s = (acc.x + acc.y) + (acc.z + acc.w);
    if (s == kNever) sink[blockIdx.x] = s;
}

template <int G>
__global__ __launch_bounds__(kBlock) void gather_rows_kernel(const float* __restrict__ table, int dim,
                                                             const int64_t* __restrict__ idx, int64_t n,
                                                             float* __restrict__ sink) {
    constexpr int NG = kBlock / G;
    const int lg = threadIdx.x % G;
    const int64_t group = (int64_t)blockIdx.x * NG + threadIdx.x / G;
    const int64_t ngroups = (int64_t)gridDim.x * NG;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t r0 = group; r0 < n; r0 += ngroups * kProbeUnroll) {
        int64_t row[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t r = r0 + u * ngroups;
            row[u] = r < n ? idx[r] : -1;
        }
        float4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = row[u] >= 0 ? *reinterpret_cast<const float4*>(table + row[u] * dim + 4 * lg)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc = f4_add(acc, v[u]);
    }
    const float s = (acc.x + acc.y) + (acc.z + acc.w);
    if (s == kNever) sink[blockIdx.x] = s;
}

// Every block reads the whole of src (n4 float4), 8 waves x 1 KiB per load
// with 8 loads in flight per lane: with src resident in L2, the rate of one
// block is the L2 -> CU rate of the single-launch forward's weight stream.
__global__ __launch_bounds__(512) void l2_stream_kernel(const float4* __restrict__ src, int64_t n4,
                                                        float* __restrict__ sink) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int64_t chunk = 512 * kProbeUnroll;
    int64_t i = threadIdx.x;
    for (; i + (kProbeUnroll - 1) * 512 < n4; i += chunk) {
        float4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * 512];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc = f4_add(acc, v[u]);
    }
    for (; i < n4; i += 512) acc = f4_add(acc, src[i]);
    const float s = (acc.x + acc.y) + (acc.z + acc.w);
    if (s == kNever) sink[blockIdx.x % 2048] = s;
}

}  // namespace

int probe_blocks() { return 256 * 8; }

hipError_t launch_l2_stream(const float* src, int64_t n_floats, int blocks, float* sink, hipStream_t s) {
    hipLaunchKernelGGL(l2_stream_kernel, dim3((unsigned)blocks), dim3(512), 0, s, reinterpret_cast<const float4*>(src),
                       n_floats / 4, sink);
    return hipGetLastError();
}

hipError_t launch_read_stream(const float* src, int64_t n_floats, float* sink, hipStream_t s) {
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)probe_blocks()), dim3(kBlock), 0, s,
                       reinterpret_cast<const float4*>(src), n_floats / 4, sink);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const float* table, int dim, const int64_t* idx, int64_t n, float* sink,
                              hipStream_t s) {
    const int g = dim / 4;
    // enough groups for 8 rows in flight each and a full chip, no more blocks than the sink holds
    switch (g) {
#define PROBE_G(G_)                                                                                   \
    case G_:                                                                                          \
        hipLaunchKernelGGL(gather_rows_kernel<G_>, dim3((unsigned)probe_blocks()), dim3(kBlock), 0, s, \
                           table, dim, idx, n, sink);                                                 \
        return hipGetLastError();
        PROBE_G(4)
        PROBE_G(8)
        PROBE_G(16)
        PROBE_G(32)
        PROBE_G(64)
#undef PROBE_G
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dlrm
