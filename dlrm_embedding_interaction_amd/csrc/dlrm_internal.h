// dlrm_internal.h -- host-side launch functions shared between the kernel
// sources and the C-ABI entry points of the DLRMv1 forward library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "dlrm_device.h"

namespace dlrm {

constexpr int kMaxDim = 1024;                       // longest embedding row supported
constexpr size_t kInteractLdsBudget = 32 * 1024;     // target LDS per interaction block
constexpr size_t kMaxLdsBytes = 64 * 1024;           // hard LDS limit per block
constexpr int kRowPad = 4;                           // floats of padding per LDS feature row

// Single-launch forward limits: Linear layers per MLP, samples per block, LDS
// per block (gfx950 gives a workgroup up to 160 KiB).
constexpr int kFusedMaxLayers = 8;
constexpr int kFusedSamples = 8;
constexpr int kMfmaDotsMinTables = 24;           // single launch: MFMA dots for this many tables up to 32
constexpr int kFusedThreads = 512;
constexpr size_t kFusedMaxLds = 160 * 1024;

// A kernel's dynamic-LDS limit is raised to the whole 160 KiB once per kernel
// and device, by whichever thread launches it there first (std::call_once:
// concurrent first launches wait for that one call).
template <typename Kernel>
hipError_t allow_full_lds(Kernel* k) {
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static hipError_t result[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    auto set = [&] {
        return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFusedMaxLds);
    };
    if (dev < 0 || dev >= kMaxDevices) return set();
    std::call_once(once[dev], [&] { result[dev] = set(); });
    return result[dev];
}

// One MLP of the single-launch forward: layer l maps dim[l] -> dim[l + 1]
// with packed weights w[l] (pack_layer_kernel layout) and bias b[l].
struct MlpArgs {
    const float* w[kFusedMaxLayers];
    const float* b[kFusedMaxLayers];
    int dim[kFusedMaxLayers + 1];
    int n_layers;
};

// Kernel arguments of the single-launch forward (about 2.5 KiB).
struct FusedArgs {
    TableArgs ta;
    MlpArgs bot, top;
    const float* small;   // packed tail: last layer's weights and bias, hidden biases (small_block_floats)
    int n_small;
    const float* packed;  // start of the packed weights and their length in floats
    int64_t n_packed;
    const float* dense;
    float* out;
    int64_t B;
    int T, D;
    int lda;     // row stride of the LDS activation buffers (set by the launcher)
    int dsplit;  // d split of the interaction dots (set by the launcher)
};

// Arguments of the device-side bag-data check.
struct CheckArgs {
    const void* idx[DLRM_MAX_TABLES];
    const void* off[DLRM_MAX_TABLES];
    int64_t nidx[DLRM_MAX_TABLES];
    int64_t rows[DLRM_MAX_TABLES];
    int idx32;
};

// Arguments of the general bag kernel (3 KiB of kernel arguments).
struct BagArgs {
    const float* w[DLRM_MAX_TABLES];
    const void* idx[DLRM_MAX_TABLES];     // int32 or int64, per the launch
    const void* off[DLRM_MAX_TABLES];
    int64_t nidx[DLRM_MAX_TABLES];
    const float* psw[DLRM_MAX_TABLES];    // per-sample weights or NULL
    int64_t pad[DLRM_MAX_TABLES];         // padding index or -1
};

bool row_shape_supported(int D);
int interact_samples_per_block(int T, int D, int64_t B);
size_t interact_lds_bytes(int T, int D, int spb);

// Bags of T tables into out (B, T, D).  aligned16: every table row and the
// output allow 16-byte access.  multi_hot: bags hold more than one index on
// average (selects deeper per-bag prefetch).
hipError_t launch_embbag_sum(const TableArgs& ta, int T, int D, int64_t B, bool aligned16, bool multi_hot,
                             float* out, hipStream_t s);

// Interaction over [x, E_0..E_{T-1}] writing Z to out[:, col_z:col_z+P] and,
// when col_x >= 0, x to out[:, col_x:col_x+D].  With ta != NULL the E rows
// are gathered from the tables (fused path); otherwise read from emb (B, T, D).
hipError_t launch_interact(const TableArgs* ta, const float* emb, int T, int D, int64_t B, bool aligned16,
                           bool multi_hot, const float* x, int64_t ld_x, float* out, int64_t ld_out, int col_x,
                           int col_z, hipStream_t s);

// Bags of one index and the interaction as a Gram matrix on the matrix cores,
// for up to 32 tables and rows of 32, 64 or 128 floats (16-byte aligned
// tables and x); Z to out[:, col_z:col_z+P], x to out[:, col_x:] when col_x >= 0.
bool gram_interact_supported(int T, int D, bool aligned16);
hipError_t launch_gram_interact(const TableArgs& ta, int T, int D, int64_t B, bool aligned16, const float* x,
                                int64_t ld_x, float* out, int64_t ld_out, int col_x, int col_z, hipStream_t s);

// General bags (mode, weights, include_last_offset, padding) into out (B, T, D).
hipError_t launch_embbag_ex(const BagArgs& ba, int T, int D, int64_t B, int mode, int last_off, bool idx32,
                            bool aligned16, bool multi_hot, float* out, hipStream_t s);

// Whole forward in one launch (kFusedSamples samples per block).  Returns
// hipErrorInvalidValue when the model is outside fused_supported.
bool fused_supported(const FusedArgs& fa, bool aligned16);
size_t fused_lds_bytes(const FusedArgs& fa, int samples);
hipError_t launch_fused_forward(FusedArgs fa, bool aligned16, bool multi_hot, hipStream_t s);
// Floats of one packed (N, K) layer, rounded up to 256 bytes, and its packing.
size_t packed_layer_floats(int N, int K);
hipError_t launch_pack_layer(const float* W, int N, int K, float* packed, hipStream_t s);

// The packed tail the single-launch kernel copies to LDS at its start: the
// one-output last layer's weights (k_last floats, rounded up to 4), its bias
// (4 floats), then the biases of every hidden layer (each rounded up to 4).
struct SmallBlock {
    const float* src[2 * kFusedMaxLayers + 2];
    int len[2 * kFusedMaxLayers + 2];
    int off[2 * kFusedMaxLayers + 2];
    int nseg;
    int total;  // floats, a multiple of 4
};
hipError_t launch_pack_small(const SmallBlock& sb, float* dst, hipStream_t s);

hipError_t launch_check_indices(const CheckArgs& ca, int T, int64_t B, int32_t* bad, hipStream_t s);

hipError_t launch_pair_index_map(int F, int32_t* i_out, int32_t* j_out, hipStream_t s);

// Measurement kernels: a sequential float4 read of n_floats (a multiple of 4)
// and a gather of n rows of `dim` floats (dim / 4 in {4, 8, 16, 32, 64}) picked
// by idx; sink holds probe_blocks() floats and is written only in theory.
int probe_blocks();
hipError_t launch_read_stream(const float* src, int64_t n_floats, float* sink, hipStream_t s);
hipError_t launch_l2_stream(const float* src, int64_t n_floats, int blocks, float* sink, hipStream_t s);
hipError_t launch_gather_rows(const float* table, int dim, const int64_t* idx, int64_t n, float* sink,
                              hipStream_t s);

// y = act(x W^T + bias): MFMA for N > 1, a dot-product kernel for N == 1.
hipError_t launch_linear(int64_t M, int64_t N, int64_t K, const float* x, int64_t ld_x, const float* W,
                         const float* bias, int act, float* y, int64_t ld_y, hipStream_t s);

}  // namespace dlrm
