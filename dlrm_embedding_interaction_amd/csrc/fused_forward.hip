// fused_forward.hip -- the whole DLRMv1 forward in one launch on gfx950.
//
// The pages' fastest path runs one kernel per forward ("dlrm --mega" on
// "luminal compare dlrm-fused-kernels...dlrm-pt2-megakernel": module doc of
// dlrm_megakernel.rs and cuda_source steps 1-7): bottom MLP with ReLU after
// every layer, bags, stacked features with x first, strict-lower-triangle
// dots, R = [x | Z], top MLP with ReLU on hidden layers and a sigmoid on the
// one-output last layer.  There one thread carries one sample through the
// whole network in registers; with 512-wide layers that cannot fit, so here a
// block of eight waves carries S samples:
//
//  * activations live in LDS, two (S, lda) ping-pong buffers, the S feature
//    stacks in a third region (S, F, D + 4);
//  * every Linear layer streams its weight rows straight from L2 into
//    registers (each weight is read once per block and used for all S
//    samples) and multiplies them on the matrix cores with
//    v_mfma_f32_4x4x1f32, one instruction being 16 blocks of 4x4x1:
//    - layers of more than 128 outputs: the instruction's A-broadcast field
//      (CBSZ = 1) lets both blocks of each pair take the weights of one of
//      them (ABID 0 or 1), so lane l = 8 m + 4 h + i holds W[4 m + i][k] for
//      two values of k (h = 0, 1), every lane holds act[sample l % 8][k] as
//      B, and one instruction covers 32 features x 8 samples x 1 k with the
//      outputs complete in the lanes (4 consecutive features of one sample);
//    - narrower layers: lane l = 16 fg + 4 kg + e supplies
//      W[f = 4 fg + e][k = 4 kg + q] as A and act[sample e][k] as B, one
//      instruction covering 16 features x 4 samples x 4 k values; the 4 k
//      groups are added afterwards with two DPP row rotations;
//  * the bags are gathered with the same lane-group code as the standalone
//    bag kernel, scheduled where waves would otherwise wait: from 8 tables
//    by waves 4-7 beside the whole bottom MLP on waves 0-3; below that, when
//    the last bottom layer has at most 64 outputs (waves 4-7 idle in it),
//    either wholly beside that layer (more bags than lane groups) or split,
//    bounds and indices at kernel start and the rows beside it;
//  * the dots reuse the interaction kernel's LDS routine, or one 32x32x2
//    MFMA tile per sample from 24 to 32 tables;
//  * nothing leaves the block but the S sigmoid outputs.
//
// Samples are independent, so blocks never communicate; the weights of one
// forward (a few MB) stay resident in every XCD's L2.
#include "dlrm_device.h"
#include "dlrm_internal.h"
#include "rowvec.h"
#include "bag_dots.h"

namespace dlrm {

// Raw buffer loads of the packed weights: a load whose offset lies past the
// buffer's size returns zeros without a memory access, so a step past a
// layer's last chunk still issues its loads (every wait keeps counting
// exactly) but costs no cache traffic.  Word 3 of the resource is the gfx9
// family's raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;
__device__ __forceinline__ floatx4 buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return __builtin_bit_cast(floatx4, v);
}

// Rotations by 4 and 8 lanes within each 16-lane row.
__device__ __forceinline__ float dpp_row_ror4(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_ror8(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

// out[s][c] = 0 for s < S and c in [c0, c1) (threads 0 .. NT-1 of the block).
template <int S, int NT = kFusedThreads>
__device__ __forceinline__ void zero_columns(float* out, int ldo, int c0, int c1) {
    const int w = c1 - c0;
    for (int i = threadIdx.x; i < S * w; i += NT) {
        const int s = i / w;
        lds_store(out + s * ldo + c0 + (i - s * w), 0.f);
    }
}

// Packed weights of one layer (N, K), zeros past N or K; each chunk is 64
// lanes x 4 floats (1 KiB, one wave load):
//  * narrow layers (N <= 128): tiles of 16 output features x 16 inputs, chunk
//    (t, kc) at float offset (t * ceil(K / 16) + kc) * 256, holding for lane
//    l = 16 fg + 4 kg + e the weights W[16 t + 4 fg + e][16 kc + 4 kg + q];
//  * wide layers (N > 128): tiles of 32 output features x 8 inputs, chunk
//    (t, kc) at float offset (t * ceil(K / 8) + kc) * 256, holding for lane
//    l = 8 m + 4 h + i the weights W[32 t + 4 m + i][8 kc + 4 h + q];
// q = 0..3.  A narrow layer of 64 outputs keeps 4 tiles for 8 waves, where 32-wide tiles
// would leave 6 of them idle.
__host__ __device__ inline bool wide_tiles(int N) { return N > 128; }

__global__ __launch_bounds__(kBlock) void pack_layer_kernel(const float* __restrict__ W, int N, int K,
                                                            float* __restrict__ packed) {
    const bool wide = wide_tiles(N);
    const int nkc = wide ? (K + 7) >> 3 : (K + 15) >> 4;
    const int64_t total = (int64_t)(wide ? (N + 31) >> 5 : (N + 15) >> 4) * nkc * 64;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= total) return;
    const int lane = (int)(i & 63);
    const int64_t tk = i >> 6;
    const int t = (int)(tk / nkc);
    const int kc = (int)(tk - (int64_t)t * nkc);
    const int n = wide ? 32 * t + 4 * (lane >> 3) + (lane & 3) : 16 * t + 4 * (lane >> 4) + (lane & 3);
    const int k0 = wide ? 8 * kc + 4 * ((lane >> 2) & 1) : 16 * kc + 4 * ((lane >> 2) & 3);
    floatx4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (n < N && k0 + q < K) ? W[(int64_t)n * K + k0 + q] : 0.f;
    *reinterpret_cast<floatx4*>(packed + i * 4) = v;
}

// out[s][n] = act(sum_k in[s][k] W[n][k] + bias[n]) for s < S, n < N, with in,
// out and bias in LDS (row strides ldi, ldo) and W packed as above (a narrow
// layer, N <= 128).  The N outputs form tiles of 16 features; wave w (of the NW waves 0 .. NW-1 that run the
// layer) takes tiles w, w + NW, ... in passes of TW tiles.  One step covers KU chunks of 16 k values; the weights of a step are
// requested PD steps ahead into a register ring whose slots are fixed at
// compile time (no register copies, so the wait before a step's MFMAs covers
// only that step's loads).  Each load of a wave is 1 KiB of contiguous packed
// weights.  in[s][k] must be zero for k in [K, round_up(K, 64)); on return
// out[s][n] is zero for n in [N, round_up(N, 64)).
template <int S, int TW, int KU, int PD, int NW>
__device__ __forceinline__ void mlp_layer(const float* in, int ldi, int K, const float* __restrict__ Wp,
                                          const float* bias, int N, bool relu, float* out, int ldo) {
    constexpr int SG = S / 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = lane & 3;
    const int kg = (lane >> 2) & 3;
    const int fg = lane >> 4;
    const int ntile = (N + 15) >> 4;
    const int nkc = (K + 15) >> 4;
    const int nkb = (K + 16 * KU - 1) / (16 * KU);
    const float* arow[SG];
#pragma unroll
    for (int sg = 0; sg < SG; ++sg) arow[sg] = in + (4 * sg + e) * ldi + 4 * kg;

    const __amdgpu_buffer_rsrc_t wr = weight_rsrc(Wp, (uint32_t)ntile * nkc * 1024u);
    for (int t0 = 0; t0 < ntile; t0 += NW * TW) {
        // a wave without a tile in this pass (or any later one) is done: its
        // k loop would only issue MFMAs on zeros, on the SIMD it shares with
        // a wave that has work (measured: the 256->64 layer's 4-tile k loop
        // ran ~5000 instead of ~3300 cycles)
        if (t0 + wave >= ntile) break;
        uint32_t wtile[TW];  // byte offset of this lane's first chunk of each tile
        floatx4 acc[TW][SG];
        float bv[TW];
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            // tiles past the last read zeros and are never stored
            const int t = t0 + wave + NW * u;
            wtile[u] = t < ntile ? ((uint32_t)t * nkc * 64u + lane) * 16u : kOutOfRange;
            // the bias of the one output this lane finishes (feature 16 t + 4 fg + kg)
            const int n = 16 * t + 4 * fg + kg;
            bv[u] = lds_load(bias + (n < N ? n : 0));
#pragma unroll
            for (int sg = 0; sg < SG; ++sg) acc[u][sg] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        floatx4 ring[PD][TW][KU];
        // Every step issues the same number of loads, so that each wait counts
        // exactly its own step; chunks past the layer's last are out of range
        // and read as zeros.
        auto loadw = [&](int kb, floatx4 (&w)[TW][KU]) {
#pragma unroll
            for (int u = 0; u < TW; ++u)
#pragma unroll
                for (int c = 0; c < KU; ++c) {
                    const int ch = kb * KU + c;
                    w[u][c] = buffer_load4(wr, ch < nkc ? wtile[u] + (uint32_t)ch * 1024u : kOutOfRange);
                }
        };
        auto step = [&](int kb, const floatx4 (&w)[TW][KU]) {
            floatx4 a[KU][SG];
#pragma unroll
            for (int c = 0; c < KU; ++c)
#pragma unroll
                for (int sg = 0; sg < SG; ++sg) a[c][sg] = lds_load4(arow[sg] + (kb * KU + c) * 16);
#pragma unroll
            for (int c = 0; c < KU; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < TW; ++u)
#pragma unroll
                        for (int sg = 0; sg < SG; ++sg)
                            acc[u][sg] =
                                __builtin_amdgcn_mfma_f32_4x4x1f32(w[u][c][q], a[c][sg][q], acc[u][sg], 0, 0, 0);
        };
#pragma unroll
        for (int p = 0; p < PD; ++p) loadw(p, ring[p]);
        // whole trips of PD steps (a loop with a single exit, so the waits
        // before each step count only that step's loads), then the rest;
        // refills past the last chunk are out of range
        const int trips = nkb / PD;
        for (int tr = 0; tr < trips; ++tr) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int kb = tr * PD + p;
                step(kb, ring[p]);
                loadw(kb + PD, ring[p]);
            }
        }
        const int rest = nkb - trips * PD;
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (p < rest) step(trips * PD + p, ring[p]);
        // VGPR r of lane 16 fg + 4 kg + e holds the partial sum over the k
        // group kg for feature 16 t + 4 fg + r and sample 4 sg + e.  Two row
        // rotations (by 4, then 8 lanes) leave the total over kg in all four
        // lanes of a group; lane kg then finishes feature 16 t + 4 fg + kg,
        // so that every lane does one output's bias, activation and store.
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int t = t0 + wave + NW * u;
            if (t >= ntile) break;
            const int n = 16 * t + 4 * fg + kg;
#pragma unroll
            for (int sg = 0; sg < SG; ++sg) {
                floatx4 v = acc[u][sg];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] += dpp_row_ror4(v[r]);
                    v[r] += dpp_row_ror8(v[r]);
                }
                // v[kg], as two levels of selects (no branches)
                const float lo = (kg & 1) ? v[1] : v[0];
                const float hi = (kg & 1) ? v[3] : v[2];
                float y = (kg & 2) ? hi : lo;
                y += bv[u];
                y = relu ? fmaxf(y, 0.f) : y;
                lds_store(out + (4 * sg + e) * ldo + n, n < N ? y : 0.f);
            }
        }
    }
    zero_columns<S, 64 * NW>(out, ldo, (N + 15) & ~15, (N + 63) & ~63);
}

// The same for a layer packed in 32-wide tiles (more than 128 outputs).  Each
// instruction multiplies 32 features by one k for 8 samples: A-broadcast
// (CBSZ = 1) hands each pair of blocks (one pair per 4 features) the weights
// held by one of them, ABID 0 taking the lanes of the 4 k values of chunk
// half h = 0 and ABID 1 those of h = 1, and every lane's B is its own sample
// l % 8.  A step reads, per chunk and group of 8 samples, two float4 of
// activations per lane (k 0-3 and 4-7 of the chunk).  The halves h = 0, 1
// accumulate apart (two independent MFMA chains per tile and group).  Lane
// l = 8 m + 4 sg + j then holds in accumulator register i the complete sum
// for feature 32 t + 4 m + i and sample 8 g + 4 sg + j, so the epilogue is
// bias, activation and one 16-byte LDS store per tile and group, with no
// cross-lane sums.
template <int S, int TW, int KU, int PD, int NW>
__device__ __forceinline__ void mlp_layer_wide(const float* in, int ldi, int K, const float* __restrict__ Wp,
                                          const float* bias, int N, bool relu, float* out, int ldo) {
    static_assert(S % 8 == 0, "groups of 8 samples");
    constexpr int SG = S / 8;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m = lane >> 3;   // outputs 4 m .. 4 m + 3 of a tile
    const int s8 = lane & 7;   // sample s8 of each group of 8
    const int ntile = (N + 31) >> 5;
    const int nkc = (K + 7) >> 3;
    const int nkb = (nkc + KU - 1) / KU;
    const float* arow[SG];
#pragma unroll
    for (int g = 0; g < SG; ++g) arow[g] = in + (8 * g + s8) * ldi;

    const __amdgpu_buffer_rsrc_t wr = weight_rsrc(Wp, (uint32_t)ntile * nkc * 1024u);
    for (int t0 = 0; t0 < ntile; t0 += NW * TW) {
        if (t0 + wave >= ntile) break;
        uint32_t wtile[TW];
        floatx4 acc[TW][SG][2];
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int t = t0 + wave + NW * u;
            wtile[u] = t < ntile ? ((uint32_t)t * nkc * 64u + lane) * 16u : kOutOfRange;
#pragma unroll
            for (int g = 0; g < SG; ++g) acc[u][g][0] = acc[u][g][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        floatx4 ring[PD][TW][KU];
        auto loadw = [&](int kb, floatx4 (&w)[TW][KU]) {
#pragma unroll
            for (int u = 0; u < TW; ++u)
#pragma unroll
                for (int c = 0; c < KU; ++c) {
                    const int ch = kb * KU + c;
                    w[u][c] = buffer_load4(wr, ch < nkc ? wtile[u] + (uint32_t)ch * 1024u : kOutOfRange);
                }
        };
        auto step = [&](int kb, const floatx4 (&w)[TW][KU]) {
            floatx4 a[KU][SG][2];
#pragma unroll
            for (int c = 0; c < KU; ++c)
#pragma unroll
                for (int g = 0; g < SG; ++g)
#pragma unroll
                    for (int h = 0; h < 2; ++h) a[c][g][h] = lds_load4(arow[g] + (kb * KU + c) * 8 + 4 * h);
#pragma unroll
            for (int c = 0; c < KU; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < TW; ++u)
#pragma unroll
                        for (int g = 0; g < SG; ++g) {
                            acc[u][g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(w[u][c][q], a[c][g][0][q], acc[u][g][0], 1, 0, 0);
                            acc[u][g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(w[u][c][q], a[c][g][1][q], acc[u][g][1], 1, 1, 0);
                        }
        };
#pragma unroll
        for (int p = 0; p < PD; ++p) loadw(p, ring[p]);
        const int trips = nkb / PD;
        for (int tr = 0; tr < trips; ++tr) {
#pragma unroll
            for (int p = 0; p < PD; ++p) {
                const int kb = tr * PD + p;
                step(kb, ring[p]);
                loadw(kb + PD, ring[p]);
            }
        }
        const int rest = nkb - trips * PD;
#pragma unroll
        for (int p = 0; p < PD; ++p)
            if (p < rest) step(trips * PD + p, ring[p]);
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int t = t0 + wave + NW * u;
            if (t >= ntile) break;
            const int n = 32 * t + 4 * m;
            const floatx4 bv = n < N ? lds_load4(bias + n) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int g = 0; g < SG; ++g) {
                const floatx4 v = acc[u][g][0] + acc[u][g][1] + bv;
                floatx4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = n + i < N ? (relu ? fmaxf(v[i], 0.f) : v[i]) : 0.f;
                lds_store4(out + (8 * g + s8) * ldo + n, y);
            }
        }
    }
    zero_columns<S, 64 * NW>(out, ldo, (N + 31) & ~31, (N + 63) & ~63);
}

// Layer dispatch: TW = tiles per wave and pass, KU chunks per step and PD
// steps in flight.  Narrow layers (16-wide tiles, chunks of 16 k) of one or
// two tiles per wave keep 2 steps (8 weight loads, 8 KiB per wave) in flight:
// measured on MI355X, deeper rings there leave the waves stalled on the CU's
// vector-memory queue, which holds up their MFMAs too (8 samples: 512->256
// layer 6.9 -> 6.3 us, 256->64 2.6 -> 2.1 us; 16 samples: batch 4096 x 4
// tables 44.3 -> 42.5 us per forward); four-tile layers keep 6 steps.  Wide
// layers (32-wide tiles, chunks of 8 k): one tile per wave keeps 2 steps of 4
// chunks, two tiles 6 steps of one chunk each (12 KiB; 8 and 24 KiB measured
// slower at 8 to 32 tables).
template <int S, int NW = kFusedThreads / 64>
__device__ __forceinline__ void mlp_layer_any(const float* in, int ldi, int K, const float* Wp, const float* bias,
                                              int N, bool relu, float* out, int ldo) {
    if (wide_tiles(N)) {
        const int tw = ((N + 31) / 32 + NW - 1) / NW;
        const int nkc = (K + 7) >> 3;
#define DLRM_WIDE(TW_, KU_, PD_)                                                     \
    {                                                                                \
        mlp_layer_wide<S, TW_, KU_, PD_, NW>(in, ldi, K, Wp, bias, N, relu, out, ldo); \
        return;                                                                      \
    }
        if (tw <= 1) DLRM_WIDE(1, 4, 2)
        if (nkc <= 1) DLRM_WIDE(2, 1, 1)
        if (S > 8 || tw <= 2) DLRM_WIDE(2, 1, 6)
        DLRM_WIDE(4, 1, 6)
#undef DLRM_WIDE
    }
    const int ntile = (N + 15) >> 4;
    const int tw = (ntile + NW - 1) / NW;
#define DLRM_LAYER(TW_, KU_, PD_)                                               \
    {                                                                           \
        mlp_layer<S, TW_, KU_, PD_, NW>(in, ldi, K, Wp, bias, N, relu, out, ldo); \
        return;                                                                 \
    }
    const int nkc = (K + 15) >> 4;
    // short rings for the short layers, so that few steps are padding
    if (tw <= 1) {
        DLRM_LAYER(1, 4, 2)
    }
    if constexpr (S > 8) {
        // 16 samples: two tiles per wave and pass at most (registers)
        if (nkc <= 1) DLRM_LAYER(2, 1, 1)
        DLRM_LAYER(2, 2, 2)
    } else {
        if (tw <= 2) DLRM_LAYER(2, 2, 2)
        if (nkc <= 1) DLRM_LAYER(4, 1, 1)
        DLRM_LAYER(4, 1, 6)
    }
#undef DLRM_LAYER
}

// y[s] = sigmoid(<in[s], w> + b) for the one-output last layer, with w staged
// in LDS: wave w takes samples w, w + NW, ...
template <int S>
__device__ __forceinline__ void last_layer(const float* in, int ldi, int K, const float* w, float b,
                                           float* __restrict__ y, int nb) {
    constexpr int NW = kFusedThreads / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int s = wave; s < nb; s += NW) {
        float acc = 0.f;
        for (int k = lane; k < K; k += 64) acc = fmaf(lds_load(in + s * ldi + k), lds_load(w + k), acc);
        acc = group_sum<64>(acc);
        if (lane == 0) y[s] = 1.f / (1.f + expf(-(acc + b)));
    }
}

// The first bottom layer when its input is at most 16 wide (the dense
// features) and it has at most 128 or more than 512 outputs runs on the
// vector ALUs instead: thread j of the nt threads from t0 computes outputs
// n = j, j + nt, ... for every sample, as a 16-term dot of the sample's
// (zero-padded) input row with the output's packed weights, then bias and
// ReLU.  Its weights are requested at kernel start (first_layer_weights), so
// that they arrive during the bag gather; with 13 inputs the layer is a few
// hundred instructions per thread, where a narrow matrix-core pass would pay a
// ring fill, an epilogue over 32 tiles and a barrier.  (129..512 outputs take
// first_layer_mfma below.)
//
// Output n = 16 t + 4 fg + e sits in lanes 16 fg + 4 kg + e of tile t, which
// hold its inputs 4 kg .. 4 kg + 3 (zero past the input width).
template <int NPRE>
__device__ __forceinline__ void first_layer_weights(const float* __restrict__ Wp, int N, int K, int j, int nt,
                                                    floatx4 (&w)[NPRE][4]) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
        const int n0 = j + i * nt;
        const int n = n0 < N ? n0 : 0;
        if (wide_tiles(N)) {
            const int t = n >> 5, r = n & 31;
            const int nkc = (K + 7) >> 3;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) {
                const int c = kg >> 1;
                w[i][kg] = c < nkc ? ld_global<floatx4>(Wp + (((size_t)t * nkc + c) * 64 + 8 * (r >> 2) + 4 * (kg & 1) + (r & 3)) * 4)
                                   : floatx4{0.f, 0.f, 0.f, 0.f};
            }
        } else {
            const int t = n >> 4, r = n & 15;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
                w[i][kg] = ld_global<floatx4>(Wp + ((size_t)t * 64 + 16 * (r >> 2) + 4 * kg + (r & 3)) * 4);
        }
    }
}

template <int S, int NPRE>
__device__ __forceinline__ void first_layer_valu(const float* in, int ldi, int K0, const float* __restrict__ Wp,
                                                 const float* bias, int N, float* out, int ldo, int t0, int nt,
                                                 const floatx4 (&wpre)[NPRE][4]) {
    const int j = threadIdx.x - t0;
    const int npad = (N + 63) & ~63;
    for (int i = 0; j + i * nt < npad; ++i) {
        const int n = j + i * nt;
        if (n >= N) {
            // columns [N, round_up(N, 64)) the next layer's k steps read
#pragma unroll
            for (int s = 0; s < S; ++s) lds_store(out + s * ldo + n, 0.f);
            continue;
        }
        floatx4 w[4];
        if (i < NPRE) {
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) w[kg] = wpre[i < NPRE ? i : 0][kg];
        } else {
            floatx4 wl[1][4];
            first_layer_weights<1>(Wp, N, K0, n, 0, wl);
#pragma unroll
            for (int kg = 0; kg < 4; ++kg) w[kg] = wl[0][kg];
        }
        const float bv = lds_load(bias + n);
        // sample s + 1's input row is requested before sample s's dots
        floatx4 a[2][4];
#pragma unroll
        for (int kg = 0; kg < 4; ++kg) a[0][kg] = lds_load4(in + 4 * kg);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            if (s + 1 < S) {
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) a[(s + 1) & 1][kg] = lds_load4(in + (s + 1) * ldi + 4 * kg);
            }
            float acc = 0.f;
#pragma unroll
            for (int kg = 0; kg < 4; ++kg)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = fmaf(a[s & 1][kg][q], w[kg][q], acc);
            lds_store(out + s * ldo + n, fmaxf(acc + bv, 0.f));
        }
    }
}

// The first bottom layer on the matrix cores when it has at most 16 inputs
// and 129..512 outputs (32-wide tiles): wave w of the nw waves that run it
// takes tiles w, w + nw, ... (2 NPRE of them), and requests all of their
// weights at kernel start -- two chunks of 8 inputs per tile, in the
// registers the vector-ALU path would use -- so that they arrive during the
// bag gather.  Then one pass of A-broadcast MFMAs as in mlp_layer_wide.
template <int NPRE>
__device__ __forceinline__ void first_layer_mfma_weights(const float* __restrict__ Wp, int N, int K, int wave, int nw,
                                                         floatx4 (&w)[NPRE][4]) {
    const int lane = threadIdx.x & 63;
    const int ntile = (N + 31) >> 5;
    const int nkc = (K + 7) >> 3;
    const __amdgpu_buffer_rsrc_t wr = weight_rsrc(Wp, (uint32_t)ntile * nkc * 1024u);
#pragma unroll
    for (int i = 0; i < 4 * NPRE; ++i) {
        const int t = wave + nw * (i >> 1), c = i & 1;
        w[i >> 2][i & 3] =
            buffer_load4(wr, t < ntile && c < nkc ? ((uint32_t)(t * nkc + c) * 64u + lane) * 16u : kOutOfRange);
    }
}

template <int S, int NPRE>
__device__ __forceinline__ void first_layer_mfma(const float* in, int ldi, const float* bias, int N, float* out,
                                                 int ldo, int wave, int nw, const floatx4 (&w)[NPRE][4]) {
    constexpr int SG = S / 8;
    constexpr int TW = 2 * NPRE;
    const int lane = threadIdx.x & 63;
    const int m = lane >> 3;
    const int s8 = lane & 7;
    const int ntile = (N + 31) >> 5;
    floatx4 acc[TW][SG][2];
#pragma unroll
    for (int u = 0; u < TW; ++u)
#pragma unroll
        for (int g = 0; g < SG; ++g) acc[u][g][0] = acc[u][g][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 a[2][SG][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int g = 0; g < SG; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h) a[c][g][h] = lds_load4(in + (8 * g + s8) * ldi + 8 * c + 4 * h);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < TW; ++u)
#pragma unroll
                for (int g = 0; g < SG; ++g) {
                    const float wq = w[(2 * u + c) >> 2][(2 * u + c) & 3][q];
                    acc[u][g][0] = __builtin_amdgcn_mfma_f32_4x4x1f32(wq, a[c][g][0][q], acc[u][g][0], 1, 0, 0);
                    acc[u][g][1] = __builtin_amdgcn_mfma_f32_4x4x1f32(wq, a[c][g][1][q], acc[u][g][1], 1, 1, 0);
                }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
        const int t = wave + nw * u;
        if (t >= ntile) break;
        const int n = 32 * t + 4 * m;
        const floatx4 bv = n < N ? lds_load4(bias + n) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < SG; ++g) {
            const floatx4 v = acc[u][g][0] + acc[u][g][1] + bv;
            floatx4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = n + i < N ? fmaxf(v[i], 0.f) : 0.f;
            lds_store4(out + (8 * g + s8) * ldo + n, y);
        }
    }
    zero_columns<S, kFusedThreads / NPRE>(out, ldo, (N + 31) & ~31, (N + 63) & ~63);
}

// Waves 0-3 of the block (the MLP team) wait here until all four have
// arrived for the k-th time (k = 1, 2, ...): an arrival counter in LDS, read
// with s_sleep between reads.  The other waves never take part, so the
// block-wide barrier cannot be used.  The wait is bounded (tens of ms), so
// that no wave can be kept forever.
constexpr int kTeamWaves = 4;
constexpr int kTeamMinTables = 8;
constexpr int kTeamSpinLimit = 1 << 20;
__device__ __forceinline__ void team_barrier(unsigned* counter, unsigned k) {
    typedef __attribute__((address_space(3))) unsigned lds_u32;
    lds_u32* c = (lds_u32*)counter;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int spin = 0; spin < kTeamSpinLimit; ++spin) {
        if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= kTeamWaves * k) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// TEAM: the bags are gathered by waves 4-7 while waves 0-3 run the bottom MLP
// (they meet at one block-wide barrier before the interaction), so that the
// gather's chain of dependent loads overlaps the bottom layers; chosen from
// 8 tables up, where the gather outlasts what 4 MLP waves lose against 8.
template <int S, int G, int U, int R, int RT, bool TEAM>
__global__ __launch_bounds__(kFusedThreads) void fused_forward_kernel(FusedArgs fa) {
    using V = Vec<4>;
    constexpr int NT = kFusedThreads;
    constexpr int NG = NT / G;
    extern __shared__ float4 lds4[];
    const int lda = fa.lda;
    const int T = fa.T, D = fa.D;
    const int F = T + 1;
    const int LDR = D + kRowPad;
    // buffers by offset from the LDS array (no pointer array: its address
    // space would be lost)
    float* const lds = reinterpret_cast<float*>(lds4);
    auto buf = [&](int i) { return lds + i * S * lda; };
    float* feat = lds + 2 * S * lda;
    float* wlast = feat + S * F * LDR;  // the packed tail: last layer's weights and bias, hidden biases
    const int klast = fa.top.dim[fa.top.n_layers - 1];
    float* bias_lds = wlast + ((klast + 3) & ~3) + 4;
    const int nbot = fa.bot.n_layers;
    const int ntop = fa.top.n_layers - 1;  // hidden top layers
    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * S;
    const int nb = (int)min((int64_t)S, fa.B - b0);

    unsigned* const team_ctr = reinterpret_cast<unsigned*>(wlast + fa.n_small);
    const int wave = tid >> 6;
    const bool valu0 = fa.bot.dim[0] <= 16;  // the first layer on the vector ALUs
    // ... or, 129 to 512 outputs wide, on the matrix cores
    const bool mfma0 = valu0 && fa.bot.dim[1] > 128 && fa.bot.dim[1] <= 512;

    // 1. dense rows into buffer 0, zeros in its columns [n0, round_up(n0, 64))
    //    that the first layer's 64-wide k steps read past n0 (every layer
    //    writes the zeros past its own width, mlp_layer), and in the rows of
    //    samples past the batch; the last layer's weights into LDS (threads
    //    0 .. nt-1)
    const int n0 = fa.bot.dim[0];
    const int w0 = (n0 + 63) & ~63;
    auto load_dense_and_tail = [&](int nt) {
        for (int i = tid; i < S * w0; i += nt) {
            const int s = i / w0;
            const int k = i - s * w0;
            lds_store(buf(0) + s * lda + k, (s < nb && k < n0) ? fa.dense[(b0 + s) * n0 + k] : 0.f);
        }
        // one contiguous copy, so that no layer waits on a bias load later
        for (int i = tid; i < (fa.n_small >> 2); i += nt)
            lds_store4(wlast + 4 * i, *reinterpret_cast<const floatx4*>(fa.small + 4 * i));
    };

    // 2. bags of this block's samples into feature rows 1..T, by threads
    //    t0 .. t0 + nt - 1
    auto gather_u = [&](auto slots, int t0, int nt) {
        constexpr int UU = decltype(slots)::value;  // bag slots per lane group and pass
        const int tt = tid - t0;
        const int lg = tt % G;
        const int g = tt / G;
        const int ng = nt / G;
        const int nbag = nb * T;
        for (int qb = 0; qb < nbag; qb += ng * UU) {
            int q[UU];
#pragma unroll
            for (int u = 0; u < UU; ++u) {
                const int qq = qb + u * ng + g;
                q[u] = qq < nbag ? qq : -1;
            }
            typename V::T acc[UU][1];
            gather_bags<4, G, 1, UU, R>(fa.ta, T, D, fa.B, b0, q, lg, acc);
#pragma unroll
            for (int u = 0; u < UU; ++u) {
                if (q[u] < 0) continue;
                const int s = q[u] / T;
                const int t = q[u] - s * T;
                if (lg * 4 < D) V::store(feat + ((size_t)s * F + 1 + t) * LDR + lg * 4, acc[u][0]);
            }
        }
    };
    auto gather_all = [&](int t0, int nt) { gather_u(std::integral_constant<int, U>{}, t0, nt); };

    // Split gather (one bag slot per lane group): at kernel start one thread per
    // bag reads its bounds and, for a bag of one index, that index, and leaves
    // the row's address in the first 8 bytes of the bag's feature row (0: an
    // empty bag; -1: a bag of several indices); later fetch_rows copies the
    // rows there.
    auto resolve_rows = [&]() {
        const int nbag = nb * T;
        if (tid < nbag) {
            const int s = tid / T;
            const int t = tid - s * T;
            const int64_t b = b0 + s;
            const int i32 = fa.ta.idx32;
            const int64_t k0 = ld_index(fa.ta.off[t], b, i32);
            const int64_t k1 = b + 1 < fa.B ? ld_index(fa.ta.off[t], b + 1, i32) : fa.ta.nidx[t];
            int64_t addr = k1 == k0 ? 0 : -1;
            if (k1 - k0 == 1) addr = reinterpret_cast<int64_t>(fa.ta.w[t] + ld_index(fa.ta.idx[t], k0, i32) * D);
            lds_store8(reinterpret_cast<int64_t*>(feat + ((size_t)s * F + 1 + t) * LDR), addr);
        }
    };
    // the rows of the resolved bags by threads t0 .. t0 + nt - 1, two bag slots
    // per lane group; a wave holding a bag of several indices sums its bags in
    // full instead
    auto fetch_rows = [&](int t0, int nt) {
        const int tt = tid - t0;
        const int lg = tt % G;
        const int g = tt / G;
        const int ng = nt / G;
        const int nbag = nb * T;
        for (int qb = 0; qb < nbag; qb += 2 * ng) {
            int q[2];
            float* slot[2];
            int64_t addr[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int qq = qb + u * ng + g;
                q[u] = qq < nbag ? qq : -1;
                const int s = q[u] >= 0 ? q[u] / T : 0;
                const int t = q[u] >= 0 ? q[u] - s * T : 0;
                slot[u] = feat + ((size_t)s * F + 1 + t) * LDR;
                addr[u] = q[u] >= 0 ? lds_load8(reinterpret_cast<const int64_t*>(slot[u])) : 0;
            }
            typename V::T v[2][1];
            if (__any(addr[0] < 0 || addr[1] < 0)) {
                gather_bags<4, G, 1, 2, R>(fa.ta, T, D, fa.B, b0, q, lg, v);
            } else {
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    v[u][0] = (addr[u] != 0 && lg * 4 < D) ? V::gload(reinterpret_cast<const float*>(addr[u]) + lg * 4)
                                                          : V::zero();
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (q[u] >= 0 && lg * 4 < D) V::store(slot[u] + lg * 4, v[u][0]);
        }
    };

    // 3. bottom MLP, ReLU after every layer
    int cur = 0;
    int boff = 0;  // this layer's biases in bias_lds
    if constexpr (TEAM) {
        if (tid == 0) lds_store(reinterpret_cast<float*>(team_ctr), 0.f);  // the counter's bits: 0
        __syncthreads();
        if (wave < kTeamWaves) {
            floatx4 w0[2][4];
            if (mfma0)
                first_layer_mfma_weights<2>(fa.bot.w[0], fa.bot.dim[1], fa.bot.dim[0], wave, kTeamWaves, w0);
            else if (valu0)
                first_layer_weights<2>(fa.bot.w[0], fa.bot.dim[1], fa.bot.dim[0], tid, 64 * kTeamWaves, w0);
            load_dense_and_tail(64 * kTeamWaves);
            team_barrier(team_ctr, 1);
            for (int l = 0; l < nbot; ++l) {
                if (l == 0 && mfma0)
                    first_layer_mfma<S, 2>(buf(cur), lda, bias_lds, fa.bot.dim[1], buf(cur ^ 1), lda, wave, kTeamWaves,
                                           w0);
                else if (l == 0 && valu0)
                    first_layer_valu<S, 2>(buf(cur), lda, fa.bot.dim[0], fa.bot.w[0], bias_lds, fa.bot.dim[1], buf(cur ^ 1), lda, 0,
                                           64 * kTeamWaves, w0);
                else
                    mlp_layer_any<S, kTeamWaves>(buf(cur), lda, fa.bot.dim[l], fa.bot.w[l], bias_lds + boff,
                                                 fa.bot.dim[l + 1], true, buf(cur ^ 1), lda);
                boff += (fa.bot.dim[l + 1] + 3) & ~3;
                cur ^= 1;
                if (l + 1 < nbot) team_barrier(team_ctr, (unsigned)l + 2);
            }
        } else {
            gather_all(64 * kTeamWaves, NT - 64 * kTeamWaves);
            for (int l = 0; l < nbot; ++l) {
                boff += (fa.bot.dim[l + 1] + 3) & ~3;
                cur ^= 1;
            }
        }
        __syncthreads();
    } else {
        // Late gather: a last bottom layer of at most 64 outputs (4 tiles)
        // leaves waves 4-7 idle, and they gather the bags beside it instead of
        // all waves before the bottom MLP, when the block has more bags than
        // the 8-wave gather's lane groups (measured at batch 2048: 5-7 tables
        // -2.5 to -3.0 us; at one bag per lane group or fewer it loses up to
        // 0.8 us, the gather then overlapping the kernel's start anyway)
        const bool late = nbot >= 2 && fa.bot.dim[nbot] <= 64 && S * T > NT / G;
        // with one bag slot per lane group the gather is split instead: bounds
        // and indices at kernel start, the rows beside that last layer
        const bool split = U == 1 && R == 1 && nbot >= 2 && fa.bot.dim[nbot] <= 64 && S * T <= NT / G;
        floatx4 w0[1][4];
        if (mfma0)
            first_layer_mfma_weights<1>(fa.bot.w[0], fa.bot.dim[1], fa.bot.dim[0], wave, NT / 64, w0);
        else if (valu0)
            first_layer_weights<1>(fa.bot.w[0], fa.bot.dim[1], fa.bot.dim[0], tid, NT, w0);
        load_dense_and_tail(NT);
        if (split)
            resolve_rows();
        else if (!late)
            gather_all(0, NT);
        __syncthreads();
        for (int l = 0; l < nbot; ++l) {
            if ((late || split) && l + 1 == nbot) {
                if (wave < kTeamWaves)
                    mlp_layer_any<S, kTeamWaves>(buf(cur), lda, fa.bot.dim[l], fa.bot.w[l], bias_lds + boff,
                                                 fa.bot.dim[l + 1], true, buf(cur ^ 1), lda);
                else if (late)
                    gather_u(std::integral_constant<int, 4>{}, 64 * kTeamWaves, NT - 64 * kTeamWaves);
                else
                    fetch_rows(64 * kTeamWaves, NT - 64 * kTeamWaves);
            } else if (l == 0 && mfma0)
                first_layer_mfma<S, 1>(buf(cur), lda, bias_lds, fa.bot.dim[1], buf(cur ^ 1), lda, wave, NT / 64, w0);
            else if (l == 0 && valu0)
                first_layer_valu<S, 1>(buf(cur), lda, fa.bot.dim[0], fa.bot.w[0], bias_lds, fa.bot.dim[1], buf(cur ^ 1), lda, 0, NT,
                                       w0);
            else
                mlp_layer_any<S>(buf(cur), lda, fa.bot.dim[l], fa.bot.w[l], bias_lds + boff, fa.bot.dim[l + 1], true,
                                 buf(cur ^ 1), lda);
            boff += (fa.bot.dim[l + 1] + 3) & ~3;
            __syncthreads();
            cur ^= 1;
        }
    }

    // 4. x into feature row 0 and into R = [x | Z] (the other buffer)
    float* Rb = buf(cur ^ 1);
    for (int i = tid; i < nb * D; i += NT) {
        const int s = i / D;
        const int d = i - s * D;
        const float v = lds_load(buf(cur) + s * lda + d);
        lds_store(feat + (size_t)s * F * LDR + d, v);
        lds_store(Rb + s * lda + d, v);
    }
    __syncthreads();

    // 5. strict-lower-triangle dots into R[:, D:D+P]
    if constexpr (RT == 32) {
        pair_dots_mfma<NT>(feat, F, D, LDR, nb, Rb + D, lda);
    } else if (RT == 0 && nb * (F * (F - 1) / 2) <= NT) {
        // few pairs (few tables): one thread per pair dot, no lane-group sums
        const int P = F * (F - 1) / 2;
        if (tid < nb * P) {
            const int s = tid / P;
            const int p = tid - s * P;
            int i, j;
            pair_from_flat(p, i, j);
            const float* si = feat + ((size_t)s * F + i) * LDR;
            const float* sj = feat + ((size_t)s * F + j) * LDR;
            float acc = 0.f;
            for (int d = 0; d < D; d += 4) {
                const floatx4 a = lds_load4(si + d), b = lds_load4(sj + d);
                acc = fmaf(a[0], b[0], acc);
                acc = fmaf(a[1], b[1], acc);
                acc = fmaf(a[2], b[2], acc);
                acc = fmaf(a[3], b[3], acc);
            }
            lds_store(Rb + s * lda + D + p, acc);
        }
    } else {
        pair_dots<4, G, 1, RT, NT>(feat, F, D, LDR, nb, Rb + D, lda, fa.dsplit);
    }
    zero_columns<S>(Rb, lda, D + F * (F - 1) / 2, (D + F * (F - 1) / 2 + 63) & ~63);
    __syncthreads();
    cur ^= 1;

    // 6. top hidden layers with ReLU, 7. last layer with sigmoid
    for (int l = 0; l < ntop; ++l) {
        mlp_layer_any<S>(buf(cur), lda, fa.top.dim[l], fa.top.w[l], bias_lds + boff, fa.top.dim[l + 1], true,
                         buf(cur ^ 1), lda);
        boff += (fa.top.dim[l + 1] + 3) & ~3;
        __syncthreads();
        cur ^= 1;
    }
    last_layer<S>(buf(cur), lda, klast, wlast, lds_load(wlast + ((klast + 3) & ~3)), fa.out + b0, nb);
}

// ---- host side ------------------------------------------------------------------

static inline int round_up_int(int v, int a) { return (v + a - 1) / a * a; }

// Row stride of the activation buffers: every width the layers read, rounded
// up to the 64 k values one weight step can cover, plus 8 floats so that the
// 4 sample rows of one read start 8 banks apart.
int fused_lda(const FusedArgs& fa) {
    int w = fa.bot.dim[0];
    for (int l = 0; l <= fa.bot.n_layers; ++l) w = w > fa.bot.dim[l] ? w : fa.bot.dim[l];
    for (int l = 0; l <= fa.top.n_layers; ++l) w = w > fa.top.dim[l] ? w : fa.top.dim[l];
    return round_up_int(w, 64) + 8;
}

size_t fused_lds_bytes(const FusedArgs& fa, int S) {
    const int F = fa.T + 1;
    // + 4 floats: the MLP team's arrival counter
    return sizeof(float) * ((size_t)2 * S * fused_lda(fa) + (size_t)S * F * (fa.D + kRowPad) + fa.n_small + 4);
}

// dst[i] for i < total: the segment of sb holding i, zero in the padding.
__global__ __launch_bounds__(kBlock) void pack_small_kernel(SmallBlock sb, float* __restrict__ dst) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= sb.total) return;
    float v = 0.f;
    for (int g = 0; g < sb.nseg; ++g)
        if (i >= sb.off[g] && i < sb.off[g] + sb.len[g]) v = sb.src[g][i - sb.off[g]];
    dst[i] = v;
}

hipError_t launch_pack_small(const SmallBlock& sb, float* dst, hipStream_t s) {
    hipLaunchKernelGGL(pack_small_kernel, dim3((unsigned)((sb.total + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, sb,
                       dst);
    return hipGetLastError();
}

template <int S, int G, int U, int R, int RT, bool TEAM>
static hipError_t launch_fused_t(const FusedArgs& fa, hipStream_t s) {
    const size_t lds = fused_lds_bytes(fa, S);
    hipError_t e = allow_full_lds(fused_forward_kernel<S, G, U, R, RT, TEAM>);
    if (e != hipSuccess) return e;
    const int64_t blocks = (fa.B + S - 1) / S;
    hipLaunchKernelGGL((fused_forward_kernel<S, G, U, R, RT, TEAM>), dim3((unsigned)blocks), dim3(kFusedThreads), lds,
                       s, fa);
    return hipGetLastError();
}

size_t packed_layer_floats(int N, int K) {
    const size_t f = wide_tiles(N) ? (size_t)((N + 31) / 32) * ((K + 7) / 8) * 256
                                   : (size_t)((N + 15) / 16) * ((K + 15) / 16) * 256;
    return (f + 63) / 64 * 64;  // each layer starts 256-byte aligned
}

hipError_t launch_pack_layer(const float* W, int N, int K, float* packed, hipStream_t s) {
    const int64_t total = (int64_t)(packed_layer_floats(N, K) / 4);
    hipLaunchKernelGGL(pack_layer_kernel, dim3((unsigned)((total + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, W, N,
                       K, packed);
    return hipGetLastError();
}

bool fused_supported(const FusedArgs& fa, bool aligned16) {
    if (!aligned16 || fa.D % 4 != 0 || fa.D < 16 || fa.D > 256) return false;
    if (fa.bot.n_layers < 1 || fa.top.n_layers < 1) return false;
    if (fa.bot.n_layers > kFusedMaxLayers || fa.top.n_layers > kFusedMaxLayers) return false;
    return fused_lds_bytes(fa, kFusedSamples) <= kFusedMaxLds;
}

// Samples per block: 8 while the batch fills at most one round of blocks
// (one per CU), 16 beyond that when the LDS allows -- a block's time is set
// by streaming every weight once, so fewer, fuller blocks win once the
// batch needs several rounds (the matrix cores then set the pace).
int fused_samples(const FusedArgs& fa) {
    if (fa.B > 2048 && fused_lds_bytes(fa, 16) <= kFusedMaxLds) return 16;
    return kFusedSamples;
}

template <int S>
static hipError_t launch_fused_s(FusedArgs& fa, bool multi_hot, hipStream_t s) {
    const int F = fa.T + 1;
    const int n4 = (F - 1 + 3) / 4;
    const int items = S * n4 * (n4 + 1) / 2;
    int dsplit = 1;
    while (dsplit < 4 && items * dsplit * 2 <= kFusedThreads && fa.D % (4 * dsplit * 2) == 0) dsplit *= 2;
    fa.dsplit = dsplit;
    const int g = pow2_at_least((fa.D + 3) / 4);
    // dots: flat pairs for few tables, 4x4 register blocks, or one 32x32
    // MFMA tile per sample for kMfmaDotsMinTables..32 tables (D a multiple
    // of 16; measured faster there, slower with fewer tables or more tiles)
    const bool mfma_dots = fa.T >= kMfmaDotsMinTables && fa.T <= 32 && fa.D % 16 == 0;
    // one-index bags: 8 bag slots per lane group, or 1 when the block's bags
    // fit one slot per group (every slot's bounds are read, used or not);
    // from kTeamMinTables tables up the bags are gathered beside the bottom
    // MLP (TEAM; F > 12 always has that many)
    static_assert(kTeamMinTables <= 12, "more than 11 tables always take the TEAM kernels");
    const bool team = fa.T >= kTeamMinTables;
#define FUSED_G(G_)                                                                                 \
    case G_:                                                                                        \
        if (F <= 12) {                                                                              \
            if (team) {                                                                             \
                if (multi_hot) return launch_fused_t<S, G_, 4, 4, 0, true>(fa, s);                  \
                return launch_fused_t<S, G_, 8, 1, 0, true>(fa, s);                                 \
            }                                                                                       \
            if (multi_hot) return launch_fused_t<S, G_, 4, 4, 0, false>(fa, s);                     \
            if (S * fa.T <= kFusedThreads / G_) return launch_fused_t<S, G_, 1, 1, 0, false>(fa, s); \
            return launch_fused_t<S, G_, 8, 1, 0, false>(fa, s);                                    \
        }                                                                                           \
        if (mfma_dots) {                                                                            \
            if (multi_hot) return launch_fused_t<S, G_, 4, 4, 32, true>(fa, s);                     \
            return launch_fused_t<S, G_, 8, 1, 32, true>(fa, s);                                    \
        }                                                                                           \
        if (multi_hot) return launch_fused_t<S, G_, 4, 4, 4, true>(fa, s);                          \
        return launch_fused_t<S, G_, 8, 1, 4, true>(fa, s);
    switch (g) {
        FUSED_G(4)
        FUSED_G(8)
        FUSED_G(16)
        FUSED_G(32)
        FUSED_G(64)
        default: return hipErrorInvalidValue;
    }
#undef FUSED_G
}

hipError_t launch_fused_forward(FusedArgs fa, bool aligned16, bool multi_hot, hipStream_t s) {
    if (!fused_supported(fa, aligned16)) return hipErrorInvalidValue;
    fa.lda = fused_lda(fa);
    if (fused_samples(fa) == 16) return launch_fused_s<16>(fa, multi_hot, s);
    return launch_fused_s<8>(fa, multi_hot, s);
}

}  // namespace dlrm
