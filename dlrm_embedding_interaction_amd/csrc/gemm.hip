// gemm.hip -- fp32 Linear layers of the DLRMv1 MLPs on gfx950 matrix cores.
//
// y = act(x W^T + bias) with W in the nn.Linear (N, K) layout: the
// addmm(bias, x, weight.t()) fast path with an absorbed ReLU / sigmoid
// consumer (linear_bias, linear_bias_relu, linear_bias_sigmoid on "luminal
// compare asglover/modal_ci_ready...vanilla-pytorch", Translator section;
// sigmoid = 1/(1+exp(-a)) as KernelSigmoid on "luminal compare
// nvidia-devcontainer-args...perf/compile-write-rayon").
//
// Both operands are K-contiguous ("NT"), so a tile of each is staged in LDS as
// [row][k] with 4 floats of padding per row.  A wave owns a (TM*MF) x (TN*MF)
// sub-tile built from MF x MF MFMA blocks:
//  * MF = 16, v_mfma_f32_16x16x4f32: for every 16-wide k slice each lane
//    reads one float4 of A and one of B from LDS and feeds their four
//    components to four MFMAs (lane l supplies A[l%16][k] and B[k][l%16] with
//    k = 4*(l/16) + q for MFMA q);
//  * MF = 32, v_mfma_f32_32x32x2f32 (the full-rate fp32 shape on gfx950):
//    each lane reads two float4 of A and two of B per 16-wide k slice and
//    feeds them to eight MFMAs (lane l supplies A[l%32][k] and B[k][l%32]
//    with k = 8*(l/32) + q for MFMA q).
// Either way the k order is a permutation that both operands share.  Two LDS
// buffers alternate between k tiles and two
// register stages hold the next two tiles in flight: while tile c is
// multiplied from one buffer, tile c+1 (fetched one tile earlier) is stored to
// the other and tile c+3 is requested, so each k tile costs one barrier and
// global latency is covered by two tiles of MFMA work.  Bias and activation
// are applied to the accumulators before the single store.  Block order is remapped so that the
// blocks one XCD runs (the hardware deals blocks to the 8 XCDs round-robin)
// cover consecutive tiles and share their rows of x in that XCD's L2.
#include "dlrm_device.h"
#include "dlrm_internal.h"

namespace dlrm {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float apply_act(float v, int act) {
    if (act == DLRM_ACT_RELU) return v > 0.f ? v : 0.f;
    if (act == DLRM_ACT_SIGMOID) return 1.f / (1.f + expf(-v));
    return v;
}

// Four consecutive floats from global memory at a 4-byte-aligned address.
// gfx9 vector-memory loads of 16 bytes need only dword alignment, so this is
// one dwordx4 load also where a row starts off a 16-byte boundary (a Linear
// weight (N, K) with K not a multiple of 4, or x with such a row stride).
__device__ __forceinline__ floatx4 load4_dword_aligned(const float* p) {
    floatx4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int MF>
struct MfmaAcc;
template <>
struct MfmaAcc<16> {
    typedef floatx4 T;
};
template <>
struct MfmaAcc<32> {
    typedef floatx16 T;
};

template <int BM, int BN, int BK, int WM, int WN, int MF, bool VA, bool VB>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bias_act_kernel(int M, int N, int K, const float* __restrict__ A,
                                                                    int64_t lda, const float* __restrict__ W,
                                                                    const float* __restrict__ bias, int act,
                                                                    float* __restrict__ Y, int64_t ldy, int tiles_m,
                                                                    int tiles_n, bool vec_y) {
    static_assert(MF == 16 || MF == 32, "16x16x4 or 32x32x2 blocks");
    using Acc = typename MfmaAcc<MF>::T;
    constexpr int NR = MF * MF / 64;  // accumulator values per lane and block
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / (WM * MF);
    constexpr int TN = BN / (WN * MF);
    constexpr int LDK = BK + 4;
    static_assert(BK % 16 == 0, "BK must be a multiple of 16");
    static_assert(TM >= 1 && TN >= 1, "wave tile too small");
    constexpr int A_V = VA ? (BM * BK / 4) / NT : (BM * BK) / NT;  // loads per thread
    constexpr int B_V = VB ? (BN * BK / 4) / NT : (BN * BK) / NT;
    static_assert(A_V >= 1 && B_V >= 1, "tile too small for the block");
    static_assert((VA ? A_V * 4 : A_V) * NT == BM * BK, "A tile must split evenly");
    static_assert((VB ? B_V * 4 : B_V) * NT == BN * BK, "B tile must split evenly");

    // two A buffers, two B buffers; the same memory stages the output tile
    constexpr int LDC = BN + 4;
    constexpr int SM_TILES = 2 * (BM + BN) * LDK;
    constexpr int SM = SM_TILES > BM * LDC ? SM_TILES : BM * LDC;
    __shared__ __attribute__((aligned(16))) float smem[SM];
    float* const Abuf[2] = {smem, smem + BM * LDK};
    float* const Bbuf[2] = {smem + 2 * BM * LDK, smem + 2 * BM * LDK + BN * LDK};

    const int nblk = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int tmi = bid / tiles_n;
    const int tni = bid - tmi * tiles_n;
    const int m0 = tmi * BM;
    const int n0 = tni * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[i][j][r] = 0.f;

    // one register stage: this thread's share of an A tile and a B tile
    struct Stage {
        floatx4 ra4[VA ? A_V : 1];
        float ra1[VA ? 1 : A_V];
        floatx4 rb4[VB ? B_V : 1];
        float rb1[VB ? 1 : B_V];
    };
    Stage st0, st1;

    auto load_tiles = [&](int k0, Stage& S_) {
        floatx4* ra4 = S_.ra4;
        float* ra1 = S_.ra1;
        floatx4* rb4 = S_.rb4;
        float* rb1 = S_.rb1;
        if constexpr (VA) {
#pragma unroll
            for (int i = 0; i < A_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / (BK / 4);
                const int k = k0 + (f - r * (BK / 4)) * 4;
                const int m = m0 + r;
                floatx4 v = {0.f, 0.f, 0.f, 0.f};
                if (m < M) {
                    const float* p = A + (int64_t)m * lda + k;
                    if (k + 3 < K) {
                        v = load4_dword_aligned(p);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k + e < K) v[e] = p[e];
                    }
                }
                ra4[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < A_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / BK;
                const int k = k0 + (f - r * BK);
                const int m = m0 + r;
                ra1[i] = (m < M && k < K) ? A[(int64_t)m * lda + k] : 0.f;
            }
        }
        if constexpr (VB) {
#pragma unroll
            for (int i = 0; i < B_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / (BK / 4);
                const int k = k0 + (f - r * (BK / 4)) * 4;
                const int n = n0 + r;
                floatx4 v = {0.f, 0.f, 0.f, 0.f};
                if (n < N) {
                    const float* p = W + (int64_t)n * K + k;
                    if (k + 3 < K) {
                        v = load4_dword_aligned(p);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k + e < K) v[e] = p[e];
                    }
                }
                rb4[i] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / BK;
                const int k = k0 + (f - r * BK);
                const int n = n0 + r;
                rb1[i] = (n < N && k < K) ? W[(int64_t)n * K + k] : 0.f;
            }
        }
    };
    auto store_tiles = [&](const Stage& S_, float* As, float* Bs) {
        const floatx4* ra4 = S_.ra4;
        const float* ra1 = S_.ra1;
        const floatx4* rb4 = S_.rb4;
        const float* rb1 = S_.rb1;
        if constexpr (VA) {
#pragma unroll
            for (int i = 0; i < A_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / (BK / 4);
                const int c = (f - r * (BK / 4)) * 4;
                *reinterpret_cast<floatx4*>(&As[r * LDK + c]) = ra4[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < A_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / BK;
                As[r * LDK + (f - r * BK)] = ra1[i];
            }
        }
        if constexpr (VB) {
#pragma unroll
            for (int i = 0; i < B_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / (BK / 4);
                const int c = (f - r * (BK / 4)) * 4;
                *reinterpret_cast<floatx4*>(&Bs[r * LDK + c]) = rb4[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < B_V; ++i) {
                const int f = i * NT + tid;
                const int r = f / BK;
                Bs[r * LDK + (f - r * BK)] = rb1[i];
            }
        }
    };

    // this lane's row within an MF-row block and its k offset in a 16-wide
    // k slice (KV float4 reads of each operand per slice)
    constexpr int KV = MF == 16 ? 1 : 2;
    const int lrow = lane & (MF - 1);
    const int lk = (lane / MF) * 4 * KV;
    const int arow0 = wm * TM * MF + lrow;
    const int brow0 = wn * TN * MF + lrow;

    auto multiply = [&](const float* As, const float* Bs) {
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            floatx4 af[TM][KV], bf[TN][KV];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int v = 0; v < KV; ++v)
                    af[i][v] = *reinterpret_cast<const floatx4*>(&As[(arow0 + i * MF) * LDK + kk + lk + 4 * v]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < KV; ++v)
                    bf[j][v] = *reinterpret_cast<const floatx4*>(&Bs[(brow0 + j * MF) * LDK + kk + lk + 4 * v]);
#pragma unroll
            for (int q = 0; q < 4 * KV; ++q)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        if constexpr (MF == 16)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][0][q], bf[j][0][q], acc[i][j],
                                                                             0, 0, 0);
                        else
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][q >> 2][q & 3],
                                                                             bf[j][q >> 2][q & 3], acc[i][j], 0, 0, 0);
                    }
        }
    };

    // tiles 0 and 1 in flight; tile 0 staged into buffer 0, tile 2 requested
    load_tiles(0, st0);
    if (BK < K) load_tiles(BK, st1);
    store_tiles(st0, Abuf[0], Bbuf[0]);
    if (2 * BK < K) load_tiles(2 * BK, st0);
    __syncthreads();
    // two k tiles per trip so that the register stage of each tile is fixed
    for (int k0 = 0; k0 < K; k0 += 2 * BK) {
        multiply(Abuf[0], Bbuf[0]);
        if (k0 + BK < K) {
            store_tiles(st1, Abuf[1], Bbuf[1]);
            if (k0 + 3 * BK < K) load_tiles(k0 + 3 * BK, st1);
        }
        __syncthreads();
        if (k0 + BK >= K) break;
        multiply(Abuf[1], Bbuf[1]);
        if (k0 + 2 * BK < K) {
            store_tiles(st0, Abuf[0], Bbuf[0]);
            if (k0 + 4 * BK < K) load_tiles(k0 + 4 * BK, st0);
        }
        __syncthreads();
    }

    // Accumulator layout of an MF x MF block: lane l holds column l % MF;
    // element r holds row 4*(l/16) + r for MF = 16 and row
    // 8*(r/4) + 4*(l/32) + r%4 for MF = 32.  Bias and activation are applied
    // there; the finished tile is staged in LDS (the loop above ended with a
    // barrier) and written back row by row, 16 bytes per lane when Y allows.
    float* const Ct = smem;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int cl = wn * TN * MF + j * MF + (lane & (MF - 1));
        const int n = n0 + cl;
        const float bv = (bias != nullptr && n < N) ? bias[n] : 0.f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int rb = MF == 16 ? (lane >> 4) * 4 + r : 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int rl = wm * TM * MF + i * MF + rb;
                Ct[rl * LDC + cl] = apply_act(acc[i][j][r] + bv, act);
            }
        }
    }
    __syncthreads();
    if (vec_y) {
        constexpr int C4 = BN / 4;
        for (int f = tid; f < BM * C4; f += NT) {
            const int rl = f / C4;
            const int c = (f - rl * C4) * 4;
            const int m = m0 + rl;
            const int n = n0 + c;
            if (m >= M || n >= N) continue;
            const floatx4 v = *reinterpret_cast<const floatx4*>(&Ct[rl * LDC + c]);
            float* dst = Y + (int64_t)m * ldy + n;
            if (n + 3 < N) {
                *reinterpret_cast<floatx4*>(dst) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < N) dst[e] = v[e];
            }
        }
    } else {
        for (int f = tid; f < BM * BN; f += NT) {
            const int rl = f / BN;
            const int c = f - rl * BN;
            const int m = m0 + rl;
            const int n = n0 + c;
            if (m < M && n < N) Y[(int64_t)m * ldy + n] = Ct[rl * LDC + c];
        }
    }
}

// One wave per row: y[m] = act(<x[m], w> + bias).
template <bool VA>
__global__ __launch_bounds__(256) void gemv_bias_act_kernel(int M, int K, const float* __restrict__ A, int64_t lda,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias, int act,
                                                            float* __restrict__ y, int64_t ldy) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // uniform per wave
    const float* a = A + row * lda;
    float acc = 0.f;
    if constexpr (VA) {
        for (int k = lane * 4; k < K; k += 256) {
            if (k + 3 < K) {
                acc = f4_dot(*reinterpret_cast<const float4*>(a + k), *reinterpret_cast<const float4*>(w + k), acc);
            } else {
                for (int e = 0; e < 4; ++e)
                    if (k + e < K) acc = fmaf(a[k + e], w[k + e], acc);
            }
        }
    } else {
        for (int k = lane; k < K; k += 64) acc = fmaf(a[k], w[k], acc);
    }
    acc = group_sum<64>(acc);
    if (lane == 0) y[row * ldy] = apply_act(acc + (bias ? bias[0] : 0.f), act);
}

template <int BM, int BN, int BK, int WM, int WN, int MF, bool VA, bool VB>
static hipError_t launch_gemm_t(int M, int N, int K, const float* x, int64_t ld_x, const float* W,
                                const float* bias, int act, float* y, int64_t ld_y, hipStream_t s) {
    const int tm = (M + BM - 1) / BM;
    const int tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_bias_act_kernel<BM, BN, BK, WM, WN, MF, VA, VB>), dim3((unsigned)(tm * tn)),
                       dim3(WM * WN * 64), 0, s, M, N, K, x, ld_x, W, bias, act, y, ld_y, tm, tn,
                       (ld_y % 4 == 0) && (((uintptr_t)y & 15u) == 0));
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int MF>
static hipError_t launch_gemm_v(bool va, bool vb, int M, int N, int K, const float* x, int64_t ld_x, const float* W,
                                const float* bias, int act, float* y, int64_t ld_y, hipStream_t s) {
    if (va && vb)
        return launch_gemm_t<BM, BN, BK, WM, WN, MF, true, true>(M, N, K, x, ld_x, W, bias, act, y, ld_y, s);
    if (va) return launch_gemm_t<BM, BN, BK, WM, WN, MF, true, false>(M, N, K, x, ld_x, W, bias, act, y, ld_y, s);
    if (vb) return launch_gemm_t<BM, BN, BK, WM, WN, MF, false, true>(M, N, K, x, ld_x, W, bias, act, y, ld_y, s);
    return launch_gemm_t<BM, BN, BK, WM, WN, MF, false, false>(M, N, K, x, ld_x, W, bias, act, y, ld_y, s);
}

static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

hipError_t launch_linear(int64_t M, int64_t N, int64_t K, const float* x, int64_t ld_x, const float* W,
                         const float* bias, int act, float* y, int64_t ld_y, hipStream_t s) {
    const bool va = (ld_x % 4 == 0) && aligned16(x);
    if (N == 1) {
        const int64_t blocks = (M + 3) / 4;
        if (va && aligned16(W))
            hipLaunchKernelGGL(gemv_bias_act_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, (int)M, (int)K,
                               x, ld_x, W, bias, act, y, ld_y);
        else
            hipLaunchKernelGGL(gemv_bias_act_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, (int)M, (int)K,
                               x, ld_x, W, bias, act, y, ld_y);
        return hipGetLastError();
    }
    // GEMM tiles take float4 loads of x and W from any 4-byte-aligned rows
    const bool vb = aligned4(W);
    const bool vx = aligned4(x);
    const int m = (int)M, n = (int)N, k = (int)K;
    // Tile choice measured on MI355X (inside HIP graphs) for the DLRM layer
    // shapes:
    //  * batches too small to give every CU four 64x64 tiles: 32x32 tiles, one
    //    16x16 block per wave;
    //  * K <= 16 (the first bottom layer, bound by writing y): 64x64 tiles of
    //    32x32 blocks with 16-wide k tiles, so that no k tile is mostly padding;
    //  * everything else (at least ~256 tiles of 128x128): 128x128 tiles, 8
    //    waves each owning a 32x64 sub-tile of 32x32 blocks, 16-wide k tiles
    //    (3-11% faster than 64x64 tiles of 16x16 blocks on the large layers).
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (t64 < 1024) return launch_gemm_v<32, 32, 32, 2, 2, 16>(vx, vb, m, n, k, x, ld_x, W, bias, act, y, ld_y, s);
    if (K <= 16) return launch_gemm_v<64, 64, 16, 2, 2, 32>(vx, vb, m, n, k, x, ld_x, W, bias, act, y, ld_y, s);
    return launch_gemm_v<128, 128, 16, 4, 2, 32>(vx, vb, m, n, k, x, ld_x, W, bias, act, y, ld_y, s);
}

}  // namespace dlrm
