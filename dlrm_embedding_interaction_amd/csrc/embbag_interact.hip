// embbag_interact.hip -- gfx950 kernels for the sparse half of the DLRMv1
// forward: multi-table sum-pooled embedding bags, the strict-lower-triangle
// pairwise-dot interaction, and the two fused (bags gathered straight into LDS,
// then dotted there).
//
// Definitions:
//  * bag sum: out[b][t] = sum of rows idx_t[k], k in [off_t[b], end_t(b)),
//    end_t(b) = off_t[b+1] or the index count for the last bag (LessonsLearned
//    "DLRM compile: EmbeddingBag translator gap" point 2 and movement.rs
//    translate_embedding_bag, on "luminal compare dlrm-fused-kernels...
//    dlrm-pt2-megakernel");
//  * interaction: Z[b][p] = <S_b[i], S_b[j]>, p = i(i-1)/2 + j, j < i < F,
//    S_b = [x_b, E_b0, ..., E_b(T-1)] (dlrm_megakernel.rs cuda_source step 4
//    on the same page; PairwiseDotLowerTriStackedKernel on "luminal compare
//    asglover/modal_ci_ready...vanilla-pytorch", cuda_lite kernels).
//
// Design on CDNA4 (not the pages' CUDA layouts):
//  * one embedding row is read by a group of G lanes, 16 bytes per lane
//    (global_load_dwordx4), so a wave64 reads 1 KiB per instruction; each
//    group keeps U bags in flight and prefetches R row indices per bag, so a
//    wave has U*R independent row loads outstanding;
//  * the fused kernel places the F vectors of each of its samples in LDS
//    (rows padded by 4 floats so that rows 16 apart are the first to share
//    banks).  With few vectors (F <= 12) every G-lane group takes one flat
//    pair index p at a time, decodes (i, j) in closed form, dots the two LDS
//    rows and reduces across the group with DPP / ds_swizzle.  With more
//    vectors each lane owns a 4x4 block of the strict lower triangle (block
//    index decoded with the same closed form) and accumulates its 16 dots
//    over d from float4 LDS reads, 8 reads per 64 FMAs and no cross-lane
//    traffic; when that leaves most lanes of a block idle, 2 or 4
//    neighbouring lanes split d for one block and add their partial blocks
//    with DPP.  The P results of a sample are staged in LDS and written as
//    one contiguous row segment.
#include "dlrm_device.h"
#include "dlrm_internal.h"
#include "rowvec.h"
#include "bag_dots.h"

namespace dlrm {

// ---- standalone multi-table bags: out (B, T, D) -------------------------------
template <int VEC, int G, int C, int U, int R>
__global__ __launch_bounds__(kBlock) void embbag_sum_kernel(TableArgs ta, int T, int D, int64_t B, float* out) {
    using V = Vec<VEC>;
    constexpr int NG = kBlock / G;
    const int lg = threadIdx.x % G;
    const int g = threadIdx.x / G;
    const int64_t nbags = B * T;
    const int64_t base = (int64_t)blockIdx.x * NG * U;
    // Local bag numbers relative to sample base_b = base / T keep int range.
    const int64_t b_base = base / T;
    const int64_t q_off = b_base * T;
    int q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t qq = base + u * NG + g;
        q[u] = (qq < nbags) ? (int)(qq - q_off) : -1;
    }
    typename V::T acc[U][C];
    gather_bags<VEC, G, C, U, R>(ta, T, D, B, b_base, q, lg, acc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (q[u] < 0) continue;
        float* o = out + (q_off + q[u]) * (int64_t)D;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int e = (c * G + lg) * VEC;
            if (e < D) V::store(o + e, acc[u][c]);
        }
    }
}

// ---- interaction, with the bags either gathered (GATHER) or read from E ------
// LDS: S[spb][F][D + kRowPad] then Zs[spb][P].  RT = 0: lane-group dots;
// RT = 4: per-lane 4x4 register blocks of the triangle, d split over dsplit
// neighbouring lanes.
template <int VEC, int G, int C, int U, int R, bool GATHER, int RT>
__global__ __launch_bounds__(kBlock) void interact_kernel(TableArgs ta, const float* __restrict__ emb, int T,
                                                          int D, int64_t B, int spb, const float* x,
                                                          int64_t ld_x, float* out, int64_t ld_out,
                                                          int col_x, int col_z, int dsplit) {
    using V = Vec<VEC>;
    constexpr int NG = kBlock / G;
    extern __shared__ float4 lds4[];
    float* S = reinterpret_cast<float*>(lds4);
    const int F = T + 1;
    const int P = F * (F - 1) / 2;
    const int LDR = D + kRowPad;
    float* Zs = S + (size_t)spb * F * LDR;
    const int tid = threadIdx.x;
    const int lg = tid % G;
    const int g = tid / G;
    const int64_t b0 = (int64_t)blockIdx.x * spb;
    const int nb = (int)min((int64_t)spb, B - b0);
    const int dv = D / VEC;

    // 1. x rows into S[s][0]
    for (int e = tid; e < nb * dv; e += kBlock) {
        const int s = e / dv;
        const int d = (e - s * dv) * VEC;
        V::store(S + (size_t)s * F * LDR + d, V::load(x + (b0 + s) * ld_x + d));
    }
    // 2. table vectors into S[s][1 + t]
    if constexpr (GATHER) {
        const int nbag = nb * T;
        for (int qb = 0; qb < nbag; qb += NG * U) {
            int q[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int qq = qb + u * NG + g;
                q[u] = qq < nbag ? qq : -1;
            }
            typename V::T acc[U][C];
            gather_bags<VEC, G, C, U, R>(ta, T, D, B, b0, q, lg, acc);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (q[u] < 0) continue;
                const int s = q[u] / T;
                const int t = q[u] - s * T;
                float* dst = S + ((size_t)s * F + 1 + t) * LDR;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int e = (c * G + lg) * VEC;
                    if (e < D) V::store(dst + e, acc[u][c]);
                }
            }
        }
    } else {
        const int per = T * dv;
        for (int e = tid; e < nb * per; e += kBlock) {
            const int s = e / per;
            const int r = e - s * per;  // element (in VEC units) within the (T, D) block
            const int t = r / dv;
            const int d = (r - t * dv) * VEC;
            V::store(S + ((size_t)s * F + 1 + t) * LDR + d, V::load(emb + ((b0 + s) * T + t) * (int64_t)D + d));
        }
    }
    __syncthreads();

    // 3. dots
    pair_dots<VEC, G, C, RT>(S, F, D, LDR, nb, Zs, P, dsplit);
    __syncthreads();

    // 4. write Z (and x) rows
    for (int e = tid; e < nb * P; e += kBlock) {
        const int s = e / P;
        const int p = e - s * P;
        out[(b0 + s) * ld_out + col_z + p] = Zs[e];
    }
    if (col_x >= 0) {
        for (int e = tid; e < nb * D; e += kBlock) {
            const int s = e / D;
            const int d = e - s * D;
            out[(b0 + s) * ld_out + col_x + d] = S[(size_t)s * F * LDR + d];
        }
    }
}

// ---- device-side validation of bag data ------------------------------------------
__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

__global__ __launch_bounds__(kBlock) void check_indices_kernel(CheckArgs ca, int T, int64_t B, int32_t* bad) {
    int64_t local = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int t = 0; t < T; ++t) {
        const int64_t rows = ca.rows[t];
        const int64_t n = ca.nidx[t];
        for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < n; k += stride) {
            const int64_t v = ld_index(ca.idx[t], k, ca.idx32);
            local += (v < 0 || v >= rows);
        }
        for (int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x; b < B; b += stride) {
            const int64_t s = ld_index(ca.off[t], b, ca.idx32);
            const int64_t e = (b + 1 < B) ? ld_index(ca.off[t], b + 1, ca.idx32) : n;
            local += (s < 0 || s > e || e > n);
        }
    }
    if (local) atomicAdd(bad, (int32_t)min(local, (int64_t)1 << 30));
}

// ---- the kernels' own pair-index decoding, exported for tests -----------------
__global__ __launch_bounds__(kBlock) void pair_map_kernel(int P, int32_t* io, int32_t* jo) {
    const int p = blockIdx.x * kBlock + threadIdx.x;
    if (p >= P) return;
    int i, j;
    pair_from_flat(p, i, j);
    io[p] = i;
    jo[p] = j;
}

// ---- host-side dispatch ---------------------------------------------------------

bool row_shape_supported(int D) { return D >= 1 && D <= kMaxDim; }

template <int VEC, int G, int C, int U, int R>
static hipError_t launch_embbag_t(const TableArgs& ta, int T, int D, int64_t B, float* out, hipStream_t s) {
    constexpr int NG = kBlock / G;
    const int64_t nbags = B * T;
    const int64_t blocks = (nbags + (int64_t)NG * U - 1) / ((int64_t)NG * U);
    hipLaunchKernelGGL((embbag_sum_kernel<VEC, G, C, U, R>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ta, T, D, B,
                       out);
    return hipGetLastError();
}

template <int VEC, int G, int C, int U, int R, bool GATHER, int RT>
static hipError_t launch_interact_t(const TableArgs& ta, const float* emb, int T, int D, int64_t B, int spb,
                                    const float* x, int64_t ld_x, float* out, int64_t ld_out, int col_x, int col_z,
                                    int dsplit, hipStream_t s) {
    const size_t lds = interact_lds_bytes(T, D, spb);
    const int64_t blocks = (B + spb - 1) / spb;
    hipLaunchKernelGGL((interact_kernel<VEC, G, C, U, R, GATHER, RT>), dim3((unsigned)blocks), dim3(kBlock), lds, s, ta,
                       emb, T, D, B, spb, x, ld_x, out, ld_out, col_x, col_z, dsplit);
    return hipGetLastError();
}


// Multi-hot bags: one bag per lane group at a time, 8 rows per step, as in
// the bag + interaction kernel (measured at 26 tables x 10^6 x 128, bag 20,
// Zipf, batch 65536: 1882 us against 1967 us with 4 bags x 4 rows).
hipError_t launch_embbag_sum(const TableArgs& ta, int T, int D, int64_t B, bool aligned16, bool multi_hot,
                             float* out, hipStream_t s) {
    const RowShape rs = row_shape(D, aligned16);
#define CALL_E(V, G, C)                                                            \
    if (multi_hot) return launch_embbag_t<V, G, C, 1, 8>(ta, T, D, B, out, s);     \
    return launch_embbag_t<V, G, C, 4, 1>(ta, T, D, B, out, s);
    DLRM_DISPATCH_ROW(rs, CALL_E);
#undef CALL_E
}

int interact_samples_per_block(int T, int D, int64_t B) {
    const int F = T + 1, P = F * (F - 1) / 2;
    const size_t per = sizeof(float) * ((size_t)F * (D + kRowPad) + P);
    int spb = (int)(kInteractLdsBudget / per);
    if (spb < 1) spb = 1;
    if (spb > 16) spb = 16;
    // keep at least ~2 blocks per CU when the batch allows it
    const int64_t want = (B + 511) / 512;
    if (want < spb) spb = (int)(want < 1 ? 1 : want);
    return spb;
}

size_t interact_lds_bytes(int T, int D, int spb) {
    const int F = T + 1, P = F * (F - 1) / 2;
    return sizeof(float) * ((size_t)spb * F * (D + kRowPad) + (size_t)spb * P);
}

hipError_t launch_interact(const TableArgs* ta, const float* emb, int T, int D, int64_t B, bool aligned16,
                           bool multi_hot, const float* x, int64_t ld_x, float* out, int64_t ld_out, int col_x,
                           int col_z, hipStream_t s) {
    // bags of one index with 4 to 32 tables: the Gram-matrix kernel (measured
    // on MI355X at batch 2048..16384, D = 64: 1.2x faster at 4 tables, 2-2.8x
    // at 8-32 tables); with 1 to 3 tables its 16-feature tile is mostly empty
    // and the lane-group kernel is as fast or faster
    if (ta && !multi_hot && T >= 4 && gram_interact_supported(T, D, aligned16))
        return launch_gram_interact(*ta, T, D, B, aligned16, x, ld_x, out, ld_out, col_x, col_z, s);
    const RowShape rs = row_shape(D, aligned16);
    const int spb = interact_samples_per_block(T, D, B);
    // one-index bags: 4 bag slots per lane group, or 1 when a block's bags fit
    // one per group (every slot's bounds are read, used or not);
    // multi-hot bags: one bag per lane group at a time, 8 row indices and rows
    // per step (measured on MI355X at 26 tables, bag 20, Zipf, batch 65536:
    // 1795 us against 1852 us with 4 bags x 4 rows, which holds more
    // registers per lane and so fewer waves per CU).
    // dot layout: lane-group dots for few vectors; otherwise per-lane 4x4
    // register blocks, with d split over 2 or 4 lanes while that leaves fewer
    // work items than threads (the slices stay multiples of the vector width).
    // (One MFMA tile per sample, as the single launch uses, measured slower
    // here: 4 waves carry up to 16 samples, and a tile computes the whole
    // square.)
    const int F = T + 1;
    const int n4 = (F - 1 + 3) / 4;
    const int items = spb * n4 * (n4 + 1) / 2;
    const int vw = (rs.vec == 4) ? 4 : 1;
    int dsplit = 1;
    while (dsplit < 4 && items * dsplit * 2 <= kBlock && D % (vw * dsplit * 2) == 0) dsplit *= 2;
    if (interact_lds_bytes(T, D, spb) > kMaxLdsBytes) return hipErrorInvalidValue;
    TableArgs dummy{};
    const TableArgs& t = ta ? *ta : dummy;
    const bool gather = (ta != nullptr);
#define CALL_I2(V, G, C, RT)                                                                                   \
    if (!gather) return launch_interact_t<V, G, C, 1, 1, false, RT>(t, emb, T, D, B, spb, x, ld_x, out, ld_out, \
                                                                    col_x, col_z, dsplit, s);                  \
    if (multi_hot) return launch_interact_t<V, G, C, 1, 8, true, RT>(t, emb, T, D, B, spb, x, ld_x, out, ld_out, \
                                                                     col_x, col_z, dsplit, s);                 \
    if (spb * T <= kBlock / G)                                                                                 \
        return launch_interact_t<V, G, C, 1, 1, true, RT>(t, emb, T, D, B, spb, x, ld_x, out, ld_out, col_x,    \
                                                          col_z, dsplit, s);                                   \
    return launch_interact_t<V, G, C, 4, 1, true, RT>(t, emb, T, D, B, spb, x, ld_x, out, ld_out, col_x, col_z, \
                                                      dsplit, s);
#define CALL_I(V, G, C)          \
    if (F <= 12) {               \
        CALL_I2(V, G, C, 0)      \
    } else {                     \
        CALL_I2(V, G, C, 4)      \
    }
    DLRM_DISPATCH_ROW(rs, CALL_I);
#undef CALL_I2
#undef CALL_I
}

hipError_t launch_pair_index_map(int F, int32_t* i_out, int32_t* j_out, hipStream_t s) {
    const int P = F * (F - 1) / 2;
    hipLaunchKernelGGL(pair_map_kernel, dim3((unsigned)((P + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, P, i_out,
                       j_out);
    return hipGetLastError();
}

hipError_t launch_check_indices(const CheckArgs& ca, int T, int64_t B, int32_t* bad, hipStream_t s) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, bad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t n = B;
    for (int t = 0; t < T; ++t) n = n > ca.nidx[t] ? n : ca.nidx[t];
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(check_indices_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, ca, T, B, bad);
    return hipGetLastError();
}

}  // namespace dlrm
