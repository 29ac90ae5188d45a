// embbag_ex.hip -- general multi-table embedding bags on gfx950: sum, mean or
// max pooling, optional per-sample weights, include_last_offset, a padding
// index per table, and 32- or 64-bit indices and offsets.
//
// Definition (LessonsLearned entry "DLRM compile: EmbeddingBag translator
// gap", point 2, on "luminal compare dlrm-fused-kernels...dlrm-pt2-megakernel":
// output[b] = reduce_op(weight[indices[offsets[b]:offsets[b+1]]]), with the
// argument set that movement.rs translate_embedding_bag reads there: mode,
// per_sample_weights, include_last_offset, padding_idx):
//   sum   sum of w_k * row(idx_k), w_k = 1 without weights
//   mean  sum of the rows / number of rows (empty bag: 0)
//   max   elementwise maximum of the rows (empty bag: 0)
// Indices equal to the table's padding index are left out of the bag.  With
// include_last_offset the offsets hold B + 1 entries and bag b ends at
// offsets[b + 1]; otherwise the last bag ends at the index count.
//
// Same layout as the plain bag kernel: one row per group of G lanes, 16 bytes
// per lane, U bags per group in flight, R row indices fetched per step.  The
// mode is a uniform run-time branch; the index width is a template argument.
#include "dlrm_device.h"
#include "dlrm_internal.h"
#include "rowvec.h"

namespace dlrm {

template <int VEC, int G, int C, int U, int R, typename IDX>
__global__ __launch_bounds__(kBlock) void embbag_ex_kernel(BagArgs ba, int T, int D, int64_t B, int mode,
                                                           int last_off, float* __restrict__ out) {
    using V = Vec<VEC>;
    constexpr int NG = kBlock / G;
    const int lg = threadIdx.x % G;
    const int g = threadIdx.x / G;
    const int64_t nbags = B * T;
    const int64_t base = (int64_t)blockIdx.x * NG * U;

    const float* wp[U];
    const IDX* ip[U];
    const float* ps[U];
    int64_t pad[U];
    int len[U], cnt[U];
    int64_t q[U];
    typename V::T acc[U][C];
    const typename V::T init = (mode == DLRM_BAG_MAX) ? V::splat(-INFINITY) : V::zero();
    int maxlen = 0;
    // Bag bounds in passes over the U slots, every load of a pass in flight
    // together: the tables' arguments, then both offsets of each bag (no load
    // under a per-slot branch, where waiting for it would also wait for every
    // older load).  A slot past the last bag reads bag 0 and gets length 0.
    const IDX* op[U];
    int64_t bb[U], nid[U];
    const float* psw[U];
    const void* ix[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        q[u] = base + u * NG + g;
        const int64_t qq = q[u] < nbags ? q[u] : 0;
        bb[u] = qq / T;
        const int t = (int)(qq - bb[u] * T);
        op[u] = reinterpret_cast<const IDX*>(ba.off[t]);
        wp[u] = ba.w[t];
        ix[u] = ba.idx[t];
        psw[u] = ba.psw[t];
        pad[u] = ba.pad[t];
        nid[u] = ba.nidx[t];
    }
    IDX s0[U], e0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t be = (last_off || bb[u] + 1 < B) ? bb[u] + 1 : bb[u];
        s0[u] = ld_global<IDX>(op[u] + bb[u]);
        e0[u] = ld_global<IDX>(op[u] + be);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t s = s0[u];
        const int64_t e = (last_off || bb[u] + 1 < B) ? (int64_t)e0[u] : nid[u];
        len[u] = q[u] < nbags ? (int)(e - s) : 0;
        cnt[u] = 0;
        ip[u] = reinterpret_cast<const IDX*>(ix[u]) + s;
        ps[u] = psw[u] ? psw[u] + s : nullptr;
        maxlen = max(maxlen, len[u]);
#pragma unroll
        for (int c = 0; c < C; ++c) acc[u][c] = init;
    }
    for (int r0 = 0; r0 < maxlen; r0 += R) {
        // indices stay in their own type until every load of the step is
        // issued: a widening inside each conditional load would wait for it
        IDX raw[R][U];
        float wt[R][U];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = r0 + rr < len[u];
                raw[rr][u] = in ? ld_global<IDX>(ip[u] + r0 + rr) : IDX(-1);
                wt[rr][u] = (in && ps[u]) ? ld_global<float>(ps[u] + r0 + rr) : 1.f;
            }
        int64_t row[R][U];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
                row[rr][u] = ((int64_t)raw[rr][u] == pad[u]) ? -1 : (int64_t)raw[rr][u];  // padding rows leave the bag
        typename V::T v[R][U][C];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int e = (c * G + lg) * VEC;
                    v[rr][u][c] = (row[rr][u] >= 0 && e < D) ? V::gload(wp[u] + row[rr][u] * D + e) : V::zero();
                }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (row[rr][u] >= 0) {
                    ++cnt[u];
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        if (mode == DLRM_BAG_MAX) acc[u][c] = V::max(acc[u][c], v[rr][u][c]);
                        else if (ps[u]) acc[u][c] = V::fma(wt[rr][u], v[rr][u][c], acc[u][c]);
                        else acc[u][c] = V::add(acc[u][c], v[rr][u][c]);
                    }
                }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (q[u] >= nbags) continue;
        float* o = out + q[u] * (int64_t)D;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int e = (c * G + lg) * VEC;
            if (e >= D) continue;
            typename V::T r = acc[u][c];
            if (cnt[u] == 0) r = V::zero();
            else if (mode == DLRM_BAG_MEAN) r = V::div(r, (float)cnt[u]);
            V::store(o + e, r);
        }
    }
}

template <int VEC, int G, int C, int U, int R, typename IDX>
static hipError_t launch_ex_t(const BagArgs& ba, int T, int D, int64_t B, int mode, int last_off, float* out,
                              hipStream_t s) {
    constexpr int NG = kBlock / G;
    const int64_t blocks = (B * T + (int64_t)NG * U - 1) / ((int64_t)NG * U);
    hipLaunchKernelGGL((embbag_ex_kernel<VEC, G, C, U, R, IDX>), dim3((unsigned)blocks), dim3(kBlock), 0, s, ba, T,
                       D, B, mode, last_off, out);
    return hipGetLastError();
}

hipError_t launch_embbag_ex(const BagArgs& ba, int T, int D, int64_t B, int mode, int last_off, bool idx32,
                            bool aligned16, bool multi_hot, float* out, hipStream_t s) {
    const RowShape rs = row_shape(D, aligned16);
#define CALL_EX(V, G, C)                                                                                   \
    if (idx32) {                                                                                           \
        if (multi_hot) return launch_ex_t<V, G, C, 4, 4, int32_t>(ba, T, D, B, mode, last_off, out, s);    \
        return launch_ex_t<V, G, C, 4, 1, int32_t>(ba, T, D, B, mode, last_off, out, s);                  \
    }                                                                                                      \
    if (multi_hot) return launch_ex_t<V, G, C, 4, 4, int64_t>(ba, T, D, B, mode, last_off, out, s);        \
    return launch_ex_t<V, G, C, 4, 1, int64_t>(ba, T, D, B, mode, last_off, out, s);
    DLRM_DISPATCH_ROW(rs, CALL_EX);
#undef CALL_EX
}

}  // namespace dlrm
