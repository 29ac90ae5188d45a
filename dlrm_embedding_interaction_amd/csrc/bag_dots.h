// bag_dots.h -- device routines shared by the bag + interaction kernel and
// the single-launch forward: the lane-group bag gather-reduce and the
// strict-lower-triangle dots over feature rows staged in LDS.
//
// Bag sum: sum of the rows idx_t[k], k in [off_t[b], end_t(b)), end_t(b) =
// off_t[b+1] or the index count for the last bag (LessonsLearned "DLRM
// compile: EmbeddingBag translator gap" point 2 on "luminal compare
// dlrm-fused-kernels...dlrm-pt2-megakernel").  Dots: Z[p] = <S[i], S[j]>,
// p = i(i-1)/2 + j, j < i < F (dlrm_megakernel.rs cuda_source step 4 on the
// same page).
#pragma once

#include "dlrm_device.h"
#include "rowvec.h"

namespace dlrm {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Explicit LDS accesses for pointers into a dynamic LDS array: the casts make
// sure the compiler emits ds_read / ds_write (a flat access is also counted
// with the global loads, so every wait for it would cover those in flight).
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) floatx4 lds_floatx4;
__device__ __forceinline__ floatx4 lds_load4(const float* p) { return *(const lds_floatx4*)(const lds_float*)p; }
__device__ __forceinline__ float lds_load(const float* p) { return *(const lds_float*)p; }
__device__ __forceinline__ void lds_store4(float* p, floatx4 v) { *(lds_floatx4*)(lds_float*)p = v; }
__device__ __forceinline__ void lds_store(float* p, float v) { *(lds_float*)p = v; }
typedef __attribute__((address_space(3))) int64_t lds_int64;
__device__ __forceinline__ int64_t lds_load8(const int64_t* p) { return *(const lds_int64*)p; }
__device__ __forceinline__ void lds_store8(int64_t* p, int64_t v) { *(lds_int64*)p = v; }


// Sum U bags per lane group.  Bag q[u] (-1 = none) is local bag number
// q = sl * T + t of sample b_base + sl.  Lane lg of the group owns elements
// (c * G + lg) * VEC .. + VEC-1 of the row for c < C.  Rows of one bag are
// added in increasing k, R of them fetched per step.  IT is the type of the
// indices and offsets (see gather_bags below).
template <int VEC, int G, int C, int U, int R, typename IT>
__device__ __forceinline__ void gather_bags_t(const TableArgs& ta, int T, int D, int64_t B, int64_t b_base,
                                              const int (&q)[U], int lg,
                                              typename Vec<VEC>::T (&acc)[U][C]) {
    using V = Vec<VEC>;
    // Bag bounds in passes over the U slots, every load of a pass in flight
    // together: first each slot's table pointers (kernel arguments indexed per
    // lane), then both of its offsets.  No load sits under a per-slot branch:
    // waiting for a load whose value the same slot needs at once would also
    // wait for every older load, one slot after the other.  A slot without a
    // bag reads sample b_base of table 0 (always valid) and gets length 0.
    const float* wp[U];
    const void* ip[U];
    const IT* op[U];
    int64_t nid[U];
    int64_t bb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int qq = q[u] >= 0 ? q[u] : 0;
        const int sl = qq / T;
        const int t = qq - sl * T;
        bb[u] = b_base + sl;
        wp[u] = ta.w[t];
        ip[u] = ta.idx[t];
        op[u] = static_cast<const IT*>(ta.off[t]);
        nid[u] = ta.nidx[t];
    }
    IT s0[U], e0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        s0[u] = ld_global<IT>(op[u] + bb[u]);
        e0[u] = ld_global<IT>(op[u] + (bb[u] + 1 < B ? bb[u] + 1 : bb[u]));
    }
    int64_t ks[U];
    int len[U];
    int maxlen = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ks[u] = s0[u];
        const int64_t e = bb[u] + 1 < B ? (int64_t)e0[u] : nid[u];
        len[u] = q[u] >= 0 ? (int)(e - ks[u]) : 0;
        maxlen = max(maxlen, len[u]);
#pragma unroll
        for (int c = 0; c < C; ++c) acc[u][c] = V::zero();
    }
    for (int r0 = 0; r0 < maxlen; r0 += R) {
        // kept in the index type until every load of the step is issued: a
        // widening inside each conditional load would wait for that load
        IT row[R][U];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
                row[rr][u] = (r0 + rr < len[u]) ? ld_global<IT>((const IT*)ip[u] + ks[u] + r0 + rr) : IT(-1);
        typename V::T v[R][U][C];
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const int e = (c * G + lg) * VEC;
                    v[rr][u][c] = (row[rr][u] >= 0 && e < D) ? V::gload(wp[u] + (int64_t)row[rr][u] * D + e) : V::zero();
                }
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (row[rr][u] >= 0) {
#pragma unroll
                    for (int c = 0; c < C; ++c) acc[u][c] = V::add(acc[u][c], v[rr][u][c]);
                }
    }
}

// gather_bags_t with the index type of the launch (one test, the same for
// every lane, around the whole gather).
template <int VEC, int G, int C, int U, int R>
__device__ __forceinline__ void gather_bags(const TableArgs& ta, int T, int D, int64_t B, int64_t b_base,
                                            const int (&q)[U], int lg, typename Vec<VEC>::T (&acc)[U][C]) {
    if (ta.idx32)
        gather_bags_t<VEC, G, C, U, R, int32_t>(ta, T, D, B, b_base, q, lg, acc);
    else
        gather_bags_t<VEC, G, C, U, R, int64_t>(ta, T, D, B, b_base, q, lg, acc);
}

// Z[s * ldz + p] = <S_s[i], S_s[j]> for s < nb and p < P = F(F-1)/2, where
// row i of sample s sits at S + (s * F + i) * LDR in LDS.  RT = 0: one G-lane
// group per flat pair index, dots reduced over the group with DPP.  RT = 4:
// 4x4 blocks of the triangle (rows i = 1 + 4I + a, columns j = 4J + b,
// J <= I; block number q = I(I+1)/2 + J decoded as the pair (I+1, J)), one
// block per lane, accumulated over d from float4 LDS reads; with dsplit > 1,
// dsplit neighbouring lanes take equal slices of d for the same block and add
// their partial blocks with DPP (xor 1, xor 2).  Block rows past F - 1 are
// read (clamped) but never stored.  NB threads of the block take part.
template <int VEC, int G, int C, int RT, int NB = kBlock>
__device__ __forceinline__ void pair_dots(const float* S, int F, int D, int LDR, int nb, float* Z, int ldz,
                                          int dsplit) {
    using V = Vec<VEC>;
    constexpr int NG = NB / G;
    const int tid = threadIdx.x;
    const int lg = tid % G;
    const int g = tid / G;
    const int P = F * (F - 1) / 2;
    const int npairs = nb * P;
    if constexpr (RT == 0) {
        for (int w = g; w < npairs; w += NG) {
            const int s = w / P;
            const int p = w - s * P;
            int i, j;
            pair_from_flat(p, i, j);
            const float* si = S + ((size_t)s * F + i) * LDR;
            const float* sj = S + ((size_t)s * F + j) * LDR;
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int e = (c * G + lg) * VEC;
                if (e < D) part = V::dot(V::load(si + e), V::load(sj + e), part);
            }
            const float tot = group_sum<G>(part);
            if (lg == 0) Z[s * ldz + p] = tot;
        }
    } else {
        const int NI = (F - 1 + RT - 1) / RT;
        const int nblk = NI * (NI + 1) / 2;
        const int dlen = D / dsplit;
        for (int w = tid; w < nb * nblk * dsplit; w += NB) {
            const int wq = w / dsplit;
            const int h = w - wq * dsplit;
            const int s = wq / nblk;
            const int q = wq - s * nblk;
            int I1, J;
            pair_from_flat(q, I1, J);
            const int i0 = 1 + RT * (I1 - 1);
            const int j0 = RT * J;
            const float* Sb = S + (size_t)s * F * LDR + h * dlen;
            const float* ri[RT];
            const float* rj[RT];
#pragma unroll
            for (int a = 0; a < RT; ++a) {
                ri[a] = Sb + min(i0 + a, F - 1) * LDR;
                rj[a] = Sb + min(j0 + a, F - 1) * LDR;
            }
            float acc[RT][RT];
#pragma unroll
            for (int a = 0; a < RT; ++a)
#pragma unroll
                for (int b = 0; b < RT; ++b) acc[a][b] = 0.f;
            for (int d = 0; d < dlen; d += VEC) {
                typename V::T u[RT], v[RT];
#pragma unroll
                for (int a = 0; a < RT; ++a) {
                    u[a] = V::load(ri[a] + d);
                    v[a] = V::load(rj[a] + d);
                }
#pragma unroll
                for (int a = 0; a < RT; ++a)
#pragma unroll
                    for (int b = 0; b < RT; ++b) acc[a][b] = V::dot(u[a], v[b], acc[a][b]);
            }
            if (dsplit > 1) {
#pragma unroll
                for (int a = 0; a < RT; ++a)
#pragma unroll
                    for (int b = 0; b < RT; ++b) {
                        acc[a][b] += dpp_quad_xor1(acc[a][b]);
                        if (dsplit > 2) acc[a][b] += dpp_quad_xor2(acc[a][b]);
                    }
            }
            if (h == 0) {
#pragma unroll
                for (int a = 0; a < RT; ++a) {
                    const int i = i0 + a;
#pragma unroll
                    for (int b = 0; b < RT; ++b) {
                        const int j = j0 + b;
                        if (i < F && j < i) Z[s * ldz + i * (i - 1) / 2 + j] = acc[a][b];
                    }
                }
            }
        }
    }
}

// Strict-lower-triangle dots on the matrix cores, for many tables: Z[s][p] =
// <S_s[i], S_s[j]>, p = i(i-1)/2 + j, j < i < F, with row i of sample s at
// S + (s * F + i) * LDR in LDS and D a multiple of 16.  Wave w of the NB
// threads takes samples w, w + NB / 64, ...  Every pair is an entry G[a][b] = <S[1 + a], S[b]>, b <= a,
// of the product of rows 1..F-1 with rows 0..F-2, computed in 32x32 tiles
// (J <= I; up to 32 tables one tile holds every pair) with
// v_mfma_f32_32x32x2f32: lane l supplies A[a = l % 32][k] = row 1 + 32 I + a
// and B[k][b = l % 32] = row 32 J + b at k = 16 c + 8 (l / 32) + q for MFMA q
// of d-chunk c (both operands share that k order), and holds tile entry
// (8 (r / 4) + 4 (l / 32) + r % 4, l % 32) in accumulator r.  Rows past F - 1
// are read clamped and never stored.
template <int NB>
__device__ __forceinline__ void pair_dots_mfma(const float* S, int F, int D, int LDR, int nb, float* Z, int ldz) {
    constexpr int NW = NB / 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int T = F - 1;
    const int nt = (T + 31) >> 5;
    const int r32 = lane & 31;
    const int h = lane >> 5;
    for (int s = wave; s < nb; s += NW) {
        const float* Sb = S + (size_t)s * F * LDR;
        float* Zs = Z + s * ldz;
        for (int I = 0; I < nt; ++I) {
            const float* ra = Sb + (1 + min(32 * I + r32, T - 1)) * LDR + 8 * h;
            for (int J = 0; J <= I; ++J) {
                const float* rb = Sb + min(32 * J + r32, T - 1) * LDR + 8 * h;
                floatx16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.f;
                // 64 values of d per group: all 16 reads first, then 32 MFMAs
                int c = 0;
                for (; c + 64 <= D; c += 64) {
                    floatx4 av[8], bv[8];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        av[2 * g] = lds_load4(ra + c + 16 * g);
                        av[2 * g + 1] = lds_load4(ra + c + 16 * g + 4);
                        bv[2 * g] = lds_load4(rb + c + 16 * g);
                        bv[2 * g + 1] = lds_load4(rb + c + 16 * g + 4);
                    }
#pragma unroll
                    for (int v = 0; v < 8; ++v)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[v][q], bv[v][q], acc, 0, 0, 0);
                }
                for (; c < D; c += 16) {
                    const floatx4 a0 = lds_load4(ra + c), a1 = lds_load4(ra + c + 4);
                    const floatx4 b0 = lds_load4(rb + c), b1 = lds_load4(rb + c + 4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[q], b0[q], acc, 0, 0, 0);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[q], b1[q], acc, 0, 0, 0);
                }
                const int bcol = 32 * J + r32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int a = 32 * I + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (a < T && bcol <= a) lds_store(Zs + (a + 1) * a / 2 + bcol, acc[r]);
                }
            }
        }
    }
}

}  // namespace dlrm
