// gram_interact.hip -- the bag gather and the strict-lower-triangle
// interaction of large batches in one kernel that keeps every feature vector
// in registers and computes the dots as a Gram matrix on the matrix cores.
//
// Definitions (as in embbag_interact.hip): bag sum out[b][t] = sum of rows
// idx_t[k], k in [off_t[b], end_t(b)) (LessonsLearned "DLRM compile:
// EmbeddingBag translator gap" point 2 on "luminal compare dlrm-fused-kernels
// ...dlrm-pt2-megakernel"); Z[b][p] = <S_b[i], S_b[j]>, p = i(i-1)/2 + j,
// j < i < F, S_b = [x_b, E_b0, ..., E_b(T-1)] (dlrm_megakernel.rs cuda_source
// step 4 on the same page).  Every such dot is entry (i, j) of the Gram matrix
// G_b = S_b S_b^T below its diagonal.
//
// Design on CDNA4:
//  * one wave owns NS consecutive samples; after one block-wide copy of the
//    tables' pointers into LDS the waves never wait for one another (no
//    further barriers), so a CU interleaves waves that are waiting for bag
//    bounds, indices or rows with waves that multiply;
//  * the wave first resolves every (sample, feature) of its chunk to the byte
//    address of one row -- x for feature 0, the bag's row for the others, 0
//    for an empty bag -- with all the bag-bound loads, then all the index
//    loads, in flight together, and keeps the addresses in its LDS;
//  * rows are read with coalesced loads: D/4 lanes cover one row, 16 bytes
//    each (a wave load is 1 KiB, whole 128-byte lines), into a register ring
//    of PD samples; each sample's rows are then written to the wave's LDS
//    and read back in the operand layout of v_mfma_f32_16x16x4f32, where lane
//    l holds feature 16 blk + (l % 16) for k slot l / 16;  16-byte chunk c of
//    row f is kept at chunk c ^ (f % (D/4)), so that neither the writes (one
//    row per 16 lanes) nor the reads (16 rows per 16 lanes) meet in a bank;
//  * LITE (rows of at most 64 floats): the rows go straight from memory into
//    the wave's LDS by 16-byte DMA copies (global_load_lds), one sample at a
//    time, with no register ring, and Z is staged where the rows were.  That
//    frees the ring's registers and LDS for 4 waves per SIMD instead of 2:
//    random row reads scale with the waves issuing them more than with the
//    bytes each has in flight (batch 16384 x 32 tables: 41.4 -> 35.8 us);
//  * the CU issues the oldest waves' requests first, so with 16 tables or
//    more (a long copy per sample) each wave lowers its issue priority
//    (s_setprio) with every sample it finishes: waves that are behind catch
//    up instead of draining the launch alone (batch 16384 x 16 tables:
//    17.9 -> 17.5 us);
//  * because G is symmetric, the same registers are both MFMA operands: tile
//    (I, J) multiplies feature block I by block J, and the tile above the
//    diagonal is never formed (NB = 2: tiles (0,0), (1,0), (1,1));
//  * accumulator r of lane l holds G[16 I + 4 (l/16) + r][16 J + l % 16];
//    entries with j < i < F are stored straight to Z, each store instruction
//    writing one contiguous run of j per 16 lanes;
//  * with F = 16 NB + 1 (16 or 32 tables) the last feature does not fit a
//    block: every lane reads that row's values for its k slots (the same LDS
//    address across 16 lanes), dots them with its own on the vector ALUs and
//    the four k slots are added with two cross-lane exchanges;
//  * a bag of more than one index sends the whole wave down a slower path
//    that sums each bag in a loop (rows added in increasing k).
#include "dlrm_device.h"
#include "dlrm_internal.h"
#include "bag_dots.h"

namespace dlrm {

namespace {

constexpr int kGramWaves = 4;
constexpr int kGramThreads = 64 * kGramWaves;
constexpr int kGramMaxTables = 32;

struct GramTable {
    const float* w;
    const void* idx;
    const void* off;
    int64_t nidx;
};

// Bytes of one wave's LDS region: the row addresses of its NS samples, one
// sample's FP staged rows, then one sample's Z (at most FP(FP-1)/2 floats).
template <int D, int FP, int NS, bool LITE>
constexpr int gram_wave_lds() {
    return (NS * FP * 8 + 15) / 16 * 16 + FP * D * 4 + (LITE ? 0 : (FP * (FP - 1) / 2 + 3) / 4 * 16);
}

// 1 KiB of zeros: where an empty bag's row is copied from
__device__ __attribute__((aligned(16))) float g_gram_zero_row[256];

template <int D, int NB, bool EXTRA, int NS, int PD, bool LITE>
__global__ __launch_bounds__(kGramThreads) __attribute__((amdgpu_waves_per_eu(LITE ? 4 : 1, 8))) void gram_interact_kernel(TableArgs ta, int T, int64_t B,
                                                                     const float* __restrict__ x, int64_t ld_x,
                                                                     float* __restrict__ out, int64_t ld_out,
                                                                     int col_x, int col_z) {
    constexpr int CPR = D / 4;                         // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                      // rows per coalesced wave load
    constexpr int FP = 16 * NB + (EXTRA ? 1 : 0);      // feature rows staged per sample
    constexpr int NLD = (FP + RPI - 1) / RPI;          // coalesced loads per lane and sample
    constexpr int NV = CPR / 4;                        // float4 per lane and feature in MFMA layout
    constexpr int NTASK = (NS * FP + 63) / 64;         // (sample, feature) lookups per lane
    extern __shared__ float4 lds4[];
    GramTable* const tabs = reinterpret_cast<GramTable*>(lds4);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int q16 = lane & 15;
    const int h = lane >> 4;
    const int F = T + 1;
    const int i32 = ta.idx32;

    // 0. the tables' pointers, once per block
    for (int t = threadIdx.x; t < T; t += kGramThreads) tabs[t] = GramTable{ta.w[t], ta.idx[t], ta.off[t], ta.nidx[t]};
    __syncthreads();
    const int64_t b0 = ((int64_t)blockIdx.x * kGramWaves + wave) * NS;
    if (b0 >= B) return;  // the whole wave; no barrier follows
    const int ns = (int)min((int64_t)NS, B - b0);
    char* const region = reinterpret_cast<char*>(lds4) + kGramMaxTables * sizeof(GramTable) +
                         wave * gram_wave_lds<D, FP, NS, LITE>();
    int64_t* const rowptr = reinterpret_cast<int64_t*>(region);                     // [NS][FP]
    float* const buf = reinterpret_cast<float*>(region + (NS * FP * 8 + 15) / 16 * 16);  // [FP][D]
    float* const zbuf = LITE ? buf : buf + FP * D;  // [P]; with LITE after every read of the rows
    const int P = F * (F - 1) / 2;
    // Z rows are written 16 bytes per lane when every row starts 16-byte aligned
    const bool vec_z = ((reinterpret_cast<uintptr_t>(out + col_z) | (uintptr_t)(ld_out * 4)) & 15) == 0;

    // 1. every (sample, feature) of the chunk to one row address: bag bounds
    //    of all lookups in flight, then all indices
    bool longbag = false;
    // Every load below is issued by every lane, from a valid address (bag
    // bounds of the chunk's first sample, the offsets array, or x's first row
    // of the chunk, when a lane has nothing to fetch), and the unwanted values
    // are dropped afterwards: loads under a per-lane branch would make the
    // compiler wait for all of them at once instead of counting them.
    auto resolve = [&](auto index_type) {
        using IT = decltype(index_type);
        int64_t st[NTASK], en[NTASK];
        bool ok[NTASK];
#pragma unroll
        for (int k = 0; k < NTASK; ++k) {
            const int q = lane + 64 * k;
            const int s = q / FP;
            const int f = q - s * FP;
            ok[k] = q < NS * FP && s < ns && f >= 1 && f < F;
            const GramTable g = tabs[ok[k] ? f - 1 : 0];
            const int64_t b = ok[k] ? b0 + s : b0;
            st[k] = ld_idx<IT>(g.off, b);
            const int64_t e = ld_idx<IT>(g.off, b + 1 < B ? b + 1 : b);
            en[k] = b + 1 < B ? e : g.nidx;
        }
#pragma unroll
        for (int k = 0; k < NTASK; ++k) {
            const int q = lane + 64 * k;
            const int s = q / FP;
            const int f = q - s * FP;
            const GramTable g = tabs[ok[k] ? f - 1 : 0];
            const int64_t len = ok[k] ? en[k] - st[k] : 0;
            longbag = longbag || len > 1;
            const int64_t b = ok[k] ? b0 + s : b0;
            const int64_t r = ld_idx<IT>(len == 1 ? g.idx : g.off, len == 1 ? st[k] : b);
            int64_t p = 0;
            if (len == 1) p = reinterpret_cast<int64_t>(g.w + r * D);
            if (q < NS * FP && s < ns && f == 0) p = reinterpret_cast<int64_t>(x + (b0 + s) * ld_x);
            if (q < NS * FP) lds_store8(rowptr + q, p);
        }
    };
    if (i32)
        resolve(int32_t{});
    else
        resolve(int64_t{});
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // this lane's row and chunk in a coalesced load, and the chunk's place in LDS
    const int lrow = lane / CPR;
    const int lchunk = lane % CPR;
    auto swz = [](int f) { return f & (CPR - 1); };

    // Sample s from its rows staged as [FP][D] (chunks permuted): the Gram
    // tiles, the extra feature's dots, Z gathered in LDS and written as one
    // contiguous row segment, and the x copy.  The operands of each 16-wide
    // slice of d are read just before their MFMAs.
    auto compute = [&](int s) {
        floatx4 acc[NB][NB];
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int J = 0; J <= I; ++J) acc[I][J] = floatx4{0.f, 0.f, 0.f, 0.f};
        float part[NB];
#pragma unroll
        for (int I = 0; I < NB; ++I) part[I] = 0.f;
        float* const xr = out + (b0 + s) * ld_out + col_x;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            floatx4 a[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                const int r = 16 * I + q16;
                a[I] = lds_load4(buf + r * D + 4 * ((4 * c + h) ^ swz(r)));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int J = 0; J <= I; ++J)
                        acc[I][J] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[I][e], a[J][e], acc[I][J], 0, 0, 0);
            if constexpr (EXTRA) {
                constexpr int fe = 16 * NB;  // the last feature, dotted on the vector ALUs
                const floatx4 ev = lds_load4(buf + fe * D + 4 * ((4 * c + h) ^ swz(fe)));
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int e = 0; e < 4; ++e) part[I] = fmaf(a[I][e], ev[e], part[I]);
            }
            // lane (0, k slot h) holds x at d = 16 c + 4 h + e
            if (col_x >= 0 && q16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) xr[16 * c + 4 * h + e] = a[0][e];
            }
        }
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int J = 0; J <= I; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * I + 4 * h + r;
                    const int jj = 16 * J + q16;
                    if (jj < i && i < F) lds_store(zbuf + i * (i - 1) / 2 + jj, acc[I][J][r]);
                }
        if constexpr (EXTRA) {
            constexpr int fe = 16 * NB;
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                float v = part[I];
                v += swizzle_xor16(v);
                v += __shfl_xor(v, 32, 64);
                if (h == 0) lds_store(zbuf + fe * (fe - 1) / 2 + 16 * I + q16, v);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float* const zr = out + (b0 + s) * ld_out + col_z;
        constexpr int PMAX = FP * (FP - 1) / 2;
        if (vec_z) {
            const int n4 = P >> 2;
#pragma unroll
            for (int k = 0; k < (PMAX / 4 + 63) / 64; ++k) {
                const int i = lane + 64 * k;
                if (i < n4) *reinterpret_cast<floatx4*>(zr + 4 * i) = lds_load4(zbuf + 4 * i);
            }
            if (lane < P - 4 * n4) zr[4 * n4 + lane] = lds_load(zbuf + 4 * n4 + lane);
        } else {
#pragma unroll
            for (int k = 0; k < (PMAX + 63) / 64; ++k) {
                const int i = lane + 64 * k;
                if (i < P) zr[i] = lds_load(zbuf + i);
            }
        }
    };
    auto stage = [&](const floatx4 (&v)[NLD]) {
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int f = RPI * k + lrow;
            if (f < FP) lds_store4(buf + f * D + 4 * lchunk, v[k]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    // the next sample's writes must not pass this sample's reads
    auto done_reading = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if (!__any(longbag)) {
        // x's first row of the chunk: where a lane with no row to fetch reads
        const char* const spare = reinterpret_cast<const char*>(x + b0 * ld_x) + 16 * lchunk;
        auto issue = [&](int s, floatx4 (&v)[NLD]) {
#pragma unroll
            for (int k = 0; k < NLD; ++k) {
                const int f = RPI * k + lrow;
                const int64_t p = lds_load8(rowptr + min(s, NS - 1) * FP + min(f, FP - 1));
                const bool take = s < ns && f < FP && p != 0;
                const floatx4 w = ld_global<floatx4>(
                    take ? reinterpret_cast<const char*>(p) + 16 * (lchunk ^ swz(f)) : spare);
                v[k] = take ? w : floatx4{0.f, 0.f, 0.f, 0.f};
            }
        };
        if constexpr (LITE) {
            // rows copied into the wave's LDS by DMA (no register ring): lane
            // l of a copy writes bytes [16 l, 16 l + 16) after the copy's
            // base, i.e. row RPI k + l / CPR, chunk l % CPR, read from the
            // swizzled chunk of the table row; lanes past the FP staged rows
            // copy nothing.  The row addresses are read from LDS before the
            // first copy (a later LDS read would wait for the copies).
#pragma unroll 1
            for (int s = 0; s < ns; ++s) {
                // A CU issues its oldest waves' requests first, so the waves
                // dispatched last fall behind and finish the launch alone.
                // From 16 tables (a long copy per sample) a wave's issue
                // priority falls with the samples it has done, so that the
                // waves behind catch up.
                if constexpr (FP > 16) {
                    switch (s) {
                        case 0: __builtin_amdgcn_s_setprio(3); break;
                        case 1: __builtin_amdgcn_s_setprio(2); break;
                        case 2: __builtin_amdgcn_s_setprio(1); break;
                        default: __builtin_amdgcn_s_setprio(0); break;
                    }
                }
                int64_t pr[NLD];
#pragma unroll
                for (int k = 0; k < NLD; ++k) {
                    const int f = RPI * k + lrow;
                    pr[k] = lds_load8(rowptr + s * FP + min(f, FP - 1));
                }
#pragma unroll
                for (int k = 0; k < NLD; ++k) {
                    const int f = RPI * k + lrow;
                    if (f < FP) {
                        const char* src = pr[k] != 0
                                              ? reinterpret_cast<const char*>(pr[k]) + 16 * (lchunk ^ swz(f))
                                              : reinterpret_cast<const char*>(g_gram_zero_row) + 16 * lchunk;
                        __builtin_amdgcn_global_load_lds(
                            (const __attribute__((address_space(1))) void*)src,
                            (__attribute__((address_space(3))) void*)(lds_float*)(buf + k * RPI * D), 16, 0, 0);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies have landed
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                compute(s);
                done_reading();
            }
        } else {
            floatx4 ring[PD][NLD];
#pragma unroll
            for (int s = 0; s < PD && s < NS; ++s) issue(s, ring[s]);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                stage(ring[s % PD]);
                if (s + PD < NS) issue(s + PD, ring[s % PD]);
                compute(s);
                done_reading();
            }
        }
    } else {
        // bags of any length: each bag summed in a loop, one sample at a time
        for (int s = 0; s < ns; ++s) {
            floatx4 v[NLD];
#pragma unroll
            for (int k = 0; k < NLD; ++k) {
                const int f = RPI * k + lrow;
                const int cc = lchunk ^ swz(f);
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
                if (f == 0) {
                    acc = ld_global<floatx4>(x + (b0 + s) * ld_x + 4 * cc);
                } else if (f < F && f < FP) {
                    const GramTable g = tabs[f - 1];
                    const int64_t b = b0 + s;
                    const int64_t k0 = ld_index(g.off, b, i32);
                    const int64_t k1 = b + 1 < B ? ld_index(g.off, b + 1, i32) : g.nidx;
                    for (int64_t kk = k0; kk < k1; ++kk) {
                        const floatx4 w = ld_global<floatx4>(g.w + ld_index(g.idx, kk, i32) * D + 4 * cc);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[e] += w[e];
                    }
                }
                v[k] = acc;
            }
            stage(v);
            compute(s);
            done_reading();
        }
    }
}

template <int D, int NB, bool EXTRA, int NS, bool LITE>
hipError_t launch_gram_t(const TableArgs& ta, int T, int64_t B, const float* x, int64_t ld_x, float* out,
                         int64_t ld_out, int col_x, int col_z, hipStream_t s) {
    constexpr int FP = 16 * NB + (EXTRA ? 1 : 0);
    constexpr int NLD = (FP + 64 / (D / 4) - 1) / (64 / (D / 4));
    // samples in flight per wave: as many as about 40 ring registers allow
    constexpr int PD = NLD <= 4 ? 3 : 2;
    constexpr size_t lds = kGramMaxTables * sizeof(GramTable) + kGramWaves * gram_wave_lds<D, FP, NS, LITE>();
    const int64_t waves = (B + NS - 1) / NS;
    const int64_t blocks = (waves + kGramWaves - 1) / kGramWaves;
    static_assert(lds <= kFusedMaxLds, "LDS of one block");
    if (lds > 64 * 1024) {
        hipError_t e = allow_full_lds(gram_interact_kernel<D, NB, EXTRA, NS, PD, LITE>);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gram_interact_kernel<D, NB, EXTRA, NS, PD, LITE>), dim3((unsigned)blocks), dim3(kGramThreads), lds,
                       s, ta, T, B, x, ld_x, out, ld_out, col_x, col_z);
    return hipGetLastError();
}

template <int D, int NB, bool EXTRA>
hipError_t launch_gram_ns(const TableArgs& ta, int T, int64_t B, const float* x, int64_t ld_x, float* out,
                          int64_t ld_out, int col_x, int col_z, hipStream_t s) {
    // samples per wave: so many that every wave is resident at once and pays
    // the bag-bound and index round trips only once (256 CUs x 4 SIMDs x the
    // waves per SIMD the registers and LDS allow: 4 with the DMA-staged rows
    // (LITE, rows of at most 64 floats) or with one 16-feature block, 2
    // otherwise); at most 8 samples per wave
    constexpr bool LITE = D <= 64;
    constexpr int64_t kResidentWaves = 1024 * (LITE || (NB == 1 && !EXTRA) ? 4 : 2);
    const int64_t want = (B + kResidentWaves - 1) / kResidentWaves;
    if (want <= 1) return launch_gram_t<D, NB, EXTRA, 1, LITE>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    if (want <= 2) return launch_gram_t<D, NB, EXTRA, 2, LITE>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    if (want <= 4) return launch_gram_t<D, NB, EXTRA, 4, LITE>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    return launch_gram_t<D, NB, EXTRA, 8, LITE>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
}

template <int D>
hipError_t launch_gram_d(const TableArgs& ta, int T, int64_t B, const float* x, int64_t ld_x, float* out,
                         int64_t ld_out, int col_x, int col_z, hipStream_t s) {
    if (T <= 15) return launch_gram_ns<D, 1, false>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    if (T == 16) return launch_gram_ns<D, 1, true>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    if (T <= 31) return launch_gram_ns<D, 2, false>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    return launch_gram_ns<D, 2, true>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
}

}  // namespace

bool gram_interact_supported(int T, int D, bool aligned16) {
    return aligned16 && T >= 1 && T <= 32 && (D == 32 || D == 64 || D == 128);
}

hipError_t launch_gram_interact(const TableArgs& ta, int T, int D, int64_t B, bool aligned16, const float* x,
                                int64_t ld_x, float* out, int64_t ld_out, int col_x, int col_z, hipStream_t s) {
    if (!gram_interact_supported(T, D, aligned16)) return hipErrorInvalidValue;
    switch (D) {
        case 32: return launch_gram_d<32>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
        case 64: return launch_gram_d<64>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
        default: return launch_gram_d<128>(ta, T, B, x, ld_x, out, ld_out, col_x, col_z, s);
    }
}

}  // namespace dlrm
