/*
 * dlrm_oracle.c -- plain, slow, fp64 CPU oracle of the DLRMv1 forward hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it: only the tests, the smoke
 * check of the entry module and the CPU-baseline leg of the benchmark do.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Every value is carried in double precision.  Model parameters and inputs
 * arrive as the fp32 / int64 tensors the GPU sees; each fp32 element is
 * widened to double exactly before use.  Loops run in the plain order of the
 * definitions; the only parallelism is an OpenMP split over independent
 * samples, which does not change any per-sample arithmetic.
 *
 * Sources (web pages on the luminal inference compiler):
 *  - "luminal compare dlrm-fused-kernels...dlrm-pt2-megakernel",
 *    file dlrm_megakernel.rs: DlrmMegaKernel::cuda_source steps 1-7 (bottom
 *    MLP with ReLU on every layer, one gather per table, strict lower
 *    triangle of dots over [x, ly_0, ...] in i-major / j-inner order,
 *    R = cat(x, zflat), top MLP with ReLU and a sigmoid on the last layer),
 *    and n_feat / n_pairs / validate.
 *  - same page, LessonsLearned entry "DLRM compile: EmbeddingBag translator
 *    gap" point 2: output[b] = sum of weight rows indices[offsets[b] :
 *    offsets[b+1]]; movement.rs translate_embedding_bag: offsets follow
 *    PyTorch's include_last_offset=False convention.
 *  - "luminal compare asglover/modal_ci_ready...vanilla-pytorch", commit
 *    message, section "Translator": Linear is addmm(bias, x, weight.t()) with
 *    alpha = beta = 1 against the (N, K) weight; the interaction is
 *    Z[:, li, lj] of bmm(cat(vectors), permute(..., [0,2,1])); section
 *    "cuda_lite kernels": pair (i, j) recovered from p by (1+sqrt(1+8p))/2.
 *  - "luminal compare nvidia-devcontainer-args...perf/compile-write-rayon",
 *    KernelSigmoid: sigmoid(x) = 1 / (1 + exp(-x)).
 *
 * Readings where the pages are silent (kept identical in DESIGN notes):
 *  - the last bag of a table ends at the index count n_indices[t];
 *  - an empty bag sums to 0;
 *  - offsets must be non-decreasing and within [0, n_indices], indices within
 *    [0, rows): anything else is reported as an error (ORACLE_E_INDEX);
 *  - vector 0 of the interaction is the post-ReLU bottom-MLP output.
 *
 * Every function returns 0 on success or a negative ORACLE_E_* code.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_E_NULL (-1)
#define ORACLE_E_SHAPE (-2)
#define ORACLE_E_INDEX (-3)
#define ORACLE_E_NOMEM (-4)

#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_SIGMOID 2

int oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Number of pairs of the strict lower triangle of an F x F matrix. */
int64_t oracle_n_pairs(int64_t n_feat) {
    if (n_feat < 1) return 0;
    return n_feat * (n_feat - 1) / 2;
}

/* Integer square root: largest r with r*r <= v (v >= 0), by bisection. */
static int64_t isqrt_floor(int64_t v) {
    int64_t lo = 0, hi = 1;
    while (hi * hi <= v) hi *= 2;
    /* invariant: lo*lo <= v < hi*hi */
    while (hi - lo > 1) {
        int64_t mid = lo + (hi - lo) / 2;
        if (mid * mid <= v) lo = mid; else hi = mid;
    }
    return lo;
}

/*
 * Closed form of the flat pair index (vanilla-pytorch page, "cuda_lite
 * kernels": i from (1 + sqrt(1 + 8p)) / 2).  Evaluated in exact integer
 * arithmetic: floor((1 + sqrt(n)) / 2) == floor((1 + isqrt(n)) / 2) for every
 * integer n >= 0, so i = (1 + isqrt(1 + 8p)) / 2 and j = p - i(i-1)/2.
 */
int oracle_pair_closed_form(int64_t p, int64_t* i_out, int64_t* j_out) {
    if (!i_out || !j_out) return ORACLE_E_NULL;
    if (p < 0) return ORACLE_E_SHAPE;
    int64_t i = (1 + isqrt_floor(1 + 8 * p)) / 2;
    *i_out = i;
    *j_out = p - i * (i - 1) / 2;
    return ORACLE_OK;
}

/*
 * Linear layer: y[m][n] = act(bias[n] + sum_k x[m][k] * W[n][k]).
 * W is (N, K) row-major (the nn.Linear layout); bias may be NULL (zero).
 * act: 0 none, 1 ReLU = max(0, a), 2 sigmoid = 1 / (1 + exp(-a)).
 */
int oracle_linear(int64_t M, int64_t N, int64_t K, const double* x, int64_t ldx,
                  const float* W, const float* bias, int act, double* y, int64_t ldy) {
    if (M < 0 || N < 1 || K < 0 || ldx < K || ldy < N) return ORACLE_E_SHAPE;
    if ((M > 0 && (!x || !y)) || !W) return ORACLE_E_NULL;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_SIGMOID) return ORACLE_E_SHAPE;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double a = bias ? (double)bias[n] : 0.0;
            for (int64_t k = 0; k < K; ++k) a += x[m * ldx + k] * (double)W[n * K + k];
            if (act == ORACLE_ACT_RELU) a = a > 0.0 ? a : 0.0;
            else if (act == ORACLE_ACT_SIGMOID) a = 1.0 / (1.0 + exp(-a));
            y[m * ldy + n] = a;
        }
    }
    return ORACLE_OK;
}

/* Bag bounds of sample b in one table; returns ORACLE_E_INDEX if malformed. */
static int bag_bounds(const int64_t* off, int64_t B, int64_t n_idx, int64_t b, int64_t* s, int64_t* e) {
    *s = off[b];
    *e = (b + 1 < B) ? off[b + 1] : n_idx;
    if (*s < 0 || *s > *e || *e > n_idx) return ORACLE_E_INDEX;
    return ORACLE_OK;
}

/*
 * Sum-pooled embedding bags for T tables:
 *   out[b][t][d] = sum_{k = s}^{e-1} W_t[idx_t[k]][d],
 * s = off_t[b], e = off_t[b+1] (or n_idx[t] for the last bag).  Output is
 * (B, T, D) row-major.  Indices and offsets are validated first.
 */
int oracle_embbag_sum(int32_t T, int64_t B, int32_t D, const float* const* W, const int64_t* rows,
                      const int64_t* const* idx, const int64_t* n_idx, const int64_t* const* off,
                      double* out) {
    if (T < 1 || B < 0 || D < 1) return ORACLE_E_SHAPE;
    if (!W || !rows || !idx || !n_idx || !off || (B > 0 && !out)) return ORACLE_E_NULL;
    for (int32_t t = 0; t < T; ++t) {
        if (!W[t] || (B > 0 && !off[t]) || (n_idx[t] > 0 && !idx[t])) return ORACLE_E_NULL;
        if (rows[t] < 1 || n_idx[t] < 0) return ORACLE_E_SHAPE;
        for (int64_t b = 0; b < B; ++b) {
            int64_t s, e;
            if (bag_bounds(off[t], B, n_idx[t], b, &s, &e)) return ORACLE_E_INDEX;
        }
        for (int64_t k = 0; k < n_idx[t]; ++k)
            if (idx[t][k] < 0 || idx[t][k] >= rows[t]) return ORACLE_E_INDEX;
    }
    int64_t b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < B; ++b) {
        for (int32_t t = 0; t < T; ++t) {
            int64_t s, e;
            bag_bounds(off[t], B, n_idx[t], b, &s, &e);
            double* o = out + (b * T + t) * (int64_t)D;
            for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t k = s; k < e; ++k) {
                const float* row = W[t] + idx[t][k] * (int64_t)D;
                for (int32_t d = 0; d < D; ++d) o[d] += (double)row[d];
            }
        }
    }
    return ORACLE_OK;
}

/*
 * General embedding bags (the reduce_op form of the same LessonsLearned entry,
 * point 2: output[b] = reduce_op(weight[indices[offsets[b]:offsets[b+1]]]),
 * with the arguments that movement.rs translate_embedding_bag and
 * dlrm_pattern.rs match_dlrm name: mode, per_sample_weights,
 * include_last_offset, padding_idx).  Definitions, per PyTorch's
 * nn.EmbeddingBag which those arguments come from:
 *   mode 0 (sum):  sum over the bag of w_k * row(idx_k)   (w_k = 1 without weights)
 *   mode 1 (mean): sum of the rows / number of rows        (empty bag: 0)
 *   mode 2 (max):  elementwise maximum of the rows          (empty bag: 0)
 *   include_last_offset: off has B + 1 entries and bag b ends at off[b + 1];
 *     otherwise off has B entries and the last bag ends at n_idx.
 *   padding_idx pad[t] >= 0: indices equal to it are left out of the bag
 *     (not summed, not counted, not maxed).
 * psw: per-sample weights per table (n_idx[t] values) or NULL; sum mode only.
 */
int oracle_embbag_ex(int32_t T, int64_t B, int32_t D, const float* const* W, const int64_t* rows,
                     const int64_t* const* idx, const int64_t* n_idx, const int64_t* const* off,
                     int32_t mode, int32_t include_last_offset, const int64_t* pad,
                     const float* const* psw, double* out) {
    if (T < 1 || B < 0 || D < 1 || mode < 0 || mode > 2) return ORACLE_E_SHAPE;
    if (!W || !rows || !idx || !n_idx || !off || (B > 0 && !out)) return ORACLE_E_NULL;
    if (psw && mode != 0) return ORACLE_E_SHAPE;
    for (int32_t t = 0; t < T; ++t) {
        if (!W[t] || !off[t] || (n_idx[t] > 0 && !idx[t]) || (psw && n_idx[t] > 0 && !psw[t])) return ORACLE_E_NULL;
        if (rows[t] < 1 || n_idx[t] < 0) return ORACLE_E_SHAPE;
        for (int64_t b = 0; b < B; ++b) {
            int64_t s = off[t][b];
            int64_t e = include_last_offset ? off[t][b + 1] : ((b + 1 < B) ? off[t][b + 1] : n_idx[t]);
            if (s < 0 || s > e || e > n_idx[t]) return ORACLE_E_INDEX;
        }
        for (int64_t k = 0; k < n_idx[t]; ++k)
            if (idx[t][k] < 0 || idx[t][k] >= rows[t]) return ORACLE_E_INDEX;
    }
    int64_t b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < B; ++b) {
        for (int32_t t = 0; t < T; ++t) {
            const int64_t s = off[t][b];
            const int64_t e = include_last_offset ? off[t][b + 1] : ((b + 1 < B) ? off[t][b + 1] : n_idx[t]);
            double* o = out + (b * T + t) * (int64_t)D;
            int64_t count = 0;
            for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
            for (int64_t k = s; k < e; ++k) {
                const int64_t r = idx[t][k];
                if (pad && pad[t] >= 0 && r == pad[t]) continue;
                const float* row = W[t] + r * (int64_t)D;
                const double w = psw ? (double)psw[t][k] : 1.0;
                for (int32_t d = 0; d < D; ++d) {
                    const double v = (double)row[d];
                    if (mode == 2) o[d] = (count == 0 || v > o[d]) ? v : o[d];
                    else o[d] += w * v;
                }
                ++count;
            }
            if (mode == 1 && count > 0)
                for (int32_t d = 0; d < D; ++d) o[d] /= (double)count;
        }
    }
    return ORACLE_OK;
}

/* Feature vector f of sample b: f = 0 is x[b], f = t+1 is E[b][t]. */
static const double* feature(const double* x, int64_t ldx, const double* E, int32_t T, int32_t D,
                             int64_t b, int32_t f) {
    if (f == 0) return x + b * ldx;
    return E + (b * T + (f - 1)) * (int64_t)D;
}

/*
 * Pairwise-dot interaction, strict lower triangle:
 *   p = 0; for i in 1..F-1: for j in 0..i-1: Z[b][p++] = <S_b[i], S_b[j]>,
 * S_b = [x_b, E[b][0], ..., E[b][T-1]], F = T + 1.  Z is (B, P), ldz >= P.
 */
int oracle_interact(int64_t B, int32_t T, int32_t D, const double* x, int64_t ldx, const double* E,
                    double* Z, int64_t ldz) {
    int32_t F = T + 1;
    int64_t P = oracle_n_pairs(F);
    if (B < 0 || T < 1 || D < 1 || ldx < D || ldz < P) return ORACLE_E_SHAPE;
    if (B > 0 && (!x || !E || !Z)) return ORACLE_E_NULL;
    int64_t b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < B; ++b) {
        int64_t p = 0;
        for (int32_t i = 1; i < F; ++i) {
            for (int32_t j = 0; j < i; ++j) {
                const double* u = feature(x, ldx, E, T, D, b, i);
                const double* v = feature(x, ldx, E, T, D, b, j);
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) acc += u[d] * v[d];
                Z[b * ldz + p] = acc;
                ++p;
            }
        }
    }
    return ORACLE_OK;
}

/* Full Gram matrix G[b][i][j] = <S_b[i], S_b[j]> for all i, j in [0, F). */
int oracle_gram(int64_t B, int32_t T, int32_t D, const double* x, int64_t ldx, const double* E,
                double* G) {
    int32_t F = T + 1;
    if (B < 0 || T < 1 || D < 1 || ldx < D) return ORACLE_E_SHAPE;
    if (B > 0 && (!x || !E || !G)) return ORACLE_E_NULL;
    for (int64_t b = 0; b < B; ++b)
        for (int32_t i = 0; i < F; ++i)
            for (int32_t j = 0; j < F; ++j) {
                const double* u = feature(x, ldx, E, T, D, b, i);
                const double* v = feature(x, ldx, E, T, D, b, j);
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) acc += u[d] * v[d];
                G[(b * F + i) * F + j] = acc;
            }
    return ORACLE_OK;
}

/* Model description for the oracle (its own layout, not the library's). */
typedef struct oracle_model {
    int32_t n_bot;               /* entries of ln_bot; n_bot - 1 layers       */
    const int64_t* ln_bot;       /* ln_bot[0] = dense width, last = D         */
    int32_t n_top;               /* entries of ln_top; n_top - 1 layers       */
    const int64_t* ln_top;       /* ln_top[0] = D + P, last = 1               */
    int32_t T;                   /* number of tables                          */
    int32_t D;                   /* embedding dim                             */
    const int64_t* rows;         /* [T]                                       */
    const float* const* emb;     /* [T] tables (rows[t], D)                   */
    const float* const* bot_w;   /* [n_bot-1] (ln_bot[l+1], ln_bot[l])        */
    const float* const* bot_b;   /* [n_bot-1] (ln_bot[l+1])                   */
    const float* const* top_w;
    const float* const* top_b;
} oracle_model;

/*
 * Shape rules of the DLRM family (dlrm_megakernel.rs, validate): at least one
 * layer per MLP, ln_bot[last] == D, ln_top[0] == D + F(F-1)/2 with F = T + 1,
 * ln_top[last] == 1, batch > 0, every width positive.
 */
int oracle_validate(const oracle_model* m, int64_t B) {
    if (!m || !m->ln_bot || !m->ln_top) return ORACLE_E_NULL;
    if (m->n_bot < 2 || m->n_top < 2 || m->T < 1 || m->D < 1 || B < 1) return ORACLE_E_SHAPE;
    for (int32_t l = 0; l < m->n_bot; ++l) if (m->ln_bot[l] < 1) return ORACLE_E_SHAPE;
    for (int32_t l = 0; l < m->n_top; ++l) if (m->ln_top[l] < 1) return ORACLE_E_SHAPE;
    if (m->ln_bot[m->n_bot - 1] != m->D) return ORACLE_E_SHAPE;
    if (m->ln_top[0] != m->D + oracle_n_pairs(m->T + 1)) return ORACLE_E_SHAPE;
    if (m->ln_top[m->n_top - 1] != 1) return ORACLE_E_SHAPE;
    return ORACLE_OK;
}

/*
 * One DLRMv1 forward pass for B samples (dlrm_megakernel.rs cuda_source):
 *  1. h = dense; each bottom layer h = ReLU(h W^T + b) (ReLU on every layer,
 *     the last included); x = h, shape (B, D).
 *  2. E = sum-pooled bags per table, (B, T, D).
 *  3-5. R = [x | Z] with Z the strict-lower-triangle dots of [x, E_0..E_{T-1}].
 *  6. each top layer but the last: h = ReLU(h W^T + b).
 *  7. last top layer (one output): y = 1 / (1 + exp(-(h w + b))).
 * Optional outputs (may be NULL): x_out (B, D), e_out (B, T, D),
 * r_out (B, D + P).  out is (B).
 */
int oracle_forward(const oracle_model* m, int64_t B, const float* dense, const int64_t* const* idx,
                   const int64_t* n_idx, const int64_t* const* off, double* out, double* x_out,
                   double* e_out, double* r_out) {
    int rc = oracle_validate(m, B);
    if (rc) return rc;
    if (!dense || !idx || !n_idx || !off || !out || !m->rows || !m->emb || !m->bot_w || !m->bot_b ||
        !m->top_w || !m->top_b)
        return ORACLE_E_NULL;
    const int32_t T = m->T, D = m->D, F = T + 1;
    const int64_t P = oracle_n_pairs(F);
    int64_t maxw = 0;
    for (int32_t l = 0; l < m->n_bot; ++l) if (m->ln_bot[l] > maxw) maxw = m->ln_bot[l];
    for (int32_t l = 0; l < m->n_top; ++l) if (m->ln_top[l] > maxw) maxw = m->ln_top[l];

    double* h0 = (double*)malloc(sizeof(double) * (size_t)(B * maxw));
    double* h1 = (double*)malloc(sizeof(double) * (size_t)(B * maxw));
    double* E = (double*)malloc(sizeof(double) * (size_t)(B * T * D));
    double* Z = (double*)malloc(sizeof(double) * (size_t)(B * (P > 0 ? P : 1)));
    if (!h0 || !h1 || !E || !Z) { rc = ORACLE_E_NOMEM; goto done; }

    /* 1. bottom MLP */
    int64_t w_in = m->ln_bot[0];
    for (int64_t i = 0; i < B * w_in; ++i) h0[i] = (double)dense[i];
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) {
        int64_t w_out = m->ln_bot[l + 1];
        rc = oracle_linear(B, w_out, w_in, h0, w_in, m->bot_w[l], m->bot_b[l], ORACLE_ACT_RELU, h1, w_out);
        if (rc) goto done;
        double* tmp = h0; h0 = h1; h1 = tmp;
        w_in = w_out;
    }
    /* h0 now holds x (B, D) */
    if (x_out) for (int64_t i = 0; i < B * D; ++i) x_out[i] = h0[i];

    /* 2. embedding bags */
    rc = oracle_embbag_sum(T, B, D, m->emb, m->rows, idx, n_idx, off, E);
    if (rc) goto done;
    if (e_out) for (int64_t i = 0; i < B * T * D; ++i) e_out[i] = E[i];

    /* 3-4. interaction */
    rc = oracle_interact(B, T, D, h0, D, E, Z, P);
    if (rc) goto done;

    /* 5. R = [x | Z] into h1 */
    int64_t wr = D + P;
    for (int64_t b = 0; b < B; ++b) {
        for (int32_t d = 0; d < D; ++d) h1[b * wr + d] = h0[b * D + d];
        for (int64_t p = 0; p < P; ++p) h1[b * wr + D + p] = Z[b * P + p];
    }
    if (r_out) for (int64_t i = 0; i < B * wr; ++i) r_out[i] = h1[i];
    { double* tmp = h0; h0 = h1; h1 = tmp; }

    /* 6-7. top MLP */
    w_in = wr;
    for (int32_t l = 0; l + 1 < m->n_top; ++l) {
        int64_t w_out = m->ln_top[l + 1];
        int last = (l + 2 == m->n_top);
        rc = oracle_linear(B, w_out, w_in, h0, w_in, m->top_w[l], m->top_b[l],
                           last ? ORACLE_ACT_SIGMOID : ORACLE_ACT_RELU, h1, w_out);
        if (rc) goto done;
        double* tmp = h0; h0 = h1; h1 = tmp;
        w_in = w_out;
    }
    for (int64_t b = 0; b < B; ++b) out[b] = h0[b];
    rc = ORACLE_OK;
done:
    free(h0); free(h1); free(E); free(Z);
    return rc;
}
