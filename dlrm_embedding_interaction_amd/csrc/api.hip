// api.hip -- extern "C" entry points of the DLRMv1 forward library
// (declared in include/dlrm_mi355x.h).  Host code only: argument validation,
// workspace planning and kernel launches on the caller's stream.  Nothing here
// allocates, copies or synchronises, so every call can be captured in a graph.
#include <stdint.h>
#include <string.h>

#include "dlrm_internal.h"

#define DLRM_API extern "C" __attribute__((visibility("default")))

using namespace dlrm;

namespace {

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
inline dlrm_status_t from_hip(hipError_t e) { return e == hipSuccess ? DLRM_OK : DLRM_E_HIP; }
inline int64_t n_pairs(int64_t f) { return f * (f - 1) / 2; }

constexpr int64_t kIntLimit = (int64_t)1 << 30;  // sizes kept well inside int for kernel indexing

// Per-table bag arguments shared by the bag entry points and the forward.
// index_bytes 4: indices and offsets are int32, 8: int64.
dlrm_status_t fill_tables(TableArgs& ta, int32_t T, int64_t B, int32_t D, const float* const* weights,
                          const int64_t* rows, const void* const* indices, const int64_t* n_indices,
                          const void* const* offsets, int32_t index_bytes, bool* aligned, bool* multi_hot) {
    memset(&ta, 0, sizeof(ta));
    if (index_bytes != 4 && index_bytes != 8) return DLRM_E_SHAPE;
    ta.idx32 = index_bytes == 4;
    bool al = (D % 4 == 0);
    bool mh = false;
    for (int32_t t = 0; t < T; ++t) {
        if (!weights[t] || !offsets[t]) return DLRM_E_NULL;
        if (rows[t] < 1 || n_indices[t] < 0 || n_indices[t] > kIntLimit * 64) return DLRM_E_SHAPE;
        if (ta.idx32 && n_indices[t] > INT32_MAX) return DLRM_E_UNSUPPORTED;
        if (n_indices[t] > 0 && !indices[t]) return DLRM_E_NULL;
        ta.w[t] = weights[t];
        ta.idx[t] = indices[t];
        ta.off[t] = offsets[t];
        ta.nidx[t] = n_indices[t];
        al = al && al16(weights[t]);
        mh = mh || (n_indices[t] > B);
    }
    *aligned = al;
    *multi_hot = mh;
    return DLRM_OK;
}

// Table pointers of the stacked layout: table t is rows [row_base[t],
// row_base[t] + rows[t]) of one (sum of rows, D) allocation.
dlrm_status_t stacked_tables(const float* stacked, const int64_t* row_base, const int64_t* rows, int32_t T,
                             int32_t D, const float** w) {
    for (int32_t t = 0; t < T; ++t) {
        if (row_base[t] < 0 || rows[t] < 1 || row_base[t] > ((int64_t)1 << 40)) return DLRM_E_SHAPE;
        w[t] = stacked + row_base[t] * (int64_t)D;
    }
    return DLRM_OK;
}

bool interaction_fits(int32_t T, int32_t D) { return interact_lds_bytes(T, D, 1) <= kMaxLdsBytes; }

// Workspace plan of the forward: R = [x | Z] (B, ldR) and two hidden
// buffers (B, ldH), each region 256-byte aligned.
struct Plan {
    int64_t P, wr, ldR, ldH;
    size_t off_r, off_h0, off_h1, total;
};

dlrm_status_t validate_model(const dlrm_model_t* m, int64_t B) {
    if (!m) return DLRM_E_NULL;
    if (!m->ln_bot || !m->ln_top) return DLRM_E_NULL;
    if (m->n_bot < 2 || m->n_top < 2 || B < 1 || m->num_tables < 1 || m->emb_dim < 1) return DLRM_E_SHAPE;
    if (m->n_bot > DLRM_MAX_LAYERS || m->n_top > DLRM_MAX_LAYERS) return DLRM_E_UNSUPPORTED;
    if (m->num_tables > DLRM_MAX_TABLES || m->emb_dim > kMaxDim) return DLRM_E_UNSUPPORTED;
    for (int32_t l = 0; l < m->n_bot; ++l)
        if (m->ln_bot[l] < 1 || m->ln_bot[l] > kIntLimit) return DLRM_E_SHAPE;
    for (int32_t l = 0; l < m->n_top; ++l)
        if (m->ln_top[l] < 1 || m->ln_top[l] > kIntLimit) return DLRM_E_SHAPE;
    if (m->ln_bot[m->n_bot - 1] != m->emb_dim) return DLRM_E_SHAPE;
    if (m->ln_top[0] != m->emb_dim + n_pairs(m->num_tables + 1)) return DLRM_E_SHAPE;
    if (m->ln_top[m->n_top - 1] != 1) return DLRM_E_SHAPE;
    if (B > kIntLimit) return DLRM_E_UNSUPPORTED;
    if (!interaction_fits(m->num_tables, m->emb_dim)) return DLRM_E_UNSUPPORTED;
    return DLRM_OK;
}

void make_plan(const dlrm_model_t* m, int64_t B, Plan* p) {
    p->P = n_pairs(m->num_tables + 1);
    p->wr = m->emb_dim + p->P;
    p->ldR = round_up(p->wr, 4);
    int64_t maxh = 0;
    for (int32_t l = 1; l + 1 < m->n_bot; ++l) maxh = maxh > m->ln_bot[l] ? maxh : m->ln_bot[l];
    for (int32_t l = 1; l + 1 < m->n_top; ++l) maxh = maxh > m->ln_top[l] ? maxh : m->ln_top[l];
    p->ldH = round_up(maxh, 4);
    const size_t r_bytes = (size_t)round_up(B * p->ldR * (int64_t)sizeof(float), 256);
    const size_t h_bytes = (size_t)round_up(B * p->ldH * (int64_t)sizeof(float), 256);
    p->off_r = 0;
    p->off_h0 = r_bytes;
    p->off_h1 = r_bytes + h_bytes;
    p->total = r_bytes + 2 * h_bytes;
}

}  // namespace

DLRM_API const char* dlrm_status_string(int32_t s) {
    switch (s) {
        case DLRM_OK: return "DLRM_OK";
        case DLRM_E_NULL: return "DLRM_E_NULL: a required pointer is NULL";
        case DLRM_E_SHAPE: return "DLRM_E_SHAPE: inconsistent or non-positive sizes";
        case DLRM_E_WORKSPACE: return "DLRM_E_WORKSPACE: workspace missing, misaligned or too small";
        case DLRM_E_UNSUPPORTED: return "DLRM_E_UNSUPPORTED: sizes beyond the library's limits";
        case DLRM_E_HIP: return "DLRM_E_HIP: a HIP launch failed";
        case DLRM_E_INDEX: return "DLRM_E_INDEX: bag indices or offsets out of range";
    }
    return "unknown dlrm_status_t";
}

DLRM_API int32_t dlrm_abi_version(void) { return DLRM_ABI_VERSION; }

DLRM_API dlrm_status_t dlrm_embbag_sum(int32_t num_tables, int64_t batch, int32_t dim, const float* const* weights,
                                       const int64_t* rows, const void* const* indices, const int64_t* n_indices,
                                       const void* const* offsets, int32_t index_bytes, float* out,
                                       void* stream) {
    if (!weights || !rows || !indices || !n_indices || !offsets || !out) return DLRM_E_NULL;
    if (num_tables < 1 || batch < 1 || dim < 1) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES || dim > kMaxDim || batch > kIntLimit) return DLRM_E_UNSUPPORTED;
    TableArgs ta;
    bool aligned, multi_hot;
    dlrm_status_t st = fill_tables(ta, num_tables, batch, dim, weights, rows, indices, n_indices, offsets,
                                   index_bytes, &aligned, &multi_hot);
    if (st != DLRM_OK) return st;
    aligned = aligned && al16(out);
    return from_hip(launch_embbag_sum(ta, num_tables, dim, batch, aligned, multi_hot, out, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_embbag_sum_stacked(int32_t num_tables, int64_t batch, int32_t dim, const float* stacked,
                                               const int64_t* row_base, const int64_t* rows,
                                               const void* const* indices, const int64_t* n_indices,
                                               const void* const* offsets, int32_t index_bytes, float* out,
                                               void* stream) {
    if (!stacked || !row_base || !rows) return DLRM_E_NULL;
    if (num_tables < 1 || dim < 1) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
    const float* w[DLRM_MAX_TABLES];
    if (stacked_tables(stacked, row_base, rows, num_tables, dim, w) != DLRM_OK) return DLRM_E_SHAPE;
    return dlrm_embbag_sum(num_tables, batch, dim, w, rows, indices, n_indices, offsets, index_bytes, out, stream);
}

DLRM_API dlrm_status_t dlrm_embbag(int32_t num_tables, int64_t batch, int32_t dim, const float* const* weights,
                                   const int64_t* rows, const void* const* indices, const int64_t* n_indices,
                                   const void* const* offsets, const dlrm_bag_options_t* opts, float* out,
                                   void* stream) {
    if (!weights || !rows || !indices || !n_indices || !offsets || !opts || !out) return DLRM_E_NULL;
    if (num_tables < 1 || batch < 1 || dim < 1) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES || dim > kMaxDim || batch > kIntLimit) return DLRM_E_UNSUPPORTED;
    if (opts->mode < DLRM_BAG_SUM || opts->mode > DLRM_BAG_MAX) return DLRM_E_SHAPE;
    if (opts->index_bytes != 4 && opts->index_bytes != 8) return DLRM_E_SHAPE;
    if (opts->per_sample_weights && opts->mode != DLRM_BAG_SUM) return DLRM_E_SHAPE;
    BagArgs ba;
    memset(&ba, 0, sizeof(ba));
    bool al = (dim % 4 == 0) && al16(out);
    bool mh = false;
    for (int32_t t = 0; t < num_tables; ++t) {
        if (!weights[t] || !offsets[t]) return DLRM_E_NULL;
        if (rows[t] < 1 || n_indices[t] < 0 || n_indices[t] > kIntLimit * 64) return DLRM_E_SHAPE;
        if (opts->index_bytes == 4 && n_indices[t] > INT32_MAX) return DLRM_E_UNSUPPORTED;
        if (n_indices[t] > 0 && !indices[t]) return DLRM_E_NULL;
        if (opts->per_sample_weights && n_indices[t] > 0 && !opts->per_sample_weights[t]) return DLRM_E_NULL;
        ba.w[t] = weights[t];
        ba.idx[t] = indices[t];
        ba.off[t] = offsets[t];
        ba.nidx[t] = n_indices[t];
        ba.psw[t] = opts->per_sample_weights ? opts->per_sample_weights[t] : nullptr;
        ba.pad[t] = (opts->padding_idx && opts->padding_idx[t] >= 0) ? opts->padding_idx[t] : -1;
        al = al && al16(weights[t]);
        mh = mh || (n_indices[t] > batch);
    }
    return from_hip(launch_embbag_ex(ba, num_tables, dim, batch, opts->mode, opts->include_last_offset ? 1 : 0,
                                     opts->index_bytes == 4, al, mh, out, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_interact_lower_tri(int64_t batch, int32_t num_tables, int32_t dim, const float* x,
                                               int64_t ld_x, const float* emb, float* out, int64_t ld_out,
                                               int32_t concat_dense, void* stream) {
    if (!x || !emb || !out) return DLRM_E_NULL;
    if (batch < 1 || num_tables < 1 || dim < 1 || ld_x < dim) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES || dim > kMaxDim || batch > kIntLimit) return DLRM_E_UNSUPPORTED;
    if (!interaction_fits(num_tables, dim)) return DLRM_E_UNSUPPORTED;
    const int64_t P = n_pairs(num_tables + 1);
    if (ld_out < (concat_dense ? dim + P : P)) return DLRM_E_SHAPE;
    const bool aligned = (dim % 4 == 0) && (ld_x % 4 == 0) && al16(x) && al16(emb);
    return from_hip(launch_interact(nullptr, emb, num_tables, dim, batch, aligned, false, x, ld_x, out, ld_out,
                                    concat_dense ? 0 : -1, concat_dense ? dim : 0, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_embbag_interact(int32_t num_tables, int64_t batch, int32_t dim,
                                            const float* const* weights, const int64_t* rows,
                                            const void* const* indices, const int64_t* n_indices,
                                            const void* const* offsets, int32_t index_bytes, const float* x,
                                            int64_t ld_x, float* out, int64_t ld_out, int32_t concat_dense,
                                            void* stream) {
    if (!weights || !rows || !indices || !n_indices || !offsets || !x || !out) return DLRM_E_NULL;
    if (num_tables < 1 || batch < 1 || dim < 1 || ld_x < dim) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES || dim > kMaxDim || batch > kIntLimit) return DLRM_E_UNSUPPORTED;
    if (!interaction_fits(num_tables, dim)) return DLRM_E_UNSUPPORTED;
    const int64_t P = n_pairs(num_tables + 1);
    if (ld_out < (concat_dense ? dim + P : P)) return DLRM_E_SHAPE;
    TableArgs ta;
    bool aligned, multi_hot;
    dlrm_status_t st = fill_tables(ta, num_tables, batch, dim, weights, rows, indices, n_indices, offsets,
                                   index_bytes, &aligned, &multi_hot);
    if (st != DLRM_OK) return st;
    aligned = aligned && (ld_x % 4 == 0) && al16(x);
    return from_hip(launch_interact(&ta, nullptr, num_tables, dim, batch, aligned, multi_hot, x, ld_x, out, ld_out,
                                    concat_dense ? 0 : -1, concat_dense ? dim : 0, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_linear_bias_act(int64_t M, int64_t N, int64_t K, const float* x, int64_t ld_x,
                                            const float* W, const float* bias, int32_t act, float* y, int64_t ld_y,
                                            void* stream) {
    if (!x || !W || !y) return DLRM_E_NULL;
    if (M < 1 || N < 1 || K < 1 || ld_x < K || ld_y < N) return DLRM_E_SHAPE;
    if (act < DLRM_ACT_NONE || act > DLRM_ACT_SIGMOID) return DLRM_E_SHAPE;
    if (M > kIntLimit || N > kIntLimit || K > kIntLimit) return DLRM_E_UNSUPPORTED;
    return from_hip(launch_linear(M, N, K, x, ld_x, W, bias, act, y, ld_y, (hipStream_t)stream));
}

DLRM_API size_t dlrm_forward_workspace_bytes(const dlrm_model_t* m, int64_t batch) {
    if (validate_model(m, batch) != DLRM_OK) return 0;
    Plan p;
    make_plan(m, batch, &p);
    return p.total;
}

namespace {

// The model's table pointers: emb_w, or the stacked layout when emb_w is NULL.
dlrm_status_t model_tables(const dlrm_model_t* m, const float** w) {
    if (!m->rows) return DLRM_E_NULL;
    if (m->emb_w) {
        for (int32_t t = 0; t < m->num_tables; ++t) w[t] = m->emb_w[t];
        return DLRM_OK;
    }
    if (!m->emb_stacked || !m->emb_row_base) return DLRM_E_NULL;
    return stacked_tables(m->emb_stacked, m->emb_row_base, m->rows, m->num_tables, m->emb_dim, w);
}

// Checks shared by every forward entry point; fills the table arguments.
dlrm_status_t forward_args(const dlrm_model_t* m, int64_t batch, const float* dense, const void* const* indices,
                           const int64_t* n_indices, const void* const* offsets, int32_t index_bytes,
                           const float* out, TableArgs& ta, bool* aligned, bool* multi_hot) {
    dlrm_status_t st = validate_model(m, batch);
    if (st != DLRM_OK) return st;
    if (!dense || !indices || !n_indices || !offsets || !out) return DLRM_E_NULL;
    if (!m->rows || !m->bot_w || !m->bot_b || !m->top_w || !m->top_b) return DLRM_E_NULL;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l)
        if (!m->bot_w[l] || !m->bot_b[l]) return DLRM_E_NULL;
    for (int32_t l = 0; l + 1 < m->n_top; ++l)
        if (!m->top_w[l] || !m->top_b[l]) return DLRM_E_NULL;
    const float* w[DLRM_MAX_TABLES];
    st = model_tables(m, w);
    if (st != DLRM_OK) return st;
    return fill_tables(ta, m->num_tables, batch, m->emb_dim, w, m->rows, indices, n_indices, offsets, index_bytes,
                       aligned, multi_hot);
}

// Segments of the packed tail (see SmallBlock).
void small_block(const dlrm_model_t* m, SmallBlock& sb) {
    memset(&sb, 0, sizeof(sb));
    const int klast = (int)m->ln_top[m->n_top - 2];
    int off = 0;
    auto add = [&](const float* src, int len, int pad_to) {
        sb.src[sb.nseg] = src;
        sb.len[sb.nseg] = len;
        sb.off[sb.nseg] = off;
        ++sb.nseg;
        off += (pad_to + 3) / 4 * 4;
    };
    add(m->top_w ? m->top_w[m->n_top - 2] : nullptr, klast, klast);
    add(m->top_b ? m->top_b[m->n_top - 2] : nullptr, 1, 4);
    for (int32_t l = 0; l + 1 < m->n_bot && l < kFusedMaxLayers; ++l)
        add(m->bot_b ? m->bot_b[l] : nullptr, (int)m->ln_bot[l + 1], (int)m->ln_bot[l + 1]);
    for (int32_t l = 0; l + 2 < m->n_top && l < kFusedMaxLayers; ++l)
        add(m->top_b ? m->top_b[l] : nullptr, (int)m->ln_top[l + 1], (int)m->ln_top[l + 1]);
    sb.total = off;
}

// Kernel arguments of the single-launch path (with packed-weight pointers
// relative to `packed`, which may be NULL when only the shape is checked);
// false when the model is outside its limits.
bool fused_args(const dlrm_model_t* m, int64_t batch, const float* dense, float* out, const TableArgs& ta,
                bool aligned, const float* packed, FusedArgs& fa) {
    if (m->n_bot - 1 > kFusedMaxLayers || m->n_top - 1 > kFusedMaxLayers) return false;
    memset(&fa, 0, sizeof(fa));
    fa.ta = ta;
    fa.bot.n_layers = m->n_bot - 1;
    fa.top.n_layers = m->n_top - 1;
    for (int32_t l = 0; l < m->n_bot; ++l) fa.bot.dim[l] = (int)m->ln_bot[l];
    for (int32_t l = 0; l < m->n_top; ++l) fa.top.dim[l] = (int)m->ln_top[l];
    size_t off = 0;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) {
        fa.bot.w[l] = packed ? packed + off : nullptr;
        fa.bot.b[l] = m->bot_b[l];
        off += packed_layer_floats(fa.bot.dim[l + 1], fa.bot.dim[l]);
    }
    for (int32_t l = 0; l + 2 < m->n_top; ++l) {
        fa.top.w[l] = packed ? packed + off : nullptr;
        fa.top.b[l] = m->top_b[l];
        off += packed_layer_floats(fa.top.dim[l + 1], fa.top.dim[l]);
    }
    SmallBlock sb;
    small_block(m, sb);
    fa.small = packed ? packed + off : nullptr;
    fa.n_small = sb.total;
    fa.packed = packed;
    fa.n_packed = (int64_t)off + sb.total;
    fa.dense = dense;
    fa.out = out;
    fa.B = batch;
    fa.T = m->num_tables;
    fa.D = m->emb_dim;
    return fused_supported(fa, aligned);
}

// Floats of the packed weights of every layer but the last, plus the tail.
size_t packed_floats(const dlrm_model_t* m) {
    size_t n = 0;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) n += packed_layer_floats((int)m->ln_bot[l + 1], (int)m->ln_bot[l]);
    for (int32_t l = 0; l + 2 < m->n_top; ++l) n += packed_layer_floats((int)m->ln_top[l + 1], (int)m->ln_top[l]);
    SmallBlock sb;
    small_block(m, sb);
    return n + ((size_t)sb.total + 63) / 64 * 64;
}

// Shape-only check of the single-launch path for a model (tables' alignment
// included); used by the packing calls.
bool model_fits_fused(const dlrm_model_t* m) {
    const float* w[DLRM_MAX_TABLES];
    if (validate_model(m, 1) != DLRM_OK || model_tables(m, w) != DLRM_OK) return false;
    bool aligned = (m->emb_dim % 4 == 0);
    for (int32_t t = 0; t < m->num_tables; ++t) aligned = aligned && w[t] && al16(w[t]);
    TableArgs ta;
    memset(&ta, 0, sizeof(ta));
    FusedArgs fa;
    return fused_args(m, 1, nullptr, nullptr, ta, aligned, nullptr, fa);
}

// Where dlrm_forward takes the single launch.  Every block streams all the
// Linear weights from L2 (so they must stay well inside one XCD's 4 MiB),
// and a block holds 8 samples (16 past batch 2048), so a forward costs about
// one block's time per round of 256 blocks; the layered GEMMs share weights
// across the whole chip.  Measured on MI355X over the batch x tables sweep
// of the 13-512-256-64 / (64+P)-512-256-1 model (both paths replayed from
// graphs of 8 steps): the single launch is faster up to batch 8192 with up
// to 16 tables, and up to 4096 with 24 to 32 tables when its dots run as one
// MFMA tile per sample (otherwise only from 1024 to 2048); past that the
// layered path, whose bag + interaction kernel forms the dots as a Gram
// matrix on the matrix cores, wins.
constexpr int64_t kFusedAutoMaxBatch = 8192;
constexpr int64_t kFusedAutoMaxWeightBytes = 3 << 20;
bool fused_preferred(const dlrm_model_t* m, int64_t batch) {
    if (batch > kFusedAutoMaxBatch) return false;
    if (m->num_tables >= 24) {
        // one MFMA tile per sample takes the dots up to 32 tables (D % 16 == 0)
        const bool gram = m->num_tables <= 32 && m->emb_dim % 16 == 0;
        return gram ? batch <= 4096 : batch >= 1024 && batch <= 2048;
    }
    return true;
}

// Bytes of all Linear weights of the model.
int64_t weight_bytes(const dlrm_model_t* m) {
    int64_t n = 0;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) n += m->ln_bot[l] * m->ln_bot[l + 1];
    for (int32_t l = 0; l + 1 < m->n_top; ++l) n += m->ln_top[l] * m->ln_top[l + 1];
    return 4 * n;
}

dlrm_status_t forward_layered(const dlrm_model_t* m, int64_t batch, const float* dense, float* out,
                              const TableArgs& ta, bool aligned, bool multi_hot, void* workspace, size_t ws_bytes,
                              hipStream_t s) {
    const int32_t T = m->num_tables, D = m->emb_dim;
    Plan p;
    make_plan(m, batch, &p);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || ws_bytes < p.total) return DLRM_E_WORKSPACE;
    char* ws = (char*)workspace;
    float* R = (float*)(ws + p.off_r);
    float* H[2] = {(float*)(ws + p.off_h0), (float*)(ws + p.off_h1)};
    int hsel = 0;

    // 1. bottom MLP, ReLU after every layer; the last layer writes x into R[:, 0:D]
    const float* in = dense;
    int64_t ld_in = m->ln_bot[0];
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) {
        const bool last = (l + 2 == m->n_bot);
        float* o = last ? R : H[hsel];
        const int64_t ld_o = last ? p.ldR : p.ldH;
        hipError_t e = launch_linear(batch, m->ln_bot[l + 1], m->ln_bot[l], in, ld_in, m->bot_w[l], m->bot_b[l],
                                     DLRM_ACT_RELU, o, ld_o, s);
        if (e != hipSuccess) return DLRM_E_HIP;
        if (!last) hsel ^= 1;
        in = o;
        ld_in = ld_o;
    }

    // 2-5. bags gathered into LDS, dots, Z written into R[:, D:D+P]
    {
        hipError_t e = launch_interact(&ta, nullptr, T, D, batch, aligned, multi_hot, R, p.ldR, R, p.ldR, -1, D, s);
        if (e != hipSuccess) return DLRM_E_HIP;
    }

    // 6-7. top MLP: ReLU on hidden layers, sigmoid on the one-output last layer
    in = R;
    ld_in = p.ldR;
    for (int32_t l = 0; l + 1 < m->n_top; ++l) {
        const bool last = (l + 2 == m->n_top);
        float* o = last ? out : H[hsel];
        const int64_t ld_o = last ? 1 : p.ldH;
        hipError_t e = launch_linear(batch, m->ln_top[l + 1], m->ln_top[l], in, ld_in, m->top_w[l], m->top_b[l],
                                     last ? DLRM_ACT_SIGMOID : DLRM_ACT_RELU, o, ld_o, s);
        if (e != hipSuccess) return DLRM_E_HIP;
        if (!last) hsel ^= 1;
        in = o;
        ld_in = ld_o;
    }
    return DLRM_OK;
}

}  // namespace

DLRM_API dlrm_status_t dlrm_forward_layered(const dlrm_model_t* m, int64_t batch, const float* dense,
                                            const void* const* indices, const int64_t* n_indices,
                                            const void* const* offsets, int32_t index_bytes, float* out,
                                            void* workspace, size_t ws_bytes, void* stream) {
    TableArgs ta;
    bool aligned, multi_hot;
    dlrm_status_t st = forward_args(m, batch, dense, indices, n_indices, offsets, index_bytes, out, ta, &aligned,
                                    &multi_hot);
    if (st != DLRM_OK) return st;
    return forward_layered(m, batch, dense, out, ta, aligned, multi_hot, workspace, ws_bytes, (hipStream_t)stream);
}

DLRM_API size_t dlrm_pack_weights_bytes(const dlrm_model_t* m) {
    if (!m || !model_fits_fused(m)) return 0;
    return packed_floats(m) * sizeof(float);
}

DLRM_API dlrm_status_t dlrm_pack_weights(const dlrm_model_t* m, float* packed, size_t bytes, void* stream) {
    if (!m || !packed) return DLRM_E_NULL;
    if (validate_model(m, 1) != DLRM_OK) return DLRM_E_SHAPE;
    if (!m->bot_w || !m->top_w) return DLRM_E_NULL;
    if (!model_fits_fused(m)) return DLRM_E_UNSUPPORTED;
    if (((uintptr_t)packed & 255u) != 0 || bytes < packed_floats(m) * sizeof(float)) return DLRM_E_WORKSPACE;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l)
        if (!m->bot_w[l]) return DLRM_E_NULL;
    for (int32_t l = 0; l + 1 < m->n_top; ++l)
        if (!m->top_w[l]) return DLRM_E_NULL;
    if (!m->bot_b || !m->top_b) return DLRM_E_NULL;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l)
        if (!m->bot_b[l]) return DLRM_E_NULL;
    for (int32_t l = 0; l + 1 < m->n_top; ++l)
        if (!m->top_b[l]) return DLRM_E_NULL;
    hipStream_t s = (hipStream_t)stream;
    size_t off = 0;
    for (int32_t l = 0; l + 1 < m->n_bot; ++l) {
        const int N = (int)m->ln_bot[l + 1], K = (int)m->ln_bot[l];
        if (launch_pack_layer(m->bot_w[l], N, K, packed + off, s) != hipSuccess) return DLRM_E_HIP;
        off += packed_layer_floats(N, K);
    }
    for (int32_t l = 0; l + 2 < m->n_top; ++l) {
        const int N = (int)m->ln_top[l + 1], K = (int)m->ln_top[l];
        if (launch_pack_layer(m->top_w[l], N, K, packed + off, s) != hipSuccess) return DLRM_E_HIP;
        off += packed_layer_floats(N, K);
    }
    SmallBlock sb;
    small_block(m, sb);
    if (launch_pack_small(sb, packed + off, s) != hipSuccess) return DLRM_E_HIP;
    return DLRM_OK;
}

DLRM_API dlrm_status_t dlrm_forward_fused(const dlrm_model_t* m, int64_t batch, const float* dense,
                                          const void* const* indices, const int64_t* n_indices,
                                          const void* const* offsets, int32_t index_bytes, float* out,
                                          void* stream) {
    TableArgs ta;
    bool aligned, multi_hot;
    dlrm_status_t st = forward_args(m, batch, dense, indices, n_indices, offsets, index_bytes, out, ta, &aligned,
                                    &multi_hot);
    if (st != DLRM_OK) return st;
    FusedArgs fa;
    if (!fused_args(m, batch, dense, out, ta, aligned, m->packed_w, fa)) return DLRM_E_UNSUPPORTED;
    if (!m->packed_w) return DLRM_E_NULL;
    if (!al16(m->packed_w)) return DLRM_E_SHAPE;
    return from_hip(launch_fused_forward(fa, aligned, multi_hot, (hipStream_t)stream));
}

DLRM_API int32_t dlrm_forward_path(const dlrm_model_t* m, int64_t batch) {
    if (!m || validate_model(m, batch) != DLRM_OK) return 0;
    if (m->packed_w && al16(m->packed_w) && fused_preferred(m, batch) &&
        weight_bytes(m) <= kFusedAutoMaxWeightBytes && model_fits_fused(m))
        return DLRM_PATH_FUSED;
    return DLRM_PATH_LAYERED;
}

DLRM_API dlrm_status_t dlrm_forward(const dlrm_model_t* m, int64_t batch, const float* dense,
                                    const void* const* indices, const int64_t* n_indices,
                                    const void* const* offsets, int32_t index_bytes, float* out, void* workspace,
                                    size_t ws_bytes, void* stream) {
    TableArgs ta;
    bool aligned, multi_hot;
    dlrm_status_t st = forward_args(m, batch, dense, indices, n_indices, offsets, index_bytes, out, ta, &aligned,
                                    &multi_hot);
    if (st != DLRM_OK) return st;
    Plan p;
    make_plan(m, batch, &p);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || ws_bytes < p.total) return DLRM_E_WORKSPACE;
    FusedArgs fa;
    if (m->packed_w && al16(m->packed_w) && fused_preferred(m, batch) &&
        weight_bytes(m) <= kFusedAutoMaxWeightBytes && fused_args(m, batch, dense, out, ta, aligned, m->packed_w, fa))
        return from_hip(launch_fused_forward(fa, aligned, multi_hot, (hipStream_t)stream));
    return forward_layered(m, batch, dense, out, ta, aligned, multi_hot, workspace, ws_bytes, (hipStream_t)stream);
}

DLRM_API dlrm_status_t dlrm_embbag_check_indices(int32_t num_tables, int64_t batch, const int64_t* rows,
                                                 const void* const* indices, const int64_t* n_indices,
                                                 const void* const* offsets, int32_t index_bytes,
                                                 int32_t* bad_count_device, void* stream) {
    if (!rows || !indices || !n_indices || !offsets || !bad_count_device) return DLRM_E_NULL;
    if (num_tables < 1 || batch < 1) return DLRM_E_SHAPE;
    if (index_bytes != 4 && index_bytes != 8) return DLRM_E_SHAPE;
    if (num_tables > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
    CheckArgs ca;
    memset(&ca, 0, sizeof(ca));
    ca.idx32 = index_bytes == 4;
    for (int32_t t = 0; t < num_tables; ++t) {
        if (!offsets[t]) return DLRM_E_NULL;
        if (n_indices[t] < 0) return DLRM_E_SHAPE;
        if (n_indices[t] > 0 && !indices[t]) return DLRM_E_NULL;
        ca.idx[t] = indices[t];
        ca.off[t] = offsets[t];
        ca.nidx[t] = n_indices[t];
        ca.rows[t] = rows[t];
    }
    return from_hip(launch_check_indices(ca, num_tables, batch, bad_count_device, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_pair_index_map(int32_t n_feat, int32_t* i_out, int32_t* j_out, void* stream) {
    if (!i_out || !j_out) return DLRM_E_NULL;
    if (n_feat < 2 || n_feat > 4096) return DLRM_E_SHAPE;
    return from_hip(launch_pair_index_map(n_feat, i_out, j_out, (hipStream_t)stream));
}

DLRM_API int64_t dlrm_probe_sink_floats(void) { return probe_blocks(); }

DLRM_API dlrm_status_t dlrm_probe_read_stream(const float* src, int64_t n_floats, float* sink, void* stream) {
    if (!src || !sink) return DLRM_E_NULL;
    if (n_floats < 4 || n_floats % 4 != 0) return DLRM_E_SHAPE;
    if (!al16(src)) return DLRM_E_SHAPE;
    return from_hip(launch_read_stream(src, n_floats, sink, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_probe_l2_stream(const float* src, int64_t n_floats, int32_t blocks, float* sink,
                                            void* stream) {
    if (!src || !sink) return DLRM_E_NULL;
    if (n_floats < 4 || n_floats % 4 != 0 || blocks < 1 || blocks > 65536) return DLRM_E_SHAPE;
    if (!al16(src)) return DLRM_E_SHAPE;
    return from_hip(launch_l2_stream(src, n_floats, blocks, sink, (hipStream_t)stream));
}

DLRM_API dlrm_status_t dlrm_probe_gather_rows(const float* table, int64_t rows, int32_t dim, const int64_t* idx,
                                              int64_t n, float* sink, void* stream) {
    if (!table || !idx || !sink) return DLRM_E_NULL;
    if (rows < 1 || n < 1 || dim < 16 || dim > 256 || (dim & (dim - 1)) != 0) return DLRM_E_SHAPE;
    if (!al16(table)) return DLRM_E_SHAPE;
    return from_hip(launch_gather_rows(table, dim, idx, n, sink, (hipStream_t)stream));
}
