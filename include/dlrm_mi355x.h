/*
 * dlrm_mi355x.h -- C ABI of the DLRMv1 forward hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * The library computes, on one GPU, the DLRMv1 inference forward described on
 * the pages "luminal compare dlrm-fused-kernels...dlrm-pt2-megakernel" (file
 * dlrm_megakernel.rs, DlrmMegaKernel::cuda_source) and "luminal compare
 * asglover/modal_ci_ready...vanilla-pytorch" (commit message, sections
 * "Translator" and "cuda_lite kernels"):
 *
 *   x  = bottom MLP(dense)            Linear + ReLU on every layer
 *   E  = per-table sum-pooled bags    (batch, tables, d)
 *   Z  = strict-lower-triangle dots   over F = tables + 1 vectors [x, E_0..]
 *   R  = [x | Z]                      (batch, d + F(F-1)/2)
 *   y  = top MLP(R)                   Linear + ReLU, last layer Linear + sigmoid
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Memory: every buffer is allocated and owned by the caller.  "device"
 *    pointers address GPU memory of the current HIP device; "host" pointers
 *    (the small per-table pointer and size arrays, the model descriptor) are
 *    read during the call only and never kept.  The library allocates
 *    nothing and frees nothing.
 *  - Layout: row-major, C-contiguous unless an explicit leading dimension
 *    (ld_*) is given, in elements.  Floating point is IEEE fp32.  Indices and
 *    offsets are integers of the width `index_bytes` gives: 8 (int64, PyTorch's
 *    torch.long) or 4 (int32, the width the pages' megakernel narrows them to:
 *    DlrmMegaKernel struct fields in dlrm_megakernel.rs, "luminal compare
 *    dlrm-fused-kernels...dlrm-pt2-megakernel"); one width for all tables of a
 *    call, indices and offsets alike.  Other widths give DLRM_E_SHAPE.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream).  Every call only enqueues work on that stream: there is no host
 *    or device synchronisation, no host<->device copy and no allocation, so
 *    calls can be captured into a HIP graph.  Calls keep no state and may run
 *    concurrently on different streams.
 *  - Errors: every call validates its arguments on the host before enqueuing
 *    anything and returns a dlrm_status_t; it never aborts or throws.  On an
 *    error nothing has been enqueued.  DLRM_E_HIP reports a failed kernel
 *    launch (hipGetLastError after the launch).
 *  - Index validity: indices in [0, rows) and offsets non-decreasing within
 *    [0, n_indices] are the caller's contract in the compute calls, as on the
 *    pages, which never check them.  dlrm_embbag_check_indices validates them
 *    on the device.
 */
#ifndef DLRM_MI355X_H
#define DLRM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dlrm_status {
    DLRM_OK = 0,
    DLRM_E_NULL = 1,        /* a required pointer is NULL                        */
    DLRM_E_SHAPE = 2,       /* sizes inconsistent, non-positive or ld too small  */
    DLRM_E_WORKSPACE = 3,   /* workspace NULL or smaller than required           */
    DLRM_E_UNSUPPORTED = 4, /* e.g. more tables than DLRM_MAX_TABLES             */
    DLRM_E_HIP = 5,         /* a HIP launch failed                               */
    DLRM_E_INDEX = 6        /* dlrm_embbag_check_indices found bad data          */
} dlrm_status_t;

/* Most tables one call accepts (their pointers travel in kernel arguments). */
#define DLRM_MAX_TABLES 64
/* Most entries in ln_bot / ln_top. */
#define DLRM_MAX_LAYERS 32

/* Activation selector of dlrm_linear_bias_act. */
#define DLRM_ACT_NONE 0
#define DLRM_ACT_RELU 1
#define DLRM_ACT_SIGMOID 2

/*
 * Model descriptor of dlrm_forward, the fields of the pages' DlrmShape /
 * DlrmMegaKernel (dlrm_megakernel.rs struct fields; dlrm_pattern.rs DlrmShape).
 * All arrays are host arrays; the weight entries are device pointers.
 *   ln_bot[0]          dense feature width, ln_bot[n_bot-1] == emb_dim
 *   ln_top[0]          == emb_dim + F(F-1)/2 with F = num_tables + 1
 *   ln_top[n_top-1]    == 1 (binary classifier)
 *   bot_w[l]           (ln_bot[l+1], ln_bot[l]) nn.Linear layout, bot_b[l] (ln_bot[l+1])
 *   top_w[l]           (ln_top[l+1], ln_top[l]),                top_b[l] (ln_top[l+1])
 *   emb_w[t]           (rows[t], emb_dim); or NULL, and then the tables are
 *                      stacked: table t is rows [emb_row_base[t],
 *                      emb_row_base[t] + rows[t]) of the one device allocation
 *                      emb_stacked (sum of rows, emb_dim), the pre-stacked
 *                      weight of StackedEmbeddingBagKernel ("luminal compare
 *                      asglover/modal_ci_ready...vanilla-pytorch", cuda_lite
 *                      kernels)
 *   packed_w           NULL, or device memory holding the weights and biases
 *                      in the order the single-launch forward reads them,
 *                      written by dlrm_pack_weights from the arrays above
 *                      (pack again after changing them)
 * Biases may not be NULL.
 */
typedef struct dlrm_model {
    int32_t n_bot;
    const int64_t* ln_bot;
    int32_t n_top;
    const int64_t* ln_top;
    int32_t num_tables;
    int32_t emb_dim;
    const int64_t* rows;
    const float* const* emb_w;
    const float* const* bot_w;
    const float* const* bot_b;
    const float* const* top_w;
    const float* const* top_b;
    const float* packed_w;
    const float* emb_stacked;
    const int64_t* emb_row_base;
} dlrm_model_t;

/*
 * dlrm_embbag_sum -- sum-pooled embedding bags of T tables in one launch.
 *
 * Defines out[b][t][:] = sum over k in [offsets[t][b], end_t(b)) of
 * weights[t][indices[t][k]][:], with end_t(b) = offsets[t][b+1] for
 * b < batch-1 and n_indices[t] for the last bag (PyTorch's
 * include_last_offset=False convention); an empty bag gives zeros.
 * Source: LessonsLearned entry "DLRM compile: EmbeddingBag translator gap",
 * point 2, and movement.rs translate_embedding_bag on "luminal compare
 * dlrm-fused-kernels...dlrm-pt2-megakernel"; the (batch, num_tables, d)
 * one-launch multi-table output of MultiTableEmbeddingBagSumKernel on "luminal
 * compare asglover/modal_ci_ready...vanilla-pytorch" (cuda_lite kernels).
 * Mode is sum; there are no per-sample weights and no padding index.
 *
 *   num_tables  T in [1, DLRM_MAX_TABLES]
 *   batch       B >= 1
 *   dim         d >= 1 (any; multiples of 4 with 16-byte aligned tables take
 *               the vector path)
 *   weights     host[T] of device pointers, table t is (rows[t], dim)
 *   rows        host[T], rows[t] >= 1 (used by the checked call only)
 *   indices     host[T] of device pointers, (n_indices[t]) integers
 *   n_indices   host[T], >= 0 (<= INT32_MAX with 4-byte indices)
 *   offsets     host[T] of device pointers, (batch) integers
 *   index_bytes 4 or 8, the width of indices and offsets
 *   out         device (batch, T, dim) fp32, written completely
 * Bag sums are accumulated in fp32 in increasing k.
 */
dlrm_status_t dlrm_embbag_sum(int32_t num_tables, int64_t batch, int32_t dim,
                              const float* const* weights, const int64_t* rows,
                              const void* const* indices, const int64_t* n_indices,
                              const void* const* offsets, int32_t index_bytes, float* out,
                              void* stream);

/*
 * dlrm_embbag_sum_stacked -- dlrm_embbag_sum over tables stacked in one
 * allocation, the pre-stacked weight layout of StackedEmbeddingBagKernel
 * ("luminal compare asglover/modal_ci_ready...vanilla-pytorch", cuda_lite
 * kernels): table t is rows [row_base[t], row_base[t] + rows[t]) of the
 * device array `stacked` (sum of rows, dim); indices stay relative to their
 * own table.  row_base and rows are host[T], row_base[t] >= 0.  Other
 * arguments, output and errors as dlrm_embbag_sum.
 */
dlrm_status_t dlrm_embbag_sum_stacked(int32_t num_tables, int64_t batch, int32_t dim,
                                      const float* stacked, const int64_t* row_base,
                                      const int64_t* rows, const void* const* indices,
                                      const int64_t* n_indices, const void* const* offsets,
                                      int32_t index_bytes, float* out, void* stream);

/* Pooling modes of dlrm_embbag. */
#define DLRM_BAG_SUM 0
#define DLRM_BAG_MEAN 1
#define DLRM_BAG_MAX 2

/*
 * Options of dlrm_embbag: the arguments of PyTorch's embedding_bag that the
 * pages' translator names and leaves to follow-up work (movement.rs
 * translate_embedding_bag and dlrm_pattern.rs match_dlrm on "luminal compare
 * dlrm-fused-kernels...dlrm-pt2-megakernel").
 *   mode                 DLRM_BAG_SUM, DLRM_BAG_MEAN or DLRM_BAG_MAX
 *   include_last_offset  0: offsets[t] hold batch entries, the last bag ends at
 *                        n_indices[t]; 1: offsets[t] hold batch + 1 entries and
 *                        bag b is [offsets[t][b], offsets[t][b+1])
 *   index_bytes          8: indices and offsets are int64; 4: int32
 *   padding_idx          host[T] or NULL; entry p >= 0 leaves the indices equal
 *                        to p out of every bag of table t (-1: none)
 *   per_sample_weights   host[T] of device pointers to n_indices[t] fp32
 *                        weights, or NULL; sum mode only
 */
typedef struct dlrm_bag_options {
    int32_t mode;
    int32_t include_last_offset;
    int32_t index_bytes;
    int32_t reserved;
    const int64_t* padding_idx;
    const float* const* per_sample_weights;
} dlrm_bag_options_t;

/*
 * dlrm_embbag -- general embedding bags of T tables in one launch:
 * out[b][t] = reduce(weights[t][i] for the indices i of bag b), with
 * reduce = sum (times the per-sample weight), mean (the sum over the number of
 * indices in the bag) or elementwise max; an empty bag gives zeros.  Source:
 * the reduce_op form of the bag on the LessonsLearned entry "DLRM compile:
 * EmbeddingBag translator gap", point 2, "luminal compare
 * dlrm-fused-kernels...dlrm-pt2-megakernel".
 * Arguments as dlrm_embbag_sum, except that indices and offsets are untyped
 * device pointers of the width opts->index_bytes gives, and opts may not be
 * NULL.  Sums accumulate in fp32 in increasing k; the mean divides the fp32
 * sum by the count.
 */
dlrm_status_t dlrm_embbag(int32_t num_tables, int64_t batch, int32_t dim, const float* const* weights,
                          const int64_t* rows, const void* const* indices, const int64_t* n_indices,
                          const void* const* offsets, const dlrm_bag_options_t* opts, float* out,
                          void* stream);

/*
 * dlrm_interact_lower_tri -- pairwise-dot feature interaction.
 *
 * For each sample b, S_b = [x_b, emb[b][0], ..., emb[b][T-1]] (F = T + 1
 * vectors of length dim) and Z[b][p] = <S_b[i], S_b[j]> for the flat pair
 * index p = i(i-1)/2 + j, 0 <= j < i < F: the strict lower triangle of
 * S_b S_b^T in row-major order, i.e. bmm(S, S^T)[:, li, lj].
 * Source: dlrm_megakernel.rs cuda_source step 4 ("luminal compare
 * dlrm-fused-kernels...dlrm-pt2-megakernel"); PairwiseDotLowerTriStackedKernel
 * and the index.Tensor peephole ("luminal compare
 * asglover/modal_ci_ready...vanilla-pytorch", Translator and cuda_lite
 * kernels).  Step 5 of the same cuda_source (R = cat(x, zflat)) is the
 * concat_dense form.
 *
 *   batch         B >= 1
 *   num_tables    T in [1, DLRM_MAX_TABLES]
 *   dim           d in [1, 1024]; one sample's F*d + P floats must fit in
 *                 64 KiB of LDS, else DLRM_E_UNSUPPORTED
 *   x             device (B, ld_x) fp32, first dim columns used, ld_x >= dim
 *   emb           device (B, T, dim) fp32
 *   out           device (B, ld_out) fp32
 *   concat_dense  0: out[b][0:P] = Z[b], ld_out >= P;
 *                 1: out[b][0:dim] = x[b], out[b][dim:dim+P] = Z[b], ld_out >= dim + P
 * Other columns of out are not touched.
 */
dlrm_status_t dlrm_interact_lower_tri(int64_t batch, int32_t num_tables, int32_t dim,
                                      const float* x, int64_t ld_x, const float* emb,
                                      float* out, int64_t ld_out, int32_t concat_dense,
                                      void* stream);

/*
 * dlrm_embbag_interact -- dlrm_embbag_sum and dlrm_interact_lower_tri fused in
 * one launch: the bag sums of each sample are gathered straight into on-chip
 * memory and dotted there, so E is never written.  Output and argument
 * meanings are those of the two calls above (same citations); the table
 * arguments follow dlrm_embbag_sum, x / out / ld_* / concat_dense follow
 * dlrm_interact_lower_tri.  x and out may point into one buffer when the
 * columns written do not overlap the x columns read (for example x = R and
 * out = R + dim with concat_dense = 0, which fills Z in beside x).
 */
dlrm_status_t dlrm_embbag_interact(int32_t num_tables, int64_t batch, int32_t dim,
                                   const float* const* weights, const int64_t* rows,
                                   const void* const* indices, const int64_t* n_indices,
                                   const void* const* offsets, int32_t index_bytes, const float* x,
                                   int64_t ld_x, float* out, int64_t ld_out, int32_t concat_dense,
                                   void* stream);

/*
 * dlrm_linear_bias_act -- y = act(x W^T + bias), i.e. addmm(bias, x, W.t())
 * with alpha = beta = 1 against the (N, K) nn.Linear weight, followed by the
 * absorbed ReLU / sigmoid consumer (linear_bias, linear_bias_relu,
 * linear_bias_sigmoid on "luminal compare asglover/modal_ci_ready...
 * vanilla-pytorch", Translator; sigmoid = 1/(1+exp(-a)) as KernelSigmoid on
 * "luminal compare nvidia-devcontainer-args...perf/compile-write-rayon").
 * Computed in fp32 on the matrix cores (MFMA) for N > 1, by a dot-product
 * kernel for N == 1.
 *
 *   M >= 1 rows, N >= 1 outputs, K >= 1 inputs
 *   x      device (M, ld_x) fp32, ld_x >= K
 *   W      device (N, K) fp32, contiguous
 *   bias   device (N) fp32, or NULL for no bias
 *   act    DLRM_ACT_NONE, DLRM_ACT_RELU or DLRM_ACT_SIGMOID
 *   y      device (M, ld_y) fp32, ld_y >= N; must not overlap x
 */
dlrm_status_t dlrm_linear_bias_act(int64_t M, int64_t N, int64_t K, const float* x, int64_t ld_x,
                                   const float* W, const float* bias, int32_t act, float* y,
                                   int64_t ld_y, void* stream);

/*
 * dlrm_forward_workspace_bytes -- device workspace dlrm_forward needs for
 * `batch` samples of model m (0 if m is invalid).  Host only.
 */
size_t dlrm_forward_workspace_bytes(const dlrm_model_t* m, int64_t batch);

/*
 * dlrm_forward -- the whole DLRMv1 forward (dlrm_megakernel.rs cuda_source
 * steps 1-7): bottom MLP with ReLU after every layer, the embedding bags of
 * every table, the strict-lower-triangle interaction over [x, E_0..E_{T-1}],
 * R = [x | Z], top MLP with ReLU after every hidden layer and a sigmoid after
 * the last (one-output) layer.  The argument set follows the megakernel's
 * input list (dense, indices per table, tables, bottom (W, b) pairs, top
 * (W, b) pairs; emit_megakernel in dlrm_pattern.rs), with bag offsets added.
 *
 *   m          host model descriptor (validated: dlrm_megakernel.rs validate)
 *   batch      B >= 1
 *   dense      device (B, ln_bot[0]) fp32
 *   indices    host[T] of device pointers (n_indices[t]) integers
 *   n_indices  host[T]
 *   offsets    host[T] of device pointers (B) integers, as dlrm_embbag_sum
 *   index_bytes  4 or 8, the width of indices and offsets
 *   out        device (B) fp32 probabilities
 *   workspace  device, >= dlrm_forward_workspace_bytes(m, B), 256-byte aligned
 * Enqueues either one kernel (the single-launch path of dlrm_forward_fused,
 * taken when m->packed_w is set, the model fits that path, its Linear weights
 * take at most 3 MiB and the batch is where it measured faster: at most 8192
 * with fewer than 24 tables, at most 4096 with 24 to 32 tables and a row
 * length that is a multiple of 16, 1024..2048 otherwise) or a few kernels
 * (dlrm_forward_layered) on `stream`; the
 * workspace must not be used by another call until they finish.  Both paths
 * compute the same function;
 * results agree to rounding.
 */
dlrm_status_t dlrm_forward(const dlrm_model_t* m, int64_t batch, const float* dense,
                           const void* const* indices, const int64_t* n_indices,
                           const void* const* offsets, int32_t index_bytes, float* out,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * dlrm_forward_noalloc -- dlrm_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and path choice as dlrm_forward
 * without the workspace: the workspace is a file-scope device array of the
 * library, dlrm_forward_noalloc_max_bytes() bytes (64 MiB) on each GPU it runs
 * on, held until the process ends.  Returns DLRM_E_UNSUPPORTED, enqueuing
 * nothing, when dlrm_forward_workspace_bytes(m, batch) exceeds that size;
 * DLRM_E_HIP if the array's address on the current device cannot be found.
 * The call itself allocates and frees nothing.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it; calls in order on one stream are safe.
 */
size_t dlrm_forward_noalloc_max_bytes(void);
dlrm_status_t dlrm_forward_noalloc(const dlrm_model_t* m, int64_t batch, const float* dense,
                                   const void* const* indices, const int64_t* n_indices,
                                   const void* const* offsets, int32_t index_bytes, float* out,
                                   void* stream);

/*
 * dlrm_forward_path -- which path dlrm_forward takes for model m and `batch`
 * samples: DLRM_PATH_FUSED (one launch), DLRM_PATH_LAYERED, or 0 when m or
 * batch is invalid.  Host only.
 */
#define DLRM_PATH_LAYERED 1
#define DLRM_PATH_FUSED 2
int32_t dlrm_forward_path(const dlrm_model_t* m, int64_t batch);

/*
 * dlrm_forward_layered -- dlrm_forward as a sequence of kernels: one MFMA
 * GEMM per Linear layer (bias and activation in its epilogue), one fused bag
 * + interaction kernel writing R = [x | Z] into the workspace, and a dot
 * product kernel with the sigmoid for the last layer.  Same arguments and
 * errors as dlrm_forward.
 */
dlrm_status_t dlrm_forward_layered(const dlrm_model_t* m, int64_t batch, const float* dense,
                                   const void* const* indices, const int64_t* n_indices,
                                   const void* const* offsets, int32_t index_bytes, float* out,
                                   void* workspace, size_t ws_bytes, void* stream);

/*
 * dlrm_pack_weights_bytes -- bytes of the packed weights of model m for the
 * single-launch forward, or 0 when m is invalid or outside that path's limits
 * (see dlrm_forward_fused).  Host only.
 *
 * dlrm_pack_weights -- write them.  Every Linear layer but the one-output
 * last layer is stored in chunks of 64 lanes x 4 floats in the operand order
 * of the kernel's matrix-core instruction, zero past the layer's edges, so
 * that one wave reads 1 KiB of contiguous memory per load: layers of at most
 * 128 outputs as tiles of 16 output features x 16 inputs, wider layers as
 * tiles of 32 output features x 8 inputs.  A tail holds the last layer's weights and bias
 * and every hidden layer's bias, which the kernel copies to LDS at once.  packed: device, >= dlrm_pack_weights_bytes(m)
 * bytes, 256-byte aligned; written asynchronously on `stream`.  The caller
 * stores the pointer in m->packed_w and packs again after changing weights.
 */
size_t dlrm_pack_weights_bytes(const dlrm_model_t* m);
dlrm_status_t dlrm_pack_weights(const dlrm_model_t* m, float* packed, size_t bytes, void* stream);

/*
 * dlrm_forward_fused -- dlrm_forward in a single kernel launch, the pages'
 * "one kernel per forward" design (dlrm_megakernel.rs module doc and
 * cuda_source steps 1-7 on "luminal compare dlrm-fused-kernels...
 * dlrm-pt2-megakernel").  Each block carries 8 samples (16 beyond batch 2048
 * when they fit) through the whole network with its activations in LDS and
 * the packed weights (m->packed_w,
 * DLRM_E_NULL when absent) read from L2; no workspace is used.  Arguments as
 * dlrm_forward without the workspace.
 * Returns DLRM_E_UNSUPPORTED, and enqueues nothing, unless emb_dim % 4 == 0,
 * 16 <= emb_dim <= 256, every table is 16-byte aligned, each MLP has at most 8
 * Linear layers and the block's LDS (2 x 8 x (widest layer rounded up to 64,
 * plus 8) + 8 x (T + 1) x (emb_dim + 4) floats, plus the last layer's weights
 * and every hidden layer's biases, each rounded up to 4 floats) fits in
 * 160 KiB.
 */
dlrm_status_t dlrm_forward_fused(const dlrm_model_t* m, int64_t batch, const float* dense,
                                 const void* const* indices, const int64_t* n_indices,
                                 const void* const* offsets, int32_t index_bytes, float* out,
                                 void* stream);

/*
 * dlrm_embbag_check_indices -- validate the bag data of dlrm_embbag_sum on the
 * device: counts indices outside [0, rows[t]) and offsets that decrease, are
 * negative or pass n_indices[t].  The count is written to *bad_count_device
 * (a device int32).  Asynchronous like every call; read the count after the
 * stream has finished.  Returns DLRM_OK when the check was enqueued.
 */
dlrm_status_t dlrm_embbag_check_indices(int32_t num_tables, int64_t batch, const int64_t* rows,
                                        const void* const* indices, const int64_t* n_indices,
                                        const void* const* offsets, int32_t index_bytes,
                                        int32_t* bad_count_device, void* stream);

/*
 * dlrm_pair_index_map -- write the interaction kernels' own flat-pair-index
 * decoding, p -> (i, j) for p in [0, F(F-1)/2), to device arrays i_out[P],
 * j_out[P] (int32).  It evaluates the closed form i = floor((1 + sqrt(1 + 8p))
 * / 2), j = p - i(i-1)/2 ("luminal compare asglover/modal_ci_ready...
 * vanilla-pytorch", cuda_lite kernels) exactly as the kernels do, so that
 * tests can compare it with the nested-loop enumeration.  2 <= F <= 4096.
 */
dlrm_status_t dlrm_pair_index_map(int32_t n_feat, int32_t* i_out, int32_t* j_out, void* stream);

/*
 * Measurement helpers (not part of the forward).  They set the bandwidth
 * ceilings the bag and interaction kernels are reported against, from kernels
 * of this library rather than a vendor copy.  Both only read memory; sink is
 * device memory of dlrm_probe_sink_floats() floats that is written only if the
 * data read sums to an impossible value.  Asynchronous on `stream`.
 *
 * dlrm_probe_read_stream -- reads n_floats (a multiple of 4, src 16-byte
 *   aligned) of device memory once, sequentially, 16 bytes per lane.
 * dlrm_probe_l2_stream -- `blocks` blocks of 512 threads each read all
 *   n_floats (a multiple of 4, src 16-byte aligned): with src small enough to
 *   stay in L2 and one block per CU, the rate at which one CU pulls L2-resident
 *   data (the single-launch forward streams its packed weights this way).
 * dlrm_probe_gather_rows -- reads the n rows idx[0..n) (int64, each in
 *   [0, rows)) of the (rows, dim) fp32 table, dim in {16, 32, 64, 128, 256},
 *   table 16-byte aligned: the access pattern of one-index bags.
 */
int64_t dlrm_probe_sink_floats(void);
dlrm_status_t dlrm_probe_read_stream(const float* src, int64_t n_floats, float* sink, void* stream);
dlrm_status_t dlrm_probe_l2_stream(const float* src, int64_t n_floats, int32_t blocks, float* sink,
                                   void* stream);
dlrm_status_t dlrm_probe_gather_rows(const float* table, int64_t rows, int32_t dim, const int64_t* idx,
                                     int64_t n, float* sink, void* stream);

/* Human-readable name of a status code (static storage).  The code is taken
 * as a plain integer so that any value a caller holds, including ones this
 * library never returns, is valid input ("unknown dlrm_status_t" for those). */
const char* dlrm_status_string(int32_t status);

/* ABI version of this header, bumped on any incompatible change. */
int32_t dlrm_abi_version(void);
#define DLRM_ABI_VERSION 3

#ifdef __cplusplus
}
#endif

#endif /* DLRM_MI355X_H */
