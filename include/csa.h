/*
 * csa.h -- C ABI of libcsa, the MI355X (gfx950) HIP library for the
 * compressed sparse attention (CSA) hot path:
 *
 *   compress -> index scores + streaming top-k -> sparse attention forward
 *   (window + selected compressed rows + sink, LSE out) -> sparse attention
 *   backward (fp32 scatter) -> compressor backward.
 *
 * Sources, cited by page title and review thread / commit message:
 *  - Megatron-LM PR #6400 "Add unfused SBHD compressed sparse attention":
 *    the compressor's fp32 softmax pooling, the gather/scatter into the compact
 *    KV, the per-head sink and head-count checks, the compressed causal mask
 *    (block j invalid for query t iff j >= (t+1)//ratio), the validity
 *    re-check with -1 padding, and the ratio dispatch of the sparse core.
 *  - torchtitan PR #4452 "Refactor Deepseek v4 to use Attention Gym's
 *    Compressed Sparse Attention": one fused softmax over the window, the
 *    selected compressed rows and the sink, returning the per-head LSE; an
 *    explicit softmax scale; the backward as the sum of a probability x
 *    grad-output product and a scaled grad-score x query product.
 *  - Megatron-LM PR #7152 "Add the min-memory DSA attention kernels": scores
 *    reduced tile by tile (memory O(tile), never O(sq * n_kv)); one full
 *    top-k as the tie rule; selected indices and scores ordered by position;
 *    selected gradients scattered back to positions in fp32; an all-or-nothing
 *    gradient gate.
 *
 * CONVENTIONS (all entry points)
 *  - Device pointers.  Every tensor argument is a device pointer to memory the
 *    caller allocated and owns.  The library allocates nothing in these calls,
 *    keeps no device state between calls, and never synchronises the stream;
 *    work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *    stream).  Calls on different streams may run concurrently.
 *  - Layout.  Contiguous, row-major, batch first:
 *      q-like  [b, sq, h, d]         (q, out, dout, dq)
 *      kv-like [b, sq, d]            (kv, x, dkv, dx)
 *      z       [b, sq, z_channels]   (dz)
 *      c       [b, n_c, d]           (c, c32, dc),   n_c = sq / ratio (floor)
 *      q_i     [b, sq, idx_heads, idx_dim];  k_i [b, n_c, idx_dim]
 *      w       [b, sq, idx_heads];   lse [b, sq, h];  sink, dsink [h]
 *      idx, score [b, sq, K'],  K' = min(topk, n_c)
 *    The *_strided calls take the layouts of the tensors they read from the
 *    caller as element strides instead: q-like, kv-like and lse for the
 *    attention (csa_attn_strides), x / dx and z / dz for the compressor
 *    (csa_compress_strides), q_i, k_i and w for the indexer
 *    (csa_index_strides).  Outputs the library hands to its own calls (c,
 *    c32, dc, idx, score) and every other tensor keep the layout above.
 *    Base pointers must be 16-byte aligned (the CSA calls return CSA_ERR_ARG,
 *    naming the argument, for any non-NULL tensor that is not; the DSA-over-GQA
 *    calls accept any element-aligned tensor).
 *  - Dtypes.  `dtype` is CSA_F32 or CSA_BF16 and applies to q, kv, c, x, z,
 *    q_i, k_i, out, dout, dq.  Always fp32: w, sink, lse, score, c32, dkv,
 *    dc, dsink, dx, dz.  All arithmetic is fp32 (scores, softmax, accumulation).
 *  - Token positions.  Query t sees the raw rows u in [max(0, t-window+1), t]
 *    (its window, inclusive of itself) and compressed block j iff
 *    j < n_valid(t) = (t+1) / ratio.  Block j covers tokens [j*ratio,
 *    (j+1)*ratio); its pooling span is [(j+1)*ratio - span, (j+1)*ratio)
 *    clipped at 0.
 *  - Packed documents (torchtitan PR #4452, its description of packed
 *    documents).  doc_ids [b, sq] int32 (nullable: one document per batch
 *    row) gives each token's document.  Window row u is a candidate of t only
 *    if doc_ids[u] == doc_ids[t]; block j (tokens [j*ratio, (j+1)*ratio))
 *    belongs to the document of token j*ratio and is selectable by the
 *    indexer, and attended in dense mode, only if that is t's document.
 *    Entries of a given index row are attended as they are.
 *  - Errors.  Every entry point validates its arguments before enqueuing any
 *    work and returns CSA_OK or a negative code; csa_last_error() then returns
 *    a message for the calling thread.  Nothing throws or aborts across the ABI.
 *    Values of floating-point inputs are not checked (NaN/Inf give unspecified
 *    results).
 *  - Gradient outputs that sum contributions (dkv, dc, dsink, dx, dz) are
 *    overwritten, not added to: every element is written by the call.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 9

enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1 };

enum csa_status {
    CSA_OK = 0,
    CSA_ERR_ARG = -1,          /* null pointer, non-positive or inconsistent size */
    CSA_ERR_SHAPE = -2,        /* shapes disagree (e.g. sink length != h)         */
    CSA_ERR_DTYPE = -3,        /* unknown dtype                                   */
    CSA_ERR_UNSUPPORTED = -4,  /* valid but outside what the kernels implement    */
    CSA_ERR_WORKSPACE = -5,    /* workspace missing or too small                  */
    CSA_ERR_HIP = -6           /* the HIP runtime reported an error on launch     */
};

/* Problem sizes shared by all calls.
 *  b, sq      batch and sequence length (>= 1)
 *  h, d       query heads on one shared KV head, head dim (key dim == value dim)
 *  ratio      compress ratio r >= 1; span L >= 1 is the pooling span (L == r:
 *             non-overlapping; L == 2r: overlapping)
 *  window     sliding window W >= 1
 *  idx_heads, idx_dim, topk   indexer heads, indexer dim and top-k (topk >= 1
 *             when the indexer is used)
 * Supported by the kernels: d in {64, 128, 512}; 1 <= h <= 64; idx_dim in
 * {32, 64, 128}; 1 <= idx_heads <= 64; K' <= 2048.  Others: CSA_ERR_UNSUPPORTED. */
typedef struct csa_dims {
    int32_t b, sq, h, d, ratio, span, window, idx_heads, idx_dim, topk;
} csa_dims;

/* Compressor forward (Megatron-LM PR #6400, review thread on the pooling
 * weights).  For block j < n_c and channel c:
 *   alpha_u = softmax over u in span(j) of z[u, c]   (z[u, 0] if z_channels == 1)
 *   c32[j, c] = sum_u alpha_u * x[u, c]               (fp32 weights and sum)
 *   y[j, c]   = c32[j, c] rounded once to dtype.
 * Epilogue (same PR: the compressor's norm after the cast; the compressed
 * rows' rotary embedding with its own base, 40000 in the layer
 * configuration), applied when norm_w != NULL or rope_dim > 0:
 *   n[j, c] = y[j, c] / sqrt(mean_c y[j, c]^2 + norm_eps) * norm_w[c]
 *             (n = y when norm_w is NULL; norm_w is fp32 [d])
 *   the last rope_dim channels of n turned in interleaved pairs (2i, 2i+1)
 *   by the angle j * rope_base^(-2i / rope_dim) (block j at position j)
 *   c[j, :] = the result rounded to dtype      (c = y without the epilogue)
 * z_channels is 1 or d; rope_dim is even, 0 <= rope_dim <= d.  c32 (the
 * pooled rows before the cast and the epilogue) may be NULL. */
int csa_compress(const csa_dims* dims, int dtype, const void* x, const void* z, int z_channels,
                 const float* norm_w, float norm_eps, int rope_dim, float rope_base,
                 void* c, float* c32, void* stream);

/* Workspace bytes csa_compress_bwd needs when the epilogue is on (device
 * memory, 16-byte aligned, caller-owned, contents on entry irrelevant): the
 * gradient of the pooled rows and per-workgroup parts of dnorm_w.  Without
 * the epilogue no workspace is used.  0 for invalid dims. */
size_t csa_compress_bwd_workspace(const csa_dims* dims);

/* Compressor backward: the gradient of csa_compress given dc (fp32,
 * [b, n_c, d]), with the same epilogue arguments; the rounding casts are
 * treated as the identity.  Through the epilogue (rotation transposed, then
 * the norm's backward on y):
 *   dy[j, :]  = gradient of sum(dc * c) with respect to y[j, :]
 *   dnorm_w[c] = sum_j dn[j, c] y[j, c] / sqrt(mean y^2 + eps)   (fp32 [d], may be NULL;
 *               must be NULL when norm_w is NULL)
 * then through the pooling, with g = dy (g = dc without the epilogue):
 *   dx[u, c] = sum_j alpha_{j,u,c} g[j, c]
 *   dz[u, c] = sum_j alpha_{j,u,c} g[j, c] (x[u, c] - c32[j, c])  (summed over c if z_channels == 1)
 * Rows u >= n_c * ratio receive zero.  ws / ws_bytes: needed only with the
 * epilogue (CSA_ERR_WORKSPACE if then NULL or smaller than
 * csa_compress_bwd_workspace(dims)). */
int csa_compress_bwd(const csa_dims* dims, int dtype, const void* x, const void* z,
                     int z_channels, const float* norm_w, float norm_eps, int rope_dim,
                     float rope_base, const float* dc, float* dx, float* dz, float* dnorm_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Element strides (in elements, not bytes) of the compressor's token rows
 * for the *_strided compressor calls, so that a sequence-major caller ([sq,
 * b, d] views) needs no transposed copy.  The channel axis stays contiguous.
 *   x_b, x_s   x and dx (dx uses the same element strides in fp32)
 *   z_b, z_s   z and dz (likewise)
 * Axes of extent > 1 must not overlap (sorted by stride, each stride at least
 * the previous one times its extent, the contiguous axis first); x strides,
 * and z strides when z_channels = d, are multiples of 16 bytes of the dtype
 * (8 bf16 or 4 fp32 elements).  Otherwise CSA_ERR_ARG naming the stride.
 * Axes of extent 1 are ignored. */
typedef struct csa_compress_strides {
    int64_t x_b, x_s;
    int64_t z_b, z_s;
} csa_compress_strides;

/* csa_compress over strided x and z (strides == NULL: the contiguous layout,
 * identical to csa_compress); c and c32 are written contiguously. */
int csa_compress_strided(const csa_dims* dims, const csa_compress_strides* strides, int dtype, const void* x,
                         const void* z, int z_channels, const float* norm_w, float norm_eps, int rope_dim,
                         float rope_base, void* c, float* c32, void* stream);

/* csa_compress_bwd over strided x, z, dx and dz (strides == NULL: identical
 * to csa_compress_bwd); dc is read contiguously.  Results are bit-identical
 * to the contiguous call on the same values. */
int csa_compress_bwd_strided(const csa_dims* dims, const csa_compress_strides* strides, int dtype,
                             const void* x, const void* z, int z_channels, const float* norm_w,
                             float norm_eps, int rope_dim, float rope_base, const float* dc, float* dx,
                             float* dz, float* dnorm_w, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes csa_index_topk needs (0: scores never leave the chip). */
size_t csa_index_topk_workspace(const csa_dims* dims);

/* Learned indexer + streaming top-k (Megatron-LM PR #6400, causal-mask thread;
 * Megatron-LM PR #7152, routing commit messages).
 *   I[t, j] = sum_h w[t, h] * relu(q_i[t, h] . k_i[j])   for j < n_valid(t)
 *   (and, with doc_ids, j in t's document: see CONVENTIONS)
 * Scores are computed tile by tile on the chip and reduced into a running
 * top-k; the [sq, n_c] score matrix is never written anywhere.  Row (b, t) of
 * idx receives the K' = min(topk, n_c) largest valid scores ordered by
 * (score desc, index asc), emitted in ascending index, then -1 for the
 * K' - min(K', n_valid(t)) remaining slots.  score (nullable) receives the
 * fp32 scores aligned with idx (-inf on -1 slots).  w is fp32 and already
 * holds any softmax scale of the indexer; w == NULL means unit weights (the
 * simplified one-head indexer).  ws may be NULL when
 * csa_index_topk_workspace() returns 0.  When sq < ratio no block exists
 * (K' = 0): the call does nothing, and k_i, idx and score may be NULL. */
int csa_index_topk(const csa_dims* dims, int dtype, const void* q_i, const void* k_i,
                   const float* w, const int32_t* doc_ids, int32_t* idx, float* score, void* ws,
                   size_t ws_bytes, void* stream);

/* Element strides of the indexer's inputs for csa_index_topk_strided (the
 * last axis of each stays contiguous):
 *   qi_b, qi_s, qi_h   q_i [b, sq, idx_heads, idx_dim]
 *   ki_b, ki_s         k_i [b, n_c, idx_dim]
 *   w_b, w_s           w   [b, sq, idx_heads] (fp32)
 * Axes of extent > 1 must not overlap; q_i and k_i strides of such axes are
 * multiples of 16 bytes of the dtype.  Otherwise CSA_ERR_ARG naming the
 * stride.  doc_ids, idx and score keep the contiguous layout. */
typedef struct csa_index_strides {
    int64_t qi_b, qi_s, qi_h;
    int64_t ki_b, ki_s;
    int64_t w_b, w_s;
} csa_index_strides;

/* csa_index_topk over strided q_i, k_i and w (strides == NULL: identical to
 * csa_index_topk).  Results are identical to the contiguous call on the same
 * values. */
int csa_index_topk_strided(const csa_dims* dims, const csa_index_strides* strides, int dtype,
                           const void* q_i, const void* k_i, const float* w, const int32_t* doc_ids,
                           int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream);

/* Sparse attention forward (Megatron-LM PR #6400 gather and sink threads;
 * torchtitan PR #4452 fused operator).  For query (b, t) and head h the
 * candidate rows are its window rows kv[b, u] and one row c[b, j] per slot
 * of idx[b, t, :] with 0 <= j < n_valid(t) (other slots, e.g. -1, are
 * skipped).  idx == NULL attends every valid compressed row (dense mode, the
 * HCA layer); c == NULL attends the window only (then idx must be NULL).
 *   l   = scale * <q[t, h], row>
 *   lse = log(exp(sink[h]) + sum exp(l))   (no sink term if sink == NULL)
 *   out[t, h] = sum exp(l - lse) * row     (the row is both key and value)
 * out has dtype, lse is fp32. */
int csa_sparse_attn_fwd(const csa_dims* dims, int dtype, const void* q, const void* kv,
                        const void* c, const int32_t* idx, const int32_t* doc_ids,
                        const float* sink, float scale,
                        void* out, float* lse, void* stream);

/* Workspace bytes csa_sparse_attn_bwd needs (device memory, 16-byte aligned,
 * owned by the caller, contents on entry irrelevant): Delta and the per-query
 * dsink terms ([b, sq, h] fp32 each) and fp32 partial rows of dkv and dc per
 * block of consecutive queries, which the call reduces in a fixed order (the
 * results do not depend on scheduling).  0 for invalid dims. */
size_t csa_sparse_attn_bwd_workspace(const csa_dims* dims);

/* Diagnostic: the number of consecutive queries per block of the backward's
 * fixed-order reduction of dkv / dc (the backward sums each block's partial
 * rows, then the blocks in order) for these dims, with (with_compressed != 0)
 * or without compressed rows.  Tests use it to give every block a query with
 * a nonzero gradient.  0 for invalid dims. */
int csa_sparse_attn_bwd_query_block(const csa_dims* dims, int with_compressed);

/* Sparse attention backward: the gradient of csa_sparse_attn_fwd given dout,
 * with out and lse from that forward (same inputs).  With
 * Delta = <dout, out> and dl = P (<dout, row> - Delta):
 *   dq[t, h] = scale * sum dl * row                          (dtype)
 *   each candidate row gets P dout[t, h] + scale * dl q[t, h], scattered in
 *   fp32 into dkv[b, u] (window rows) or dc[b, j] (compressed rows);
 *   repeated indices across queries accumulate without loss of fp32 precision
 *   dsink[h] = -sum_{b,t} exp(sink[h] - lse) Delta          (fp32)
 * Gradient gate (Megatron-LM PR #7152): dq, dkv and dc are all non-NULL, or
 * all NULL (no-op apart from dsink); dc must be NULL when c is NULL.  dsink
 * may be NULL (required NULL when sink is NULL).  lse gradient is zero.
 * ws / ws_bytes: the workspace (CSA_ERR_WORKSPACE if NULL or smaller than
 * csa_sparse_attn_bwd_workspace(dims)). */
int csa_sparse_attn_bwd(const csa_dims* dims, int dtype, const void* q, const void* kv,
                        const void* c, const int32_t* idx, const int32_t* doc_ids,
                        const float* sink, float scale,
                        const void* out, const float* lse, const void* dout, void* dq,
                        float* dkv, float* dc, float* dsink, void* ws, size_t ws_bytes,
                        void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * backward as csa_sparse_attn_bwd, same arguments minus the workspace, which
 * here is a fixed array of CSA_BWD_SCRATCH_BYTES in the library's device
 * memory (one copy per GPU the library runs on, held until the process
 * ends; its address is looked up on the first call on each device).  The
 * call allocates nothing.  Returns CSA_ERR_UNSUPPORTED when the dims need more
 * scratch than that (csa_sparse_attn_bwd_workspace(dims) bytes; the bench
 * workload b 1, sq 4096, h 64, d 128, n_c 1024 needs 44.5 MiB).  Nothing in
 * the scratch needs to start at zero: every element is written before it is
 * read.  Calls that overlap on one GPU (different streams, or threads) share
 * the one array and race: serialise them. */
#define CSA_BWD_SCRATCH_BYTES ((size_t)64 << 20)
int csa_sparse_attn_bwd_noalloc(const csa_dims* dims, int dtype, const void* q, const void* kv,
                                const void* c, const int32_t* idx, const int32_t* doc_ids,
                                const float* sink, float scale, const void* out, const float* lse,
                                const void* dout, void* dq, float* dkv, float* dc, float* dsink,
                                void* stream);

/* Element strides (in elements, not bytes) of the attention tensors for the
 * *_strided calls, so that a caller holding sequence-major tensors (the
 * SBHD layout of Megatron-LM PR #6400: [sq, b, h, d]) passes views instead
 * of transposed copies.  The last axis (d for q-like and kv-like, h for lse)
 * stays contiguous.
 *   q_b, q_s, q_h   q, out, dout and dq (one layout for all four)
 *   kv_b, kv_s      kv and dkv (dkv uses the same element strides in fp32)
 *   lse_b, lse_s    lse
 * Axes of extent > 1 must not overlap (sorted by stride, each stride at least
 * the previous one times its extent, the contiguous axis first); q-like and
 * kv-like strides of such axes are multiples of 16 bytes (8 bf16 or 4 fp32
 * elements).  Otherwise CSA_ERR_ARG naming the stride.  Axes of extent 1 are
 * ignored.  c, dc, idx, doc_ids, sink and dsink keep the contiguous layout. */
typedef struct csa_attn_strides {
    int64_t q_b, q_s, q_h;
    int64_t kv_b, kv_s;
    int64_t lse_b, lse_s;
} csa_attn_strides;

/* csa_sparse_attn_fwd over strided q, kv, out and lse (strides == NULL: the
 * contiguous layout, identical to csa_sparse_attn_fwd). */
int csa_sparse_attn_fwd_strided(const csa_dims* dims, const csa_attn_strides* strides, int dtype,
                                const void* q, const void* kv, const void* c, const int32_t* idx,
                                const int32_t* doc_ids, const float* sink, float scale, void* out,
                                float* lse, void* stream);

/* csa_sparse_attn_bwd over strided q, kv, out, lse, dout, dq and dkv
 * (strides == NULL: identical to csa_sparse_attn_bwd).  The workspace is
 * the same size (csa_sparse_attn_bwd_workspace(dims)) and the results are
 * bit-identical to the contiguous call on the same values. */
int csa_sparse_attn_bwd_strided(const csa_dims* dims, const csa_attn_strides* strides, int dtype,
                                const void* q, const void* kv, const void* c, const int32_t* idx,
                                const int32_t* doc_ids, const float* sink, float scale,
                                const void* out, const float* lse, const void* dout, void* dq,
                                float* dkv, float* dc, float* dsink, void* ws, size_t ws_bytes,
                                void* stream);

/* Workspace bytes csa_indexer_loss needs when gradients are requested
 * (device memory, 16-byte aligned, owned by the caller, contents on entry
 * irrelevant): dI ([b, sq, K'] fp32) and fp32 partial rows of dk_i per block
 * of consecutive queries, reduced in a fixed order.  0 for invalid dims. */
size_t csa_indexer_loss_workspace(const csa_dims* dims);

/* Indexer distillation loss and its gradients (the indexer's training path;
 * torchtitan PR #4452, lightning indexer and indexer distillation loss;
 * Megatron-LM PR #6400, teacher normalisation thread; Megatron-LM PR #7152,
 * reuse of the routing scores and fp32 scatter of selected gradients).
 * For row (b, t) the support is the slots s of idx[b, t, :] (the output of
 * csa_index_topk) with 0 <= j_s < n_valid(t); with lse the per-head LSE of
 * csa_sparse_attn_fwd for the same row:
 *   mass[s]    = sum_h exp(scale * <q[t, h], c[j_s]> - lse[t, h])
 *   target     = mass / sum(mass)            (all zero on an empty support)
 *   predict    = softmax over the support of score[b, t, s] (the fp32 scores
 *                csa_index_topk wrote beside idx: the student's logits)
 *   kl[b, t]   = sum_s target (log target - log predict)          (fp32)
 * The teacher is detached.  With dkl ([b, sq] fp32, the upstream gradient of
 * each row's kl) and a = <q_i[t, h], k_i[j_s]>:
 *   dI[s]      = dkl[t] * (predict[s] * sum(target) - target[s])
 *   dw[t, h]   = sum_s dI[s] * relu(a)                            (fp32)
 *   dq_i[t, h] = sum_s dI[s] * w[t, h] * [a > 0] * k_i[j_s]        (dtype)
 *   dk_i[j]    = sum over (t, s) with j_s = j of dI * w * [a > 0] * q_i[t, h]
 *                summed over h, accumulated in fp32                (fp32)
 * Layouts as in CONVENTIONS; lse [b, sq, h], score [b, sq, K'] fp32.
 * kl may be NULL.  Gradient gate: dkl, dq_i, dw and dk_i are all non-NULL
 * (then q_i, k_i, w and the workspace are required) or all NULL (the call
 * only writes kl).  Every element of the outputs is overwritten.  ws /
 * ws_bytes: CSA_ERR_WORKSPACE if gradients are requested and ws is NULL or
 * smaller than csa_indexer_loss_workspace(dims). */
int csa_indexer_loss(const csa_dims* dims, int dtype, const void* q, const void* c,
                     const float* lse, const void* q_i, const void* k_i, const float* w,
                     const int32_t* idx, const float* score, float scale,
                     const float* dkl, float* kl, void* dq_i, float* dw, float* dk_i,
                     void* ws, size_t ws_bytes, void* stream);

/* Dense warm-up form of the indexer distillation loss (Megatron-LM PR #7152,
 * the commit adding the dense warm-up tile plan: the dense teacher scores
 * every attention head against all keys, under a planned memory budget).
 * Same as csa_indexer_loss with the support of row (b, t) every valid block
 * j < n_valid(t) instead of the selected slots, and the student's logits
 * I[t, j] = sum_h w[t, h] * relu(<q_i[t, h], k_i[j]>) formed inside the call
 * (no idx or score input; topk is ignored):
 *   mass[j]  = sum_h exp(scale * <q[t, h], c[j]> - lse[t, h])
 *   target   = mass / sum(mass),  predict = softmax_j I[t, j]
 *   kl[b, t] = sum_j target (log target - log predict)
 *   dI[j]    = dkl[t] * (predict[j] - target[j])   (rows with blocks)
 *   dw, dq_i, dk_i as in csa_indexer_loss over every valid block.
 * lse is the per-head LSE of the warm-up's attention (e.g. csa_sparse_attn_fwd
 * with idx == NULL, every valid block attended).  No packed documents.
 * The queries run in chunks; the workspace holds, per chunk, two fp32 rows of
 * n_c entries per query and the chunk's fp32 partial rows of dk_i.  The call
 * plans the largest chunk that fits ws_bytes (so memory follows the budget,
 * not sq * n_c) and needs at least csa_indexer_loss_dense_workspace(dims, 0)
 * bytes (CSA_ERR_WORKSPACE otherwise), also when only kl is requested.
 * csa_indexer_loss_dense_workspace(dims, budget) returns the bytes the plan
 * for that budget uses (at most budget unless budget is below that minimum;
 * 0 for invalid dims).  dk_i accumulates over the chunks in a fixed order.
 * Gradient gate, kl, layouts and the 16-byte alignment as in
 * csa_indexer_loss. */
size_t csa_indexer_loss_dense_workspace(const csa_dims* dims, size_t budget);
int csa_indexer_loss_dense(const csa_dims* dims, int dtype, const void* q, const void* c,
                           const float* lse, const void* q_i, const void* k_i, const float* w,
                           float scale, const float* dkl, float* kl, void* dq_i, float* dw,
                           float* dk_i, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------ simplified DSA over GQA
 * Megatron-LM PR #7152 (description and commit messages): a one-head indexer
 * without per-head weights selects K' = min(topk, sq) keys per query at full
 * resolution -- csa_index_topk with ratio 1, idx_heads 1 and w == NULL (unit
 * weights), so n_valid(t) = t + 1 -- and attention runs over the selected
 * keys only, with separate keys and values per key/value head:
 *   query head h reads key/value head g = h / (h / h_kv)
 *   l   = scale * <q[t, h], k[j, g]>  over the slots j of idx[b, t, :] with
 *         0 <= j <= t (other slots skipped; a repeated j counts once per slot)
 *   lse = log sum exp(l), out[t, h] = sum exp(l - lse) v[j, g]
 *   (no valid slot: out = 0, lse = -inf, no gradient)
 * No window rows and no sink.  Layouts (row-major, last dim contiguous):
 * q / out / dout / dq [b, sq, h, d_qk or d_v], k / dk [b, sq, h_kv, d_qk],
 * v / dv [b, sq, h_kv, d_v], lse [b, sq, h] fp32, idx [b, sq, K'] int32;
 * dk and dv are fp32 and accumulate every selecting query (fixed order).
 * h / h_kv <= 64; d_qk + d_v in {64, 128, 256, 512} for bf16, {64, 128} for
 * fp32; K' <= 2048. */
typedef struct csa_gqa_dims {
    int32_t b, sq, h, h_kv, d_qk, d_v, topk;
} csa_gqa_dims;

/* Workspace bytes of csa_dsa_gqa_fwd (backward == 0) or csa_dsa_gqa_bwd
 * (backward != 0): device memory, 256-byte aligned, caller-owned, contents on
 * entry irrelevant.  0 for invalid dims. */
size_t csa_dsa_gqa_workspace(const csa_gqa_dims* dims, int dtype, int backward);

/* Forward of the attention above. */
int csa_dsa_gqa_fwd(const csa_gqa_dims* dims, int dtype, const void* q, const void* k,
                    const void* v, const int32_t* idx, float scale, void* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/* Backward, given dout and the forward's out and lse (same inputs):
 *   dP = <dout, v>, Delta = <dout, out>, dl = P (dP - Delta)
 *   dq[t, h] = scale sum dl k[j, g]                         (dtype)
 *   dk[j, g] += scale dl q[t, h],  dv[j, g] += P dout[t, h]  (fp32)
 * dq, dk and dv are all required. */
int csa_dsa_gqa_bwd(const csa_gqa_dims* dims, int dtype, const void* q, const void* k,
                    const void* v, const int32_t* idx, float scale, const void* out,
                    const float* lse, const void* dout, void* dq, float* dk, float* dv,
                    void* ws, size_t ws_bytes, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* csa_last_error(void);

/* CSA_ABI_VERSION of the loaded library. */
int csa_version(void);

/* ---------------------------------------------------------------- timing
 * Benchmark hook, not part of the computation.  Kernel ids of the entry
 * points above (one entry point may launch several kernels):
 *   csa_compress          -> CSA_K_COMPRESS_FWD, CSA_K_COMPRESS_EPI (epilogue)
 *   csa_compress_bwd      -> CSA_K_COMPRESS_EPI (epilogue), CSA_K_COMPRESS_BWD
 *   csa_index_topk        -> CSA_K_INDEX_TOPK
 *   csa_sparse_attn_fwd   -> CSA_K_ATTN_FWD
 *   csa_sparse_attn_bwd   -> CSA_K_ATTN_DQ (dq, Delta, dsink), CSA_K_ATTN_ROWS
 *                            (per-query-block dkv / dc partials), CSA_K_ATTN_REDUCE
 *   csa_indexer_loss      -> CSA_K_LOSS_QUERY (teacher, kl, dI, dq_i, dw),
 *                            CSA_K_LOSS_KEYS (per-query-block dk_i partials),
 *                            CSA_K_LOSS_REDUCE
 * csa_timing_enable(k) makes every later launch of kernel k, from any thread,
 * record one hipEvent before and one after it on the launch stream; -1
 * switches timing off.  Returns CSA_ERR_ARG for an unknown id.
 * csa_timing_read() waits for the recorded events, returns the number of
 * timed launches and the sum of their durations in milliseconds, and forgets
 * them; CSA_ERR_HIP if an event could not be read.  The events are created by
 * the library on first use and reused; they are the only resource it keeps. */
enum csa_kernel_id {
    CSA_K_COMPRESS_FWD = 0, CSA_K_COMPRESS_BWD = 1, CSA_K_INDEX_TOPK = 2, CSA_K_ATTN_FWD = 3,
    CSA_K_ATTN_DQ = 4, CSA_K_ATTN_ROWS = 5, CSA_K_ATTN_REDUCE = 6, CSA_K_LOSS_QUERY = 7,
    CSA_K_LOSS_KEYS = 8, CSA_K_LOSS_REDUCE = 9, CSA_K_COMPRESS_EPI = 10
};
int csa_timing_enable(int kernel);
int csa_timing_read(int* launches, double* total_ms);
/* Short name of a kernel id ("" if unknown). */
const char* csa_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
