/*
 * csa_oracle.c -- plain fp64 CPU oracle for the compressed sparse attention
 * (CSA) hot path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it to check and to time the HIP library.
 * The product path never calls, links or loads it.
 *
 * Every function computes the plain definition of one step, in fp64, from the
 * exact values of the (fp32- or bf16-rounded) inputs.  No blocking, fusion or
 * reordering: loops follow the definitions one to one.  Shares no code,
 * header, table or helper with the HIP path.
 *
 * Sources (the pages this follows; cited by title and thread / message):
 *  [PR6400-pool]   Megatron-LM PR #6400 "Add unfused SBHD compressed sparse
 *                  attention", review thread on the compressor's pooling
 *                  weights (softmax in fp32, fp32 weighted sum, one cast).
 *  [PR6400-gather] same PR, review thread on the sparse-attention gather and
 *                  its backward (index_select / index_add into the compact KV).
 *  [PR6400-sink]   same PR, review thread on the per-head attention sink and
 *                  head counts (sink logit joins the softmax denominator).
 *  [PR6400-mask]   same PR, review thread on the per-forward causal mask:
 *                  block j is masked for query t iff j >= (t+1)//ratio; the
 *                  validity re-check and the -1 padding of invalid slots.
 *  [PR6400-core]   same PR, review thread on the sparse-core docstring
 *                  (ratio > 1 compresses; ratio 4 with no dense mode uses the
 *                  learned indexer; otherwise all valid compressed rows).
 *  [PR6400-window] same PR, review thread on duplicated sliding-window logits
 *                  (window indices form the first window_size score columns).
 *  [TT4452-op]     torchtitan PR #4452 "Refactor Deepseek v4 to use Attention
 *                  Gym's CSA": the fused operator (window + selected compressed
 *                  rows + sink in one softmax, per-head LSE returned) and the
 *                  comment on its backward as a sum of two products.
 *  [TT4452-docs]   same PR, its description of packed documents: with
 *                  doc_ids [b, S], the window keeps only keys of the query's
 *                  document, and indexer entry j (tokens [j*r, (j+1)*r)) belongs
 *                  to the document of token j*r and is selectable by t iff that
 *                  document is t's and j < (t+1)//r.
 *  [PR7152-route]  Megatron-LM PR #7152 "Add the min-memory DSA attention
 *                  kernels", commit messages on routing: one full top-k (not
 *                  chunked) is the tie rule; indices/scores ordered by position.
 *  [PR7152-scatter] same PR, first commit message: selected gradients are
 *                  scattered back to positions, accumulated in fp32.
 *
 * Readings where the pages leave a step open (also listed in the design notes):
 *  - window of query t: rows u in [t-W+1, t] clipped at 0 (inclusive of t);
 *  - block j covers tokens [j*r, (j+1)*r); pooling span L ends where the block
 *    ends: R(j) = [(j+1)*r - L, (j+1)*r) clipped at 0; n_c = floor(S/r);
 *  - pooling scores are per row and channel (z_channels == D) or one per row
 *    (z_channels == 1, broadcast over channels);
 *  - key == value: one gathered row feeds both the logit and the output;
 *  - the sink is an unscaled per-head logit in the denominator only;
 *  - indexer score I[t,j] = sum_h w[t,h] * relu(q_i[t,h] . k_i[j]);
 *    top-k order is (score desc, index asc); output ascending index, then -1;
 *  - every slot of an index row is one candidate (a repeated index in one row
 *    counts once per slot); slots outside [0, n_valid(t)) are ignored;
 *  - packed documents (doc != NULL): the window and the indexer follow
 *    [TT4452-docs]; entries of a given index row are taken as given (the
 *    attention leaves the selected branch to the indexer), while the dense
 *    mode (no index rows) applies the indexer's document rule to every block.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR (-1)

static int64_t n_valid_blocks(int64_t t, int64_t r) { return (t + 1) / r; }

/* Tokens t and u of batch row bi are in the same packed document [TT4452-docs]
 * (always, without document ids). */
static int same_doc(const int32_t* doc, int64_t S, int64_t bi, int64_t t, int64_t u)
{
    return !doc || doc[bi * S + t] == doc[bi * S + u];
}

/* ------------------------------------------------------------------ a1 --- */
/* Softmax pooling [PR6400-pool]: for block j and channel c,
 *   alpha_u = softmax_{u in R(j)} Z[u, c]      (c -> 0 when z_channels == 1)
 *   C[j, c] = sum_{u in R(j)} alpha_u * X[u, c]
 * X [b,S,D], Z [b,S,zc] -> C [b,n_c,D] (unrounded). */
int csa_oracle_compress(int64_t b, int64_t S, int64_t D, int64_t r, int64_t L, int64_t zc,
                        const double* X, const double* Z, double* C)
{
    if (r < 1 || L < 1 || (zc != 1 && zc != D)) return ORACLE_ERR;
    int64_t nc = S / r;
    for (int64_t bi = 0; bi < b; ++bi)
        for (int64_t j = 0; j < nc; ++j) {
            int64_t hi = (j + 1) * r;
            int64_t lo = hi - L < 0 ? 0 : hi - L;
            for (int64_t c = 0; c < D; ++c) {
                int64_t zcol = zc == 1 ? 0 : c;
                double m = -INFINITY;
                for (int64_t u = lo; u < hi; ++u) {
                    double z = Z[(bi * S + u) * zc + zcol];
                    if (z > m) m = z;
                }
                double den = 0.0;
                for (int64_t u = lo; u < hi; ++u) den += exp(Z[(bi * S + u) * zc + zcol] - m);
                double acc = 0.0;
                for (int64_t u = lo; u < hi; ++u) {
                    double alpha = exp(Z[(bi * S + u) * zc + zcol] - m) / den;
                    acc += alpha * X[(bi * S + u) * D + c];
                }
                C[(bi * nc + j) * D + c] = acc;
            }
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ a6 --- */
/* Backward of the pooling above.  With alpha = softmax(z) and C = sum alpha x:
 *   dX[u,c] += alpha_u dC[j,c]
 *   dZ[u,c] += alpha_u dC[j,c] (X[u,c] - C[j,c])   (summed over c if zc == 1)
 * The single cast to the working dtype is taken as the identity.
 * dX [b,S,D], dZ [b,S,zc] are overwritten. */
int csa_oracle_compress_bwd(int64_t b, int64_t S, int64_t D, int64_t r, int64_t L, int64_t zc,
                            const double* X, const double* Z, const double* dC,
                            double* dX, double* dZ)
{
    if (r < 1 || L < 1 || (zc != 1 && zc != D)) return ORACLE_ERR;
    int64_t nc = S / r;
    memset(dX, 0, sizeof(double) * b * S * D);
    memset(dZ, 0, sizeof(double) * b * S * zc);
    for (int64_t bi = 0; bi < b; ++bi)
        for (int64_t j = 0; j < nc; ++j) {
            int64_t hi = (j + 1) * r;
            int64_t lo = hi - L < 0 ? 0 : hi - L;
            for (int64_t c = 0; c < D; ++c) {
                int64_t zcol = zc == 1 ? 0 : c;
                double m = -INFINITY;
                for (int64_t u = lo; u < hi; ++u) {
                    double z = Z[(bi * S + u) * zc + zcol];
                    if (z > m) m = z;
                }
                double den = 0.0;
                for (int64_t u = lo; u < hi; ++u) den += exp(Z[(bi * S + u) * zc + zcol] - m);
                double cj = 0.0;
                for (int64_t u = lo; u < hi; ++u)
                    cj += exp(Z[(bi * S + u) * zc + zcol] - m) / den * X[(bi * S + u) * D + c];
                double g = dC[(bi * nc + j) * D + c];
                for (int64_t u = lo; u < hi; ++u) {
                    double alpha = exp(Z[(bi * S + u) * zc + zcol] - m) / den;
                    dX[(bi * S + u) * D + c] += alpha * g;
                    dZ[(bi * S + u) * zc + zcol] += alpha * g * (X[(bi * S + u) * D + c] - cj);
                }
            }
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ a2 --- */
/* Indexer scores for a list of query rows [PR6400-mask, PR7152-route]:
 *   I[n, j] = sum_h W[n,h] * max(0, sum_e QI[n,h,e] * KI[b_n, j, e])  for valid j
 *   I[n, j] = -inf                                                     otherwise
 * j is valid for t iff j < n_valid(t) and (with doc [b,S]) token j*r is in
 * t's document [TT4452-docs].  QI [nrows,HI,DI] and W [nrows,HI] hold the
 * listed rows; KI is [b,n_c,DI].  I is [nrows, n_c]. */
int csa_oracle_index_scores(int64_t nc, int64_t r, int64_t HI, int64_t DI,
                            const double* QI, const double* KI, const double* W,
                            int64_t nrows, const int64_t* rows_b, const int64_t* rows_t,
                            int64_t S, const int32_t* doc, double* I)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < nrows; ++n) {
        int64_t nv = n_valid_blocks(rows_t[n], r);
        const double* kb = KI + rows_b[n] * nc * DI;
        for (int64_t j = 0; j < nc; ++j) {
            if (j >= nv || !same_doc(doc, S, rows_b[n], rows_t[n], j * r)) { I[n * nc + j] = -INFINITY; continue; }
            double s = 0.0;
            for (int64_t h = 0; h < HI; ++h) {
                double dot = 0.0;
                for (int64_t e = 0; e < DI; ++e) dot += QI[(n * HI + h) * DI + e] * kb[j * DI + e];
                s += W[n * HI + h] * (dot > 0.0 ? dot : 0.0);
            }
            I[n * nc + j] = s;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ a3 --- */
/* One full top-k per row [PR7152-route]: among valid j (as for the scores)
 * sort by (I desc, j asc), keep the first min(K', number valid) and emit them
 * in ascending j, then -1 padding up to K' = min(K, n_c) [PR6400-mask].
 * Scores are aligned with the indices; padded slots carry -inf. */
typedef struct { double s; int64_t j; } oracle_cand;

static int cand_cmp(const void* a, const void* b)
{
    const oracle_cand* x = (const oracle_cand*)a;
    const oracle_cand* y = (const oracle_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int int_cmp(const void* a, const void* b)
{
    int64_t x = ((const oracle_cand*)a)->j, y = ((const oracle_cand*)b)->j;
    return (x > y) - (x < y);
}

int csa_oracle_topk(int64_t nc, int64_t r, int64_t K, int64_t nrows, const int64_t* rows_b,
                    const int64_t* rows_t, int64_t S, const int32_t* doc, const double* I,
                    int32_t* idx, double* score)
{
    int64_t kp = K < nc ? K : nc;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        oracle_cand* buf = (oracle_cand*)malloc(sizeof(oracle_cand) * (nc > 0 ? nc : 1));
        if (!buf) err = ORACLE_ERR;
#pragma omp for schedule(dynamic, 8)
        for (int64_t n = 0; n < nrows; ++n) {
            if (!buf) continue;
            int64_t nv = n_valid_blocks(rows_t[n], r);
            if (nv > nc) nv = nc;
            int64_t nval = 0;
            for (int64_t j = 0; j < nv; ++j) {
                if (!same_doc(doc, S, rows_b[n], rows_t[n], j * r)) continue;
                buf[nval].s = I[n * nc + j]; buf[nval].j = j; ++nval;
            }
            nv = nval;
            qsort(buf, (size_t)nv, sizeof(oracle_cand), cand_cmp);
            int64_t m = kp < nv ? kp : nv;
            qsort(buf, (size_t)m, sizeof(oracle_cand), int_cmp);
            for (int64_t s = 0; s < kp; ++s) {
                idx[n * kp + s] = s < m ? (int32_t)buf[s].j : -1;
                score[n * kp + s] = s < m ? buf[s].s : -INFINITY;
            }
        }
        free(buf);
    }
    return err;
}

/* ------------------------------------------------------------------ a4 --- */
/* Candidate rows of query (b, t) [PR6400-gather, PR6400-window, TT4452-op]:
 * the window rows KV[b, u], u in [max(0, t-W+1), t], then one compressed row
 * C[b, j] per slot whose j satisfies 0 <= j < n_valid(t) (idx == NULL: every
 * j < n_valid(t), the dense-over-compressed mode of [PR6400-core]).  With
 * doc, window rows of other documents drop out, and so do dense-mode blocks
 * whose first token is in another document [TT4452-docs].
 * Returns the number of candidates and fills ptrs with row addresses. */
static int64_t gather_rows(int64_t bi, int64_t t, int64_t S, int64_t D, int64_t W, int64_t r,
                           int64_t nc, int64_t kp, const double* KV, const double* C,
                           const int32_t* idx_row, const int32_t* doc, const double** ptrs,
                           int64_t* is_c, int64_t* where)
{
    int64_t n = 0;
    int64_t u0 = t - W + 1 < 0 ? 0 : t - W + 1;
    for (int64_t u = u0; u <= t; ++u) {
        if (!same_doc(doc, S, bi, t, u)) continue;
        ptrs[n] = KV + (bi * S + u) * D; is_c[n] = 0; where[n] = u; ++n;
    }
    int64_t nv = n_valid_blocks(t, r);
    if (nv > nc) nv = nc;
    if (idx_row) {
        for (int64_t s = 0; s < kp; ++s) {
            int64_t j = idx_row[s];
            if (j < 0 || j >= nv) continue;
            ptrs[n] = C + (bi * nc + j) * D; is_c[n] = 1; where[n] = j; ++n;
        }
    } else {
        for (int64_t j = 0; j < nv; ++j) {
            if (!same_doc(doc, S, bi, t, j * r)) continue;
            ptrs[n] = C + (bi * nc + j) * D; is_c[n] = 1; where[n] = j; ++n;
        }
    }
    return n;
}

/* Sparse attention forward for listed query rows [PR6400-gather, PR6400-sink, TT4452-op]:
 *   l_c  = scale * <Q[t,h], row_c>
 *   LSE  = log(exp(sink_h) + sum_c exp(l_c))       (no sink term if sink == NULL)
 *   P_c  = exp(l_c - LSE),   O[t,h] = sum_c P_c row_c
 * Q [nrows,H,D] holds the listed rows, idx [nrows,kp] their index rows (or NULL),
 * KV [b,S,D], C [b,n_c,D].  O [nrows,H,D], LSE [nrows,H]. */
int csa_oracle_attn_fwd(int64_t S, int64_t H, int64_t D, int64_t W, int64_t r, int64_t nc,
                        int64_t kp, const double* Q, const double* KV, const double* C,
                        const int32_t* idx, const double* sink, double scale,
                        int64_t nrows, const int64_t* rows_b, const int64_t* rows_t,
                        const int32_t* doc, double* O, double* LSE)
{
    int64_t maxc = W + (idx ? kp : nc);
    int err = ORACLE_OK;
#pragma omp parallel
    {
        const double** ptrs = (const double**)malloc(sizeof(double*) * maxc);
        int64_t* is_c = (int64_t*)malloc(sizeof(int64_t) * maxc);
        int64_t* where = (int64_t*)malloc(sizeof(int64_t) * maxc);
        double* l = (double*)malloc(sizeof(double) * maxc);
        if (!ptrs || !is_c || !where || !l) err = ORACLE_ERR;
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < nrows; ++n) {
            if (!ptrs || !is_c || !where || !l) continue;
            int64_t nc_n = gather_rows(rows_b[n], rows_t[n], S, D, W, r, nc, kp, KV, C,
                                       idx ? idx + n * kp : NULL, doc, ptrs, is_c, where);
            for (int64_t h = 0; h < H; ++h) {
                const double* q = Q + (n * H + h) * D;
                double m = sink ? sink[h] : -INFINITY;
                for (int64_t c = 0; c < nc_n; ++c) {
                    double dot = 0.0;
                    for (int64_t e = 0; e < D; ++e) dot += q[e] * ptrs[c][e];
                    l[c] = scale * dot;
                    if (l[c] > m) m = l[c];
                }
                double den = sink ? exp(sink[h] - m) : 0.0;
                for (int64_t c = 0; c < nc_n; ++c) den += exp(l[c] - m);
                double lse = m + log(den);
                LSE[n * H + h] = lse;
                double* o = O + (n * H + h) * D;
                for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
                for (int64_t c = 0; c < nc_n; ++c) {
                    double p = exp(l[c] - lse);
                    for (int64_t e = 0; e < D; ++e) o[e] += p * ptrs[c][e];
                }
            }
        }
        free(ptrs); free(is_c); free(where); free(l);
    }
    return err;
}

/* ------------------------------------------------------------------ a5 --- */
/* Sparse attention backward for listed query rows: the closed-form gradient
 * of the forward above with respect to Q, the gathered rows and the sink.
 *   Delta   = <dO[t,h], O[t,h]>
 *   dl_c    = P_c (<dO[t,h], row_c> - Delta)
 *   dQ[t,h] = scale * sum_c dl_c row_c
 *   row_c  += P_c dO[t,h] + scale * dl_c Q[t,h]    (key part plus value part,
 *             the sum of two products of [TT4452-op]; accumulated into the
 *             compact dKV / dC buffers as in [PR6400-gather], [PR7152-scatter])
 *   dsink_h -= exp(sink_h - LSE) Delta
 * The forward is recomputed here from the same inputs.  dQ [nrows,H,D] is
 * overwritten; dKV [b,S,D], dC [b,n_c,D] and dsink [H] are accumulated into
 * (the caller zeroes them). */
/* One query row's backward: dQ of the row is written, its contributions to
 * the gathered rows and the sink are added into dKV / dC / dsink. */
static void attn_bwd_row(int64_t n, int64_t S, int64_t H, int64_t D, int64_t W, int64_t r, int64_t nc,
                         int64_t kp, const double* Q, const double* KV, const double* C,
                         const int32_t* idx, const double* sink, double scale,
                         const int64_t* rows_b, const int64_t* rows_t, const int32_t* doc,
                         const double* dO, double* dQ, double* dKV, double* dC, double* dsink,
                         const double** ptrs, int64_t* is_c, int64_t* where, double* l, double* o)
{
    int64_t bi = rows_b[n];
    int64_t nc_n = gather_rows(bi, rows_t[n], S, D, W, r, nc, kp, KV, C,
                               idx ? idx + n * kp : NULL, doc, ptrs, is_c, where);
    for (int64_t h = 0; h < H; ++h) {
        const double* q = Q + (n * H + h) * D;
        const double* go = dO + (n * H + h) * D;
        double* gq = dQ + (n * H + h) * D;
        /* forward recompute */
        double m = sink ? sink[h] : -INFINITY;
        for (int64_t c = 0; c < nc_n; ++c) {
            double dot = 0.0;
            for (int64_t e = 0; e < D; ++e) dot += q[e] * ptrs[c][e];
            l[c] = scale * dot;
            if (l[c] > m) m = l[c];
        }
        double den = sink ? exp(sink[h] - m) : 0.0;
        for (int64_t c = 0; c < nc_n; ++c) den += exp(l[c] - m);
        double lse = m + log(den);
        for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
        for (int64_t c = 0; c < nc_n; ++c) {
            double p = exp(l[c] - lse);
            for (int64_t e = 0; e < D; ++e) o[e] += p * ptrs[c][e];
        }
        /* backward */
        double delta = 0.0;
        for (int64_t e = 0; e < D; ++e) delta += go[e] * o[e];
        for (int64_t e = 0; e < D; ++e) gq[e] = 0.0;
        for (int64_t c = 0; c < nc_n; ++c) {
            double p = exp(l[c] - lse);
            double dp = 0.0;
            for (int64_t e = 0; e < D; ++e) dp += go[e] * ptrs[c][e];
            double dl = p * (dp - delta);
            double* dst = is_c[c] ? dC + (bi * nc + where[c]) * D : dKV + (bi * S + where[c]) * D;
            for (int64_t e = 0; e < D; ++e) {
                gq[e] += scale * dl * ptrs[c][e];
                dst[e] += p * go[e] + scale * dl * q[e];
            }
        }
        if (sink && dsink) dsink[h] -= exp(sink[h] - lse) * delta;
    }
}

/* Rows are dealt to BWD_CHUNKS chunks (row n to chunk n % BWD_CHUNKS); each
 * chunk adds its rows, in row order, into a buffer of its own, and the chunk
 * buffers are then added into dKV / dC / dsink in chunk order.  The chunks
 * run on the available threads; the sum is grouped the same way whatever the
 * thread count, so the result is deterministic. */
#define BWD_CHUNKS 16

int csa_oracle_attn_bwd(int64_t S, int64_t H, int64_t D, int64_t W, int64_t r, int64_t nc,
                        int64_t kp, const double* Q, const double* KV, const double* C,
                        const int32_t* idx, const double* sink, double scale,
                        int64_t nrows, const int64_t* rows_b, const int64_t* rows_t,
                        const int32_t* doc, const double* dO, double* dQ, double* dKV, double* dC,
                        double* dsink)
{
    if (nrows <= 0) return ORACLE_OK;
    int64_t maxc = W + (idx ? kp : nc);
    int64_t nb = 0;
    for (int64_t n = 0; n < nrows; ++n)
        if (rows_b[n] + 1 > nb) nb = rows_b[n] + 1;
    const int64_t nch = nrows < BWD_CHUNKS ? nrows : BWD_CHUNKS;
    const int64_t n_kv = nb * S * D, n_c = nb * nc * D, per = n_kv + n_c + H;
    double* part = (double*)calloc((size_t)(nch * per), sizeof(double));
    if (!part) return ORACLE_ERR;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        const double** ptrs = (const double**)malloc(sizeof(double*) * maxc);
        int64_t* is_c = (int64_t*)malloc(sizeof(int64_t) * maxc);
        int64_t* where = (int64_t*)malloc(sizeof(int64_t) * maxc);
        double* l = (double*)malloc(sizeof(double) * maxc);
        double* o = (double*)malloc(sizeof(double) * D);
        if (!ptrs || !is_c || !where || !l || !o) err = ORACLE_ERR;
#pragma omp for schedule(dynamic, 1)
        for (int64_t k = 0; k < nch; ++k) {
            if (!ptrs || !is_c || !where || !l || !o) continue;
            double* pk = part + k * per;
            for (int64_t n = k; n < nrows; n += nch)
                attn_bwd_row(n, S, H, D, W, r, nc, kp, Q, KV, C, idx, sink, scale, rows_b, rows_t, doc, dO,
                             dQ, pk, pk + n_kv, pk + n_kv + n_c, ptrs, is_c, where, l, o);
        }
        free(ptrs); free(is_c); free(where); free(l); free(o);
    }
    if (err == ORACLE_OK) {
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < n_kv; ++e)
            for (int64_t k = 0; k < nch; ++k) dKV[e] += part[k * per + e];
        if (dC) {
#pragma omp parallel for schedule(static)
            for (int64_t e = 0; e < n_c; ++e)
                for (int64_t k = 0; k < nch; ++k) dC[e] += part[k * per + n_kv + e];
        }
        if (sink && dsink)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t k = 0; k < nch; ++k) dsink[h] += part[k * per + n_kv + n_c + h];
    }
    free(part);
    return err;
}
