/*
 * CPU oracle for block-sparse attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct fp64 definitions of every step of the
 * block-sparse attention path.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path
 * never does.  It shares no code, header, table or helper with the GPU
 * library.
 *
 * Inputs are the same bfloat16 tensors the GPU consumes (uint16 bit
 * patterns, widened exactly), laid out contiguously as [B][H][N][D].
 * Every reduction runs in a fixed sequential order per output element, and
 * OpenMP only distributes independent outputs, so results do not depend on
 * the thread count.
 *
 * Sources (page title, section):
 *  - "Block Sparse Attention in multimodal DiT" write-up (lmnt.cn), 2.2:
 *    each block is mean-pooled to one vector, a small linear layer projects
 *    it, query-block / key-block similarity is scored and the top-k key
 *    blocks per query block are kept.  2.3: rows and columns that involve
 *    text stay dense.  3.1: the kept blocks are computed FlashAttention-style
 *    (exactly the dense softmax restricted to the kept set).
 *  - DiTFastAttnV2 notes, "Head-wise Arrow Attention" / "Head-wise Caching" /
 *    "Fused Kernel": vision-vision region keeps a diagonal local window,
 *    every region touching text stays dense; per head one of full, arrow(w)
 *    or skip (reuse the cached output).
 *  - SparseD notes, "Isolated selection": A' = avgpool(A, block) of the
 *    post-softmax attention map, top-rho% blocks chosen separately over the
 *    prefill and the generation columns and unioned.
 *
 * Readings where the pages leave a step open (documented with the tests):
 *  - a partial last block (N not a multiple of the block size) pools over
 *    the tokens it holds; avgpool divides by the actual counts;
 *  - a block that holds any text token is a text block;
 *  - the arrow window is measured in whole blocks, |i - j| <= w;
 *  - top-k ties keep the lower column index;
 *  - a row with no kept key gives O = 0 and LSE = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ECAPACITY (-3)
#define OR_ENOMEM (-4)

#define HEAD_FULL 0
#define HEAD_ARROW 1
#define HEAD_SKIP 2

static double widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int64_t nblocks(int64_t N, int64_t beta) { return (N + beta - 1) / beta; }

static int64_t block_len(int64_t N, int64_t beta, int64_t i)
{
    int64_t lo = i * beta, hi = lo + beta;
    if (hi > N) hi = N;
    return hi - lo;
}

/* ------------------------------------------------------------------------
 * Mean pooling: pooled[b][h][i][:] = (1/n_i) * sum_{t in block i} x[b][h][t][:]
 * ---------------------------------------------------------------------- */
int oracle_pool_mean(const uint16_t *x, int64_t B, int64_t H, int64_t N, int64_t D,
                     int64_t beta, double *pooled)
{
    if (!x || !pooled || B <= 0 || H <= 0 || N <= 0 || D <= 0 || beta <= 0) return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    const int64_t total = B * H * nB;
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        const int64_t bh = item / nB, i = item % nB;
        const int64_t n_i = block_len(N, beta, i);
        double *out = pooled + item * D;
        for (int64_t d = 0; d < D; ++d) {
            double s = 0.0;
            for (int64_t t = i * beta; t < i * beta + n_i; ++t)
                s += widen_bf16(x[(bh * N + t) * D + d]);
            out[d] = s / (double)n_i;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------
 * Content-driven block score (block-sparse DiT write-up, 2.2):
 *   p_i  = W^T qbar_i,  p'_j = W^T kbar_j,  S_ij = p_i . p'_j
 * W is [D][r] row-major, one matrix for queries and keys and all heads.
 * ---------------------------------------------------------------------- */
int oracle_scores_meanpool_proj(const uint16_t *q, const uint16_t *k,
                                int64_t B, int64_t H, int64_t N, int64_t D, int64_t beta,
                                const float *w, int64_t r, double *S)
{
    if (!q || !k || !w || !S || r <= 0) return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    double *qbar = malloc(sizeof(double) * B * H * nB * D);
    double *kbar = malloc(sizeof(double) * B * H * nB * D);
    double *pq = malloc(sizeof(double) * B * H * nB * r);
    double *pk = malloc(sizeof(double) * B * H * nB * r);
    int rc = OR_OK;
    if (!qbar || !kbar || !pq || !pk) { rc = OR_ENOMEM; goto done; }
    if ((rc = oracle_pool_mean(q, B, H, N, D, beta, qbar)) != OR_OK) goto done;
    if ((rc = oracle_pool_mean(k, B, H, N, D, beta, kbar)) != OR_OK) goto done;

    const int64_t total = B * H * nB;
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        for (int64_t m = 0; m < r; ++m) {
            double a = 0.0, c = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                a += (double)w[d * r + m] * qbar[item * D + d];
                c += (double)w[d * r + m] * kbar[item * D + d];
            }
            pq[item * r + m] = a;
            pk[item * r + m] = c;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        const int64_t bh = item / nB;
        for (int64_t j = 0; j < nB; ++j) {
            double s = 0.0;
            for (int64_t m = 0; m < r; ++m)
                s += pq[item * r + m] * pk[(bh * nB + j) * r + m];
            S[item * nB + j] = s;
        }
    }
done:
    free(qbar); free(kbar); free(pq); free(pk);
    return rc;
}

/* ------------------------------------------------------------------------
 * Gradient of the content-driven block score (block-sparse DiT write-up,
 * 2.2, where the projection is trained jointly with the model).  The pages
 * give no loss, so this is the vector-Jacobian product of the score map for
 * a caller's upstream gradient dS = dL/dS [B][H][nB][nB]:
 *   S_ij = p_i . p'_j,  p_i = W^T qbar_i,  p'_j = W^T kbar_j
 *   dL/dp_i  = sum_j dS_ij p'_j          dL/dp'_j = sum_i dS_ij p_i
 *   dL/dW    = sum_{b,h} ( sum_i qbar_i (dL/dp_i)^T + sum_j kbar_j (dL/dp'_j)^T )
 *   dL/dqbar_i = W dL/dp_i,   dL/dkbar_j = W dL/dp'_j
 * dW is [D][r] row-major; dqbar, dkbar are [B][H][nB][D] (either may be
 * NULL).  The gradient of a token of block i is dL/dqbar_i / n_i.
 * ---------------------------------------------------------------------- */
int oracle_score_grad(const uint16_t *q, const uint16_t *k,
                      int64_t B, int64_t H, int64_t N, int64_t D, int64_t beta,
                      const float *w, int64_t r, const double *dS,
                      double *dW, double *dqbar, double *dkbar)
{
    if (!q || !k || !w || !dS || !dW || r <= 0) return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    const int64_t total = B * H * nB;
    double *qbar = malloc(sizeof(double) * total * D);
    double *kbar = malloc(sizeof(double) * total * D);
    double *pq = malloc(sizeof(double) * total * r);
    double *pk = malloc(sizeof(double) * total * r);
    double *gq = malloc(sizeof(double) * total * r);
    double *gk = malloc(sizeof(double) * total * r);
    int rc = OR_OK;
    if (!qbar || !kbar || !pq || !pk || !gq || !gk) { rc = OR_ENOMEM; goto done; }
    if ((rc = oracle_pool_mean(q, B, H, N, D, beta, qbar)) != OR_OK) goto done;
    if ((rc = oracle_pool_mean(k, B, H, N, D, beta, kbar)) != OR_OK) goto done;

    /* the projections, as in the score itself */
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        for (int64_t m = 0; m < r; ++m) {
            double a = 0.0, c = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                a += (double)w[d * r + m] * qbar[item * D + d];
                c += (double)w[d * r + m] * kbar[item * D + d];
            }
            pq[item * r + m] = a;
            pk[item * r + m] = c;
        }
    }
    /* dL/dp_i over the row i of dS, dL/dp'_j over the column j */
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        const int64_t bh = item / nB, x = item % nB;
        for (int64_t m = 0; m < r; ++m) {
            double a = 0.0, c = 0.0;
            for (int64_t y = 0; y < nB; ++y) {
                a += dS[(bh * nB + x) * nB + y] * pk[(bh * nB + y) * r + m];
                c += dS[(bh * nB + y) * nB + x] * pq[(bh * nB + y) * r + m];
            }
            gq[item * r + m] = a;
            gk[item * r + m] = c;
        }
    }
    /* dW: the outer products summed over every block of every head */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < D * r; ++e) {
        const int64_t d = e / r, m = e % r;
        double s = 0.0;
        for (int64_t item = 0; item < total; ++item)
            s += qbar[item * D + d] * gq[item * r + m] + kbar[item * D + d] * gk[item * r + m];
        dW[e] = s;
    }
    /* the pooled blocks' gradients */
#pragma omp parallel for schedule(static)
    for (int64_t item = 0; item < total; ++item) {
        for (int64_t d = 0; d < D; ++d) {
            double a = 0.0, c = 0.0;
            for (int64_t m = 0; m < r; ++m) {
                a += (double)w[d * r + m] * gq[item * r + m];
                c += (double)w[d * r + m] * gk[item * r + m];
            }
            if (dqbar) dqbar[item * D + d] = a;
            if (dkbar) dkbar[item * D + d] = c;
        }
    }
done:
    free(qbar); free(kbar); free(pq); free(pk); free(gq); free(gk);
    return rc;
}

/* ------------------------------------------------------------------------
 * Exact block score (SparseD notes, isolated selection):
 *   A_ts = softmax_s(scale * Q_t . K_s) over all N keys of the head;
 *   S_ij = (1 / (n_i n_j)) * sum_{t in block i} sum_{s in block j} A_ts.
 * Computed one query row at a time (the notes compute A' chunk by chunk
 * over Q).  `rows` lists flat query-block rows (b*H + h)*nB + i; NULL means
 * all of them in order.  Output S_rows is [n_rows][nB].
 * ---------------------------------------------------------------------- */
int oracle_scores_exact_avgpool(const uint16_t *q, const uint16_t *k,
                                int64_t B, int64_t H, int64_t N, int64_t D, int64_t beta,
                                double scale, const int64_t *rows, int64_t n_rows,
                                double *S_rows)
{
    if (!q || !k || !S_rows || B <= 0 || H <= 0 || N <= 0 || D <= 0 || beta <= 0)
        return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    if (!rows) n_rows = B * H * nB;
    for (int64_t x = 0; x < n_rows; ++x) {
        int64_t row = rows ? rows[x] : x;
        if (row < 0 || row >= B * H * nB) return OR_EINVAL;
    }
    /* one partial row of block sums per query token, reduced afterwards in
       token order so that the result does not depend on the thread count */
    const int64_t tok = n_rows * beta;
    double *part = calloc((size_t)(tok * nB), sizeof(double));
    if (!part) return OR_ENOMEM;
    int rc = OR_OK;
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * N);
        double *qt = malloc(sizeof(double) * D);
        if (!z || !qt) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t u = 0; u < tok; ++u) {
                const int64_t x = u / beta, tt = u % beta;
                const int64_t row = rows ? rows[x] : x;
                const int64_t bh = row / nB, i = row % nB;
                const int64_t t = i * beta + tt;
                if (t >= N) continue;
                for (int64_t d = 0; d < D; ++d) qt[d] = widen_bf16(q[(bh * N + t) * D + d]);
                double m = -INFINITY;
                for (int64_t s = 0; s < N; ++s) {
                    const uint16_t *ks = k + (bh * N + s) * D;
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += qt[d] * widen_bf16(ks[d]);
                    z[s] = scale * acc;
                    if (z[s] > m) m = z[s];
                }
                double l = 0.0;
                for (int64_t s = 0; s < N; ++s) l += exp(z[s] - m);
                double *p = part + u * nB;
                for (int64_t s = 0; s < N; ++s) p[s / beta] += exp(z[s] - m) / l;
            }
        }
        free(z);
        free(qt);
    }
    if (rc == OR_OK) {
        for (int64_t x = 0; x < n_rows; ++x) {
            const int64_t row = rows ? rows[x] : x;
            const int64_t i = row % nB;
            const int64_t n_i = block_len(N, beta, i);
            for (int64_t j = 0; j < nB; ++j) {
                double s = 0.0;
                for (int64_t tt = 0; tt < n_i; ++tt) s += part[(x * beta + tt) * nB + j];
                S_rows[x * nB + j] = s / ((double)n_i * (double)block_len(N, beta, j));
            }
        }
    }
    free(part);
    return rc;
}

/* ------------------------------------------------------------------------
 * Top-k block selection (write-up 2.2 and 2.3; SparseD isolated selection).
 * For each listed row (its query-block index qblock[x] and its nB scores):
 *   - a text query block (qblock < text_blocks) keeps every column;
 *   - otherwise keep F = {j < text_blocks} united with, for each group g
 *     (column range [c_g, e_g), budget k_g), the first k_g columns of that
 *     range ordered by descending score, lower column first on equal scores.
 * A NaN score carries no evidence for its block: it ranks after every
 * number (-inf included), NaNs among themselves by lower column.
 * Output: CSR over the listed rows, columns ascending.  Returns nnz >= 0 or
 * a negative error.
 * ---------------------------------------------------------------------- */
typedef struct { double s; int32_t j; } scored_col;

static int cmp_scored(const void *a, const void *b)
{
    const scored_col *x = a, *y = b;
    const int xn = isnan(x->s), yn = isnan(y->s);
    if (xn != yn) return xn ? 1 : -1;
    if (!xn) {
        if (x->s > y->s) return -1;
        if (x->s < y->s) return 1;
    }
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

int64_t oracle_select_rows(const double *S_rows, const int32_t *qblock, int64_t n_rows,
                           int64_t nB, int64_t text_blocks, const int32_t *groups, int64_t n_groups,
                           int32_t *row_ptr, int32_t *col_idx, int64_t capacity)
{
    if (!S_rows || !qblock || !row_ptr || nB <= 0 || text_blocks < 0 || n_groups < 0)
        return OR_EINVAL;
    for (int64_t g = 0; g < n_groups; ++g) {
        int32_t c0 = groups[3 * g], c1 = groups[3 * g + 1], kk = groups[3 * g + 2];
        if (c0 < 0 || c1 > nB || c0 >= c1 || kk < 0 || kk > c1 - c0) return OR_EINVAL;
    }
    unsigned char *keep = malloc((size_t)nB);
    scored_col *buf = malloc(sizeof(scored_col) * (size_t)nB);
    if (!keep || !buf) { free(keep); free(buf); return OR_ENOMEM; }
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int64_t x = 0; x < n_rows; ++x) {
        const double *s = S_rows + x * nB;
        memset(keep, 0, (size_t)nB);
        if (qblock[x] < text_blocks) {
            memset(keep, 1, (size_t)nB);
        } else {
            for (int64_t j = 0; j < nB && j < text_blocks; ++j) keep[j] = 1;
            for (int64_t g = 0; g < n_groups; ++g) {
                int32_t c0 = groups[3 * g], c1 = groups[3 * g + 1], kk = groups[3 * g + 2];
                int64_t n = 0;
                for (int32_t j = c0; j < c1; ++j) { buf[n].s = s[j]; buf[n].j = j; ++n; }
                qsort(buf, (size_t)n, sizeof(scored_col), cmp_scored);
                for (int64_t a = 0; a < kk; ++a) keep[buf[a].j] = 1;
            }
        }
        for (int64_t j = 0; j < nB; ++j) {
            if (!keep[j]) continue;
            if (col_idx) {
                if (nnz >= capacity) { free(keep); free(buf); return OR_ECAPACITY; }
                col_idx[nnz] = (int32_t)j;
            }
            ++nnz;
        }
        row_ptr[x + 1] = (int32_t)nnz;
    }
    free(keep);
    free(buf);
    return nnz;
}

/* ------------------------------------------------------------------------
 * Arrow layout (DiTFastAttnV2 notes, head-wise arrow attention):
 *   ARROW head: keep(i, j) = i < T_b or j < T_b or |i - j| <= w_h
 *   FULL head : keep every (i, j)
 *   SKIP head : no rows are computed (every row is empty)
 * Rows are ordered (b, h, i); columns ascending.  Returns nnz or an error.
 * ---------------------------------------------------------------------- */
int64_t oracle_arrow(int64_t B, int64_t H, int64_t nB, int64_t text_blocks,
                     const int8_t *modes, const int32_t *windows,
                     int32_t *row_ptr, int32_t *col_idx, int64_t capacity)
{
    if (B <= 0 || H <= 0 || nB <= 0 || text_blocks < 0 || !modes || !windows || !row_ptr)
        return OR_EINVAL;
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            if (modes[h] != HEAD_FULL && modes[h] != HEAD_ARROW && modes[h] != HEAD_SKIP)
                return OR_EINVAL;
            if (modes[h] == HEAD_ARROW && windows[h] < 0) return OR_EINVAL;
            for (int64_t i = 0; i < nB; ++i) {
                for (int64_t j = 0; j < nB; ++j) {
                    int kp;
                    if (modes[h] == HEAD_SKIP) kp = 0;
                    else if (modes[h] == HEAD_FULL) kp = 1;
                    else kp = (i < text_blocks) || (j < text_blocks) ||
                              (llabs(i - j) <= (int64_t)windows[h]);
                    if (!kp) continue;
                    if (col_idx) {
                        if (nnz >= capacity) return OR_ECAPACITY;
                        col_idx[nnz] = (int32_t)j;
                    }
                    ++nnz;
                }
                row_ptr[(b * H + h) * nB + i + 1] = (int32_t)nnz;
            }
        }
    return nnz;
}

/* ------------------------------------------------------------------------
 * Block-sparse attention forward, by definition:
 *   z_s = scale * Q_t . K_s   if key block floor(s/beta) is kept for query
 *                             block floor(t/beta) of this head, else -inf
 *   m = max_s z_s,  l = sum_s e^{z_s - m},
 *   O_t = sum_s e^{z_s - m} V_s / l,   LSE_t = m + ln l.
 * SKIP heads (modes != NULL and modes[h] == SKIP) return the cached row
 * unchanged (O from o_cache, LSE from lse_cache, NaN when lse_cache is NULL).
 * `rows` lists flat token rows (b*H + h)*N + t; NULL means every row.
 * Outputs O [n_rows][D], LSE [n_rows].
 * ---------------------------------------------------------------------- */
int oracle_forward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   int64_t B, int64_t H, int64_t N, int64_t D, int64_t beta,
                   const int32_t *row_ptr, const int32_t *col_idx,
                   const int8_t *modes, const uint16_t *o_cache, const float *lse_cache,
                   double scale, const int64_t *rows, int64_t n_rows,
                   double *O, double *LSE)
{
    if (!q || !k || !v || !row_ptr || !O || !LSE || B <= 0 || H <= 0 || N <= 0 || D <= 0 ||
        beta <= 0)
        return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    if (row_ptr[0] != 0) return OR_EINVAL;
    for (int64_t r = 0; r < B * H * nB; ++r) {
        if (row_ptr[r + 1] < row_ptr[r]) return OR_EINVAL;
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            if (!col_idx || col_idx[e] < 0 || col_idx[e] >= nB) return OR_EINVAL;
    }
    if (!rows) n_rows = B * H * N;
    for (int64_t x = 0; x < n_rows; ++x) {
        int64_t row = rows ? rows[x] : x;
        if (row < 0 || row >= B * H * N) return OR_EINVAL;
        int64_t h = (row / N) % H;
        if (modes && modes[h] == HEAD_SKIP && !o_cache) return OR_EINVAL;
    }
    int rc = OR_OK;
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * N);
        unsigned char *kept = malloc((size_t)nB);
        if (!z || !kept) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t row = rows ? rows[x] : x;
                const int64_t bh = row / N, t = row % N, h = bh % H;
                double *o = O + x * D;
                if (modes && modes[h] == HEAD_SKIP) {
                    for (int64_t d = 0; d < D; ++d) o[d] = widen_bf16(o_cache[row * D + d]);
                    LSE[x] = lse_cache ? (double)lse_cache[row] : NAN;
                    continue;
                }
                const int64_t r = bh * nB + t / beta;
                memset(kept, 0, (size_t)nB);
                for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) kept[col_idx[e]] = 1;
                double m = -INFINITY;
                for (int64_t s = 0; s < N; ++s) {
                    if (!kept[s / beta]) { z[s] = -INFINITY; continue; }
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        acc += widen_bf16(q[row * D + d]) * widen_bf16(k[(bh * N + s) * D + d]);
                    z[s] = scale * acc;
                    if (z[s] > m) m = z[s];
                }
                if (m == -INFINITY) {
                    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                    LSE[x] = -INFINITY;
                    continue;
                }
                double l = 0.0;
                for (int64_t s = 0; s < N; ++s)
                    if (z[s] != -INFINITY) l += exp(z[s] - m);
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (z[s] == -INFINITY) continue;
                    const double p = exp(z[s] - m);
                    for (int64_t d = 0; d < D; ++d) o[d] += p * widen_bf16(v[(bh * N + s) * D + d]);
                }
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
                LSE[x] = m + log(l);
            }
        }
        free(z);
        free(kept);
    }
    return rc;
}

/* ------------------------------------------------------------------------
 * FP8 (OCP E4M3) quantisation and the forward on quantised inputs.
 *
 * E4M3, by its definition: 1 sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent field 0 holds subnormals m * 2^-9; field 15 with
 * mantissa 7 is NaN (no infinities); the largest finite value is
 * 1.75 * 2^8 = 448.  Encoding rounds to nearest, ties to even mantissa.
 *
 * Scaled quantisation of a group of values x with amax = max |x| (all in
 * fp32, the precision the codes are decided in):
 *   scale = amax / 448,  inv = 448 / amax   (both 0 when amax == 0),
 *   code  = E4M3(x * inv),   dequantised value = decode(code) * scale.
 * Groups: Q per token (over d); K per 64-key tile of a head (64 keys x d,
 * the last tile holding the keys that exist); V per channel d over all N
 * keys of a head.
 * ---------------------------------------------------------------------- */
double oracle_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

uint8_t oracle_e4m3_encode(float x)
{
    if (isnan(x)) return 0x7F;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const double a = fabs((double)x);
    if (a > 464.0) return (uint8_t)(sign | 0x7F);   /* past the rounding range of 448: NaN */
    /* the finite non-negative codes 0x00 .. 0x7E are increasing in value:
       find the first code >= a, then take the nearer neighbour, ties to the
       even code (even mantissa) */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) < a) lo = mid + 1;
        else hi = mid;
    }
    int c = lo;
    if (c > 0) {
        const double up = oracle_e4m3_decode((uint8_t)c) - a;
        const double dn = a - oracle_e4m3_decode((uint8_t)(c - 1));
        if (dn < up || (dn == up && ((c - 1) & 1) == 0)) c = c - 1;
    }
    return (uint8_t)(sign | c);
}

void oracle_e4m3_encode_array(const float *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_array(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

static void quant_group_scale(float amax, float *scale, float *inv)
{
    if (amax > 0.f) {
        *scale = amax / 448.0f;
        *inv = 448.0f / amax;
    } else {
        *scale = 0.f;
        *inv = 0.f;
    }
}

static float widen_bf16_f(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int oracle_quantize_fp8(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int64_t B, int64_t H, int64_t N, int64_t D,
                        uint8_t *q8, float *q_scale, uint8_t *k8, float *k_scale,
                        uint8_t *v8, float *v_scale)
{
    if (!q || !k || !v || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || B <= 0 || H <= 0 ||
        N <= 0 || D <= 0)
        return OR_EINVAL;
    const int64_t NT = (N + 63) / 64;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        for (int64_t t = 0; t < N; ++t) {   /* Q: per token */
            const uint16_t *x = q + (bh * N + t) * D;
            float amax = 0.f;
            for (int64_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(widen_bf16_f(x[d])));
            float sc, inv;
            quant_group_scale(amax, &sc, &inv);
            q_scale[bh * N + t] = sc;
            for (int64_t d = 0; d < D; ++d) q8[(bh * N + t) * D + d] = oracle_e4m3_encode(widen_bf16_f(x[d]) * inv);
        }
        for (int64_t T = 0; T < NT; ++T) {   /* K: per 64-key tile */
            const int64_t t0 = T * 64, t1 = (t0 + 64 < N) ? t0 + 64 : N;
            float amax = 0.f;
            for (int64_t t = t0; t < t1; ++t)
                for (int64_t d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(widen_bf16_f(k[(bh * N + t) * D + d])));
            float sc, inv;
            quant_group_scale(amax, &sc, &inv);
            k_scale[bh * NT + T] = sc;
            for (int64_t t = t0; t < t1; ++t)
                for (int64_t d = 0; d < D; ++d)
                    k8[(bh * N + t) * D + d] = oracle_e4m3_encode(widen_bf16_f(k[(bh * N + t) * D + d]) * inv);
        }
        for (int64_t d = 0; d < D; ++d) {   /* V: per channel */
            float amax = 0.f;
            for (int64_t t = 0; t < N; ++t) amax = fmaxf(amax, fabsf(widen_bf16_f(v[(bh * N + t) * D + d])));
            float sc, inv;
            quant_group_scale(amax, &sc, &inv);
            v_scale[bh * D + d] = sc;
            for (int64_t t = 0; t < N; ++t)
                v8[(bh * N + t) * D + d] = oracle_e4m3_encode(widen_bf16_f(v[(bh * N + t) * D + d]) * inv);
        }
    }
    return OR_OK;
}

/* The forward of oracle_forward on the dequantised inputs
 * q = decode(q8) * q_scale[token], k = decode(k8) * k_scale[tile],
 * v = decode(v8) * v_scale[channel]; every head computed (no modes). */
int oracle_forward_fp8(const uint8_t *q8, const float *q_scale, const uint8_t *k8, const float *k_scale,
                       const uint8_t *v8, const float *v_scale, int64_t B, int64_t H, int64_t N, int64_t D,
                       int64_t beta, const int32_t *row_ptr, const int32_t *col_idx, double scale,
                       const int64_t *rows, int64_t n_rows, double *O, double *LSE)
{
    if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !row_ptr || !O || !LSE || B <= 0 ||
        H <= 0 || N <= 0 || D <= 0 || beta <= 0)
        return OR_EINVAL;
    const int64_t nB = nblocks(N, beta), NT = (N + 63) / 64;
    if (row_ptr[0] != 0) return OR_EINVAL;
    for (int64_t r = 0; r < B * H * nB; ++r) {
        if (row_ptr[r + 1] < row_ptr[r]) return OR_EINVAL;
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            if (!col_idx || col_idx[e] < 0 || col_idx[e] >= nB) return OR_EINVAL;
    }
    if (!rows) n_rows = B * H * N;
    for (int64_t x = 0; x < n_rows; ++x) {
        const int64_t row = rows ? rows[x] : x;
        if (row < 0 || row >= B * H * N) return OR_EINVAL;
    }
    int rc = OR_OK;
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * N);
        unsigned char *kept = malloc((size_t)nB);
        if (!z || !kept) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t row = rows ? rows[x] : x;
                const int64_t bh = row / N, t = row % N;
                double *o = O + x * D;
                const int64_t r = bh * nB + t / beta;
                memset(kept, 0, (size_t)nB);
                for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) kept[col_idx[e]] = 1;
                const double qs = q_scale[row];
                double m = -INFINITY;
                for (int64_t s = 0; s < N; ++s) {
                    if (!kept[s / beta]) { z[s] = -INFINITY; continue; }
                    const double ks = k_scale[bh * NT + s / 64];
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        acc += (oracle_e4m3_decode(q8[row * D + d]) * qs) *
                               (oracle_e4m3_decode(k8[(bh * N + s) * D + d]) * ks);
                    z[s] = scale * acc;
                    if (z[s] > m) m = z[s];
                }
                if (m == -INFINITY) {
                    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                    LSE[x] = -INFINITY;
                    continue;
                }
                double l = 0.0;
                for (int64_t s = 0; s < N; ++s)
                    if (z[s] != -INFINITY) l += exp(z[s] - m);
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (z[s] == -INFINITY) continue;
                    const double pw = exp(z[s] - m);
                    for (int64_t d = 0; d < D; ++d)
                        o[d] += pw * (oracle_e4m3_decode(v8[(bh * N + s) * D + d]) * v_scale[bh * D + d]);
                }
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
                LSE[x] = m + log(l);
            }
        }
        free(z);
        free(kept);
    }
    return rc;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Two-dimensional neighbourhood attention (GNA notes, section 1.1: a
 * window around each query on the latent grid, with a stride by which
 * groups of queries share one window; stride 1 is the sliding window, a
 * stride equal to the window gives blocked attention).  Per axis of length
 * L with window k and stride s, query position i sees the k positions from
 *     start(i) = clamp(s * floor(i / s) + floor(s / 2) - floor(k / 2), 0, L - k),
 * the window of the centre of i's stride group, shifted inside the axis.
 * The sequence is text_len text tokens, then the R x C image grid in
 * row-major order; text queries see every key and every query sees the
 * text keys (regions involving text stay dense).
 * ---------------------------------------------------------------------- */
int64_t oracle_na_start(int64_t i, int64_t L, int64_t k, int64_t s)
{
    int64_t a = s * (i / s) + s / 2 - k / 2;
    if (a > L - k) a = L - k;
    if (a < 0) a = 0;
    return a;
}

typedef struct {
    int64_t T, R, C, kh, kw, sh, sw;
} na_geom;

/* natural-order tokens: does query tq see key tk */
static int na_token_keep(int64_t tq, int64_t tk, const na_geom *g)
{
    if (tq < g->T || tk < g->T) return 1;
    const int64_t pq = tq - g->T, pk = tk - g->T;
    const int64_t rq = pq / g->C, cq = pq % g->C, rk = pk / g->C, ck = pk % g->C;
    const int64_t r0 = oracle_na_start(rq, g->R, g->kh, g->sh), c0 = oracle_na_start(cq, g->C, g->kw, g->sw);
    return rk >= r0 && rk < r0 + g->kh && ck >= c0 && ck < c0 + g->kw;
}

static int na_check(int64_t N, int64_t T, int64_t R, int64_t C, int64_t kh, int64_t kw, int64_t sh, int64_t sw)
{
    return T >= 0 && R > 0 && C > 0 && N == T + R * C && kh >= 1 && kh <= R && kw >= 1 && kw <= C && sh >= 1 &&
           sw >= 1;
}

/* Dense softmax attention under the neighbourhood mask, natural token order. */
int oracle_forward_neighborhood(const uint16_t *q, const uint16_t *k, const uint16_t *v, int64_t B, int64_t H,
                                int64_t N, int64_t D, int64_t text_len, int64_t R, int64_t C, int64_t kh,
                                int64_t kw, int64_t sh, int64_t sw, double scale, const int64_t *rows,
                                int64_t n_rows, double *O, double *LSE)
{
    if (!q || !k || !v || !O || !LSE || B <= 0 || H <= 0 || D <= 0 || !na_check(N, text_len, R, C, kh, kw, sh, sw))
        return OR_EINVAL;
    if (!rows) n_rows = B * H * N;
    for (int64_t x = 0; x < n_rows; ++x) {
        const int64_t row = rows ? rows[x] : x;
        if (row < 0 || row >= B * H * N) return OR_EINVAL;
    }
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
    int rc = OR_OK;
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * N);
        if (!z) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t row = rows ? rows[x] : x;
                const int64_t bh = row / N, t = row % N;
                double *o = O + x * D;
                double m = -INFINITY;
                for (int64_t s = 0; s < N; ++s) {
                    if (!na_token_keep(t, s, &g)) { z[s] = -INFINITY; continue; }
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        acc += widen_bf16(q[row * D + d]) * widen_bf16(k[(bh * N + s) * D + d]);
                    z[s] = scale * acc;
                    if (z[s] > m) m = z[s];
                }
                double l = 0.0;
                for (int64_t s = 0; s < N; ++s)
                    if (z[s] != -INFINITY) l += exp(z[s] - m);
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (z[s] == -INFINITY) continue;
                    const double p = exp(z[s] - m);
                    for (int64_t d = 0; d < D; ++d) o[d] += p * widen_bf16(v[(bh * N + s) * D + d]);
                }
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
                LSE[x] = m + log(l);
            }
        }
        free(z);
    }
    return rc;
}

/* Tile-major order (GNA notes, section 2.2, token permutation): text
 * tokens first and unchanged, then the image tiles of th x tw tokens in
 * row-major order of tiles, each tile's tokens row-major.  perm[p] is the
 * natural index of the token at permuted position p. */
int oracle_tile_permutation(int64_t text_len, int64_t R, int64_t C, int64_t th, int64_t tw, int64_t *perm)
{
    if (!perm || text_len < 0 || R <= 0 || C <= 0 || th <= 0 || tw <= 0 || R % th || C % tw) return OR_EINVAL;
    for (int64_t t = 0; t < text_len; ++t) perm[t] = t;
    const int64_t tpr = C / tw;
    for (int64_t p = 0; p < R * C; ++p) {
        const int64_t tile = p / (th * tw), o = p % (th * tw);
        const int64_t r = (tile / tpr) * th + o / tw, c = (tile % tpr) * tw + o % tw;
        perm[text_len + p] = text_len + r * C + c;
    }
    return OR_OK;
}

/* Block layout of one head in tile-major order, by brute force over token
 * pairs: block pair (i, j) is absent when no query of block i sees a key of
 * block j, "full" (flag 0) when every query sees every key, else "partial"
 * (flag 1).  Blocks are th*tw tokens; text_len must be a multiple of that.
 * Columns ascend within a row. */
int oracle_neighborhood_layout(int64_t text_len, int64_t R, int64_t C, int64_t th, int64_t tw, int64_t kh,
                               int64_t kw, int64_t sh, int64_t sw, int32_t *row_ptr, int32_t *col_idx,
                               uint8_t *flags, int64_t capacity)
{
    const int64_t beta = th * tw, N = text_len + R * C;
    if (!row_ptr || !col_idx || !flags || text_len % beta || !na_check(N, text_len, R, C, kh, kw, sh, sw) ||
        R % th || C % tw)
        return OR_EINVAL;
    const int64_t nB = N / beta;
    int64_t *perm = malloc(sizeof(int64_t) * N);
    int64_t *cnt = malloc(sizeof(int64_t) * nB * nB);
    if (!perm || !cnt) { free(perm); free(cnt); return OR_ENOMEM; }
    oracle_tile_permutation(text_len, R, C, th, tw, perm);
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nB; ++i)
        for (int64_t j = 0; j < nB; ++j) {
            int64_t c = 0;
            for (int64_t a = 0; a < beta; ++a)
                for (int64_t b = 0; b < beta; ++b) c += na_token_keep(perm[i * beta + a], perm[j * beta + b], &g);
            cnt[i * nB + j] = c;
        }
    int64_t nnz = 0;
    int rc = OR_OK;
    row_ptr[0] = 0;
    for (int64_t i = 0; i < nB && rc == OR_OK; ++i) {
        for (int64_t j = 0; j < nB; ++j) {
            const int64_t c = cnt[i * nB + j];
            if (c == 0) continue;
            if (nnz >= capacity) { rc = OR_ECAPACITY; break; }
            col_idx[nnz] = (int32_t)j;
            flags[nnz] = c == beta * beta ? 0 : 1;
            ++nnz;
        }
        row_ptr[i + 1] = (int32_t)nnz;
    }
    free(perm);
    free(cnt);
    return rc;
}

/* ------------------------------------------------------------------------
 * Backward of the block-sparse forward (the gradient of the dense softmax
 * restricted to the kept blocks), fp64 throughout, on fp64 inputs.
 * With z_ts = scale * Q_t.K_s on kept (t, s), P = softmax_s(z), O = P V:
 *   dV_s  = sum_t P_ts dO_t
 *   dP_ts = dO_t . V_s,   Delta_t = sum_s P_ts dP_ts  (= dO_t . O_t)
 *   dS_ts = P_ts (dP_ts - Delta_t)
 *   dQ_t  = scale * sum_s dS_ts K_s,   dK_s = scale * sum_t dS_ts Q_t
 * A row with no kept key contributes nothing.  oracle_forward_f64 is the
 * forward on the same fp64 inputs (for finite-difference checks).
 * ---------------------------------------------------------------------- */
static int bw_check_csr(int64_t rows, int64_t nB, const int32_t *row_ptr, const int32_t *col_idx)
{
    if (!row_ptr || row_ptr[0] != 0) return 0;
    for (int64_t r = 0; r < rows; ++r) {
        if (row_ptr[r + 1] < row_ptr[r]) return 0;
        for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)
            if (!col_idx || col_idx[e] < 0 || col_idx[e] >= nB) return 0;
    }
    return 1;
}

/* probabilities of row t of head bh: p[s] (0 where not kept); returns 0 for
 * a row with no kept key */
static int bw_row_probs(const double *q, const double *k, int64_t N, int64_t D, int64_t beta, int64_t nB,
                        int64_t bh, int64_t t, const int32_t *row_ptr, const int32_t *col_idx, double scale,
                        unsigned char *kept, double *p, double *lse)
{
    const int64_t r = bh * nB + t / beta;
    memset(kept, 0, (size_t)nB);
    for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) kept[col_idx[e]] = 1;
    double m = -INFINITY;
    for (int64_t s = 0; s < N; ++s) {
        if (!kept[s / beta]) { p[s] = -INFINITY; continue; }
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += q[(bh * N + t) * D + d] * k[(bh * N + s) * D + d];
        p[s] = scale * acc;
        if (p[s] > m) m = p[s];
    }
    if (m == -INFINITY) return 0;
    double l = 0.0;
    for (int64_t s = 0; s < N; ++s) l += p[s] == -INFINITY ? 0.0 : exp(p[s] - m);
    for (int64_t s = 0; s < N; ++s) p[s] = p[s] == -INFINITY ? 0.0 : exp(p[s] - m) / l;
    if (lse) *lse = m + log(l);
    return 1;
}

int oracle_forward_f64(const double *q, const double *k, const double *v, int64_t B, int64_t H, int64_t N,
                       int64_t D, int64_t beta, const int32_t *row_ptr, const int32_t *col_idx, double scale,
                       double *O, double *LSE)
{
    if (!q || !k || !v || !O || !LSE || B <= 0 || H <= 0 || N <= 0 || D <= 0 || beta <= 0) return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    if (!bw_check_csr(B * H * nB, nB, row_ptr, col_idx)) return OR_EINVAL;
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        unsigned char *kept = malloc((size_t)nB);
        if (!p || !kept) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t row = 0; row < B * H * N; ++row) {
                const int64_t bh = row / N, t = row % N;
                double *o = O + row * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
                if (!bw_row_probs(q, k, N, D, beta, nB, bh, t, row_ptr, col_idx, scale, kept, p, &LSE[row])) {
                    LSE[row] = -INFINITY;
                    continue;
                }
                for (int64_t s = 0; s < N; ++s)
                    if (p[s] != 0.0)
                        for (int64_t d = 0; d < D; ++d) o[d] += p[s] * v[(bh * N + s) * D + d];
            }
        }
        free(p);
        free(kept);
    }
    return rc;
}

int oracle_backward_f64(const double *q, const double *k, const double *v, const double *dO, int64_t B, int64_t H,
                        int64_t N, int64_t D, int64_t beta, const int32_t *row_ptr, const int32_t *col_idx,
                        double scale, double *dQ, double *dK, double *dV)
{
    if (!q || !k || !v || !dO || !dQ || !dK || !dV || B <= 0 || H <= 0 || N <= 0 || D <= 0 || beta <= 0)
        return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    if (!bw_check_csr(B * H * nB, nB, row_ptr, col_idx)) return OR_EINVAL;
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        double *dp = malloc(sizeof(double) * N);
        unsigned char *kept = malloc((size_t)nB);
        if (!p || !dp || !kept) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
            /* one (b, h) per iteration: dK, dV of a head are touched by its rows only */
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                memset(dK + bh * N * D, 0, sizeof(double) * N * D);
                memset(dV + bh * N * D, 0, sizeof(double) * N * D);
                for (int64_t t = 0; t < N; ++t) {
                    double *dq = dQ + (bh * N + t) * D;
                    for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
                    if (!bw_row_probs(q, k, N, D, beta, nB, bh, t, row_ptr, col_idx, scale, kept, p, NULL))
                        continue;
                    const double *go = dO + (bh * N + t) * D;
                    double delta = 0.0;
                    for (int64_t s = 0; s < N; ++s) {
                        if (p[s] == 0.0) { dp[s] = 0.0; continue; }
                        double acc = 0.0;
                        for (int64_t d = 0; d < D; ++d) acc += go[d] * v[(bh * N + s) * D + d];
                        dp[s] = acc;
                        delta += p[s] * acc;
                    }
                    for (int64_t s = 0; s < N; ++s) {
                        if (p[s] == 0.0) continue;
                        const double ds = p[s] * (dp[s] - delta);
                        for (int64_t d = 0; d < D; ++d) {
                            dV[(bh * N + s) * D + d] += p[s] * go[d];
                            dq[d] += scale * ds * k[(bh * N + s) * D + d];
                            dK[(bh * N + s) * D + d] += scale * ds * q[(bh * N + t) * D + d];
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
        free(kept);
    }
    return rc;
}

/* dQ of selected query rows only (flat row indices into [B*H*N]): row t's
 * gradient needs only row t of P and dP, so rows of a full-size problem can
 * be checked one by one.  Same formulas as oracle_backward_f64. */
int oracle_backward_dq_rows(const double *q, const double *k, const double *v, const double *dO, int64_t B,
                            int64_t H, int64_t N, int64_t D, int64_t beta, const int32_t *row_ptr,
                            const int32_t *col_idx, double scale, const int64_t *rows, int64_t n_rows, double *dQ)
{
    if (!q || !k || !v || !dO || !rows || !dQ || B <= 0 || H <= 0 || N <= 0 || D <= 0 || beta <= 0)
        return OR_EINVAL;
    const int64_t nB = nblocks(N, beta);
    if (!bw_check_csr(B * H * nB, nB, row_ptr, col_idx)) return OR_EINVAL;
    for (int64_t x = 0; x < n_rows; ++x)
        if (rows[x] < 0 || rows[x] >= B * H * N) return OR_EINVAL;
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        double *dp = malloc(sizeof(double) * N);
        unsigned char *kept = malloc((size_t)nB);
        if (!p || !dp || !kept) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t bh = rows[x] / N, t = rows[x] % N;
                double *dq = dQ + x * D;
                for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
                if (!bw_row_probs(q, k, N, D, beta, nB, bh, t, row_ptr, col_idx, scale, kept, p, NULL)) continue;
                const double *go = dO + (bh * N + t) * D;
                double delta = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (p[s] == 0.0) { dp[s] = 0.0; continue; }
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += go[d] * v[(bh * N + s) * D + d];
                    dp[s] = acc;
                    delta += p[s] * acc;
                }
                for (int64_t s = 0; s < N; ++s) {
                    if (p[s] == 0.0) continue;
                    const double ds = p[s] * (dp[s] - delta);
                    for (int64_t d = 0; d < D; ++d) dq[d] += scale * ds * k[(bh * N + s) * D + d];
                }
            }
        }
        free(p);
        free(dp);
        free(kept);
    }
    return rc;
}

/* ------------------------------------------------------------------------
 * Backward of the 2-D neighbourhood attention (GNA notes, 1.1), natural
 * token order, fp64 inputs: the gradient of the dense softmax under the
 * token mask na_token_keep (the same formulas as oracle_backward_f64 with
 * that mask in place of the kept blocks).  oracle_forward_neighborhood_f64
 * is the forward on the same fp64 inputs (for finite-difference checks).
 * Every query keeps at least the keys of its window, so no row is empty.
 * ---------------------------------------------------------------------- */
static void na_row_probs(const double *q, const double *k, int64_t N, int64_t D, int64_t bh, int64_t t,
                         const na_geom *g, double scale, double *p, double *lse)
{
    double m = -INFINITY;
    for (int64_t s = 0; s < N; ++s) {
        if (!na_token_keep(t, s, g)) { p[s] = -INFINITY; continue; }
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += q[(bh * N + t) * D + d] * k[(bh * N + s) * D + d];
        p[s] = scale * acc;
        if (p[s] > m) m = p[s];
    }
    double l = 0.0;
    for (int64_t s = 0; s < N; ++s) {
        p[s] = p[s] == -INFINITY ? 0.0 : exp(p[s] - m);
        l += p[s];
    }
    for (int64_t s = 0; s < N; ++s) p[s] /= l;
    if (lse) *lse = m + log(l);
}

int oracle_forward_neighborhood_f64(const double *q, const double *k, const double *v, int64_t B, int64_t H,
                                    int64_t N, int64_t D, int64_t text_len, int64_t R, int64_t C, int64_t kh,
                                    int64_t kw, int64_t sh, int64_t sw, double scale, double *O, double *LSE)
{
    if (!q || !k || !v || !O || !LSE || B <= 0 || H <= 0 || D <= 0 || !na_check(N, text_len, R, C, kh, kw, sh, sw))
        return OR_EINVAL;
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        if (!p) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t row = 0; row < B * H * N; ++row) {
                const int64_t bh = row / N, t = row % N;
                na_row_probs(q, k, N, D, bh, t, &g, scale, p, &LSE[row]);
                for (int64_t d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t s = 0; s < N; ++s)
                        if (p[s] != 0.0) acc += p[s] * v[(bh * N + s) * D + d];
                    O[row * D + d] = acc;
                }
            }
        }
        free(p);
    }
    return rc;
}

/* The same forward for the flat query rows rows[0..nrows) ((b*H + h)*N + t)
 * only: O [nrows][D], LSE [nrows]. */
int oracle_forward_neighborhood_f64_rows(const double *q, const double *k, const double *v, int64_t B, int64_t H,
                                         int64_t N, int64_t D, int64_t text_len, int64_t R, int64_t C, int64_t kh,
                                         int64_t kw, int64_t sh, int64_t sw, double scale, const int64_t *rows,
                                         int64_t nrows, double *O, double *LSE)
{
    if (!q || !k || !v || !O || !LSE || !rows || nrows < 0 || B <= 0 || H <= 0 || D <= 0 ||
        !na_check(N, text_len, R, C, kh, kw, sh, sw))
        return OR_EINVAL;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= B * H * N) return OR_EINVAL;
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        if (!p) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < nrows; ++i) {
                const int64_t bh = rows[i] / N, t = rows[i] % N;
                na_row_probs(q, k, N, D, bh, t, &g, scale, p, &LSE[i]);
                for (int64_t d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t s = 0; s < N; ++s)
                        if (p[s] != 0.0) acc += p[s] * v[(bh * N + s) * D + d];
                    O[i * D + d] = acc;
                }
            }
        }
        free(p);
    }
    return rc;
}

int oracle_backward_neighborhood_f64(const double *q, const double *k, const double *v, const double *dO, int64_t B,
                                     int64_t H, int64_t N, int64_t D, int64_t text_len, int64_t R, int64_t C,
                                     int64_t kh, int64_t kw, int64_t sh, int64_t sw, double scale, double *dQ,
                                     double *dK, double *dV)
{
    if (!q || !k || !v || !dO || !dQ || !dK || !dV || B <= 0 || H <= 0 || D <= 0 ||
        !na_check(N, text_len, R, C, kh, kw, sh, sw))
        return OR_EINVAL;
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        double *dp = malloc(sizeof(double) * N);
        if (!p || !dp) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
            /* one (b, h) per iteration: dK, dV of a head are touched by its rows only */
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * H; ++bh) {
                memset(dK + bh * N * D, 0, sizeof(double) * N * D);
                memset(dV + bh * N * D, 0, sizeof(double) * N * D);
                for (int64_t t = 0; t < N; ++t) {
                    double *dq = dQ + (bh * N + t) * D;
                    const double *go = dO + (bh * N + t) * D;
                    na_row_probs(q, k, N, D, bh, t, &g, scale, p, NULL);
                    double delta = 0.0;
                    for (int64_t s = 0; s < N; ++s) {
                        if (p[s] == 0.0) { dp[s] = 0.0; continue; }
                        double acc = 0.0;
                        for (int64_t d = 0; d < D; ++d) acc += go[d] * v[(bh * N + s) * D + d];
                        dp[s] = acc;
                        delta += p[s] * acc;
                    }
                    for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
                    for (int64_t s = 0; s < N; ++s) {
                        if (p[s] == 0.0) continue;
                        const double ds = p[s] * (dp[s] - delta);
                        for (int64_t d = 0; d < D; ++d) {
                            dV[(bh * N + s) * D + d] += p[s] * go[d];
                            dq[d] += scale * ds * k[(bh * N + s) * D + d];
                            dK[(bh * N + s) * D + d] += scale * ds * q[(bh * N + t) * D + d];
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
    }
    return rc;
}

/* dQ of selected query rows (flat indices into [B*H*N], natural order) of
 * the neighbourhood backward: the same arithmetic as
 * oracle_backward_neighborhood_f64 restricted to those rows. */
int oracle_backward_neighborhood_dq_rows(const double *q, const double *k, const double *v, const double *dO,
                                         int64_t B, int64_t H, int64_t N, int64_t D, int64_t text_len, int64_t R,
                                         int64_t C, int64_t kh, int64_t kw, int64_t sh, int64_t sw, double scale,
                                         const int64_t *rows, int64_t n_rows, double *dQ)
{
    if (!q || !k || !v || !dO || !rows || !dQ || B <= 0 || H <= 0 || D <= 0 ||
        !na_check(N, text_len, R, C, kh, kw, sh, sw))
        return OR_EINVAL;
    for (int64_t x = 0; x < n_rows; ++x)
        if (rows[x] < 0 || rows[x] >= B * H * N) return OR_EINVAL;
    const na_geom g = {text_len, R, C, kh, kw, sh, sw};
    int rc = OR_OK;
#pragma omp parallel
    {
        double *p = malloc(sizeof(double) * N);
        double *dp = malloc(sizeof(double) * N);
        if (!p || !dp) {
#pragma omp atomic write
            rc = OR_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t x = 0; x < n_rows; ++x) {
                const int64_t bh = rows[x] / N, t = rows[x] % N;
                double *dq = dQ + x * D;
                const double *go = dO + (bh * N + t) * D;
                na_row_probs(q, k, N, D, bh, t, &g, scale, p, NULL);
                double delta = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (p[s] == 0.0) { dp[s] = 0.0; continue; }
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += go[d] * v[(bh * N + s) * D + d];
                    dp[s] = acc;
                    delta += p[s] * acc;
                }
                for (int64_t d = 0; d < D; ++d) dq[d] = 0.0;
                for (int64_t s = 0; s < N; ++s) {
                    if (p[s] == 0.0) continue;
                    const double ds = p[s] * (dp[s] - delta);
                    for (int64_t d = 0; d < D; ++d) dq[d] += scale * ds * k[(bh * N + s) * D + d];
                }
            }
        }
        free(p);
        free(dp);
    }
    return rc;
}
