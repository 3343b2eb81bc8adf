/*
 * sol_oracle.c -- plain fp64 CPU oracle of the Sol-Attn forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the HIP library is
 * tested against, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the pages this follows; citations name the page and its equation):
 *   [VE]  "Sol-Attn" visual paper explainer (mxino.github.io): "The complete
 *         idea in one pass", Eq. (4), Eq. (5), Eq. (9), Eq. (10), Eq. (11),
 *         "Key consequence".
 *   [ABS] Sol-Attn paper abstract (Hugging Face papers page).
 *   [P1]  Sol-Attn explainer (papers.ananclaw.com), "Attention(Q,K,V)" formula.
 *
 * Notation: H heads, L tokens, head dim d, block size B, N = ceil(L/B) blocks,
 * n_j = valid tokens of block j (B except for a ragged last block),
 * c = 1/sqrt(d).  Tensors are [H][L][d] row-major float (the exact values the
 * GPU received, bf16 values widened losslessly to float); all arithmetic here
 * is double.
 *
 * Every function is a direct, unblocked transcription of one step of the
 * method.  OpenMP only distributes independent (head, block) or (head, row)
 * items; each output element is computed by one thread in a fixed order, so
 * results are deterministic.
 *
 * Parity status: every function below is pinned by tests/test_oracle_pins.py
 * (closed forms, invariants, special cases reducing to textbook attention,
 * brute force on tiny inputs, the pages' Gaussian density example).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

static int64_t nblk(int L, int B) { return ((int64_t)L + B - 1) / B; }

/* Number of valid tokens in block j (the last block may be ragged). */
static int blk_len(int L, int B, int64_t j)
{
    int64_t lo = j * (int64_t)B;
    int64_t hi = lo + B;
    if (hi > L) hi = L;
    return (int)(hi - lo);
}

static int bad_shape(int H, int L, int d, int B)
{
    return H < 1 || L < 1 || d < 1 || B < 1;
}

/*
 * Step 1 -- pooling.  [VE] "Pool Q, K and V into blocks": the pooled query
 * and key of a block are the mean of its token vectors (Eq. (5) legend: "mean
 * query vector", "mean key vector"); the pooled value is the SUM of its token
 * values (Eq. (10) legend: "summed values").  Means run over the n_j valid
 * tokens of the block.
 *
 * Outputs are [H][N][d] doubles.
 */
int sol_oracle_pool(const float* q, const float* k, const float* v,
                    int H, int L, int d, int B,
                    double* qbar, double* kbar, double* vsum)
{
    if (bad_shape(H, L, d, B) || !q || !k || !v || !qbar || !kbar || !vsum)
        return ORACLE_EINVAL;
    const int64_t N = nblk(L, B);
#pragma omp parallel for collapse(2) schedule(static)
    for (int h = 0; h < H; ++h) {
        for (int64_t j = 0; j < N; ++j) {
            const int n = blk_len(L, B, j);
            const int64_t t0 = j * (int64_t)B;
            double* qb = qbar + ((int64_t)h * N + j) * d;
            double* kb = kbar + ((int64_t)h * N + j) * d;
            double* vs = vsum + ((int64_t)h * N + j) * d;
            for (int c = 0; c < d; ++c) {
                double sq = 0.0, sk = 0.0, sv = 0.0;
                for (int t = 0; t < n; ++t) {
                    const int64_t off = ((int64_t)h * L + t0 + t) * d + c;
                    sq += (double)q[off];
                    sk += (double)k[off];
                    sv += (double)v[off];
                }
                qb[c] = sq / (double)n;
                kb[c] = sk / (double)n;
                vs[c] = sv;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Step 2 -- proxy scores, threshold statistics, threshold and selected set,
 * for every (head h, query block i).
 *
 *   proxy      s_ij  = c * qbar_i . kbar_j      ([VE] Eq. (11), right-hand
 *              side; the 1/sqrt(d) scale of [P1]'s attention formula applies
 *              to every logit)
 *   statistics mu_i  = (1/N) sum_j s_ij,  sigma_i^2 = (1/N) sum_j (s_ij-mu_i)^2
 *              (population moments over all N key blocks, [VE] Eq. (5))
 *   threshold  tau_i = mu_i + beta * sigma_i                ([VE] Eq. (4))
 *   selection  S_i   = { j : s_ij > tau_i }  (strict)       ([VE] Eq. (4))
 *
 * beta = -inf selects every block and beta = +inf selects none; both are
 * taken literally (tau = -inf / +inf) so that sigma = 0 never produces
 * inf * 0.
 *
 * Outputs: shat [H][N][N] (may be NULL), mu/sigma/tau [H][N] (each may be
 * NULL), sel [H][N][N] bytes 0/1 (may be NULL), kept [H][N] (may be NULL).
 */
int sol_oracle_route(const double* qbar, const double* kbar,
                     int H, int N, int d, double beta,
                     double* shat, double* mu, double* sigma, double* tau,
                     uint8_t* sel, int32_t* kept)
{
    if (H < 1 || N < 1 || d < 1 || !qbar || !kbar || isnan(beta))
        return ORACLE_EINVAL;
    const double c = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)N);
        if (!row) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for collapse(2) schedule(static)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < N; ++i) {
                if (!row) continue;
                const double* qi = qbar + ((int64_t)h * N + i) * d;
                for (int j = 0; j < N; ++j) {
                    const double* kj = kbar + ((int64_t)h * N + j) * d;
                    double s = 0.0;
                    for (int x = 0; x < d; ++x) s += qi[x] * kj[x];
                    row[j] = c * s;
                }
                /* a constant row's mean is its common value and its variance
                   is 0 (Eq. (5) with every s_ij equal); a sum of N equal fp64
                   terms divided by N need not give the value back, so such
                   a row takes these exact statistics directly */
                int flat = 1;
                for (int j = 1; j < N; ++j) flat &= row[j] == row[0];
                double m = 0.0, var = 0.0;
                if (flat) {
                    m = row[0];
                } else {
                    for (int j = 0; j < N; ++j) m += row[j];
                    m /= (double)N;
                    for (int j = 0; j < N; ++j) var += (row[j] - m) * (row[j] - m);
                    var /= (double)N;
                }
                const double sg = sqrt(var > 0.0 ? var : 0.0);
                double t;
                if (isinf(beta)) t = beta; /* -inf: keep all, +inf: keep none */
                else t = m + beta * sg;
                int cnt = 0;
                const int64_t base = ((int64_t)h * N + i) * (int64_t)N;
                for (int j = 0; j < N; ++j) {
                    const int s_in = row[j] > t;
                    cnt += s_in;
                    if (sel) sel[base + j] = (uint8_t)s_in;
                    if (shat) shat[base + j] = row[j];
                }
                const int64_t hi_idx = (int64_t)h * N + i;
                if (mu) mu[hi_idx] = m;
                if (sigma) sigma[hi_idx] = sg;
                if (tau) tau[hi_idx] = t;
                if (kept) kept[hi_idx] = cnt;
            }
        }
        free(row);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Eq. (5) moment form of the threshold statistics ([VE] Eq. (5)): per head,
 * the mean pooled key m_K = (1/N) sum_j kbar_j and the second moment
 * C = (1/N) sum_j kbar_j^T kbar_j (d x d); then, with the proxy scale c,
 *   mu_i = c * qbar_i m_K^T,   sigma_i^2 = c^2 * qbar_i C qbar_i^T - mu_i^2.
 * A second, independent route to the statistics of sol_oracle_route (the
 * pages call it the efficient form); used as a pin, not by the merge.
 */
int sol_oracle_moments(const double* qbar, const double* kbar,
                       int H, int N, int d, double* mu, double* sigma2)
{
    if (H < 1 || N < 1 || d < 1 || !qbar || !kbar || !mu || !sigma2)
        return ORACLE_EINVAL;
    const double c = 1.0 / sqrt((double)d);
    double* mk = (double*)malloc(sizeof(double) * (size_t)d);
    double* C = (double*)malloc(sizeof(double) * (size_t)d * (size_t)d);
    if (!mk || !C) { free(mk); free(C); return ORACLE_ENOMEM; }
    for (int h = 0; h < H; ++h) {
        const double* kh = kbar + (int64_t)h * N * d;
        for (int a = 0; a < d; ++a) {
            double s = 0.0;
            for (int j = 0; j < N; ++j) s += kh[(int64_t)j * d + a];
            mk[a] = s / (double)N;
        }
#pragma omp parallel for schedule(static)
        for (int a = 0; a < d; ++a) {
            for (int b = 0; b < d; ++b) {
                double s = 0.0;
                for (int j = 0; j < N; ++j)
                    s += kh[(int64_t)j * d + a] * kh[(int64_t)j * d + b];
                C[(int64_t)a * d + b] = s / (double)N;
            }
        }
#pragma omp parallel for schedule(static)
        for (int i = 0; i < N; ++i) {
            const double* qi = qbar + ((int64_t)h * N + i) * d;
            double m = 0.0;
            for (int a = 0; a < d; ++a) m += qi[a] * mk[a];
            double quad = 0.0;
            for (int a = 0; a < d; ++a) {
                double r = 0.0;
                for (int b = 0; b < d; ++b) r += C[(int64_t)a * d + b] * qi[b];
                quad += qi[a] * r;
            }
            mu[(int64_t)h * N + i] = c * m;
            sigma2[(int64_t)h * N + i] = c * c * quad - (c * m) * (c * m);
        }
    }
    free(mk);
    free(C);
    return ORACLE_OK;
}

/*
 * Fixed-budget comparator ([ABS]: the routing the abstract contrasts with,
 * one share of key blocks for every query block, ranked by proxy score):
 * every query block keeps the
 * k key blocks with the largest proxy scores s_ij = c * qbar_i . kbar_j (the
 * same proxy as sol_oracle_route), k the same for every (h, i).  Ties in the
 * score go to the lower block index (the pages do not say).
 *
 * Outputs: shat [H][N][N] (may be NULL), kth [H][N] = the k-th largest score
 * (+inf when k = 0; may be NULL), sel [H][N][N] bytes 0/1 (may be NULL),
 * kept [H][N] = k (may be NULL).  0 <= k <= N.
 */
typedef struct { double s; int j; } score_ix;

static int by_score_then_index(const void* a, const void* b)
{
    const score_ix* x = (const score_ix*)a;
    const score_ix* y = (const score_ix*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

int sol_oracle_route_topk(const double* qbar, const double* kbar, int H, int N, int d, int k,
                          double* shat, double* kth, uint8_t* sel, int32_t* kept)
{
    if (H < 1 || N < 1 || d < 1 || !qbar || !kbar || k < 0 || k > N)
        return ORACLE_EINVAL;
    const double c = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        score_ix* row = (score_ix*)malloc(sizeof(score_ix) * (size_t)N);
        if (!row) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for collapse(2) schedule(static)
        for (int h = 0; h < H; ++h) {
            for (int i = 0; i < N; ++i) {
                if (!row) continue;
                const double* qi = qbar + ((int64_t)h * N + i) * d;
                const int64_t base = ((int64_t)h * N + i) * (int64_t)N;
                for (int j = 0; j < N; ++j) {
                    const double* kj = kbar + ((int64_t)h * N + j) * d;
                    double s = 0.0;
                    for (int x = 0; x < d; ++x) s += qi[x] * kj[x];
                    row[j].s = c * s;
                    row[j].j = j;
                    if (shat) shat[base + j] = c * s;
                }
                qsort(row, (size_t)N, sizeof(score_ix), by_score_then_index);
                if (sel) {
                    for (int j = 0; j < N; ++j) sel[base + j] = 0;
                    for (int x = 0; x < k; ++x) sel[base + row[x].j] = 1;
                }
                const int64_t hi_idx = (int64_t)h * N + i;
                if (kth) kth[hi_idx] = k > 0 ? row[k - 1].s : INFINITY;
                if (kept) kept[hi_idx] = k;
            }
        }
        free(row);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/*
 * Step 3 -- the merge: exact attention over selected blocks and the
 * approximate correction over unselected blocks, in one softmax.
 *
 * For a query token r of query block i (head h), per [VE] Eq. (9) and
 * Eq. (10), read row by row (Q_i there is the query-token matrix, so the
 * approximate logit is per query token, not the block proxy):
 *   exact logits        a_rt = c * q_r . k_t      for t in a block j of S_i
 *   approximate logits  g_rj = c * q_r . kbar_j   for j in U_i (unselected)
 *   D_r = sum_{j in U_i} n_j exp(g_rj) + sum_{j in S_i} sum_{t in j} exp(a_rt)
 *   N_r = sum_{j in U_i} exp(g_rj) vsum_j + sum_{j in S_i} sum_{t in j} exp(a_rt) v_t
 *   out_r = N_r / D_r                     ([VE] "Key consequence")
 * The factor written B in Eq. (9) is the number of tokens the block stands
 * for, n_j, which differs from B only for a ragged last block.  All
 * exponentials are taken relative to the row maximum M_r of every logit
 * above, which cancels in N_r / D_r.
 *
 * sel is [H][N][N] bytes (1 = exact).  rows lists (h, r) pairs (n_rows of
 * them); rows == NULL means every (h, r) in order, and out is then
 * [H][L][d]; otherwise out is [n_rows][d].
 *
 * drop_approx != 0 gives the keep-or-drop scheme the pages contrast with
 * ([VE] "Place it among nearby methods", ordinary block sparse attention:
 * every unselected block contributes zero; [ABS] keep-or-drop): the
 * terms over U_i are left out of both sums, and a row whose S_i is empty
 * (D_r = 0) is set to zero (the pages do not say).
 */
int sol_oracle_merge_ex(const float* q, const float* k, const float* v,
                        const double* kbar, const double* vsum,
                        int H, int L, int d, int B, const uint8_t* sel, int drop_approx,
                        int64_t n_rows, const int32_t* rows, double* out)
{
    if (bad_shape(H, L, d, B) || !q || !k || !v || !kbar || !vsum || !sel || !out)
        return ORACLE_EINVAL;
    const int64_t N = nblk(L, B);
    const int64_t total = rows ? n_rows : (int64_t)H * L;
    if (rows) {
        for (int64_t x = 0; x < n_rows; ++x)
            if (rows[2 * x] < 0 || rows[2 * x] >= H || rows[2 * x + 1] < 0 || rows[2 * x + 1] >= L)
                return ORACLE_EINVAL;
    }
    const double c = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        /* per-thread logit buffers: one per token (exact) and per block (approx) */
        double* a_tok = (double*)malloc(sizeof(double) * (size_t)L);
        double* g_blk = (double*)malloc(sizeof(double) * (size_t)N);
        double* num = (double*)malloc(sizeof(double) * (size_t)d);
        if (!a_tok || !g_blk || !num) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t x = 0; x < total; ++x) {
            if (!a_tok || !g_blk || !num) continue;
            const int h = rows ? rows[2 * x] : (int)(x / L);
            const int r = rows ? rows[2 * x + 1] : (int)(x % L);
            const int64_t i = r / B;
            const float* qr = q + ((int64_t)h * L + r) * d;
            const uint8_t* srow = sel + ((int64_t)h * N + i) * N;
            double M = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                const int n = blk_len(L, B, j);
                if (srow[j]) {
                    for (int t = 0; t < n; ++t) {
                        const int64_t tok = j * (int64_t)B + t;
                        const float* kt = k + ((int64_t)h * L + tok) * d;
                        double s = 0.0;
                        for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kt[e];
                        a_tok[tok] = c * s;
                        if (a_tok[tok] > M) M = a_tok[tok];
                    }
                } else if (!drop_approx) {
                    const double* kb = kbar + ((int64_t)h * N + j) * d;
                    double s = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * kb[e];
                    g_blk[j] = c * s;
                    if (g_blk[j] > M) M = g_blk[j];
                }
            }
            double D = 0.0;
            for (int e = 0; e < d; ++e) num[e] = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                const int n = blk_len(L, B, j);
                if (srow[j]) {
                    /* exact term of Eq. (9) / Eq. (10) */
                    for (int t = 0; t < n; ++t) {
                        const int64_t tok = j * (int64_t)B + t;
                        const double w = exp(a_tok[tok] - M);
                        const float* vt = v + ((int64_t)h * L + tok) * d;
                        D += w;
                        for (int e = 0; e < d; ++e) num[e] += w * (double)vt[e];
                    }
                } else if (!drop_approx) {
                    /* approximate term of Eq. (9) / Eq. (10) */
                    const double w = exp(g_blk[j] - M);
                    const double* vs = vsum + ((int64_t)h * N + j) * d;
                    D += (double)n * w;
                    for (int e = 0; e < d; ++e) num[e] += w * vs[e];
                }
            }
            double* o = out + x * d;
            for (int e = 0; e < d; ++e) o[e] = D > 0.0 ? num[e] / D : 0.0;
        }
        free(a_tok);
        free(g_blk);
        free(num);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

int sol_oracle_merge(const float* q, const float* k, const float* v,
                     const double* kbar, const double* vsum,
                     int H, int L, int d, int B, const uint8_t* sel,
                     int64_t n_rows, const int32_t* rows, double* out)
{
    return sol_oracle_merge_ex(q, k, v, kbar, vsum, H, L, d, B, sel, 0, n_rows, rows, out);
}

/*
 * Textbook dense softmax attention, softmax(Q K^T / sqrt(d)) V ([P1]
 * "Attention(Q, K, V)"), for the listed (h, r) rows.  The speedup baseline's
 * reference and the beta = -inf special case of the merge.
 */
int sol_oracle_dense(const float* q, const float* k, const float* v,
                     int H, int L, int d,
                     int64_t n_rows, const int32_t* rows, double* out)
{
    if (H < 1 || L < 1 || d < 1 || !q || !k || !v || !out) return ORACLE_EINVAL;
    const int64_t total = rows ? n_rows : (int64_t)H * L;
    if (rows) {
        for (int64_t x = 0; x < n_rows; ++x)
            if (rows[2 * x] < 0 || rows[2 * x] >= H || rows[2 * x + 1] < 0 || rows[2 * x + 1] >= L)
                return ORACLE_EINVAL;
    }
    const double c = 1.0 / sqrt((double)d);
    int err = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double* num = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s || !num) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t x = 0; x < total; ++x) {
            if (!s || !num) continue;
            const int h = rows ? rows[2 * x] : (int)(x / L);
            const int r = rows ? rows[2 * x + 1] : (int)(x % L);
            const float* qr = q + ((int64_t)h * L + r) * d;
            double M = -INFINITY;
            for (int t = 0; t < L; ++t) {
                const float* kt = k + ((int64_t)h * L + t) * d;
                double acc = 0.0;
                for (int e = 0; e < d; ++e) acc += (double)qr[e] * (double)kt[e];
                s[t] = c * acc;
                if (s[t] > M) M = s[t];
            }
            double D = 0.0;
            for (int e = 0; e < d; ++e) num[e] = 0.0;
            for (int t = 0; t < L; ++t) {
                const double w = exp(s[t] - M);
                const float* vt = v + ((int64_t)h * L + t) * d;
                D += w;
                for (int e = 0; e < d; ++e) num[e] += w * (double)vt[e];
            }
            double* o = out + x * d;
            for (int e = 0; e < d; ++e) o[e] = num[e] / D;
        }
        free(s);
        free(num);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

int sol_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
