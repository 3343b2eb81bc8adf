/*
 * oracle_sanitize_driver.c -- exercises every function of the fp64 oracle
 * (oracle/sol_oracle.c) on small, ragged and degenerate shapes, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitized.py compiles and runs it).  Memory errors,
 * leaks and undefined behaviour abort the run; a few invariants of the
 * method are checked on the way:
 *   - rows of V = 1 give out = 1 for every selection (the merged softmax
 *     weights sum to one: "Sol-Attn" visual explainer, Eq. (9), Eq. (10));
 *   - beta = -inf (every block exact) equals dense softmax attention;
 *   - the fixed budget keeps exactly k blocks per row;
 *   - invalid arguments are rejected with a nonzero code.
 * Prints "OK" and returns 0 when everything passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int sol_oracle_pool(const float* q, const float* k, const float* v, int H, int L, int d, int B,
                    double* qbar, double* kbar, double* vsum);
int sol_oracle_route(const double* qbar, const double* kbar, int H, int N, int d, double beta,
                     double* shat, double* mu, double* sigma, double* tau, uint8_t* sel,
                     int32_t* kept);
int sol_oracle_moments(const double* qbar, const double* kbar, int H, int N, int d, double* mu,
                       double* sigma2);
int sol_oracle_route_topk(const double* qbar, const double* kbar, int H, int N, int d, int k,
                          double* shat, double* kth, uint8_t* sel, int32_t* kept);
int sol_oracle_merge_ex(const float* q, const float* k, const float* v, const double* kbar,
                        const double* vsum, int H, int L, int d, int B, const uint8_t* sel,
                        int drop_approx, int64_t n_rows, const int32_t* rows, double* out);
int sol_oracle_merge(const float* q, const float* k, const float* v, const double* kbar,
                     const double* vsum, int H, int L, int d, int B, const uint8_t* sel,
                     int64_t n_rows, const int32_t* rows, double* out);
int sol_oracle_dense(const float* q, const float* k, const float* v, int H, int L, int d,
                     int64_t n_rows, const int32_t* rows, double* out);
int sol_oracle_num_threads(void);

static int failures = 0;
#define CHECK(cond, ...)                         \
    do {                                         \
        if (!(cond)) {                           \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");               \
            ++failures;                          \
        }                                        \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float urand(void) {  /* uniform in [-1, 1) from a 64-bit LCG */
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(rng >> 11) / 4503599627370496.0 - 1.0);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void run_shape(int H, int L, int d, int B) {
    const int N = (L + B - 1) / B;
    const size_t nt = (size_t)H * L * d, np = (size_t)H * N * d, nn = (size_t)H * N * N;
    float* q = xmalloc(sizeof(float) * nt);
    float* k = xmalloc(sizeof(float) * nt);
    float* v = xmalloc(sizeof(float) * nt);
    float* ones = xmalloc(sizeof(float) * nt);
    for (size_t x = 0; x < nt; ++x) {
        q[x] = 2.0f * urand();
        k[x] = 2.0f * urand();
        v[x] = urand();
        ones[x] = 1.0f;
    }
    double* qbar = xmalloc(sizeof(double) * np);
    double* kbar = xmalloc(sizeof(double) * np);
    double* vsum = xmalloc(sizeof(double) * np);
    double* vsum1 = xmalloc(sizeof(double) * np);
    double* s1 = xmalloc(sizeof(double) * np);
    double* s2 = xmalloc(sizeof(double) * np);
    CHECK(sol_oracle_pool(q, k, v, H, L, d, B, qbar, kbar, vsum) == 0, "pool H=%d L=%d", H, L);
    CHECK(sol_oracle_pool(q, k, ones, H, L, d, B, s1, s2, vsum1) == 0, "pool V=1");

    double* shat = xmalloc(sizeof(double) * nn);
    double* mu = xmalloc(sizeof(double) * H * N);
    double* sg = xmalloc(sizeof(double) * H * N);
    double* tau = xmalloc(sizeof(double) * H * N);
    uint8_t* sel = xmalloc(nn);
    int32_t* kept = xmalloc(sizeof(int32_t) * H * N);
    double* out = xmalloc(sizeof(double) * (nt + 3 * (size_t)d));  /* all rows, or 3 listed rows */
    double* ref = xmalloc(sizeof(double) * nt);
    const double betas[4] = {-INFINITY, 0.0, 1.0, INFINITY};
    for (int b = 0; b < 4; ++b) {
        CHECK(sol_oracle_route(qbar, kbar, H, N, d, betas[b], shat, mu, sg, tau, sel, kept) == 0, "route");
        CHECK(sol_oracle_route(qbar, kbar, H, N, d, betas[b], NULL, NULL, NULL, NULL, sel, NULL) == 0,
              "route without optional outputs");
        for (int drop = 0; drop < 2; ++drop) {
            CHECK(sol_oracle_merge_ex(q, k, ones, kbar, vsum1, H, L, d, B, sel, drop, 0, NULL, out) == 0,
                  "merge_ex V=1");
            for (size_t x = 0; x < nt; ++x) {
                /* dropping leaves an empty row at 0; otherwise the weights sum to 1 */
                const int h = (int)(x / ((size_t)L * d)), r = (int)((x / d) % L);
                int any = 0;
                for (int j = 0; j < N; ++j) any |= sel[((size_t)h * N + r / B) * N + j];
                const double want = (drop && !any) ? 0.0 : 1.0;
                if (fabs(out[x] - want) > 1e-12) {
                    CHECK(0, "V=1 row weights: got %.17g want %.17g (drop=%d)", out[x], want, drop);
                    break;
                }
            }
        }
        CHECK(sol_oracle_merge(q, k, v, kbar, vsum, H, L, d, B, sel, 0, NULL, out) == 0, "merge");
        if (b == 0) {
            CHECK(sol_oracle_dense(q, k, v, H, L, d, 0, NULL, ref) == 0, "dense");
            double e = 0.0;
            for (size_t x = 0; x < nt; ++x) e = fmax(e, fabs(out[x] - ref[x]));
            CHECK(e <= 1e-12, "beta=-inf merge vs dense: %.3g", e);
        }
    }
    /* a few rows: first, last, and one in the middle of the last head */
    int32_t rows[6] = {0, 0, H - 1, L - 1, H - 1, L / 2};
    CHECK(sol_oracle_merge_ex(q, k, v, kbar, vsum, H, L, d, B, sel, 1, 3, rows, out) == 0, "merge rows");
    CHECK(sol_oracle_dense(q, k, v, H, L, d, 3, rows, out) == 0, "dense rows");
    CHECK(sol_oracle_moments(qbar, kbar, H, N, d, mu, sg) == 0, "moments");
    double* kth = xmalloc(sizeof(double) * H * N);
    const int ks[3] = {0, 1, N};
    for (int t = 0; t < 3; ++t) {
        CHECK(sol_oracle_route_topk(qbar, kbar, H, N, d, ks[t], shat, kth, sel, kept) == 0, "topk");
        for (int x = 0; x < H * N; ++x) CHECK(kept[x] == ks[t], "topk kept %d != %d", kept[x], ks[t]);
        CHECK(sol_oracle_route_topk(qbar, kbar, H, N, d, ks[t], NULL, NULL, sel, NULL) == 0, "topk sparse outputs");
    }
    /* invalid arguments */
    CHECK(sol_oracle_pool(NULL, k, v, H, L, d, B, qbar, kbar, vsum) != 0, "pool NULL");
    CHECK(sol_oracle_route(qbar, kbar, H, N, d, NAN, NULL, NULL, NULL, NULL, sel, NULL) != 0, "route NaN");
    CHECK(sol_oracle_route_topk(qbar, kbar, H, N, d, N + 1, NULL, NULL, sel, NULL) != 0, "topk k > N");
    CHECK(sol_oracle_merge_ex(q, k, v, kbar, vsum, 0, L, d, B, sel, 0, 0, NULL, out) != 0, "merge H=0");
    CHECK(sol_oracle_dense(q, k, v, H, 0, d, 0, NULL, out) != 0, "dense L=0");

    free(q); free(k); free(v); free(ones); free(qbar); free(kbar); free(vsum); free(vsum1);
    free(s1); free(s2); free(shat); free(mu); free(sg); free(tau); free(sel); free(kept); free(out);
    free(ref); free(kth);
}

int main(void) {
    CHECK(sol_oracle_num_threads() >= 1, "threads");
    run_shape(1, 1, 4, 4);     /* one token, one block */
    run_shape(2, 37, 8, 8);    /* ragged last block of 5 */
    run_shape(2, 64, 16, 64);  /* one full block */
    run_shape(3, 50, 4, 1);    /* B = 1 */
    run_shape(1, 130, 8, 32);  /* ragged last block of 2 */
    if (failures) {
        fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    printf("OK\n");
    return 0;
}
