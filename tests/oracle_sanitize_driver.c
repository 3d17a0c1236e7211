/*
 * Driver for the sanitizer run of the oracle's C routines (built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py together with
 * oracle/nufft_oracle.c).  It calls every exported routine on small inputs,
 * including coordinates in the folded ranges [pi, 3 pi) and [-3 pi, -pi),
 * grids smaller than the kernel (stencils that wrap more than once), empty
 * point sets and rejected points, and checks that the parallel spreading and
 * interpolation forms equal the serial ones exactly.  Exit status 0 = all
 * checks passed; the sanitizers abort the process on any memory or
 * undefined-behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_spread(int d, const int64_t* n, int w, double beta, int64_t M, const double* const* X,
                  const double* c, double* b);
int oracle_interp(int d, const int64_t* n, int w, double beta, int64_t M, const double* const* X,
                  const double* b, double* c);
int oracle_spread_par(int d, const int64_t* n, int w, double beta, int64_t M, const double* const* X,
                      const double* c, double* b, int threads);
int oracle_interp_par(int d, const int64_t* n, int w, double beta, int64_t M, const double* const* X,
                      const double* b, double* c, int threads);
int oracle_binsort(int d, const int64_t* n, const int64_t* m, int64_t M, const double* const* X,
                   int64_t* bin, int64_t* counts, int64_t* perm);
int64_t oracle_subproblems(int64_t nbins, const int64_t* counts, int64_t cap, int64_t* out);
int oracle_direct_type1(int d, const int64_t* N, int64_t M, const double* const* X, const double* c,
                        int64_t nsel, const int64_t* sel, double* f);
int oracle_direct_type2(int d, const int64_t* N, int64_t M, const double* const* X, const double* f,
                        int64_t nsel, const int64_t* sel, double* c);
int oracle_type1_bhat_at(int d, const int64_t* n, int w, double beta, int64_t M, const double* const* X,
                         const double* c, int64_t nk, const int64_t* kvec, double* bhat);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(double lo, double hi)
{
    /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return lo + (hi - lo) * ((double)(z >> 11) / 9007199254740992.0);
}

static int failures = 0;
#define CHECK(cond, what)                                              \
    do {                                                               \
        if (!(cond)) { fprintf(stderr, "FAIL: %s\n", what); ++failures; } \
    } while (0)

static void run_case(int d, const int64_t* n, int w, int64_t M)
{
    const double PI = 3.141592653589793;
    double* X[3] = {NULL, NULL, NULL};
    for (int i = 0; i < d; ++i) {
        X[i] = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
        for (int64_t j = 0; j < M; ++j) X[i][j] = uniform(-3 * PI, 3 * PI);
    }
    if (M > 2) {
        X[0][0] = -3 * PI + 1e-12;
        X[0][1] = nextafter(-PI, -4.0);
        X[0][2] = 3 * PI - 1e-9;
    }
    int64_t cells = 1;
    for (int i = 0; i < d; ++i) cells *= n[i];
    double* c = (double*)malloc(sizeof(double) * 2 * (size_t)(M > 0 ? M : 1));
    for (int64_t j = 0; j < 2 * M; ++j) c[j] = uniform(-1, 1);
    double* b1 = (double*)calloc(2 * (size_t)cells, sizeof(double));
    double* b2 = (double*)calloc(2 * (size_t)cells, sizeof(double));
    const double beta = 2.30 * w;
    const double* const* XC = (const double* const*)X;
    CHECK(oracle_spread(d, n, w, beta, M, XC, c, b1) == 0, "spread");
    CHECK(oracle_spread_par(d, n, w, beta, M, XC, c, b2, 3) == 0, "spread_par");
    CHECK(memcmp(b1, b2, sizeof(double) * 2 * (size_t)cells) == 0, "spread_par equals spread");
    double* c1 = (double*)malloc(sizeof(double) * 2 * (size_t)(M > 0 ? M : 1));
    double* c2 = (double*)malloc(sizeof(double) * 2 * (size_t)(M > 0 ? M : 1));
    CHECK(oracle_interp(d, n, w, beta, M, XC, b1, c1) == 0, "interp");
    CHECK(oracle_interp_par(d, n, w, beta, M, XC, b1, c2, 2) == 0, "interp_par");
    CHECK(M == 0 || memcmp(c1, c2, sizeof(double) * 2 * (size_t)M) == 0, "interp_par equals interp");

    int64_t m[3] = {1, 1, 1}, nb = 1;
    for (int i = 0; i < d; ++i) {
        m[i] = n[i] > 3 ? n[i] / 3 : 1;
        nb *= (n[i] + m[i] - 1) / m[i];
    }
    int64_t* bin = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    int64_t* counts = (int64_t*)malloc(sizeof(int64_t) * (size_t)nb);
    CHECK(oracle_binsort(d, n, m, M, XC, bin, counts, perm) == 0, "binsort");
    int64_t tot = 0;
    for (int64_t k = 0; k < nb; ++k) tot += counts[k];
    CHECK(tot == M, "counts sum to M");
    for (int64_t j = 1; j < M; ++j)
        CHECK(bin[perm[j - 1]] < bin[perm[j]] || (bin[perm[j - 1]] == bin[perm[j]] && perm[j - 1] < perm[j]),
              "perm is the stable sort of the bins");
    int64_t ns = oracle_subproblems(nb, counts, 5, NULL);
    int64_t* sub = (int64_t*)malloc(sizeof(int64_t) * 3 * (size_t)(ns > 0 ? ns : 1));
    CHECK(oracle_subproblems(nb, counts, 5, sub) == ns, "subproblems");

    int64_t N[3] = {1, 1, 1}, modes = 1;
    for (int i = 0; i < d; ++i) {
        N[i] = n[i] / 2 > 0 ? n[i] / 2 : 1;
        modes *= N[i];
    }
    double* f = (double*)malloc(sizeof(double) * 2 * (size_t)modes);
    CHECK(oracle_direct_type1(d, N, M, XC, c, 0, NULL, f) == 0, "direct type 1");
    double* cc = (double*)malloc(sizeof(double) * 2 * (size_t)(M > 0 ? M : 1));
    CHECK(oracle_direct_type2(d, N, M, XC, f, 0, NULL, cc) == 0, "direct type 2");
    int64_t kv[6] = {0, 1, -1, 2, 3, -2};
    double bh[4];
    CHECK(oracle_type1_bhat_at(d, n, w, beta, M, XC, c, 2, kv, bh) == 0, "type1_bhat_at");

    /* a rejected point (outside [-3 pi, 3 pi)) */
    if (M > 0) {
        double keep = X[0][M - 1];
        X[0][M - 1] = 20.0;
        CHECK(oracle_spread_par(d, n, w, beta, M, XC, c, b2, 2) == -2, "bad point rejected (spread_par)");
        CHECK(oracle_binsort(d, n, m, M, XC, bin, counts, perm) == -2, "bad point rejected (binsort)");
        X[0][M - 1] = keep;
    }
    free(cc); free(f); free(sub); free(counts); free(perm); free(bin);
    free(c2); free(c1); free(b2); free(b1); free(c);
    for (int i = 0; i < d; ++i) free(X[i]);
}

int main(void)
{
    const int64_t n1a[1] = {40}, n1b[1] = {5};
    const int64_t n2a[2] = {24, 18}, n2b[2] = {4, 6};
    const int64_t n3a[3] = {12, 10, 8}, n3b[3] = {4, 3, 5};
    run_case(1, n1a, 7, 300);
    run_case(1, n1b, 9, 50);
    run_case(2, n2a, 6, 400);
    run_case(2, n2b, 13, 60);
    run_case(3, n3a, 5, 300);
    run_case(3, n3b, 10, 40);
    run_case(3, n3a, 4, 0);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all checks passed\n");
    return 0;
}
