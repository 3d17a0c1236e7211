/*
 * Plain CPU oracle for the 2D/3D type 1 and type 2 NUFFT (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source,
 * header, table or helper with the GPU library; the two agree only because
 * both follow the same published definitions:
 *
 *   "cuFINUFFT: a load-balanced GPU library for general-purpose nonuniform
 *    FFTs" (Shih, Wright, Anden, Blaschke, Barnett), Sec. I eqs. (1)-(3)
 *   (the exact sums), Sec. II eqs. (4)-(12) (ES kernel, spreading, FFT,
 *   correction, interpolation) and Sec. III-A (bins and the "inside a bin"
 *   rule).
 *
 * Everything is fp64, IEEE round-to-nearest, compiled without FP contraction
 * and without fast-math.  Loops are written in the order the equations state
 * them; nothing is blocked, fused or reordered for speed.  The only
 * parallelism (OpenMP) is over independent outputs of the exact sums, over
 * point ranges of the sampled type 1 evaluation (partial sums added in range
 * order), and in the parallel spreading / interpolation forms, which give the
 * serial forms' results bit for bit (see there); the bin-sort is serial.  Arrays of complex
 * numbers are interleaved (re, im).  Grids are stored with the first index
 * fastest: cell (l1, l2, l3) sits at l1 + n1*(l2 + n2*l3).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The double nearest pi. */
static const double PI_D = 3.141592653589793115997963468544185161590576171875;

#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_BAD_POINT (-2)

/*
 * Fine-grid coordinate of a point along one dimension.
 *
 * cuFINUFFT paper, Sec. III-A: a point is "inside" the bin holding
 * l = floor((x + pi)/h), h = 2 pi / n.  We use the same origin (grid cell l
 * at position l*h - pi) for spreading and interpolation as well, and fold the
 * sign change this causes into the correction factors.  The scaled coordinate
 * is t = (x + pi) * s with s = n / (2 pi), formed as two separately rounded
 * fp64 operations.  One periodic fold brings l into [0, n).
 */
static int grid_coord(double x, int64_t n, double s, double* t_out, int64_t* l_out)
{
    double t = (x + PI_D) * s;
    if (!(t == t)) return ORACLE_BAD_POINT;          /* NaN */
    double fl = floor(t);
    if (fl < -(double)n || fl >= 2.0 * (double)n) return ORACLE_BAD_POINT;
    int64_t l = (int64_t)fl;
    if (l >= n) { l -= n; t -= (double)n; }
    else if (l < 0) { l += n; t += (double)n; }
    *t_out = t;
    *l_out = l;
    return ORACLE_OK;
}

/* s_i = n_i / (2 pi), rounded once. */
double oracle_grid_scale(int64_t n) { return (double)n / (2.0 * PI_D); }

/* ES kernel, cuFINUFFT paper eq. (5): exp(beta (sqrt(1 - z^2) - 1)) on |z| <= 1, else 0. */
double oracle_es_kernel(double z, double beta)
{
    if (fabs(z) > 1.0) return 0.0;
    return exp(beta * (sqrt(1.0 - z * z) - 1.0));
}

static int64_t pmod(int64_t a, int64_t n)
{
    int64_t r = a % n;
    return r < 0 ? r + n : r;
}

/*
 * Kernel weights and cells of one point along one dimension.
 *
 * Eq. (8): psi(x) = phi_beta(x / alpha), alpha = w pi / n, periodised.  In grid
 * units the argument for cell l is z = (l - t) * 2 / w, so the support is the
 * w cells starting at l0 = ceil(t - w/2).  The cell index is taken mod n
 * (periodisation).
 */
static void stencil_1d(double t, int64_t n, int w, double beta, double* phi, int64_t* cell)
{
    double l0 = ceil(t - 0.5 * (double)w);
    for (int q = 0; q < w; ++q) {
        double z = ((l0 + (double)q) - t) * (2.0 / (double)w);
        phi[q] = oracle_es_kernel(z, beta);
        cell[q] = pmod((int64_t)l0 + q, n);
    }
}

/*
 * Type 1 step 1, spreading (eq. (7)):
 *   b_l = sum_j c_j psi_per(l h - pi - x_j)   for every fine cell l.
 * X[i] holds coordinate i of all M points; c and b are interleaved complex.
 * b must be zeroed by the caller (or hold a grid to accumulate into).
 */
int oracle_spread(int d, const int64_t* n, int w, double beta, int64_t M,
                  const double* const* X, const double* c, double* b)
{
    if (d < 1 || d > 3 || w < 1 || w > 32 || M < 0) return ORACLE_BAD_ARG;
    int64_t nn[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) nn[i] = n[i];
    double phi[3][32];
    int64_t cell[3][32];
    int wd[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) wd[i] = w;
    for (int64_t j = 0; j < M; ++j) {
        for (int i = 0; i < 3; ++i) { phi[i][0] = 1.0; cell[i][0] = 0; }
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l) != ORACLE_OK)
                return ORACLE_BAD_POINT;
            stencil_1d(t, nn[i], w, beta, phi[i], cell[i]);
        }
        double cre = c[2 * j], cim = c[2 * j + 1];
        for (int q3 = 0; q3 < wd[2]; ++q3)
            for (int q2 = 0; q2 < wd[1]; ++q2)
                for (int q1 = 0; q1 < wd[0]; ++q1) {
                    double k = phi[0][q1] * phi[1][q2] * phi[2][q3];
                    int64_t idx = cell[0][q1] + nn[0] * (cell[1][q2] + nn[1] * cell[2][q3]);
                    b[2 * idx] += cre * k;
                    b[2 * idx + 1] += cim * k;
                }
    }
    return ORACLE_OK;
}

/*
 * Type 2 step 3, interpolation (the sum after eq. (12)):
 *   c_j = sum_l b_l psi_per(l h - pi - x_j).
 */
int oracle_interp(int d, const int64_t* n, int w, double beta, int64_t M,
                  const double* const* X, const double* b, double* c)
{
    if (d < 1 || d > 3 || w < 1 || w > 32 || M < 0) return ORACLE_BAD_ARG;
    int64_t nn[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) nn[i] = n[i];
    double phi[3][32];
    int64_t cell[3][32];
    int wd[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) wd[i] = w;
    for (int64_t j = 0; j < M; ++j) {
        for (int i = 0; i < 3; ++i) { phi[i][0] = 1.0; cell[i][0] = 0; }
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l) != ORACLE_OK)
                return ORACLE_BAD_POINT;
            stencil_1d(t, nn[i], w, beta, phi[i], cell[i]);
        }
        double sre = 0.0, sim = 0.0;
        for (int q3 = 0; q3 < wd[2]; ++q3)
            for (int q2 = 0; q2 < wd[1]; ++q2)
                for (int q1 = 0; q1 < wd[0]; ++q1) {
                    double k = phi[0][q1] * phi[1][q2] * phi[2][q3];
                    int64_t idx = cell[0][q1] + nn[0] * (cell[1][q2] + nn[1] * cell[2][q3]);
                    sre += b[2 * idx] * k;
                    sim += b[2 * idx + 1] * k;
                }
        c[2 * j] = sre;
        c[2 * j + 1] = sim;
    }
    return ORACLE_OK;
}

/*
 * Parallel forms of the two steps above, for large inputs.  Both give exactly
 * the serial result, bit for bit, because every output is still summed over
 * the same terms in the same order:
 *  - spreading: the grid is cut along its slowest dimension into one slab per
 *    thread; each thread walks all points in index order and adds only the
 *    contributions whose cell lies in its own slab (so no two threads write a
 *    cell, and each cell receives its terms in the serial order);
 *  - interpolation: every point's sum is independent; threads take points.
 * threads <= 0 means all available threads.
 */
int oracle_spread_par(int d, const int64_t* n, int w, double beta, int64_t M,
                      const double* const* X, const double* c, double* b, int threads)
{
    if (d < 1 || d > 3 || w < 1 || w > 32 || M < 0) return ORACLE_BAD_ARG;
    int64_t nn[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) nn[i] = n[i];
    for (int64_t j = 0; j < M; ++j)
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l) != ORACLE_OK)
                return ORACLE_BAD_POINT;
        }
    int T = 1;
#ifdef _OPENMP
    T = threads > 0 ? threads : omp_get_max_threads();
#endif
    (void)threads;
    const int slow = d - 1;
    int wd[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) wd[i] = w;
#pragma omp parallel num_threads(T)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        const int64_t lo = nn[slow] * tid / T, hi = nn[slow] * (tid + 1) / T;
        double phi[3][32];
        int64_t cell[3][32];
        for (int64_t j = 0; j < M; ++j) {
            double ts; int64_t ls;
            grid_coord(X[slow][j], nn[slow], oracle_grid_scale(nn[slow]), &ts, &ls);
            /* does the support along the slow dimension meet this slab? */
            const int64_t l0 = (int64_t)ceil(ts - 0.5 * (double)w);
            int meets = 0;
            for (int q = 0; q < w && !meets; ++q) {
                const int64_t cq = pmod(l0 + q, nn[slow]);
                meets = (cq >= lo && cq < hi);
            }
            if (!meets) continue;
            for (int i = 0; i < 3; ++i) { phi[i][0] = 1.0; cell[i][0] = 0; }
            for (int i = 0; i < d; ++i) {
                double t; int64_t l;
                grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l);
                stencil_1d(t, nn[i], w, beta, phi[i], cell[i]);
            }
            double cre = c[2 * j], cim = c[2 * j + 1];
            for (int q3 = 0; q3 < wd[2]; ++q3)
                for (int q2 = 0; q2 < wd[1]; ++q2)
                    for (int q1 = 0; q1 < wd[0]; ++q1) {
                        const int64_t cs = (slow == 2) ? cell[2][q3] : (slow == 1) ? cell[1][q2] : cell[0][q1];
                        if (cs < lo || cs >= hi) continue;
                        double k = phi[0][q1] * phi[1][q2] * phi[2][q3];
                        int64_t idx = cell[0][q1] + nn[0] * (cell[1][q2] + nn[1] * cell[2][q3]);
                        b[2 * idx] += cre * k;
                        b[2 * idx + 1] += cim * k;
                    }
        }
    }
    return ORACLE_OK;
}

int oracle_interp_par(int d, const int64_t* n, int w, double beta, int64_t M,
                      const double* const* X, const double* b, double* c, int threads)
{
    if (d < 1 || d > 3 || w < 1 || w > 32 || M < 0) return ORACLE_BAD_ARG;
    int64_t nn[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) nn[i] = n[i];
    for (int64_t j = 0; j < M; ++j)
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l) != ORACLE_OK)
                return ORACLE_BAD_POINT;
        }
    int T = 1;
#ifdef _OPENMP
    T = threads > 0 ? threads : omp_get_max_threads();
#endif
    (void)threads;
    int wd[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) wd[i] = w;
#pragma omp parallel for num_threads(T) schedule(static)
    for (int64_t j = 0; j < M; ++j) {
        double phi[3][32];
        int64_t cell[3][32];
        for (int i = 0; i < 3; ++i) { phi[i][0] = 1.0; cell[i][0] = 0; }
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            grid_coord(X[i][j], nn[i], oracle_grid_scale(nn[i]), &t, &l);
            stencil_1d(t, nn[i], w, beta, phi[i], cell[i]);
        }
        double sre = 0.0, sim = 0.0;
        for (int q3 = 0; q3 < wd[2]; ++q3)
            for (int q2 = 0; q2 < wd[1]; ++q2)
                for (int q1 = 0; q1 < wd[0]; ++q1) {
                    double k = phi[0][q1] * phi[1][q2] * phi[2][q3];
                    int64_t idx = cell[0][q1] + nn[0] * (cell[1][q2] + nn[1] * cell[2][q3]);
                    sre += b[2 * idx] * k;
                    sim += b[2 * idx + 1] * k;
                }
        c[2 * j] = sre;
        c[2 * j + 1] = sim;
    }
    return ORACLE_OK;
}

/*
 * Bin-sort of the points (Sec. III-A, GM-sort and SM step 1).
 *
 * The fine grid is cut into bins of m1 x m2 (x m3) cells, ordered with the x
 * index fastest.  Point j lies in the bin holding its cell l_i = floor(t_i).
 * Outputs: bin[j]; counts[b] = number of points in bin b; perm = the points
 * listed bin by bin, which is how the page reads the list out "in bin
 * ordering".  The page leaves the order inside a bin open; the reading taken
 * here is the stable one, increasing original index, so perm is the stable
 * counting sort of bin[] (a library may order a bin's points differently as
 * long as each bin keeps exactly its own points).
 */
int oracle_binsort(int d, const int64_t* n, const int64_t* m, int64_t M, const double* const* X,
                   int64_t* bin, int64_t* counts, int64_t* perm)
{
    if (d < 1 || d > 3 || M < 0) return ORACLE_BAD_ARG;
    int64_t nb[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) {
        if (n[i] < 1 || m[i] < 1) return ORACLE_BAD_ARG;
        nb[i] = (n[i] + m[i] - 1) / m[i];
    }
    int64_t nbins = nb[0] * nb[1] * nb[2];
    int64_t* next = (int64_t*)calloc((size_t)(nbins > 0 ? nbins : 1), sizeof(int64_t));
    if (!next) return ORACLE_BAD_ARG;
    for (int64_t b = 0; b < nbins; ++b) counts[b] = 0;
    for (int64_t j = 0; j < M; ++j) {
        int64_t bi[3] = {0, 0, 0};
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], n[i], oracle_grid_scale(n[i]), &t, &l) != ORACLE_OK) {
                free(next);
                return ORACLE_BAD_POINT;
            }
            bi[i] = l / m[i];
        }
        bin[j] = bi[0] + nb[0] * (bi[1] + nb[1] * bi[2]);
        counts[bin[j]] += 1;
    }
    /* exclusive prefix sum of the counts: where each bin's run starts */
    int64_t run = 0;
    for (int64_t b = 0; b < nbins; ++b) { next[b] = run; run += counts[b]; }
    /* read the points out in bin order, ascending j inside a bin */
    for (int64_t j = 0; j < M; ++j) perm[next[bin[j]]++] = j;
    free(next);
    return ORACLE_OK;
}

/*
 * Subproblems (Sec. III-A, SM step 1): each bin's sorted points are cut into
 * consecutive chunks of at most `cap` points, bins taken in order.  Writes
 * (bin, start, length) triples; returns the number of subproblems, or a
 * negative code.  `out` may be NULL to only count.
 */
int64_t oracle_subproblems(int64_t nbins, const int64_t* counts, int64_t cap, int64_t* out)
{
    if (cap < 1) return ORACLE_BAD_ARG;
    int64_t ns = 0, start = 0;
    for (int64_t b = 0; b < nbins; ++b) {
        for (int64_t s = 0; s < counts[b]; s += cap) {
            if (out) {
                out[3 * ns] = b;
                out[3 * ns + 1] = start + s;
                out[3 * ns + 2] = (counts[b] - s < cap) ? counts[b] - s : cap;
            }
            ++ns;
        }
        start += counts[b];
    }
    return ns;
}

/* Mode index k_i of position idx along a dimension with N_i modes, I_N of eq. (2). */
static int64_t mode_of(int64_t idx, int64_t N) { return idx - N / 2; }

/*
 * Exact type 1 sum, eq. (1):  f_k = sum_j c_j exp(-i k.x_j), k in I_N.
 * Modes are evaluated at the flat output positions listed in `sel` (nsel of
 * them), or at every position when sel == NULL.  f is written at those
 * positions (f has prod(N) complex entries when sel == NULL, nsel otherwise).
 */
int oracle_direct_type1(int d, const int64_t* N, int64_t M, const double* const* X,
                        const double* c, int64_t nsel, const int64_t* sel, double* f)
{
    if (d < 1 || d > 3 || M < 0) return ORACLE_BAD_ARG;
    int64_t NN[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) NN[i] = N[i];
    int64_t total = NN[0] * NN[1] * NN[2];
    int64_t count = sel ? nsel : total;
    for (int64_t s = 0; s < count; ++s) {
        int64_t pos = sel ? sel[s] : s;
        if (pos < 0 || pos >= total) return ORACLE_BAD_ARG;
    }
    /* each output is one serial sum; outputs are independent (threads over outputs) */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < count; ++s) {
        int64_t pos = sel ? sel[s] : s;
        int64_t k1 = mode_of(pos % NN[0], NN[0]);
        int64_t k2 = mode_of((pos / NN[0]) % NN[1], NN[1]);
        int64_t k3 = mode_of(pos / (NN[0] * NN[1]), NN[2]);
        double sre = 0.0, sim = 0.0;
        for (int64_t j = 0; j < M; ++j) {
            double ph = (double)k1 * X[0][j];
            if (d > 1) ph += (double)k2 * X[1][j];
            if (d > 2) ph += (double)k3 * X[2][j];
            double co = cos(ph), si = sin(ph);
            /* c_j * exp(-i ph) */
            sre += c[2 * j] * co + c[2 * j + 1] * si;
            sim += c[2 * j + 1] * co - c[2 * j] * si;
        }
        f[2 * s] = sre;
        f[2 * s + 1] = sim;
    }
    return ORACLE_OK;
}

/*
 * Exact type 2 sum, eq. (3):  c_j = sum_{k in I_N} f_k exp(+i k.x_j).
 * Points are the indices in `sel` (nsel of them) or all M when sel == NULL.
 */
int oracle_direct_type2(int d, const int64_t* N, int64_t M, const double* const* X,
                        const double* f, int64_t nsel, const int64_t* sel, double* c)
{
    if (d < 1 || d > 3 || M < 0) return ORACLE_BAD_ARG;
    int64_t NN[3] = {1, 1, 1};
    for (int i = 0; i < d; ++i) NN[i] = N[i];
    int64_t total = NN[0] * NN[1] * NN[2];
    int64_t count = sel ? nsel : M;
    for (int64_t s = 0; s < count; ++s) {
        int64_t j = sel ? sel[s] : s;
        if (j < 0 || j >= M) return ORACLE_BAD_ARG;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < count; ++s) {
        int64_t j = sel ? sel[s] : s;
        double sre = 0.0, sim = 0.0;
        for (int64_t pos = 0; pos < total; ++pos) {
            int64_t k1 = mode_of(pos % NN[0], NN[0]);
            int64_t k2 = mode_of((pos / NN[0]) % NN[1], NN[1]);
            int64_t k3 = mode_of(pos / (NN[0] * NN[1]), NN[2]);
            double ph = (double)k1 * X[0][j];
            if (d > 1) ph += (double)k2 * X[1][j];
            if (d > 2) ph += (double)k3 * X[2][j];
            double co = cos(ph), si = sin(ph);
            /* f_k * exp(+i ph) */
            sre += f[2 * pos] * co - f[2 * pos + 1] * si;
            sim += f[2 * pos + 1] * co + f[2 * pos] * si;
        }
        c[2 * s] = sre;
        c[2 * s + 1] = sim;
    }
    return ORACLE_OK;
}

/*
 * Type 1 steps 1-2 evaluated at chosen frequencies only, for large problems
 * where the whole fine grid is too costly on the CPU.
 *
 * Step 2 (eq. (9)) at one frequency k is bhat_k = sum_l b_l exp(-2 pi i l.k/n).
 * Inserting step 1 (eq. (7)) and exchanging the two finite sums gives
 *   bhat_k = sum_j c_j prod_i ( sum_q phi_{i,q}(x_j) exp(-2 pi i cell_{i,q} k_i / n_i) ),
 * because psi is a tensor product (eq. (8)).  kvec holds nk frequency tuples
 * (k1, k2[, k3]) (any integers); bhat receives nk complex values (no
 * correction factor applied).
 */
int oracle_type1_bhat_at(int d, const int64_t* n, int w, double beta, int64_t M,
                         const double* const* X, const double* c,
                         int64_t nk, const int64_t* kvec, double* bhat)
{
    if (d < 1 || d > 3 || w < 1 || w > 32 || M < 0 || nk < 0) return ORACLE_BAD_ARG;
    for (int64_t s = 0; s < 2 * nk; ++s) bhat[s] = 0.0;
    for (int64_t j = 0; j < M; ++j)
        for (int i = 0; i < d; ++i) {
            double t; int64_t l;
            if (grid_coord(X[i][j], n[i], oracle_grid_scale(n[i]), &t, &l) != ORACLE_OK)
                return ORACLE_BAD_POINT;
        }
    int nthreads = 1;
#ifdef _OPENMP
    nthreads = omp_get_max_threads();
#endif
    /* points are split into nthreads contiguous ranges; each range's partial sums are added
       in range order at the end */
    double* part = (double*)calloc((size_t)nthreads * 2 * (size_t)(nk > 0 ? nk : 1), sizeof(double));
    if (!part) return ORACLE_BAD_ARG;
    /* twiddles exp(-2 pi i r / n_i), r = 0..n_i-1, one table per dimension */
    double* tw[3] = {NULL, NULL, NULL};
    for (int i = 0; i < d; ++i) {
        tw[i] = (double*)malloc(sizeof(double) * 2 * (size_t)n[i]);
        if (!tw[i]) { free(part); for (int q = 0; q < i; ++q) free(tw[q]); return ORACLE_BAD_ARG; }
        for (int64_t r = 0; r < n[i]; ++r) {
            double ang = -2.0 * PI_D * (double)r / (double)n[i];
            tw[i][2 * r] = cos(ang);
            tw[i][2 * r + 1] = sin(ang);
        }
    }
#pragma omp parallel num_threads(nthreads)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        int64_t j0 = M * tid / nthreads, j1 = M * (tid + 1) / nthreads;
        double* acc = part + (size_t)tid * 2 * (size_t)nk;
        double phi[3][32];
        int64_t cell[3][32];
        for (int64_t j = j0; j < j1; ++j) {
            for (int i = 0; i < d; ++i) {
                double t; int64_t l;
                grid_coord(X[i][j], n[i], oracle_grid_scale(n[i]), &t, &l);
                stencil_1d(t, n[i], w, beta, phi[i], cell[i]);
            }
            for (int64_t s = 0; s < nk; ++s) {
                double pre = c[2 * j], pim = c[2 * j + 1];
                for (int i = 0; i < d; ++i) {
                    int64_t k = kvec[d * s + i];
                    double are = 0.0, aim = 0.0;
                    for (int q = 0; q < w; ++q) {
                        /* exp(-2 pi i cell k / n), with cell*k reduced mod n exactly first */
                        int64_t r = pmod(pmod(cell[i][q], n[i]) * pmod(k, n[i]), n[i]);
                        are += phi[i][q] * tw[i][2 * r];
                        aim += phi[i][q] * tw[i][2 * r + 1];
                    }
                    double nre = pre * are - pim * aim;
                    double nim = pre * aim + pim * are;
                    pre = nre; pim = nim;
                }
                acc[2 * s] += pre;
                acc[2 * s + 1] += pim;
            }
        }
    }
    for (int t = 0; t < nthreads; ++t)
        for (int64_t s = 0; s < 2 * nk; ++s) bhat[s] += part[(size_t)t * 2 * (size_t)nk + s];
    free(part);
    for (int i = 0; i < d; ++i) free(tw[i]);
    return ORACLE_OK;
}
