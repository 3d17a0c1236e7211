// Type 3 (nonuniform to nonuniform) helper kernels.  The transform itself is carried by an inner
// type 1 plan (spreading, eq. (7), onto a fine grid sized from the data) and an inner type 2
// plan (eqs. (11), (12) and the interpolation sum, evaluating the grid's Fourier sum at the
// scaled targets); these kernels do what is particular to type 3:
//  * min / max of each coordinate array (centres and half-widths of sources and targets);
//  * the scaled coordinates y = (x - C) / gamma and theta = ((s - D) gamma) h;
//  * per-source phase exp(i D.(x - C)) and per-target factor
//    prod_i (2/w) / phihat(alpha_i xi_i) exp(i (xi_i (h_i floor(n_i/2) - pi) + s_i C_i)),
//    xi = (s - D) gamma, alpha = w h / 2 (the kernel's Fourier transform, eq. (4), by
//    Gauss-Legendre quadrature after z = sin(theta), with a table built on the host);
//  * the complex products c' = c pre and f = post cin.
// Coordinate arithmetic is fp64 with explicit rounding (no contraction), so the scaled
// coordinates are reproducible bit for bit.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kBlock = 256;

template <typename T>
__global__ void __launch_bounds__(kBlock) k_minmax(const T* __restrict__ a, int64_t n, double* __restrict__ part) {
    __shared__ double slo[kBlock], shi[kBlock];
    double lo = __builtin_inf(), hi = -__builtin_inf();
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
        const double v = (double)a[i];
        if (!isfinite(v)) bad = true;
        lo = fmin(lo, v);
        hi = fmax(hi, v);
    }
    if (bad) lo = __builtin_nan("");
    slo[threadIdx.x] = lo;
    shi[threadIdx.x] = hi;
    __syncthreads();
    for (int s = kBlock / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            const double a2 = slo[threadIdx.x + s], b2 = shi[threadIdx.x + s];
            slo[threadIdx.x] = (isnan(slo[threadIdx.x]) || isnan(a2)) ? __builtin_nan("") : fmin(slo[threadIdx.x], a2);
            shi[threadIdx.x] = fmax(shi[threadIdx.x], b2);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[2 * blockIdx.x] = slo[0];
        part[2 * blockIdx.x + 1] = shi[0];
    }
}

// y = (((x - ctr) / div) * mul1) * mul2, each operation rounded in fp64, the result rounded to T
template <typename T>
__global__ void __launch_bounds__(kBlock) k_scale(const T* __restrict__ x, int64_t n, double ctr, double div,
                                                  double mul1, double mul2, T* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n) y[i] = (T)__dmul_rn(__dmul_rn(__ddiv_rn(__dsub_rn((double)x[i], ctr), div), mul1), mul2);
}

struct T3Geom {
    int dim;
    double C[3], D[3], gamma[3], alpha[3], off[3];   // off = h floor(n/2) - pi
    double corr;                                     // 2 / w
};

// pre_j = exp(i sum_i D_i (x_ij - C_i))
template <typename T>
__global__ void __launch_bounds__(kBlock) k_pre(T3Geom g, const T* __restrict__ x0, const T* __restrict__ x1,
                                                const T* __restrict__ x2, int64_t M, cplx<T>* __restrict__ pre) {
    const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (j >= M) return;
    const T* xs[3] = {x0, x1, x2};
    double ph = 0.0;
    for (int i = 0; i < g.dim; ++i) ph = __dadd_rn(ph, __dmul_rn(g.D[i], __dsub_rn((double)xs[i][j], g.C[i])));
    double sn, cs;
    sincos(ph, &sn, &cs);
    cplx<T> v;
    v.re = (T)cs;
    v.im = (T)sn;
    pre[j] = v;
}

// post_k = prod_i (2/w) / phihat(alpha_i xi_i) * exp(i sum_i (xi_i off_i + s_i C_i)),
// phihat(u) = sum_q tw[q] cos(u ts[q])
template <typename T>
__global__ void __launch_bounds__(kBlock) k_post(T3Geom g, const T* __restrict__ s0, const T* __restrict__ s1,
                                                 const T* __restrict__ s2, int64_t K, const double* __restrict__ tab,
                                                 int nq, cplx<T>* __restrict__ post) {
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (k >= K) return;
    const T* ss[3] = {s0, s1, s2};
    double amp = 1.0, ph = 0.0;
    for (int i = 0; i < g.dim; ++i) {
        const double s = (double)ss[i][k];
        const double xi = __dmul_rn(__dsub_rn(s, g.D[i]), g.gamma[i]);
        const double u = g.alpha[i] * xi;
        double acc = 0.0;
        for (int q = 0; q < nq; ++q) acc += tab[nq + q] * cos(u * tab[q]);
        amp *= g.corr / acc;
        ph += xi * g.off[i] + s * g.C[i];
    }
    double sn, cs;
    sincos(ph, &sn, &cs);
    cplx<T> v;
    v.re = (T)(amp * cs);
    v.im = (T)(amp * sn);
    post[k] = v;
}

// out = a * b (complex)
template <typename T>
__global__ void __launch_bounds__(kBlock) k_cmul(const cplx<T>* __restrict__ a, const cplx<T>* __restrict__ b,
                                                 int64_t n, cplx<T>* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    const cplx<T> x = a[i], y = b[i];
    cplx<T> r;
    r.re = x.re * y.re - x.im * y.im;
    r.im = x.re * y.im + x.im * y.re;
    out[i] = r;
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kBlock - 1) / kBlock); }

}  // namespace

int t3_minmax_blocks() { return 512; }

hipError_t launch_t3_minmax(int prec, const void* a, int64_t n, double* part, hipStream_t st) {
    if (prec == 0) k_minmax<float><<<t3_minmax_blocks(), kBlock, 0, st>>>((const float*)a, n, part);
    else k_minmax<double><<<t3_minmax_blocks(), kBlock, 0, st>>>((const double*)a, n, part);
    return hipGetLastError();
}

hipError_t launch_t3_scale(int prec, const void* x, int64_t n, double ctr, double div, double mul1, double mul2,
                           void* y, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (prec == 0)
        k_scale<float><<<blocks_for(n), kBlock, 0, st>>>((const float*)x, n, ctr, div, mul1, mul2, (float*)y);
    else
        k_scale<double><<<blocks_for(n), kBlock, 0, st>>>((const double*)x, n, ctr, div, mul1, mul2, (double*)y);
    return hipGetLastError();
}

hipError_t launch_t3_factors(int prec, int dim, const double* C, const double* D, const double* gamma,
                             const double* alpha, const double* off, double corr, const void* const* x, int64_t M,
                             void* pre, const void* const* s, int64_t K, const double* tab, int nq, void* post,
                             hipStream_t st) {
    T3Geom g{};
    g.dim = dim;
    for (int i = 0; i < 3; ++i) {
        g.C[i] = i < dim ? C[i] : 0.0;
        g.D[i] = i < dim ? D[i] : 0.0;
        g.gamma[i] = i < dim ? gamma[i] : 1.0;
        g.alpha[i] = i < dim ? alpha[i] : 0.0;
        g.off[i] = i < dim ? off[i] : 0.0;
    }
    g.corr = corr;
    if (M > 0) {
        if (prec == 0)
            k_pre<float><<<blocks_for(M), kBlock, 0, st>>>(g, (const float*)x[0], (const float*)x[1], (const float*)x[2],
                                                           M, (cplx<float>*)pre);
        else
            k_pre<double><<<blocks_for(M), kBlock, 0, st>>>(g, (const double*)x[0], (const double*)x[1],
                                                            (const double*)x[2], M, (cplx<double>*)pre);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (K > 0) {
        if (prec == 0)
            k_post<float><<<blocks_for(K), kBlock, 0, st>>>(g, (const float*)s[0], (const float*)s[1], (const float*)s[2],
                                                            K, tab, nq, (cplx<float>*)post);
        else
            k_post<double><<<blocks_for(K), kBlock, 0, st>>>(g, (const double*)s[0], (const double*)s[1],
                                                             (const double*)s[2], K, tab, nq, (cplx<double>*)post);
    }
    return hipGetLastError();
}

hipError_t launch_t3_cmul(int prec, const void* a, const void* b, int64_t n, void* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (prec == 0)
        k_cmul<float><<<blocks_for(n), kBlock, 0, st>>>((const cplx<float>*)a, (const cplx<float>*)b, n,
                                                        (cplx<float>*)out);
    else
        k_cmul<double><<<blocks_for(n), kBlock, 0, st>>>((const cplx<double>*)a, (const cplx<double>*)b, n,
                                                         (cplx<double>*)out);
    return hipGetLastError();
}

}  // namespace nufft
