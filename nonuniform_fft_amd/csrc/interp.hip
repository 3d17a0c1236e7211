// Type 2 step 3: interpolation from the fine grid at the nonuniform points
// (cuFINUFFT paper, Sec. II-B, the weighted sum that follows eq. (12); kernel as in eq. (8)).
//
// GM-sort scheme (Sec. III-B): one thread per point in bin-sorted order, so neighbouring lanes
// read neighbouring grid cells; each thread gathers its w^d cells, sums along x first, and
// writes c at the point's original index.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kInterpBlock = 128;

template <typename T, int DIM, int W>
__global__ void __launch_bounds__(kInterpBlock) k_interp_gm(GeomArgs g, const cplx<T>* __restrict__ grid,
                                                            cplx<T>* __restrict__ c) {
    const int64_t i = (int64_t)blockIdx.x * kInterpBlock + threadIdx.x;
    if (i >= g.M) return;
    const T beta = (T)g.beta;
    T ker[DIM][W];
    int idx[DIM][W];
#pragma unroll
    for (int d = 0; d < DIM; ++d) {
        double t = grid_t((double)((const T*)g.xs[d])[i], g.s[d]);
        int l;
        fold_t(t, g.n[d], l);
        int l0 = es_weights<T, W>(t, beta, ker[d]);
#pragma unroll
        for (int q = 0; q < W; ++q) {
            int v = l0 + q;
            v = (v < 0) ? v + g.n[d] : (v >= g.n[d] ? v - g.n[d] : v);
            idx[d][q] = v;
        }
    }
    const int n1 = g.n[0], n2 = g.n[1];
    T are = 0, aim = 0;
#pragma unroll
    for (int q3 = 0; q3 < (DIM == 3 ? W : 1); ++q3) {
        for (int q2 = 0; q2 < W; ++q2) {
            T wr = ker[1][q2];
            size_t row = (size_t)idx[1][q2];
            if (DIM == 3) {
                wr *= ker[DIM - 1][q3];
                row += (size_t)n2 * (size_t)idx[DIM - 1][q3];
            }
            const cplx<T>* src = grid + row * (size_t)n1;
            T rre = 0, rim = 0;
#pragma unroll
            for (int q1 = 0; q1 < W; ++q1) {
                const cplx<T> v = src[idx[0][q1]];
                rre += v.re * ker[0][q1];
                rim += v.im * ker[0][q1];
            }
            are += rre * wr;
            aim += rim * wr;
        }
    }
    cplx<T> out;
    out.re = are;
    out.im = aim;
    c[g.perm[i]] = out;
}

template <typename T, int DIM>
hipError_t interp_dim(const GeomArgs& g, const void* grid, void* c, hipStream_t st) {
    if (g.M <= 0) return hipSuccess;
    dim3 grd((unsigned)((g.M + kInterpBlock - 1) / kInterpBlock));
    switch (g.w) {
#define NUFFT_CASE(WW)                                                                          \
    case WW:                                                                                    \
        k_interp_gm<T, DIM, WW><<<grd, kInterpBlock, 0, st>>>(g, (const cplx<T>*)grid, (cplx<T>*)c); \
        return hipGetLastError();
        NUFFT_CASE(2) NUFFT_CASE(3) NUFFT_CASE(4) NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7)
        NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10) NUFFT_CASE(11) NUFFT_CASE(12) NUFFT_CASE(13)
        NUFFT_CASE(14) NUFFT_CASE(15) NUFFT_CASE(16)
#undef NUFFT_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_interp(int prec, const GeomArgs& g, const void* grid, void* c, hipStream_t st) {
    if (prec == 0) return g.dim == 2 ? interp_dim<float, 2>(g, grid, c, st) : interp_dim<float, 3>(g, grid, c, st);
    return g.dim == 2 ? interp_dim<double, 2>(g, grid, c, st) : interp_dim<double, 3>(g, grid, c, st);
}

}  // namespace nufft
