// Correction steps (cuFINUFFT paper, Sec. II): type 1 step 3, truncation to I_N and scaling by
// p_k (eq. (10)); type 2 step 1, pre-correction and zero padding onto the fine grid (eq. (11)).
// p_k = p_1(k1) p_2(k2) [p_3(k3)] is separable; the per-dimension vectors are computed on the
// host once per plan (one thread per mode or cell, coalesced along the fastest dimension).  1D
// plans run the 2D kernels: their second dimension has N2 = n2 = 1 and p_2 = 1.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kBlock = 256;

template <typename T, int DIM>
__global__ void __launch_bounds__(kBlock) k_deconvolve(int N1, int N2, int N3, int n1, int n2, int n3,
                                                       const T* __restrict__ p,
                                                       const cplx<T>* __restrict__ fhat,
                                                       cplx<T>* __restrict__ f) {
    // vector blockIdx.y of a many-vector launch
    fhat += (int64_t)blockIdx.y * n1 * n2 * n3;
    f += (int64_t)blockIdx.y * N1 * N2 * N3;
    const int64_t total = (int64_t)N1 * N2 * N3;
    const int64_t pos = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (pos >= total) return;
    const int i1 = (int)(pos % N1);
    const int64_t r = pos / N1;
    const int i2 = (int)(r % N2);
    const int i3 = (int)(r / N2);
    int k1 = i1 - N1 / 2, k2 = i2 - N2 / 2, k3 = i3 - N3 / 2;
    int l1 = k1 < 0 ? k1 + n1 : k1;
    int l2 = k2 < 0 ? k2 + n2 : k2;
    int l3 = k3 < 0 ? k3 + n3 : k3;
    T s = p[i1] * p[N1 + i2];
    if (DIM == 3) s *= p[N1 + N2 + i3];
    else l3 = 0;
    const cplx<T> v = fhat[(size_t)l1 + (size_t)n1 * ((size_t)l2 + (size_t)n2 * (size_t)l3)];
    cplx<T> o;
    o.re = v.re * s;
    o.im = v.im * s;
    f[pos] = o;
}

template <typename T, int DIM>
__global__ void __launch_bounds__(kBlock) k_precorrect_pad(int N1, int N2, int N3, int n1, int n2, int n3, FastDiv fd1, FastDiv fd2,
                                                           const T* __restrict__ p,
                                                           const cplx<T>* __restrict__ f,
                                                           cplx<T>* __restrict__ fhat) {
    // vector blockIdx.y of a many-vector launch
    fhat += (int64_t)blockIdx.y * n1 * n2 * n3;
    f += (int64_t)blockIdx.y * N1 * N2 * N3;
    const int64_t total = (int64_t)n1 * n2 * n3;
    const int64_t cell = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (cell >= total) return;
    int l1, l2, l3;
    if (total < (int64_t(1) << 31)) {   // 32-bit multiply-high division (fd = reciprocals of n1, n2)
        const int c32 = (int)cell;
        const int r = fast_div(c32, fd1);
        l1 = c32 - r * n1;
        l3 = fast_div(r, fd2);
        l2 = r - l3 * n2;
    } else {
        l1 = (int)(cell % n1);
        const int64_t r = cell / n1;
        l2 = (int)(r % n2);
        l3 = (int)(r / n2);
    }
    // mode k of cell l: k = l on the nonnegative part of I_N, k = l - n on the negative part
    auto mode_index = [](int l, int N, int n) -> int {
        if (l < N - N / 2) return l + N / 2;
        if (l >= n - N / 2) return l - n + N / 2;
        return -1;
    };
    const int i1 = mode_index(l1, N1, n1);
    const int i2 = mode_index(l2, N2, n2);
    const int i3 = (DIM == 3) ? mode_index(l3, N3, n3) : 0;
    cplx<T> o;
    o.re = 0;
    o.im = 0;
    if (i1 >= 0 && i2 >= 0 && i3 >= 0) {
        T s = p[i1] * p[N1 + i2];
        if (DIM == 3) s *= p[N1 + N2 + i3];
        const cplx<T> v = f[(size_t)i1 + (size_t)N1 * ((size_t)i2 + (size_t)N2 * (size_t)i3)];
        o.re = v.re * s;
        o.im = v.im * s;
    }
    fhat[cell] = o;
}

// fp32 variant for an even n1: each thread fills two neighbouring cells of one row (l1 even) with
// one 16-byte store, so a wave writes 1 KiB per instruction instead of 512 B.  The launcher takes
// it only when the fine grid's base is 16-byte aligned; n1 even makes every row, and every
// vector's grid in a many-vector launch, start on a 16-byte boundary as well.
template <int DIM>
__global__ void __launch_bounds__(kBlock) k_precorrect_pad_pair(int N1, int N2, int N3, int n1, int n2, int n3,
                                                                FastDiv fdh1, FastDiv fd2,
                                                                const float* __restrict__ p,
                                                                const cplx<float>* __restrict__ f,
                                                                float4* __restrict__ fhat) {
    const int h1 = n1 >> 1;                              // cell pairs per row
    const int64_t pairs = (int64_t)h1 * n2 * n3;
    fhat += (int64_t)blockIdx.y * pairs;
    f += (int64_t)blockIdx.y * N1 * N2 * N3;
    const int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (q >= pairs) return;
    int l1, l2, l3;
    if (pairs < (int64_t(1) << 31)) {
        const int q32 = (int)q;
        const int r = fast_div(q32, fdh1);
        l1 = 2 * (q32 - r * h1);
        l3 = fast_div(r, fd2);
        l2 = r - l3 * n2;
    } else {
        l1 = 2 * (int)(q % h1);
        const int64_t r = q / h1;
        l2 = (int)(r % n2);
        l3 = (int)(r / n2);
    }
    auto mode_index = [](int l, int N, int n) -> int {
        if (l < N - N / 2) return l + N / 2;
        if (l >= n - N / 2) return l - n + N / 2;
        return -1;
    };
    const int i2 = mode_index(l2, N2, n2);
    const int i3 = (DIM == 3) ? mode_index(l3, N3, n3) : 0;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i2 >= 0 && i3 >= 0) {
        // same product order as the one-cell kernel, (p_1 p_2) p_3, so both give identical values
        const float p2 = p[N1 + i2];
        const float p3 = (DIM == 3) ? p[N1 + N2 + i3] : 1.f;
        const size_t row = (size_t)N1 * ((size_t)i2 + (size_t)N2 * (size_t)i3);
        const int ia = mode_index(l1, N1, n1);
        const int ib = mode_index(l1 + 1, N1, n1);
        if (ia >= 0) {
            const cplx<float> v = f[row + ia];
            float s = p[ia] * p2;
            if (DIM == 3) s *= p3;
            o.x = v.re * s;
            o.y = v.im * s;
        }
        if (ib >= 0) {
            const cplx<float> v = f[row + ib];
            float s = p[ib] * p2;
            if (DIM == 3) s *= p3;
            o.z = v.re * s;
            o.w = v.im * s;
        }
    }
    fhat[q] = o;
}

}  // namespace

hipError_t launch_deconvolve(int prec, int dim, const int64_t* N, const int64_t* n, const void* pcorr,
                             const void* fhat, void* f, hipStream_t st, int nv) {
    int N3 = dim == 3 ? (int)N[2] : 1, n3 = dim == 3 ? (int)n[2] : 1;
    int64_t total = N[0] * N[1] * (int64_t)N3;
    if (total == 0) return hipSuccess;
    dim3 g((unsigned)((total + kBlock - 1) / kBlock), (unsigned)nv);
    if (prec == 0) {
        if (dim <= 2) k_deconvolve<float, 2><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], 1, (int)n[0], (int)n[1], 1, (const float*)pcorr, (const cplx<float>*)fhat, (cplx<float>*)f);
        else k_deconvolve<float, 3><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], N3, (int)n[0], (int)n[1], n3, (const float*)pcorr, (const cplx<float>*)fhat, (cplx<float>*)f);
    } else {
        if (dim <= 2) k_deconvolve<double, 2><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], 1, (int)n[0], (int)n[1], 1, (const double*)pcorr, (const cplx<double>*)fhat, (cplx<double>*)f);
        else k_deconvolve<double, 3><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], N3, (int)n[0], (int)n[1], n3, (const double*)pcorr, (const cplx<double>*)fhat, (cplx<double>*)f);
    }
    return hipGetLastError();
}

hipError_t launch_precorrect_pad(int prec, int dim, const int64_t* N, const int64_t* n, const void* pcorr,
                                 const void* f, void* fhat, hipStream_t st, int nv) {
    int N3 = dim == 3 ? (int)N[2] : 1, n3 = dim == 3 ? (int)n[2] : 1;
    int64_t total = n[0] * n[1] * (int64_t)n3;
    dim3 g((unsigned)((total + kBlock - 1) / kBlock), (unsigned)nv);
    if (prec == 0 && n[0] % 2 == 0 && reinterpret_cast<uintptr_t>(fhat) % 16 == 0) {
        const int64_t pairs = total / 2;
        dim3 gp((unsigned)((pairs + kBlock - 1) / kBlock), (unsigned)nv);
        const FastDiv fdh1 = make_fastdiv((int)(n[0] / 2)), fd2 = make_fastdiv((int)n[1]);
        if (dim <= 2) k_precorrect_pad_pair<2><<<gp, kBlock, 0, st>>>((int)N[0], (int)N[1], 1, (int)n[0], (int)n[1], 1, fdh1, fd2, (const float*)pcorr, (const cplx<float>*)f, (float4*)fhat);
        else k_precorrect_pad_pair<3><<<gp, kBlock, 0, st>>>((int)N[0], (int)N[1], N3, (int)n[0], (int)n[1], n3, fdh1, fd2, (const float*)pcorr, (const cplx<float>*)f, (float4*)fhat);
    } else if (prec == 0) {
        if (dim <= 2) k_precorrect_pad<float, 2><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], 1, (int)n[0], (int)n[1], 1, make_fastdiv((int)n[0]), make_fastdiv((int)n[1]), (const float*)pcorr, (const cplx<float>*)f, (cplx<float>*)fhat);
        else k_precorrect_pad<float, 3><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], N3, (int)n[0], (int)n[1], n3, make_fastdiv((int)n[0]), make_fastdiv((int)n[1]), (const float*)pcorr, (const cplx<float>*)f, (cplx<float>*)fhat);
    } else {
        if (dim <= 2) k_precorrect_pad<double, 2><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], 1, (int)n[0], (int)n[1], 1, make_fastdiv((int)n[0]), make_fastdiv((int)n[1]), (const double*)pcorr, (const cplx<double>*)f, (cplx<double>*)fhat);
        else k_precorrect_pad<double, 3><<<g, kBlock, 0, st>>>((int)N[0], (int)N[1], N3, (int)n[0], (int)n[1], n3, make_fastdiv((int)n[0]), make_fastdiv((int)n[1]), (const double*)pcorr, (const cplx<double>*)f, (cplx<double>*)fhat);
    }
    return hipGetLastError();
}

}  // namespace nufft
