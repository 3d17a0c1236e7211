// Internal declarations of the gfx950 NUFFT library: plan state, kernel launchers and the
// device helpers every kernel shares (grid coordinates, ES kernel weights).
#pragma once

#include <hip/hip_runtime.h>
#include <rocfft/rocfft.h>

#include <cstdint>
#include <type_traits>
#include <string>

#include "../../include/nufft_amd.h"

namespace nufft {

// Largest kernel width supported (the tolerance rule is clamped to [2, 16]).
constexpr int kMaxW = 16;
constexpr int kMinW = 2;

// The double nearest pi (bit-identical to M_PI).
constexpr double kPi = 3.141592653589793115997963468544185161590576171875;

// ------------------------------------------------------------------------------------------------
// Device helpers
// ------------------------------------------------------------------------------------------------

// Scaled coordinate t = (x + pi) * s, s = n / (2 pi), as two separately rounded fp64 operations
// (no contraction), so that the bin of every point is reproducible bit for bit.
__device__ __forceinline__ double grid_t(double x, double s) {
    return __dmul_rn(__dadd_rn(x, kPi), s);
}

// One periodic fold of t into [0, n).  Returns false for NaN or values outside [-n, 2n).
__device__ __forceinline__ bool fold_t(double& t, int n, int& l) {
    double fl = floor(t);
    if (!(fl >= -(double)n && fl < 2.0 * (double)n)) return false;
    l = (int)fl;
    if (l >= n) { l -= n; t = __dsub_rn(t, (double)n); }
    else if (l < 0) { l += n; t = __dadd_rn(t, (double)n); }
    return true;
}

// (s1, s2, s3) of cell index k = s1 + p1 (s2 + p2 s3), advanced by a fixed stride without division.
struct CellWalk {
    int s1, s2, s3, d1, d2, d3, p1, p2;
    __device__ CellWalk(int k, int stride, int p1_, int p2_) : p1(p1_), p2(p2_) {
        s1 = k % p1; int r = k / p1; s2 = r % p2; s3 = r / p2;
        d1 = stride % p1; r = stride / p1; d2 = r % p2; d3 = r / p2;
    }
    __device__ void next() {
        s1 += d1; int c = s1 >= p1; s1 -= c ? p1 : 0;
        s2 += d2 + c; c = s2 >= p2; s2 -= c ? p2 : 0;
        s3 += d3 + c;
    }
};

// Periodic wrap of a padded-tile coordinate onto [0, n).  A padded bin can reach past the grid
// end by up to m + w cells, which is more than one period on small grids, hence the loops.
__device__ __forceinline__ int wrap_grid(int v, int n) {
    while (v >= n) v -= n;
    while (v < 0) v += n;
    return v;
}

// The same wrap for v in [-n, 2n) without branches: of v - n, v and v + n, the one in [0, n) is
// the smallest as an unsigned number (the others are negative or at least n).
__device__ __forceinline__ int wrap_step(int v, int n) {
    const unsigned a = (unsigned)v, b = (unsigned)(v - n), c = (unsigned)(v + n);
    return (int)min(min(a, b), c);
}

template <bool FAST>
__device__ __forceinline__ int wrap_pad(int v, int n) {
    if constexpr (FAST) return wrap_step(v, n);
    else return wrap_grid(v, n);
}

// Linear fine-grid index of cell (g1, g2, g3); FAST when the grid has fewer than 2^32 cells.
template <bool FAST>
__device__ __forceinline__ size_t grid_index(int g1, int g2, int g3, const int* n) {
    if constexpr (FAST)
        return (uint32_t)g1 + (uint32_t)n[0] * ((uint32_t)g2 + (uint32_t)n[1] * (uint32_t)g3);
    else
        return (size_t)g1 + (size_t)n[0] * ((size_t)g2 + (size_t)n[1] * (size_t)g3);
}

// Whether a padded tile can take the FAST forms above: origin[i] + s, s in [0, p[i]), stays in
// [-n[i], 2 n[i]) along the first dim dimensions (every grid at least as large as the tile), and
// the grid's cells are indexable in 32 bits.  The result is uniform over a workgroup.
__device__ __forceinline__ bool tile_fast(const int* origin, const int* p, const int* n, int dim) {
    bool ok = (uint64_t)n[0] * (uint64_t)(dim >= 2 ? n[1] : 1) * (uint64_t)(dim == 3 ? n[2] : 1) < (1ull << 32);
    for (int i = 0; i < dim; ++i) ok = ok && origin[i] >= -n[i] && origin[i] + p[i] <= 2 * n[i];
    return ok;
}

// e^x in fp64 for x in [-64, 0], the range of the ES kernel's exponent beta (sqrt(1 - z^2) - 1).
// Cody-Waite reduction x = k ln2 + r, |r| <= ln2 / 2, with ln2 split into LN2_HI (its first 32
// significant bits, so k LN2_HI is exact) and LN2_LO = ln2 - LN2_HI; e^r from its Taylor series
// to degree 12 (truncation error below 2.3e-16 relative on that interval); then scaled by 2^k.
// No special cases: the argument range rules out overflow, underflow and NaN.
__device__ __forceinline__ double exp_es(double x) {
    constexpr double kLog2e = 1.4426950408889634;              // 1 / ln2
    constexpr double kLn2Hi = 0x1.62e42fee00000p-1;
    constexpr double kLn2Lo = 0x1.a39ef35793c76p-33;
    const double k = rint(x * kLog2e);
    const double r = __fma_rn(-k, kLn2Lo, __fma_rn(-k, kLn2Hi, x));
    double p = 1.0 / 479001600.0;                                // 1/12!
    p = __fma_rn(p, r, 1.0 / 39916800.0);
    p = __fma_rn(p, r, 1.0 / 3628800.0);
    p = __fma_rn(p, r, 1.0 / 362880.0);
    p = __fma_rn(p, r, 1.0 / 40320.0);
    p = __fma_rn(p, r, 1.0 / 5040.0);
    p = __fma_rn(p, r, 1.0 / 720.0);
    p = __fma_rn(p, r, 1.0 / 120.0);
    p = __fma_rn(p, r, 1.0 / 24.0);
    p = __fma_rn(p, r, 1.0 / 6.0);
    p = __fma_rn(p, r, 0.5);
    p = __fma_rn(p, r, 1.0);
    p = __fma_rn(p, r, 1.0);
    return ldexp(p, (int)k);
}

// sqrt(x) for x in [0, 1] in fp64: the hardware square root (about 2^-23 relative error) refined
// by one Newton step s + (x - s^2) / (2 s), which squares the relative error (below 1e-15 here);
// x = 0 gives 0.  The refinement's reciprocal may be approximate: its error only scales the
// already small correction.
__device__ __forceinline__ double sqrt_unit(double x) {
    const double s = __builtin_amdgcn_sqrt(x);
    const double e = __fma_rn(-s, s, x);
    const double r = __builtin_amdgcn_rcp(s);
    return (x > 0.0) ? __fma_rn(e, 0.5 * r, s) : 0.0;
}

// ES kernel weights (cuFINUFFT paper eq. (5), rescaled as in eq. (8)) of a point with folded
// scaled coordinate t along one dimension: the support is the W cells starting at
// l0 = ceil(t - W/2); weight q has argument z = (l0 + q - t) * 2/W.  The offset l0 - t is
// formed in fp64 and the rest in the plan precision T (fp32 uses the hardware square root and
// exp2-based exponential, whose relative errors -- about 1e-7, and 1e-6 at the smallest weights --
// are far below the fp32 output tolerance).
template <typename T, int W>
__device__ __forceinline__ int es_weights(double t, T beta, T* phi) {
    double l0d = ceil(__dsub_rn(t, 0.5 * (double)W));
    T delta = (T)__dsub_rn(l0d, t);
    const T scale = (T)2 / (T)W;
#pragma unroll
    for (int q = 0; q < W; ++q) {
        T z = (delta + (T)q) * scale;
        T zz = z * z;
        if constexpr (sizeof(T) == 4)
            phi[q] = (zz <= 1.0f) ? __expf(beta * (__builtin_amdgcn_sqrtf(1.0f - zz) - 1.0f)) : 0.0f;
        else
            phi[q] = (zz <= (T)1) ? exp_es(beta * (sqrt_unit((T)1 - zz) - (T)1)) : (T)0;
    }
    return (int)l0d;
}

template <typename T> struct cplx { T re, im; };

// A kernel-support start l0 inside a padded tile must lie in [0, hi]; the bin-sort and the
// kernels place every point so that it does.  A start outside is counted in *err (a plan-owned
// counter the tests read back) and clamped, so a disagreement shows up as a count instead of
// as an out-of-bounds access.
__device__ __forceinline__ int checked_start(int l0, int hi, unsigned int* err) {
    if (l0 < 0 || l0 > hi) {
        atomicAdd(err, 1u);
        l0 = min(max(l0, 0), hi);
    }
    return l0;
}

// ------------------------------------------------------------------------------------------------
// Plan
// ------------------------------------------------------------------------------------------------

struct DevBuf {
    void* p = nullptr;
    size_t bytes = 0;
};

}  // namespace nufft

struct nufft_plan_s {
    int type = 0, dim = 0, prec = 0;   // prec 0 = fp32, 1 = fp64
    int64_t N[3] = {1, 1, 1};
    int64_t n[3] = {1, 1, 1};
    int w = 0;
    double beta = 0, eps = 0;
    double sigma = 2.0;                 // fine-grid upsampling factor
    double s[3] = {0, 0, 0};            // n_i / (2 pi)
    hipStream_t stream = nullptr;
    int device = 0;
    nufft_opts opts{};
    int method = NUFFT_METHOD_SM;

    // bin geometry
    int m[3] = {1, 1, 1};
    int nb[3] = {1, 1, 1};
    int64_t nbins = 0;
    int cap = 0;
    int nbits = 0;                      // bits of the largest sort key
    int colw = 0;                       // column order inside bins (see SortArgs)
    int colstep = 1;
    int ncol = 1;

    size_t bytes_in_use = 0;
    std::string last_error;

    // plan-owned device memory
    nufft::DevBuf grid;                 // fine grid, n^d complex
    nufft::DevBuf grid2;                // the FFT's output grid (out-of-place transforms)
    nufft::DevBuf pcorr;                // correction factors p_1 | p_2 | p_3 in precision T
    nufft::DevBuf fft_work;

    // points (setpts)
    int64_t M = -1;
    int64_t nsub = 0;
    nufft::DevBuf xs;                   // sorted coordinates, d arrays of M (precision T)
    nufft::DevBuf perm;                 // int32[M]
    nufft::DevBuf counts;               // int32[nbins]
    nufft::DevBuf offsets;              // int32[nbins + 1]
    nufft::DevBuf sub;                  // int32[3 * nsub] (bin, start, len)
    nufft::DevBuf range_err;            // unsigned int: stencil starts found outside their tile
    nufft::DevBuf sort_tmp;             // radix-sort scratch
    size_t sort_tmp_cap = 0;
    size_t pts_cap = 0;                 // capacity (points) of xs / perm

    // type 3: an inner type 1 plan spreads the scaled sources onto its fine grid (t3_n), an inner
    // type 2 plan evaluates that grid's Fourier sum at the scaled targets
    nufft_plan t3_spread = nullptr;
    nufft_plan t3_eval = nullptr;
    int64_t t3_n[3] = {0, 0, 0};
    int64_t K = -1;                     // targets (type 3)
    nufft::DevBuf t3_part;              // min / max partials
    nufft::DevBuf t3_y;                 // scaled sources, d arrays of M
    nufft::DevBuf t3_theta;             // scaled targets, d arrays of K
    nufft::DevBuf t3_pre;               // per-source phases (M complex)
    nufft::DevBuf t3_post;              // per-target factors (K complex)
    nufft::DevBuf t3_cp;                // phased strengths (M complex)
    nufft::DevBuf t3_cin;               // inner type 2 output (K complex)
    nufft::DevBuf t3_tab;               // quadrature table for phihat

    // many-vector batches: nv fine grids, and (fp64) the strengths gathered in sorted order
    nufft::DevBuf grid_many;
    nufft::DevBuf grid_many2;
    nufft::DevBuf c_many;

    // rocFFT
    rocfft_plan fft_fwd = nullptr;
    rocfft_plan fft_bwd = nullptr;
    rocfft_plan fft_many[2] = {nullptr, nullptr};   // batched forward / backward
    int fft_many_nv[2] = {0, 0};
    rocfft_execution_info fft_info = nullptr;

    // timing
    // stage timing (opts.timing): a ring of event sets, one set per step (a setpts, or an
    // execute of a direction already recorded in the current set), read without host syncs
    // until nufft_get_stage_times averages the steps recorded since its last call
    static constexpr int kEvRing = 16;
    hipEvent_t ev[kEvRing][16] = {};
    unsigned char ev_rec[kEvRing] = {};   // bits: 1 type 1 stages, 2 type 2 stages, 4 sort
    int ev_cur = 0;
    int ev_n = 0;                         // sets used since the last readout (<= kEvRing)
    bool ev_ok = false;
    void* host_tail = nullptr;            // pinned 128 B: setpts reads the subproblem count and bad-point flag here
    double stage_ms[8] = {0, 0, 0, 0, 0, 0, 0, 0};
};

namespace nufft {

// Kernel launchers (defined in the .hip files).  All return hipError_t of the launch.

// binsort.hip
// Division by a fixed d >= 1 as a multiply-high: q = (umulhi(x, mul) + x) >> shift with
// shift = ceil(log2 d), mul = floor(2^32 (2^shift - d) / d) + 1, exact for 0 <= x < 2^32.
struct FastDiv {
    uint32_t mul;
    int shift;
};
inline FastDiv make_fastdiv(int d) {
    int s = 0;
    while ((uint32_t(1) << s) < (uint32_t)d) ++s;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - (uint64_t)d)) / (uint64_t)d + 1;
    return {(uint32_t)m, s};
}
__device__ __forceinline__ int fast_div(int x, FastDiv f) {
    return (int)(((uint64_t)__umulhi((uint32_t)x, f.mul) + (uint64_t)(uint32_t)x) >> f.shift);
}

struct SortArgs {
    int dim;
    int prec;
    int64_t M;
    const void* x[3];
    int n[3];
    double s[3];
    int m[3];
    int nb[3];
    int nbins;
    int nbits;
    int cap;
    int colw;      // > 0: order points inside a bin by the x-y column block where their kernel
                   //       support starts, then by its z start (3D; colw = kernel width),
                   //       0: by original index only
    int colstep;   // column block edge s: support starts c_i in [0, m_i] grouped as c_i / s
    int ncol;      // keys per bin, ceil((m1 + 1) / s) ceil((m2 + 1) / s) (m3 + 1), else 1
    FastDiv fdm[3];  // division by m_i and by colstep (set by launch_sort)
    FastDiv fdc;
};
// Bytes of scratch the sort needs for M points and the plan's bin count.
size_t sort_scratch_bytes(int64_t M, int nbins, int dim, int prec);
// Clears nwords 32-bit words with a kernel (no memset node when the stream is captured).
hipError_t launch_zero_words(void* p, int64_t nwords, hipStream_t st);
// Runs bin index + radix sort + counts/offsets + subproblem counts.  Writes perm, counts,
// offsets and the coordinates in sorted order (xs_out: dim arrays of M, plan precision);
// writes the number of subproblems into *nsub_dev (device int64) and a nonzero value into
// *bad_dev when a point is invalid (*bad_dev must be zeroed by the caller).  Then the caller
// reads back and calls launch_build_subproblems_from.
hipError_t launch_sort(const SortArgs& a, int32_t* perm, int32_t* counts, int32_t* offsets,
                       void* xs_out, void* scratch, size_t scratch_bytes, int64_t* nsub_dev,
                       int* bad_dev, hipStream_t st);
// (bin, start, len) rows from the per-bin subproblem prefix left in the sort scratch.
// Points in the caller's order (GM method): checks and copies the coordinates into xs_out,
// perm = identity; no binning.
hipError_t launch_identity_order(const SortArgs& a, int32_t* perm, void* xs_out, int* bad_dev, hipStream_t st);
hipError_t launch_build_subproblems_from(int64_t M, int nbins, int dim, int prec, int cap, int64_t nsub,
                                         const int32_t* counts, const int32_t* offsets,
                                         const void* scratch, int32_t* sub, hipStream_t st);

// spread.hip / interp.hip / deconv.hip
struct GeomArgs {
    int dim;
    int w;
    int n[3];
    double s[3];
    int m[3];
    int nb[3];
    double beta;
    int64_t M;
    const void* xs[3];     // sorted coordinates
    const int32_t* perm;
    const int32_t* cperm;  // spreading reads strength cperm[j] for sorted point j; null: c is sorted
    const int32_t* sub;    // (bin, start, len)
    int64_t nsub;
    // many-vector launches: nv vectors along blockIdx.y; vector v reads / writes c + v cvs and
    // grid + v gvs (strides in complex values; nv = 1 for a single transform)
    int nv;
    int64_t cvs, gvs;
    // count of stencil starts found outside their subproblem's padded tile (clamped; the sort and
    // the kernels agree on every bin, so this stays 0)
    unsigned int* range_err;
};
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// columns: the points of each bin are in column order (3D), so the column-run kernel may run.
// c_scratch: device scratch of at least nv M complex values (fp64 plans gather c into it in
// sorted order before spreading).
hipError_t launch_spread(int prec, int method, const GeomArgs& g, const void* c, void* grid,
                         hipStream_t st, bool columns, void* c_scratch);
hipError_t launch_interp(int prec, int method, const GeomArgs& g, const void* grid, void* c,
                         hipStream_t st);
size_t interp_tile_bytes(int prec, int dim, int w, const int* m);
// nv vectors: fhat holds nv fine grids, f nv mode arrays, back to back.
hipError_t launch_deconvolve(int prec, int dim, const int64_t* N, const int64_t* n,
                             const void* pcorr, const void* fhat, void* f, hipStream_t st, int nv = 1);
hipError_t launch_precorrect_pad(int prec, int dim, const int64_t* N, const int64_t* n,
                                 const void* pcorr, const void* f, void* fhat, hipStream_t st, int nv = 1);
// Type 3 helpers (t3.hip).  minmax: per-block (min, max) pairs of one array into part
// (t3_minmax_blocks() pairs; min is NaN when the block saw a non-finite value).
int t3_minmax_blocks();
hipError_t launch_t3_minmax(int prec, const void* a, int64_t n, double* part, hipStream_t st);
// y = (((x - ctr) / div) * mul1) * mul2 in fp64, rounded to the plan precision
hipError_t launch_t3_scale(int prec, const void* x, int64_t n, double ctr, double div, double mul1, double mul2,
                           void* y, hipStream_t st);
// per-source phases pre (M complex) and per-target factors post (K complex); tab holds nq
// quadrature abscissae sin(theta_q) then nq weights for phihat(u) = sum_q wt_q cos(u sin(theta_q))
hipError_t launch_t3_factors(int prec, int dim, const double* C, const double* D, const double* gamma,
                             const double* alpha, const double* off, double corr, const void* const* x, int64_t M,
                             void* pre, const void* const* s, int64_t K, const double* tab, int nq, void* post,
                             hipStream_t st);
hipError_t launch_t3_cmul(int prec, const void* a, const void* b, int64_t n, void* out, hipStream_t st);
// Largest LDS tile (bytes) the SM spreading kernel may use.
size_t spread_lds_limit();
size_t spread_tile_bytes(int prec, int dim, int w, const int* m);
// LDS bytes of the 3D column-run spreading kernel for bins m (0 if it cannot run: m3 > 8).
size_t spread_col_lds_bytes(int prec, int w, const int* m);
int spread_col_per_cu(int prec, int w);   // workgroups of the column kernel meant to share a CU
// Whether 3D spreading with this kernel width uses the column-run kernel (needs the column order).
bool spread_uses_columns(int dim, int w);
int spread_col_step(int w);   // column block edge the 3D column kernel groups points by

}  // namespace nufft
