// Type 2 step 3: interpolation from the fine grid at the nonuniform points
// (cuFINUFFT paper, Sec. II-B, the weighted sum that follows eq. (12); kernel as in eq. (8)).
//
// Two schemes on the bin-sorted points of setpts:
//  * GM-sort (Sec. III-B): one thread per point in bin-sorted order, so neighbouring lanes read
//    neighbouring grid cells; each thread gathers its w^d cells from the fine grid in HBM.
//  * SM (the read-side counterpart of the SM spreading subproblems): one workgroup per
//    subproblem copies the padded bin of the fine grid into LDS with coalesced row reads, then
//    each lane evaluates one point from LDS.
// Both sum along x first and write c at the point's original index.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kInterpBlock = 128;

template <typename T, int DIM, int W>
__global__ void __launch_bounds__(kInterpBlock) k_interp_gm(GeomArgs g, const cplx<T>* __restrict__ grid,
                                                            cplx<T>* __restrict__ c) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
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
    if constexpr (DIM == 1) {
#pragma unroll
        for (int q1 = 0; q1 < W; ++q1) {
            const cplx<T> v = grid[idx[0][q1]];
            are += v.re * ker[0][q1];
            aim += v.im * ker[0][q1];
        }
    } else {
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
    }
    cplx<T> out;
    out.re = are;
    out.im = aim;
    c[g.perm[i]] = out;
}

// 3D: 768 lanes.  fp64 tiles leave room for one workgroup per CU (three wavefronts per SIMD);
// fp32 tiles for two (six per SIMD), which measured faster than 512 or 1024 lanes at w = 6.
// fp64 up to w = 12 takes 1024 lanes (at most 128 VGPRs, a few spilled at w = 10): 3D 256^3
// fp64 w = 10 interpolation 37.4 -> 36.3 ms.  fp32 below w = 5, whose small tiles fit four
// times, takes 512 lanes (32 wavefronts per CU instead of 24): 3D 128^3 w = 3 0.377 -> 0.358 ms.
template <typename T, int DIM, int W>
constexpr int kInterpSmBlock =
    (DIM == 3) ? ((sizeof(T) == 8 && W <= 12) ? 1024 : (sizeof(T) == 4 && W < 5) ? 512 : 768) : 512;

// Bank-aware order of the points inside a chunk (ORD, fp64 3D).  Every LDS read of a point is
// its stencil start plus an offset that is the same for all lanes of the read instruction, so
// how often the lanes of one read collide on an LDS bank depends only on the starts' cell
// addresses modulo R = kBankCells (16 cells of 16 bytes span the 64 four-byte banks).  In sorted
// order those residues are random, and a read waits on its most loaded bank.  ORD counts the
// chunk's points (one per lane of the workgroup) per residue class and lays them out rank-major:
// one point of every class, classes ascending, then a second point of every class that has one,
// and so on; lane i takes position i, so every run of R lanes holds R distinct residues until
// the classes run out.  Which lane evaluates a point changes nothing in its result.
//
// Measured (3D, N = 256^3, M = 2^27, eps = 1e-9, w = 10): 36.2 -> 31.4 ms.  The same order did not
// pay for its three barriers per chunk in fp32, whose interpolation issues few LDS bytes per
// VALU instruction (3D 128^3 w = 6: 0.78 -> 1.11 ms), nor for 2D fp64 (w = 13: 0.30 -> 0.33 ms).
template <typename T>
constexpr int kBankCells = 256 / (int)sizeof(cplx<T>);

// fp32 tiles in 2D and 3D are read in 16-byte pairs of cells.  A row of a point's stencil
// starts at any cell, so a lane reads the kPairReads aligned pairs from the even cell at or
// below its start and multiplies them by the x weights shifted by the start's parity (zero on
// the one or two cells outside the stencil).  That moves up to two cells more per row than
// 8-byte reads, but ds_read_b128 delivers about twice the bytes per clock of ds_read_b64 and the
// rows collide less often on the banks.  3D fp32, N = 128^3, M = 2^24 interpolation: w = 5 0.55 ->
// 0.49 ms, w = 6 0.80 -> 0.65 ms, w = 7 1.33 -> 0.96 ms, w = 8 2.77 -> 1.61 ms.  The x pitch
// of these tiles is even (rows start 16-byte aligned; the extra column is zero) and four zero
// cells follow the tile, so the last row's pairs stay inside the tile.
template <typename T, int DIM>
constexpr bool kPairRows = sizeof(T) == 4 && DIM >= 2;
template <int W>
constexpr int kPairReads = (W + 2) / 2;   // pairs covering w + 1 cells
constexpr int kPairPad = 4;                // zero cells after a paired tile

template <typename T, int DIM>
constexpr bool kInterpOrder = sizeof(T) == 8 && DIM == 3;

// LDS bytes of the ORD bookkeeping after the tile: lane -> point slot, residue counts, and per
// rank the number of earlier points and the mask of classes still present.
template <typename T, int DIM, int W>
constexpr size_t interp_order_bytes() {
    return (size_t)(3 * kInterpSmBlock<T, DIM, W> + kBankCells<T>) * 4;
}

template <typename T, int DIM, int W, bool ORD>
__global__ void __launch_bounds__((kInterpSmBlock<T, DIM, W>)) k_interp_sm(GeomArgs g, const cplx<T>* __restrict__ grid,
                                                              cplx<T>* __restrict__ c, int p1, int p2,
                                                              int p3) {
    constexpr int NB = kInterpSmBlock<T, DIM, W>;
    constexpr int R = kBankCells<T>;
    static_assert(R <= 32, "class masks are 32 bits");
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    extern __shared__ __align__(16) unsigned char smem[];
    cplx<T>* tile = (cplx<T>*)smem;
    constexpr bool PAIRS = kPairRows<T, DIM>;
    const int pc = PAIRS ? (p1 + 1) & ~1 : p1, pp = pc * p2;
    const int P = pc * p2 * p3;   // cells of the tile, x pitch pc
    int32_t* slot = (int32_t*)(smem + (((size_t)P * sizeof(cplx<T>) + 15) & ~(size_t)15));
    int32_t* cnt = slot + NB;
    int32_t* before = cnt + R;
    uint32_t* present = (uint32_t*)(before + NB);
    const int tid = threadIdx.x;
    const int sid = blockIdx.x;
    const int bin = g.sub[3 * sid + 0];
    const int start = g.sub[3 * sid + 1];
    const int len = g.sub[3 * sid + 2];
    int origin[3] = {0, 0, 0};
    {
        int b0 = bin % g.nb[0];
        int b1 = (bin / g.nb[0]) % g.nb[1];
        int b2 = bin / (g.nb[0] * g.nb[1]);
        origin[0] = b0 * g.m[0] - W / 2;
        if (DIM >= 2) origin[1] = b1 * g.m[1] - W / 2;
        if (DIM == 3) origin[2] = b2 * g.m[2] - W / 2;
    }
    // the coordinates of this thread's first point are requested before the tile copy, and
    // each later point's one chunk ahead, so their latency overlaps other work
    T xn[DIM];
    int32_t on = 0;   // output index (original order) of the next point
    if (tid < len) {
#pragma unroll
        for (int d = 0; d < DIM; ++d) xn[d] = ((const T*)g.xs[d])[(int64_t)start + tid];
        if (!ORD) on = g.perm[(int64_t)start + tid];
    }
    if (ORD && tid < R) cnt[tid] = 0;
    // copy the padded bin (with periodic wrap) into LDS; consecutive lanes read consecutive x
    const int pd[3] = {p1, p2, p3};
    auto copy = [&](auto fast) {
        constexpr bool FAST = decltype(fast)::value;
        CellWalk cw(tid, NB, pc, p2);
        for (int k = tid; k < P; k += NB, cw.next()) {
            if (PAIRS && cw.s1 >= p1) {
                tile[k] = cplx<T>{(T)0, (T)0};   // the pitch column of an odd row length
                continue;
            }
            const int g1 = wrap_pad<FAST>(origin[0] + cw.s1, g.n[0]);
            const int g2 = (DIM >= 2) ? wrap_pad<FAST>(origin[1] + cw.s2, g.n[1]) : 0;
            const int g3 = (DIM == 3) ? wrap_pad<FAST>(origin[2] + cw.s3, g.n[2]) : 0;
            tile[k] = grid[grid_index<FAST>(g1, g2, g3, g.n)];
        }
    };
    if (tile_fast(origin, pd, g.n, DIM)) copy(std::true_type{});
    else copy(std::false_type{});
    if (PAIRS && tid < kPairPad) tile[P + tid] = cplx<T>{(T)0, (T)0};
    __syncthreads();
    const T beta = (T)g.beta;
    for (int c0 = 0; c0 < len; c0 += NB) {
        const int nv = min(NB, len - c0);
        T xc[DIM];
#pragma unroll
        for (int d = 0; d < DIM; ++d) xc[d] = xn[d];
        int32_t oc = on;
        bool live = tid < nv;
        if constexpr (ORD) {
            // residue class of this thread's point (sorted position c0 + tid) and its rank there
            int r = 0, rank = 0;
            if (live) {
                int base = 0;
#pragma unroll
                for (int d = 0; d < DIM; ++d) {
                    double t = grid_t((double)xc[d], g.s[d]);
                    int l;
                    fold_t(t, g.n[d], l);
                    const int s0 = (int)ceil(__dsub_rn(t, 0.5 * (double)W)) - origin[d];
                    base += s0 * (d == 0 ? 1 : (d == 1 ? pc : pp));
                }
                r = base & (R - 1);
                rank = atomicAdd(&cnt[r], 1);
            }
            if (c0 + NB + tid < len) {
#pragma unroll
                for (int d = 0; d < DIM; ++d) xn[d] = ((const T*)g.xs[d])[(int64_t)start + c0 + NB + tid];
            }
            __syncthreads();
            if (tid < 64) {
                // per rank k: the points of lower rank, and the classes holding more than k points
                int most = 0;
                for (int q = 0; q < R; ++q) most = max(most, cnt[q]);
                for (int k = tid; k < most; k += 64) {
                    int sb = 0;
                    uint32_t pm = 0;
                    for (int q = 0; q < R; ++q) {
                        const int cq = cnt[q];
                        sb += min(cq, k);
                        pm |= (cq > k ? 1u : 0u) << q;
                    }
                    before[k] = sb;
                    present[k] = pm;
                }
                // the counts were read above by this same wavefront; clear them for the next chunk
                if (tid < R) cnt[tid] = 0;
            }
            __syncthreads();
            if (live) slot[before[rank] + __popc(present[rank] & ((1u << r) - 1u))] = tid;
            __syncthreads();
            if (live) {
                const int64_t j = (int64_t)start + c0 + slot[tid];
#pragma unroll
                for (int d = 0; d < DIM; ++d) xc[d] = ((const T*)g.xs[d])[j];
                oc = g.perm[j];
            }
        } else {
            if (c0 + NB + tid < len) {
                const int64_t jn = (int64_t)start + c0 + NB + tid;
#pragma unroll
                for (int d = 0; d < DIM; ++d) xn[d] = ((const T*)g.xs[d])[jn];
                on = g.perm[jn];
            }
        }
        if (!live) continue;
        T ker[DIM][W];
        int l0[3] = {0, 0, 0};
#pragma unroll
        for (int d = 0; d < DIM; ++d) {
            double t = grid_t((double)xc[d], g.s[d]);
            int l;
            fold_t(t, g.n[d], l);
            l0[d] = checked_start(es_weights<T, W>(t, beta, ker[d]) - origin[d], pd[d] - W, g.range_err);
        }
        T are = 0, aim = 0;
        if constexpr (DIM == 1) {
            const cplx<T>* row = tile + l0[0];
#pragma unroll
            for (int q1 = 0; q1 < W; ++q1) {
                const cplx<T> v = row[q1];
                are += v.re * ker[0][q1];
                aim += v.im * ker[0][q1];
            }
        } else if constexpr (PAIRS) {
            constexpr int NQ = kPairReads<W>;
            const int par = l0[0] & 1;
            T kxw[2 * NQ];
#pragma unroll
            for (int k = 0; k < 2 * NQ; ++k) {
                const T a = (k < W) ? ker[0][k] : (T)0;
                const T b = (k >= 1 && k - 1 < W) ? ker[0][k - 1] : (T)0;
                kxw[k] = par ? b : a;
            }
            // pc and pp are even, so every row of the stencil starts on a 16-byte boundary
            const float4* b4 = (const float4*)(tile + (l0[0] - par) + l0[1] * pc + (DIM == 3 ? l0[2] * pp : 0));
#pragma unroll
            for (int q3 = 0; q3 < (DIM == 3 ? W : 1); ++q3) {
                T pre = 0, pim = 0;
#pragma unroll
                for (int q2 = 0; q2 < W; ++q2) {
                    const float4* r = b4 + ((q2 * pc + q3 * pp) >> 1);
                    T rre = 0, rim = 0;
#pragma unroll
                    for (int h = 0; h < NQ; ++h) {
                        const float4 v = r[h];
                        rre += v.x * kxw[2 * h];
                        rim += v.y * kxw[2 * h];
                        rre += v.z * kxw[2 * h + 1];
                        rim += v.w * kxw[2 * h + 1];
                    }
                    pre += rre * ker[1][q2];
                    pim += rim * ker[1][q2];
                }
                const T kz = (DIM == 3) ? ker[DIM - 1][q3] : (T)1;
                are += pre * kz;
                aim += pim * kz;
            }
        } else {
#pragma unroll
        for (int q3 = 0; q3 < (DIM == 3 ? W : 1); ++q3) {
            T pre = 0, pim = 0;
#pragma unroll
            for (int q2 = 0; q2 < W; ++q2) {
                const cplx<T>* row = tile + l0[0] + (l0[1] + q2) * pc + (DIM == 3 ? (l0[2] + q3) * pp : 0);
                T rre = 0, rim = 0;
#pragma unroll
                for (int q1 = 0; q1 < W; ++q1) {
                    const cplx<T> v = row[q1];
                    rre += v.re * ker[0][q1];
                    rim += v.im * ker[0][q1];
                }
                pre += rre * ker[1][q2];
                pim += rim * ker[1][q2];
            }
            const T kz = (DIM == 3) ? ker[DIM - 1][q3] : (T)1;
            are += pre * kz;
            aim += pim * kz;
        }
        }
        cplx<T> out;
        out.re = are;
        out.im = aim;
        c[oc] = out;
    }
}

template <typename T, int DIM, int W>
hipError_t interp_w(int method, const GeomArgs& g, const void* grid, void* c, hipStream_t st) {
    if (g.M <= 0) return hipSuccess;
    if (method == NUFFT_METHOD_GM_SORT || method == NUFFT_METHOD_GM) {
        dim3 grd((unsigned)((g.M + kInterpBlock - 1) / kInterpBlock), (unsigned)g.nv);
        k_interp_gm<T, DIM, W><<<grd, kInterpBlock, 0, st>>>(g, (const cplx<T>*)grid, (cplx<T>*)c);
        return hipGetLastError();
    }
    if (g.nsub <= 0) return hipSuccess;
    const int p1 = g.m[0] + W, p2 = (DIM >= 2) ? g.m[1] + W : 1, p3 = (DIM == 3) ? g.m[2] + W : 1;
    const size_t tile = kPairRows<T, DIM> ? ((size_t)((p1 + 1) & ~1) * p2 * p3 + kPairPad) * sizeof(cplx<T>)
                                          : (size_t)p1 * p2 * p3 * sizeof(cplx<T>);
    if (tile > spread_lds_limit()) return hipErrorInvalidConfiguration;
    // the bank-aware order needs its bookkeeping beside the tile; a tile too large for both runs
    // in sorted order
    const size_t lds_ord = ((tile + 15) & ~(size_t)15) + interp_order_bytes<T, DIM, W>();
    auto go = [&](auto ord) -> hipError_t {
        constexpr bool ORD = decltype(ord)::value;
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void*)k_interp_sm<T, DIM, W, ORD>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)spread_lds_limit());
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        k_interp_sm<T, DIM, W, ORD><<<dim3((unsigned)g.nsub, (unsigned)g.nv), (kInterpSmBlock<T, DIM, W>),
                                      ORD ? lds_ord : tile, st>>>(g, (const cplx<T>*)grid, (cplx<T>*)c, p1, p2, p3);
        return hipGetLastError();
    };
    if constexpr (kInterpOrder<T, DIM>) {
        if (lds_ord <= spread_lds_limit()) return go(std::true_type{});
    }
    return go(std::false_type{});
}

template <typename T, int DIM>
hipError_t interp_dim(int method, const GeomArgs& g, const void* grid, void* c, hipStream_t st) {
    switch (g.w) {
#define NUFFT_CASE(WW) case WW: return interp_w<T, DIM, WW>(method, g, grid, c, st);
        NUFFT_CASE(2) NUFFT_CASE(3) NUFFT_CASE(4) NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7)
        NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10) NUFFT_CASE(11) NUFFT_CASE(12) NUFFT_CASE(13)
        NUFFT_CASE(14) NUFFT_CASE(15) NUFFT_CASE(16)
#undef NUFFT_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_interp(int prec, int method, const GeomArgs& g, const void* grid, void* c,
                         hipStream_t st) {
    if (prec == 0)
        return g.dim == 1   ? interp_dim<float, 1>(method, g, grid, c, st)
               : g.dim == 2 ? interp_dim<float, 2>(method, g, grid, c, st)
                            : interp_dim<float, 3>(method, g, grid, c, st);
    return g.dim == 1   ? interp_dim<double, 1>(method, g, grid, c, st)
           : g.dim == 2 ? interp_dim<double, 2>(method, g, grid, c, st)
                        : interp_dim<double, 3>(method, g, grid, c, st);
}

size_t interp_tile_bytes(int prec, int dim, int w, const int* m) {
    size_t cells = 1;
    for (int i = 0; i < dim; ++i) cells *= (size_t)(m[i] + w);
    if (prec == 0 && dim >= 2) {
        // paired rows: even x pitch and the zero cells after the tile
        cells = cells / (size_t)(m[0] + w) * (size_t)((m[0] + w + 1) & ~1) + kPairPad;
    }
    return cells * 2 * (prec == 0 ? sizeof(float) : sizeof(double));
}

}  // namespace nufft
