// Type 1 step 1: spreading of the nonuniform points onto the fine grid
// (cuFINUFFT paper, Sec. II-A eq. (7) with the periodised tensor-product ES kernel of eq. (8)).
//
// Two schemes, both on the bin-sorted points of setpts (Sec. III-A):
//  * SM: one workgroup per subproblem (at most `cap` sorted points of one bin).  The workgroup
//    accumulates into an LDS copy of its padded bin (the bin plus the kernel's reach on each
//    side, eq. (13)-(14)), then adds the padded bin into the fine grid with periodic wrap
//    (eq. (15)).
//  * GM-sort: one thread per sorted point adding its w^d contributions straight into the fine
//    grid with global atomics.
//
// gfx950 notes.  LDS float atomics are slow on this part (ds_add_f32 measured ~0.33 lane-op per
// clock per CU against ~7.8 for ds_add_f64), so the LDS tile accumulates in fp64 for both
// precisions: each complex update is two ds_add_f64 into separate real/imaginary planes.  Work
// in a chunk of staged points is split into (point, q1, q2) items -- the x-y patch of a point's
// stencil -- and each item walks the w cells along z, so a wavefront's lanes hit one or two
// w x w patches whose rows are spread over the LDS banks by the padded row pitch.  Workgroups
// of 1024 lanes keep 16 wavefronts per CU even when one padded bin fills most of the LDS.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kSpreadBlock = 1024;   // 16 wavefronts: one workgroup keeps a CU busy on its own
constexpr int kGmBlock = 128;

// One staged point of the point-patch kernel: its x and y weights, strength, the tile offset of
// its stencil start (l0x + l0y pc + l0z pp) and, in 3D, its z weights widened to fp64.  Records
// of 20 or 22 words put the x (or y) weights of up to 16 neighbouring points on distinct banks.
template <typename T, int DIM, int W>
struct SmRec {
    static constexpr int kWP = (W + 3) & ~3;                      // padded row of T weights (16 B aligned)
    static constexpr int kWD = (W + 1) & ~1;                      // padded row of fp64 z weights
    T kx[kWP];
    T ky[kWP];
    cplx<T> cv;
    int base;
    int pad_;
    double kz[DIM == 3 ? kWD : 1];
};

// Points staged per round: about 24 KB of LDS.
template <typename T, int DIM, int W>
struct SmCfg {
    static constexpr int kPerPoint = (int)sizeof(SmRec<T, DIM, W>);
    static constexpr int kRaw = 24576 / kPerPoint;
    static constexpr int kChunk = kRaw >= 256 ? 256 : (kRaw < 32 ? 32 : (kRaw & ~31));
};

template <typename T, int DIM, int W>
struct Stage {
    using C = SmCfg<T, DIM, W>;
    static constexpr int CH = C::kChunk;
    SmRec<T, DIM, W> rec[CH];
};

// A copy of a per-lane value that the optimizer cannot split into scalar and vector parts.
__device__ __forceinline__ uint32_t vector_copy(uint32_t v) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// LDS tile of a padded bin: separate fp64 planes for real and imaginary parts, row pitch pc with
// pc = W (mod 16), so the w x w patch of one point's x-y stencil covers the 16 bank pairs evenly.
__host__ __device__ inline int tile_row_pitch(int p1, int w) {
    int pc = p1;
    while (((pc - w) % 16 + 16) % 16 != 0) ++pc;
    return pc;
}

// TWO: compiled for two workgroups per CU (at most 64 VGPRs, with spills if need be); the
// launcher takes it when two tiles fit in LDS but the plain build's registers would not let
// the second workgroup in.
template <typename T, int DIM, int W, bool TWO>
__global__ void __launch_bounds__(kSpreadBlock) __attribute__((amdgpu_waves_per_eu(TWO ? 8 : 1)))
k_spread_sm(GeomArgs g, const cplx<T>* __restrict__ c, cplx<T>* __restrict__ grid, int p1, int p2, int p3,
            int pc) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    using St = Stage<T, DIM, W>;
    constexpr int CH = St::CH;
    constexpr int WW = W * W;
    constexpr int PPP = kSpreadBlock / WW;          // points per pass of the workgroup
    extern __shared__ __align__(16) unsigned char smem[];
    const int pp = pc * p2;                          // plane pitch
    const int PL = pp * p3;                          // padded cells
    double* tre = (double*)smem;
    double* tim = tre + PL;
    St* st = (St*)(tim + PL);

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
        origin[1] = b1 * g.m[1] - W / 2;
        if (DIM == 3) origin[2] = b2 * g.m[2] - W / 2;
    }
    const int pd[3] = {p1, p2, p3};
    for (int k = threadIdx.x; k < 2 * PL; k += kSpreadBlock) tre[k] = 0.0;

    // this thread's fixed slot (q1, q2) of the x-y stencil patch, and its tile offset
    const int t = threadIdx.x;
    const int p_first = t / WW;
    const int slot = t - p_first * WW;
    const int q2 = slot / W;
    const int q1 = slot - q2 * W;
    const int qoff = q1 + q2 * pc;
    const bool active = p_first < PPP;

    const T beta = (T)g.beta;
    // staging thread (point sp, dimension si < DIM; in 3D four lanes per point, the fourth idle,
    // so that a point's lanes sit in one aligned quad): its raw coordinate and strength for the
    // next chunk are requested while the current chunk is accumulated
    constexpr int SPW = (DIM == 3) ? 4 : DIM;
    static_assert(SPW * CH <= kSpreadBlock, "one staging lane per point and dimension");
    const int sp = threadIdx.x / SPW, si = threadIdx.x - (threadIdx.x / SPW) * SPW;
    const int spitch = (si == 0) ? 1 : (si == 1 ? pc : pp);
    T xr = (T)0;
    cplx<T> cr;
    cr.re = (T)0;
    cr.im = (T)0;
    auto fetch = [&](int c0) {
        if (si < DIM && sp < min(CH, len - c0)) {
            const int64_t j = (int64_t)start + c0 + sp;
            xr = ((const T*)g.xs[si])[j];
            if (si == 0) cr = c[g.cperm ? g.cperm[j] : j];
        }
    };
    using Rec = SmRec<T, DIM, W>;
    using LRec = __attribute__((address_space(3))) const Rec;
    using LT = __attribute__((address_space(3))) const T;
    constexpr uint32_t kStep = (uint32_t)(PPP * sizeof(Rec));
    fetch(0);
    for (int c0 = 0; c0 < len; c0 += CH) {
        const int np = min(CH, len - c0);
        __syncthreads();   // previous chunk consumed (and tile zeroed on the first round)
        // stage kernel weights: one thread per (point, dimension); the point's lanes add up the
        // tile offset of its stencil start
        int part = 0;
        if (si < DIM && sp < np) {
            Rec& r = st->rec[sp];
            double tt = grid_t((double)xr, g.s[si]);
            int l;
            fold_t(tt, g.n[si], l);
            T ker[W];
            const int l0 = checked_start(es_weights<T, W>(tt, beta, ker) - origin[si], pd[si] - W, g.range_err);
            if (si == 0) {
#pragma unroll
                for (int q = 0; q < W; ++q) r.kx[q] = ker[q];
                r.cv = cr;
            } else if (si == 1) {
#pragma unroll
                for (int q = 0; q < W; ++q) r.ky[q] = ker[q];
            } else {
#pragma unroll
                for (int q = 0; q < W; ++q) r.kz[DIM == 3 ? q : 0] = (double)ker[q];
            }
            part = l0 * spitch;
        }
        part += __shfl_xor(part, 1);
        if (DIM == 3) part += __shfl_xor(part, 2);
        if (si == 0 && sp < np) st->rec[sp].base = part;
        if (c0 + CH < len) fetch(c0 + CH);
        __syncthreads();
        if (active && p_first < np) {
            // this item's record fields as whole vector registers, advanced PPP records at a time
            uint32_t ar = vector_copy((uint32_t)(uintptr_t)(LRec*)&st->rec[p_first]);
            uint32_t ax = vector_copy((uint32_t)(uintptr_t)(LT*)&st->rec[p_first].kx[q1]);
            uint32_t ay = vector_copy((uint32_t)(uintptr_t)(LT*)&st->rec[p_first].ky[q2]);
            for (int p = p_first; p < np; p += PPP) {
                // read everything this item needs before the first atomic, so the LDS counter
                // waits only on these reads and the atomics then issue back to back
                LRec* R = (LRec*)(uintptr_t)ar;
                cplx<T> cv;
                cv.re = R->cv.re;
                cv.im = R->cv.im;
                const int base = R->base + qoff;
                double kz[DIM == 3 ? W : 1];
                if (DIM == 3) {
#pragma unroll
                    for (int q3 = 0; q3 < W; ++q3) kz[q3] = R->kz[DIM == 3 ? q3 : 0];
                }
                const T wxy = *(LT*)(uintptr_t)ax * *(LT*)(uintptr_t)ay;
                ar += kStep;
                ax += kStep;
                ay += kStep;
                const double vre = (double)(cv.re * wxy);
                const double vim = (double)(cv.im * wxy);
                if (DIM == 2) {
                    atomicAdd(tre + base, vre);
                    atomicAdd(tim + base, vim);
                } else {
#pragma unroll
                    for (int q3 = 0; q3 < W; ++q3) {
                        atomicAdd(tre + base + q3 * pp, vre * kz[q3]);
                        atomicAdd(tim + base + q3 * pp, vim * kz[q3]);
                    }
                }
            }
        }
    }
    __syncthreads();
    // flush the padded bin with periodic wrap (eq. (15)): lane pairs take one cell, the even lane
    // its real and the odd lane its imaginary part, consecutive pairs consecutive x, so one
    // atomic instruction covers contiguous grid bytes
    const int P = p1 * p2 * p3;
    auto flush = [&](auto fast) {
        constexpr bool FAST = decltype(fast)::value;
        const int comp = threadIdx.x & 1;
        const double* src = comp ? tim : tre;
        CellWalk cw(threadIdx.x >> 1, kSpreadBlock / 2, p1, p2);
        for (int k = threadIdx.x >> 1; k < P; k += kSpreadBlock / 2, cw.next()) {
            const double v = src[cw.s1 + cw.s2 * pc + cw.s3 * pp];
            if (v == 0.0) continue;
            const int g1 = wrap_pad<FAST>(origin[0] + cw.s1, g.n[0]);
            const int g2 = wrap_pad<FAST>(origin[1] + cw.s2, g.n[1]);
            const int g3 = (DIM == 3) ? wrap_pad<FAST>(origin[2] + cw.s3, g.n[2]) : 0;
            const size_t gi = grid_index<FAST>(g1, g2, g3, g.n);
            unsafeAtomicAdd((T*)grid + 2 * gi + comp, (T)v);
        }
    };
    if (tile_fast(origin, pd, g.n, DIM)) flush(std::true_type{});
    else flush(std::false_type{});
}

// ------------------------------------------------------------------------------------------
// 3D column-run spreading.
//
// The lanes of a wavefront (or of kSlotWaves wavefronts) own a B x B block of x-y columns of
// the padded bin and keep the whole z-line of each column (8 + w cells) in registers, in the
// transform's precision (a run's sum is added to the LDS bin, also in the transform's
// precision, when the run ends).  A
// point whose kernel support starts at column (c1, c2) fits in the block at origin
// (s floor(c1 / s), s floor(c2 / s)) with s = B - w + 1, so setpts orders the points of a bin
// by that column block and a wavefront accumulates every point of a block in registers; the
// lines are added to the LDS padded bin only when the block changes (about s^2 m3 points per
// run).  The point's x and y weights are staged as zero-padded B-wide windows, so each lane
// reads its own two weights and all lanes stay live in the flush.  All lanes work on the same
// point, so its z offset inside the line is wave-uniform: a scalar branch picks the w
// registers it updates, and each point costs 2 w FMAs per lane.  The LDS bin is stored
// z-fastest in separate real and imaginary planes (cell = (x + y p1) pz + z) so a line is
// flushed with fixed offsets (an odd pz puts the lanes of a flush on distinct banks).  Blocks of
// different wavefronts overlap, so the flush is atomic.
// Per-point weights are staged per wavefront (no workgroup barrier inside the loop).
// ------------------------------------------------------------------------------------------
// column block edge per kernel width: one wavefront for w <= 6, two up to 10, three above
__host__ __device__ constexpr int col_block_edge(int w) { return w <= 6 ? 8 : (w <= 10 ? 11 : (w == 11 ? 12 : 13)); }

// fp64 z-lines need twice the registers per lane, so 768 lanes.  fp32 plans keep the bin in
// fp32 and up to w = 8 run 768 lanes, so that two workgroups share a CU (LDS and registers):
// 3D fp32, N = 128^3, M = 2^24 spreads in 1.36 ms instead of 1.72 ms at w = 6 (with one
// 1024-lane workgroup on an fp64 bin), 1.26 instead of 1.71 ms at w = 5, 2.32 instead of
// 3.10 ms at w = 7 and 2.83 instead of 3.46 ms at w = 8.
template <typename T, int W>
constexpr int kColBlock = (sizeof(T) == 4 && W > 8) ? 1024 : 768;

// workgroups of the column kernel meant to share one CU (the bins are chosen to fit, and the
// kernel is built for the registers that allow it)
template <typename T, int W>
constexpr int kColPerCu = (sizeof(T) == 4 && W <= 8) ? 2 : 1;

template <typename T, int W>
struct ColCfg {
    static constexpr int kZ = 8 + W;                        // z extent of the padded bin (m3 = 8)
    // z pitch of the LDS bin: odd, so the lanes of a line flush fall on distinct banks, except
    // for fp32 bins up to w = 6, where the unpadded pitch leaves room for 21-point stages with two
    // workgroups per CU (the flush is rare; w = 6 spread 1.39 -> 1.35 ms)
    static constexpr int kPZ = (sizeof(T) == 4 && W <= 6) ? kZ : (kZ | 1);
    static constexpr int kB = col_block_edge(W);            // column block edge
    static constexpr int kS = kB - W + 1;                   // support starts per block edge
    static constexpr int kBlock = kColBlock<T, W>;
    static constexpr int kWaves = kBlock / 64;
    static constexpr int kSlotWaves = (kB * kB + 63) / 64;  // wavefronts sharing one slice
    // points staged per round (3 lanes each), sized so that with two fp32 workgroups per CU
    // the stages of 12 wavefronts and the bin fit twice in the LDS: 16 x 16 x 8 bins at
    // w <= 6 (80,416 bytes at w = 6), 16 x 8 x 8 at w = 7 and 8
    static constexpr int kPiece = (sizeof(T) == 4) ? (W == 8 ? 16 : 21) : 6;
    static constexpr int kWZ = (sizeof(T) == 4) ? ((W + 3) & ~3) : ((W + 1) & ~1);  // 16-byte rows
};

template <typename T, int W>
struct ColStage {
    using C = ColCfg<T, W>;
    // a point's z weights then its strength, in one 16-byte-aligned row: every lane reads the
    // row from one address
    static constexpr int kRow = (W + 2 + 3) & ~3;
    T kzc[C::kPiece][kRow];
    // x and y weights placed in the point's block window (zero elsewhere); the odd row pitch puts
    // the staging lanes' stores on distinct banks
    T kx[C::kPiece][C::kB | 1];
    T ky[C::kPiece][C::kB | 1];
};

template <int V>
struct IntC {
    static constexpr int value = V;
};

// A copy of a wave-uniform value that the optimizer cannot see through.
__device__ __forceinline__ int uniform_copy(int v) {
    int r;
    asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
    return r;
}

// Clears a register in place (a plain assignment of 0 lets the allocator rotate the whole
// register line through copies at the loop head).
__device__ __forceinline__ void zero_in_place(double& v) { asm volatile("v_mov_b64 %0, 0" : "+v"(v)); }
__device__ __forceinline__ void zero_in_place(float& v) { asm volatile("v_mov_b32 %0, 0" : "+v"(v)); }

// Adds a register z-line into an LDS bin line t[0..Z).  fp64 bins use the LDS float atomic.
// fp32 bins use compare-and-swap: the LDS fp32 atomic add runs at a third of a lane per clock
// per CU on this part, a read plus compare-and-swap at about 6.6 (as fast as the fp64 add).
// The reads and swaps are issued in batches of Z/2 so their latencies overlap; a swap that
// lost a race with another wavefront (an overlapping column block) is retried.
template <int Z>
__device__ __forceinline__ void lds_line_add(double* t, const float (&a)[Z]) {
#pragma unroll
    for (int z = 0; z < Z; ++z) atomicAdd(t + z, (double)a[z]);
}
template <int Z>
__device__ __forceinline__ void lds_line_add(double* t, const double (&a)[Z]) {
#pragma unroll
    for (int z = 0; z < Z; ++z) atomicAdd(t + z, a[z]);
}
template <int Z>
__device__ __forceinline__ void lds_line_add(float* t, const float (&a)[Z]) {
    unsigned int* u = (unsigned int*)t;
    constexpr int H = (Z + 1) / 2;
#pragma unroll
    for (int h = 0; h < Z; h += H) {
        constexpr int n = H;
        unsigned int want[n], got[n];
#pragma unroll
        for (int i = 0; i < n; ++i)
            if (h + i < Z) want[i] = u[h + i];
#pragma unroll
        for (int i = 0; i < n; ++i)
            if (h + i < Z) got[i] = atomicCAS(u + h + i, want[i], __float_as_uint(__uint_as_float(want[i]) + a[h + i]));
#pragma unroll
        for (int i = 0; i < n; ++i) {
            if (h + i >= Z) continue;
            while (got[i] != want[i]) {
                want[i] = got[i];
                got[i] = atomicCAS(u + h + i, want[i], __float_as_uint(__uint_as_float(want[i]) + a[h + i]));
            }
        }
    }
}

// Adds the point's w z-weights times v into the register line at the wave-uniform offset Z0.
template <int W, int Z, int Z0, typename A>
__device__ __forceinline__ void col_acc(A (&are)[Z], A (&aim)[Z], const A (&kz)[W], A vre, A vim) {
#pragma unroll
    for (int q = 0; q < W; ++q) {
        are[Z0 + q] = fma(vre, kz[q], are[Z0 + q]);
        aim[Z0 + q] = fma(vim, kz[q], aim[Z0 + q]);
    }
}

// One point's operands for a lane of a column block: its x and y window weights, the z weights
// and the strength, read from a stage.
template <typename T, int W>
struct ColPt {
    cplx<T> cv;
    T kx, ky;
    T kz[W];
    template <typename Stage>
    __device__ __forceinline__ void load(const Stage& st, int p, int q1, int q2) {
        cv = st.cv[p];
        kx = st.kx[p][q1];
        ky = st.ky[p][q2];
#pragma unroll
        for (int q = 0; q < W; ++q) kz[q] = st.kz[p][q];
    }
    template <int Z, int Z0>
    __device__ __forceinline__ void add(T (&are)[Z], T (&aim)[Z]) const {
        const T wxy = kx * ky;
        col_acc<W, Z, Z0>(are, aim, kz, cv.re * wxy, cv.im * wxy);
    }
};

// Adds a column kernel's padded bin (z fastest with pitch PZ, z extent pd[2]) to the fine grid
// with periodic wrap (eq. (15)).  Lane pairs take one cell (the even lane its real part, the odd
// lane its imaginary part), consecutive pairs consecutive x, then y, then z, so one atomic
// instruction covers contiguous grid bytes: 3D fp32 w = 6, M = 2^24 spread 1.36 -> 1.30 ms
// against one lane per cell and two atomic instructions.
template <typename T, int BLOCK, int PZ, typename TT>
__device__ __forceinline__ void flush_columns(const GeomArgs& g, const TT* tre, const TT* tim,
                                              cplx<T>* grid, const int* origin, const int* pd, int p1, int p2) {
    const int P = p1 * p2 * pd[2];
    auto run = [&](auto fast) {
        constexpr bool FAST = decltype(fast)::value;
        const int comp = threadIdx.x & 1;
        const TT* src = comp ? tim : tre;
        CellWalk cw(threadIdx.x >> 1, BLOCK / 2, p1, p2);
        for (int k = threadIdx.x >> 1; k < P; k += BLOCK / 2, cw.next()) {
            const TT v = src[(cw.s1 + cw.s2 * p1) * PZ + cw.s3];
            if (v == (TT)0) continue;
            const int g1 = wrap_pad<FAST>(origin[0] + cw.s1, g.n[0]);
            const int g2 = wrap_pad<FAST>(origin[1] + cw.s2, g.n[1]);
            const int g3 = wrap_pad<FAST>(origin[2] + cw.s3, g.n[2]);
            const size_t gi = grid_index<FAST>(g1, g2, g3, g.n);
            unsafeAtomicAdd((T*)grid + 2 * gi + comp, (T)v);
        }
    };
    if (tile_fast(origin, pd, g.n, 3)) run(std::true_type{});
    else run(std::false_type{});
}

template <typename T, int W>
__global__ void __launch_bounds__((kColBlock<T, W>)) __attribute__((amdgpu_waves_per_eu(kColPerCu<T, W> == 2 ? 6 : 1)))
k_spread_col(GeomArgs g, const cplx<T>* __restrict__ c,
                                                                     cplx<T>* __restrict__ grid, int p1, int p2) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    using C = ColCfg<T, W>;
    using St = ColStage<T, W>;
    constexpr int Z = C::kZ;
    constexpr int PZ = C::kPZ;
    constexpr int B = C::kB;
    constexpr int S = C::kS;
    constexpr int SW = C::kSlotWaves;
    constexpr int SLICES = C::kWaves / SW;
    constexpr int PIECE = C::kPiece;
    constexpr int BLOCK = C::kBlock;
    extern __shared__ __align__(16) unsigned char smem[];
    const int PL = p1 * p2 * PZ;
    T* tre = (T*)smem;                       // real and imaginary planes, cell (x + y p1) pz + z
    T* tim = tre + PL;
    St* stages = (St*)(tim + PL);

    const int sid = blockIdx.x;
    const int bin = g.sub[3 * sid + 0];
    const int start = g.sub[3 * sid + 1];
    const int len = g.sub[3 * sid + 2];
    int origin[3];
    {
        int b0 = bin % g.nb[0];
        int b1 = (bin / g.nb[0]) % g.nb[1];
        int b2 = bin / (g.nb[0] * g.nb[1]);
        origin[0] = b0 * g.m[0] - W / 2;
        origin[1] = b1 * g.m[1] - W / 2;
        origin[2] = b2 * g.m[2] - W / 2;
    }
    const int pd[3] = {p1, p2, Z};
    for (int k = threadIdx.x; k < 2 * PL; k += BLOCK) tre[k] = (T)0;
    __syncthreads();

    // the wavefront index is uniform: say so, so the slice bounds and the point loop stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int slice = wave / SW, sub_wave = wave - slice * SW;
    St* ws = stages + wave;
    const int slot = sub_wave * 64 + lane;
    // lanes past the B x B block run along (column (0, 0)'s weights) but never flush
    const bool valid = (slot < B * B) && (slice < SLICES);
    const int q2 = valid ? slot / B : 0;
    const int q1 = valid ? slot - q2 * B : 0;
    const int per = (len + SLICES - 1) / SLICES;
    const int a = (slice < SLICES) ? min(len, slice * per) : len;
    const int b = (slice < SLICES) ? min(len, a + per) : len;

    T are[Z], aim[Z];
#pragma unroll
    for (int z = 0; z < Z; ++z) {
        are[z] = (T)0;
        aim[z] = (T)0;
    }
    int cur = -1, cell = 0;
    bool live = false;   // this lane's column lies inside the padded bin
    const T beta = (T)g.beta;
    // staging lane (point sp, dimension si); the raw coordinate and strength of the next piece
    // are loaded into registers while the current piece is processed
    // (the permutation entry that selects a strength is requested one piece earlier still)
    const int sp = lane / 3, si = lane - (lane / 3) * 3;
    T xr = (T)0;
    cplx<T> cr;
    cr.re = (T)0;
    cr.im = (T)0;
    int32_t pr = 0;
    auto perm_of = [&](int64_t j) -> int32_t { return g.cperm ? g.cperm[j] : (int32_t)j; };
    if (lane < min(PIECE, b - a) * 3) {
        const int64_t j = (int64_t)start + a + sp;
        xr = ((const T*)g.xs[si])[j];
        if (si == 0) cr = c[perm_of(j)];
    }
    if (si == 0 && lane < min(PIECE, b - a - PIECE) * 3) pr = perm_of((int64_t)start + a + PIECE + sp);
    for (int p0 = a; p0 < b; p0 += PIECE) {
        const int np = min(PIECE, b - p0);
        int l0 = 0;
        if (lane < np * 3) {
            double tt = grid_t((double)xr, g.s[si]);
            int l;
            fold_t(tt, g.n[si], l);
            T ker[W];
            l0 = checked_start(es_weights<T, W>(tt, beta, ker) - origin[si], pd[si] - W, g.range_err);
            if (si < 2) {
                // x or y: the block index, and the weights placed in the block's window
                const int blk = l0 / S;
                const int off = l0 - blk * S;
                T* win = (si == 0) ? ws->kx[sp] : ws->ky[sp];
#pragma unroll
                for (int q = 0; q < B; ++q) win[q] = (T)0;
#pragma unroll
                for (int q = 0; q < W; ++q) win[off + q] = ker[q];
                if (si == 0) {
                    ws->kzc[sp][W] = cr.re;
                    ws->kzc[sp][W + 1] = cr.im;
                }
                l0 = blk;
            } else {
#pragma unroll
                for (int q = 0; q < W; ++q) ws->kzc[sp][q] = ker[q];
            }
        }
        // lane 3 sp packs the point's x block | y block << 8 | z start << 16
        const int ly = __shfl(l0, lane + 1);
        const int lz = __shfl(l0, lane + 2);
        const int key = l0 | (ly << 8) | (lz << 16);
        {
            const int pn = p0 + PIECE;
            if (lane < min(PIECE, b - pn) * 3) {
                const int64_t j = (int64_t)start + pn + sp;
                xr = ((const T*)g.xs[si])[j];
                if (si == 0) cr = c[pr];
            }
            if (si == 0 && lane < min(PIECE, b - pn - PIECE) * 3) pr = perm_of((int64_t)start + pn + PIECE + sp);
        }
        // the staged piece is written and read by this wavefront only
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // The points arrive grouped by (column block, z start).  One scalar dispatch on the z
        // start covers a whole group, whose points then cost only their loads and 2 w FMAs.
        auto group = [&](auto z0c, int p, int kp) -> int {
            constexpr int Z0 = decltype(z0c)::value;
            using LT = __attribute__((address_space(3))) const T;
            constexpr uint32_t kRowBytes = (uint32_t)sizeof(ws->kx[0]);
            // this lane's x and y weight addresses as whole vector registers, advanced one staged
            // point at a time (left to itself the compiler re-adds the stage base on every point)
            uint32_t ax = vector_copy((uint32_t)(uintptr_t)(LT*)&ws->kx[p][q1]);
            uint32_t ay = vector_copy((uint32_t)(uintptr_t)(LT*)&ws->ky[p][q2]);
            // lane of the next point's key, kept in a scalar register
            int kl = uniform_copy(3 * p + 3);
            ColPt<T, W> A;
            while (true) {
#pragma unroll
                for (int q = 0; q < W; ++q) A.kz[q] = ws->kzc[p][q];
                A.cv.re = ws->kzc[p][W];
                A.cv.im = ws->kzc[p][W + 1];
                A.kx = *(LT*)(uintptr_t)ax;
                A.ky = *(LT*)(uintptr_t)ay;
                A.template add<Z, Z0>(are, aim);
                ++p;
                ax += kRowBytes;
                ay += kRowBytes;
                if (p >= np || __builtin_amdgcn_readlane(key, kl) != kp) break;
                kl = uniform_copy(kl + 3);
            }
            return p;
        };
        int p = 0;
        while (p < np) {
            const int kp = __builtin_amdgcn_readlane(key, 3 * p);
            const int col = kp & 0xffff;
            if (col != cur) {
                if (cur >= 0 && live) {
                    lds_line_add<Z>(tre + cell, are);
                    lds_line_add<Z>(tim + cell, aim);
                }
#pragma unroll
                for (int z = 0; z < Z; ++z) {
                    zero_in_place(are[z]);
                    zero_in_place(aim[z]);
                }
                cur = col;
                const int cx = (col & 0xff) * S + q1, cy = (col >> 8) * S + q2;
                live = valid && cx < p1 && cy < p2;
                cell = (cx + cy * p1) * PZ;
            }
            // nine independent uniform branches; each tests its own opaque copy of the offset
            // so the compiler cannot fold them into one multiway branch, whose merge points
            // copy the register line
            const int z0 = kp >> 16;
            if (uniform_copy(z0) == 0) p = group(IntC<0>{}, p, kp);
            if (uniform_copy(z0) == 1) p = group(IntC<1>{}, p, kp);
            if (uniform_copy(z0) == 2) p = group(IntC<2>{}, p, kp);
            if (uniform_copy(z0) == 3) p = group(IntC<3>{}, p, kp);
            if (uniform_copy(z0) == 4) p = group(IntC<4>{}, p, kp);
            if (uniform_copy(z0) == 5) p = group(IntC<5>{}, p, kp);
            if (uniform_copy(z0) == 6) p = group(IntC<6>{}, p, kp);
            if (uniform_copy(z0) == 7) p = group(IntC<7>{}, p, kp);
            if (uniform_copy(z0) == 8) p = group(IntC<8>{}, p, kp);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (cur >= 0 && live) {
        lds_line_add<Z>(tre + cell, are);
        lds_line_add<Z>(tim + cell, aim);
    }
    __syncthreads();
    // add the padded bin to the fine grid with periodic wrap (eq. (15))
    flush_columns<T, BLOCK, PZ>(g, tre, tim, grid, origin, pd, p1, p2);
}

// ------------------------------------------------------------------------------------------
// Column runs with workgroup staging (fp64 plans).
//
// The same register-line accumulation, but the per-point weights are computed once per
// workgroup with one lane per weight: a piece holds the next kWgPiece points of every slice,
// every thread evaluates one (slice, point, dimension, q) weight, and a workgroup barrier hands
// the piece to the slices' wavefronts.  fp64 exp and sqrt are long instruction sequences, so
// evaluating each weight once, on full wavefronts, matters more than the barrier: with
// per-wavefront staging only 3 lanes per point work, and the wavefronts of a slice (two or
// three at these widths) repeat each other's work.  The stage is double-buffered (one barrier
// per piece) and the raw coordinates and strengths of the piece after next are loaded into
// registers while the current one is consumed.  The strengths must arrive in sorted order.
// ------------------------------------------------------------------------------------------
template <typename T, int W>
struct WgStage {
    using C = ColCfg<T, W>;
    static constexpr int kPiece = 6;
    T kz[kPiece][C::kWZ];
    cplx<T> cv[kPiece];
    T kx[kPiece][C::kB | 1];
    T ky[kPiece][C::kB | 1];
    int kp[kPiece][4];           // x block, y block, z start
};

template <typename T, int W>
__global__ void __launch_bounds__((kColBlock<T, W>)) k_spread_col_wg(GeomArgs g, const cplx<T>* __restrict__ c,
                                                                        cplx<T>* __restrict__ grid, int p1, int p2) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    using C = ColCfg<T, W>;
    using St = WgStage<T, W>;
    constexpr int Z = C::kZ;
    constexpr int PZ = C::kPZ;
    constexpr int B = C::kB;
    constexpr int S = C::kS;
    constexpr int SW = C::kSlotWaves;
    constexpr int SLICES = C::kWaves / SW;
    constexpr int PIECE = St::kPiece;
    constexpr int BLOCK = C::kBlock;
    constexpr int ITEMS = SLICES * PIECE * 3 * W;              // weights per piece
    constexpr int IT = (ITEMS + BLOCK - 1) / BLOCK;            // weights per thread per piece
    extern __shared__ __align__(16) unsigned char smem[];
    const int PL = p1 * p2 * PZ;
    double* tre = (double*)smem;             // real and imaginary planes, cell (x + y p1) pz + z
    double* tim = tre + PL;
    St* stages = (St*)(tim + PL);            // [2][SLICES]

    const int sid = blockIdx.x;
    const int bin = g.sub[3 * sid + 0];
    const int start = g.sub[3 * sid + 1];
    const int len = g.sub[3 * sid + 2];
    int origin[3];
    {
        int b0 = bin % g.nb[0];
        int b1 = (bin / g.nb[0]) % g.nb[1];
        int b2 = bin / (g.nb[0] * g.nb[1]);
        origin[0] = b0 * g.m[0] - W / 2;
        origin[1] = b1 * g.m[1] - W / 2;
        origin[2] = b2 * g.m[2] - W / 2;
    }
    const int pd[3] = {p1, p2, Z};
    for (int k = threadIdx.x; k < 2 * PL; k += BLOCK) tre[k] = 0.0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int slice = wave / SW, sub_wave = wave - slice * SW;
    const int slot = sub_wave * 64 + lane;
    const bool valid = (slot < B * B) && (slice < SLICES);
    const int q2 = valid ? slot / B : 0;
    const int q1 = valid ? slot - q2 * B : 0;
    const int per = (len + SLICES - 1) / SLICES;      // points per slice (the last may have fewer)
    const int npieces = (per + PIECE - 1) / PIECE;    // the same for every wavefront
    const T beta = (T)g.beta;

    // this thread's staging items: (slice, point, dimension, q), the same in every piece, so they
    // are decoded once and kept packed (q | d << 5 | p << 7 | s << 11, or -1 past the last item);
    // and their raw inputs (the strengths arrive in sorted order)
    static_assert(W < 32 && PIECE < 16 && SLICES < 64, "item fields");
    T xr[IT], crr[IT], cri[IT];
    int item[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int i = threadIdx.x + it * BLOCK;
        if (i >= ITEMS) {
            item[it] = -1;
        } else {
            const int q = i % W, r = i / W;
            item[it] = q | ((r % 3) << 5) | (((r / 3) % PIECE) << 7) | ((r / 3 / PIECE) << 11);
        }
    }
    auto item_point = [&](int it, int k, int& s_, int& p_, int& d_, int& q_) -> int64_t {
        const int v = item[it];
        if (v < 0) return -1;
        q_ = v & 31;
        d_ = (v >> 5) & 3;
        p_ = (v >> 7) & 15;
        s_ = v >> 11;
        const int ps = s_ * per + k * PIECE + p_;              // point index in the subproblem
        if (k * PIECE + p_ >= per || ps >= len) return -1;
        return (int64_t)start + ps;
    };
    auto fetch = [&](int k) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            int s_, p_, d_, q_;
            const int64_t j = item_point(it, k, s_, p_, d_, q_);
            if (j >= 0) {
                xr[it] = ((const T*)g.xs[d_])[j];
                if (d_ == 0 && q_ == 0) {
                    const cplx<T> cv = c[g.cperm ? g.cperm[j] : j];
                    crr[it] = cv.re;
                    cri[it] = cv.im;
                }
            }
        }
    };
    auto stage = [&](int k, St* buf) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            int s_, p_, d_, q_;
            const int64_t j = item_point(it, k, s_, p_, d_, q_);
            if (j < 0) continue;
            St& st = buf[s_];
            double tt = grid_t((double)xr[it], g.s[d_]);
            int l;
            fold_t(tt, g.n[d_], l);
            // the weight for offset q of eq. (8), as in es_weights
            const double l0d = ceil(__dsub_rn(tt, 0.5 * (double)W));
            const T delta = (T)__dsub_rn(l0d, tt);
            const T zq = (delta + (T)q_) * ((T)2 / (T)W);
            const T zz = zq * zq;
            T phi;
            if constexpr (sizeof(T) == 4)
                phi = (zz <= 1.0f) ? __expf(beta * (__builtin_amdgcn_sqrtf(1.0f - zz) - 1.0f)) : 0.0f;
            else
                phi = (zz <= (T)1) ? exp_es(beta * (sqrt_unit((T)1 - zz) - (T)1)) : (T)0;
            // the start is checked once per (point, dimension), by its q = 0 item
            const int l0 = (q_ == 0) ? checked_start((int)l0d - origin[d_], pd[d_] - W, g.range_err)
                                     : min(max((int)l0d - origin[d_], 0), pd[d_] - W);
            if (d_ < 2) {
                const int blk = l0 / S;
                const int off = l0 - blk * S;
                T* win = (d_ == 0) ? st.kx[p_] : st.ky[p_];
                win[off + q_] = phi;
                if (q_ < B - W) win[q_ < off ? q_ : q_ + W] = (T)0;
                if (q_ == 0) st.kp[p_][d_] = blk;
                if (d_ == 0 && q_ == 0) {
                    st.cv[p_].re = crr[it];
                    st.cv[p_].im = cri[it];
                }
            } else {
                st.kz[p_][q_] = phi;
                if (q_ == 0) st.kp[p_][2] = l0;
            }
        }
    };

    T are[Z], aim[Z];
#pragma unroll
    for (int z = 0; z < Z; ++z) {
        are[z] = (T)0;
        aim[z] = (T)0;
    }
    int cur = -1, cell = 0;
    bool live = false;

    fetch(0);
    stage(0, stages);
    fetch(1);
    __syncthreads();
    for (int k = 0; k < npieces; ++k) {
        St* now = stages + (k & 1) * SLICES;
        if (k + 1 < npieces) {
            stage(k + 1, stages + ((k + 1) & 1) * SLICES);
            fetch(k + 2);
        }
        const int p0 = slice * per + k * PIECE;
        const int np = (slice < SLICES) ? max(0, min(PIECE, min(len, slice * per + per) - p0)) : 0;
        if (np > 0) {
            const St& ws = now[slice];
            int key = 0;
            if (lane < np) key = ws.kp[lane][0] | (ws.kp[lane][1] << 8) | (ws.kp[lane][2] << 16);
            auto group = [&](auto z0c, int p, int kp) -> int {
                constexpr int Z0 = decltype(z0c)::value;
                ColPt<T, W> A;
                do {
                    A.load(ws, p, q1, q2);
                    A.template add<Z, Z0>(are, aim);
                    ++p;
                } while (p < np && __builtin_amdgcn_readlane(key, p) == kp);
                return p;
            };
            int p = 0;
            while (p < np) {
                const int kp = __builtin_amdgcn_readlane(key, p);
                const int col = kp & 0xffff;
                if (col != cur) {
                    if (cur >= 0 && live) {
#pragma unroll
                        for (int z = 0; z < Z; ++z) {
                            atomicAdd(tre + cell + z, (double)are[z]);
                            atomicAdd(tim + cell + z, (double)aim[z]);
                        }
                    }
#pragma unroll
                    for (int z = 0; z < Z; ++z) {
                        zero_in_place(are[z]);
                        zero_in_place(aim[z]);
                    }
                    cur = col;
                    const int cx = (col & 0xff) * S + q1, cy = (col >> 8) * S + q2;
                    live = valid && cx < p1 && cy < p2;
                    cell = (cx + cy * p1) * PZ;
                }
                const int z0 = kp >> 16;
                if (uniform_copy(z0) == 0) p = group(IntC<0>{}, p, kp);
                if (uniform_copy(z0) == 1) p = group(IntC<1>{}, p, kp);
                if (uniform_copy(z0) == 2) p = group(IntC<2>{}, p, kp);
                if (uniform_copy(z0) == 3) p = group(IntC<3>{}, p, kp);
                if (uniform_copy(z0) == 4) p = group(IntC<4>{}, p, kp);
                if (uniform_copy(z0) == 5) p = group(IntC<5>{}, p, kp);
                if (uniform_copy(z0) == 6) p = group(IntC<6>{}, p, kp);
                if (uniform_copy(z0) == 7) p = group(IntC<7>{}, p, kp);
                if (uniform_copy(z0) == 8) p = group(IntC<8>{}, p, kp);
            }
        }
        // piece k + 1 is staged and piece k consumed before either buffer is reused
        __syncthreads();
    }
    if (cur >= 0 && live) {
#pragma unroll
        for (int z = 0; z < Z; ++z) {
            atomicAdd(tre + cell + z, (double)are[z]);
            atomicAdd(tim + cell + z, (double)aim[z]);
        }
    }
    __syncthreads();
    // add the padded bin to the fine grid with periodic wrap (eq. (15))
    flush_columns<T, BLOCK, PZ>(g, tre, tim, grid, origin, pd, p1, p2);
}

// fp64 plans stage per workgroup; fp32 plans per wavefront
template <typename T>
constexpr bool kWgStaging = sizeof(T) == 8;

template <typename T, int W>
size_t col_lds_bytes(const int* m) {
    using C = ColCfg<T, W>;
    // fp64 plans (workgroup staging) and fp32 plans keep the bin in their own precision
    const size_t tile = (size_t)(m[0] + W) * (m[1] + W) * C::kPZ * 2 * sizeof(T);
    if constexpr (kWgStaging<T>)
        return tile + sizeof(WgStage<T, W>) * 2 * (C::kWaves / C::kSlotWaves);
    return tile + sizeof(ColStage<T, W>) * C::kWaves;
}

size_t col_lds_bytes_rt(int prec, int w, const int* m) {
    switch (w) {
#define NUFFT_CASE(WW) case WW: return prec == 0 ? col_lds_bytes<float, WW>(m) : col_lds_bytes<double, WW>(m);
        NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7) NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10)
        NUFFT_CASE(11) NUFFT_CASE(12)
#undef NUFFT_CASE
        default: return 0;
    }
}

template <typename T, int W>
hipError_t spread_col_w(const GeomArgs& g, const void* c, void* grid, hipStream_t st) {
    if (g.M <= 0 || g.nsub <= 0) return hipSuccess;
    if (g.m[2] != 8) return hipErrorInvalidConfiguration;
    const int p1 = g.m[0] + W, p2 = g.m[1] + W;
    const size_t lds = col_lds_bytes<T, W>(g.m);
    if (lds > spread_lds_limit()) return hipErrorInvalidConfiguration;
    const void* fn;
    if constexpr (kWgStaging<T>)
        fn = (const void*)k_spread_col_wg<T, W>;
    else
        fn = (const void*)k_spread_col<T, W>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)spread_lds_limit());
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if constexpr (kWgStaging<T>)
        k_spread_col_wg<T, W><<<dim3((unsigned)g.nsub, (unsigned)g.nv), ColCfg<T, W>::kBlock, lds, st>>>(
            g, (const cplx<T>*)c, (cplx<T>*)grid, p1, p2);
    else
        k_spread_col<T, W><<<dim3((unsigned)g.nsub, (unsigned)g.nv), ColCfg<T, W>::kBlock, lds, st>>>(
            g, (const cplx<T>*)c, (cplx<T>*)grid, p1, p2);
    return hipGetLastError();
}

template <typename T>
hipError_t spread_col(const GeomArgs& g, const void* c, void* grid, hipStream_t st) {
    switch (g.w) {
#define NUFFT_CASE(WW) case WW: return spread_col_w<T, WW>(g, c, grid, st);
        NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7) NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10)
        NUFFT_CASE(11) NUFFT_CASE(12)
#undef NUFFT_CASE
        default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------------------------------------
// 1D SM spreading: one workgroup per subproblem and one lane per point.  A lane evaluates its
// w weights and adds its w complex contributions into the fp64 LDS copy of the padded bin
// (m + w cells, real and imaginary planes); the bin is then added into the fine grid with
// periodic wrap (eq. (15)).  The next point's coordinate and strength are requested one
// iteration ahead.
// ------------------------------------------------------------------------------------------
constexpr int kSpread1Block = 512;

template <typename T, int W>
__global__ void __launch_bounds__(kSpread1Block) k_spread_sm1(GeomArgs g, const cplx<T>* __restrict__ c,
                                                              cplx<T>* __restrict__ grid, int p1) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    extern __shared__ __align__(16) unsigned char smem[];
    double* tre = (double*)smem;
    double* tim = tre + p1;
    const int sid = blockIdx.x;
    const int bin = g.sub[3 * sid + 0];
    const int start = g.sub[3 * sid + 1];
    const int len = g.sub[3 * sid + 2];
    const int origin = bin * g.m[0] - W / 2;
    T xn = (T)0;
    cplx<T> cn;
    cn.re = (T)0;
    cn.im = (T)0;
    auto fetch = [&](int i) {
        const int64_t j = (int64_t)start + i;
        xn = ((const T*)g.xs[0])[j];
        cn = c[g.cperm ? g.cperm[j] : j];
    };
    if ((int)threadIdx.x < len) fetch(threadIdx.x);
    for (int k = threadIdx.x; k < 2 * p1; k += kSpread1Block) tre[k] = 0.0;
    __syncthreads();
    const T beta = (T)g.beta;
    for (int i = threadIdx.x; i < len; i += kSpread1Block) {
        const T xc = xn;
        const cplx<T> cv = cn;
        if (i + kSpread1Block < len) fetch(i + kSpread1Block);
        double t = grid_t((double)xc, g.s[0]);
        int l;
        fold_t(t, g.n[0], l);
        T ker[W];
        const int l0 = checked_start(es_weights<T, W>(t, beta, ker) - origin, p1 - W, g.range_err);
#pragma unroll
        for (int q = 0; q < W; ++q) {
            atomicAdd(tre + l0 + q, (double)(cv.re * ker[q]));
            atomicAdd(tim + l0 + q, (double)(cv.im * ker[q]));
        }
    }
    __syncthreads();
    // lane pairs take one cell: the even lane its real part, the odd lane its imaginary part
    auto flush = [&](auto fast) {
        constexpr bool FAST = decltype(fast)::value;
        const int comp = threadIdx.x & 1;
        const double* src = comp ? tim : tre;
        for (int k = threadIdx.x >> 1; k < p1; k += kSpread1Block / 2) {
            const double v = src[k];
            if (v == 0.0) continue;
            const int gi = wrap_pad<FAST>(origin + k, g.n[0]);
            unsafeAtomicAdd((T*)grid + 2 * (size_t)gi + comp, (T)v);
        }
    };
    if (tile_fast(&origin, &p1, g.n, 1)) flush(std::true_type{});
    else flush(std::false_type{});
}

template <typename T, int DIM, int W>
__global__ void __launch_bounds__(kGmBlock) k_spread_gm(GeomArgs g, const cplx<T>* __restrict__ c,
                                                        cplx<T>* __restrict__ grid) {
    // vector blockIdx.y of a many-vector launch (strides in complex values)
    c += (int64_t)blockIdx.y * g.cvs;
    grid += (int64_t)blockIdx.y * g.gvs;
    const int64_t i = (int64_t)blockIdx.x * kGmBlock + threadIdx.x;
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
    const cplx<T> v = c[g.cperm ? g.cperm[i] : i];
    if constexpr (DIM == 1) {
#pragma unroll
        for (int q1 = 0; q1 < W; ++q1) {
            unsafeAtomicAdd(&grid[idx[0][q1]].re, v.re * ker[0][q1]);
            unsafeAtomicAdd(&grid[idx[0][q1]].im, v.im * ker[0][q1]);
        }
        return;
    } else {
    const int n1 = g.n[0], n2 = g.n[1];
#pragma unroll
    for (int q3 = 0; q3 < (DIM == 3 ? W : 1); ++q3) {
        for (int q2 = 0; q2 < W; ++q2) {
            T wr = ker[1][q2];
            size_t row = (size_t)idx[1][q2];
            if (DIM == 3) {
                wr *= ker[DIM - 1][q3];
                row += (size_t)n2 * (size_t)idx[DIM - 1][q3];
            }
            const T vre = v.re * wr, vim = v.im * wr;
            cplx<T>* dst = grid + row * (size_t)n1;
#pragma unroll
            for (int q1 = 0; q1 < W; ++q1) {
                unsafeAtomicAdd(&dst[idx[0][q1]].re, vre * ker[0][q1]);
                unsafeAtomicAdd(&dst[idx[0][q1]].im, vim * ker[0][q1]);
            }
        }
    }
    }
}

// cs[i] = c[perm[i]]: the strengths in the bin-sorted order the spreading kernels walk.
__global__ void __launch_bounds__(256) k_gather_c(const int32_t* __restrict__ perm, const cplx<double>* __restrict__ c,
                                                  cplx<double>* __restrict__ cs, int64_t M) {
    c += (int64_t)blockIdx.y * M;
    cs += (int64_t)blockIdx.y * M;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < M) cs[i] = c[perm[i]];
}

__global__ void k_fill_zero(uint4* __restrict__ p, size_t n16) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

template <typename T, int DIM, int W>
size_t stage_bytes() { return sizeof(Stage<T, DIM, W>); }

template <typename T, int DIM, int W>
hipError_t spread_w(int method, const GeomArgs& g, const void* c, void* grid, hipStream_t st) {
    if (g.M <= 0) return hipSuccess;
    if (method == NUFFT_METHOD_GM_SORT || method == NUFFT_METHOD_GM) {
        dim3 grd((unsigned)((g.M + kGmBlock - 1) / kGmBlock), (unsigned)g.nv);
        k_spread_gm<T, DIM, W><<<grd, kGmBlock, 0, st>>>(g, (const cplx<T>*)c, (cplx<T>*)grid);
        return hipGetLastError();
    }
    if (g.nsub <= 0) return hipSuccess;
    if constexpr (DIM == 1) {
        const int p1 = g.m[0] + W;
        const size_t lds = (size_t)p1 * 2 * sizeof(double);
        if (lds > spread_lds_limit()) return hipErrorInvalidConfiguration;
        static bool attr_set1 = false;
        if (!attr_set1) {
            hipError_t e = hipFuncSetAttribute((const void*)k_spread_sm1<T, W>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)spread_lds_limit());
            if (e != hipSuccess) return e;
            attr_set1 = true;
        }
        k_spread_sm1<T, W><<<dim3((unsigned)g.nsub, (unsigned)g.nv), kSpread1Block, lds, st>>>(g, (const cplx<T>*)c,
                                                                              (cplx<T>*)grid, p1);
        return hipGetLastError();
    } else {
    const int p1 = g.m[0] + W, p2 = g.m[1] + W, p3 = (DIM == 3) ? g.m[2] + W : 1;
    const int pc = tile_row_pitch(p1, W);
    const size_t lds = (size_t)pc * p2 * p3 * 2 * sizeof(double) + sizeof(Stage<T, DIM, W>);
    if (lds > spread_lds_limit()) return hipErrorInvalidConfiguration;
    auto go = [&](auto two) -> hipError_t {
        constexpr bool TWO = decltype(two)::value;
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute((const void*)k_spread_sm<T, DIM, W, TWO>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)spread_lds_limit());
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        k_spread_sm<T, DIM, W, TWO><<<dim3((unsigned)g.nsub, (unsigned)g.nv), kSpreadBlock, lds, st>>>(
            g, (const cplx<T>*)c, (cplx<T>*)grid, p1, p2, p3, pc);
        return hipGetLastError();
    };
    // fp64 tiles that fit twice in LDS run the two-workgroup build (the plain one needs 60-110
    // VGPRs, one workgroup per CU): 2D fp64 w = 13, N = 1024^2, M = 2^22: 1.48 -> 1.21 ms
    if constexpr (sizeof(T) == 8) {
        if (2 * lds <= spread_lds_limit()) return go(std::true_type{});
    }
    return go(std::false_type{});
    }
}

template <typename T, int DIM>
hipError_t spread_dim(int method, const GeomArgs& g, const void* c, void* grid, hipStream_t st) {
    switch (g.w) {
#define NUFFT_CASE(WW) case WW: return spread_w<T, DIM, WW>(method, g, c, grid, st);
        NUFFT_CASE(2) NUFFT_CASE(3) NUFFT_CASE(4) NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7)
        NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10) NUFFT_CASE(11) NUFFT_CASE(12) NUFFT_CASE(13)
        NUFFT_CASE(14) NUFFT_CASE(15) NUFFT_CASE(16)
#undef NUFFT_CASE
        default: return hipErrorInvalidValue;
    }
}

template <typename T, int DIM>
size_t stage_bytes_dim(int w) {
    switch (w) {
#define NUFFT_CASE(WW) case WW: return stage_bytes<T, DIM, WW>();
        NUFFT_CASE(2) NUFFT_CASE(3) NUFFT_CASE(4) NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7)
        NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10) NUFFT_CASE(11) NUFFT_CASE(12) NUFFT_CASE(13)
        NUFFT_CASE(14) NUFFT_CASE(15) NUFFT_CASE(16)
#undef NUFFT_CASE
        default: return 0;
    }
}

}  // namespace

size_t spread_lds_limit() { return 160 * 1024; }

size_t spread_tile_bytes(int prec, int dim, int w, const int* m) {
    if (dim == 1) return (size_t)(m[0] + w) * 2 * sizeof(double);
    size_t cells = (size_t)tile_row_pitch(m[0] + w, w);
    for (int i = 1; i < dim; ++i) cells *= (size_t)(m[i] + w);
    size_t stage = (prec == 0) ? (dim == 2 ? stage_bytes_dim<float, 2>(w) : stage_bytes_dim<float, 3>(w))
                               : (dim == 2 ? stage_bytes_dim<double, 2>(w) : stage_bytes_dim<double, 3>(w));
    return cells * 2 * sizeof(double) + stage;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    if (bytes % 16 != 0 || ((uintptr_t)p % 16) != 0) return hipMemsetAsync(p, 0, bytes, st);
    size_t n16 = bytes / 16;
    unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 256 * 64);
    k_fill_zero<<<blocks, 256, 0, st>>>((uint4*)p, n16);
    return hipGetLastError();
}

// below w = 5 the per-point overhead of a column run outweighs its savings: the point-patch
// kernel is faster there
bool spread_uses_columns(int dim, int w) { return dim == 3 && w >= 5 && w <= 12; }

// support starts per column-block edge; defined (and at least 1) only where spread_uses_columns holds
int spread_col_step(int w) { return col_block_edge(w) - w + 1; }

size_t spread_col_lds_bytes(int prec, int w, const int* m) {
    if (!spread_uses_columns(3, w) || m[2] != 8) return 0;
    return col_lds_bytes_rt(prec, w, m);
}

int spread_col_per_cu(int prec, int w) {
    switch (w) {
#define NUFFT_CASE(WW) case WW: return prec == 0 ? kColPerCu<float, WW> : kColPerCu<double, WW>;
        NUFFT_CASE(5) NUFFT_CASE(6) NUFFT_CASE(7) NUFFT_CASE(8) NUFFT_CASE(9) NUFFT_CASE(10)
        NUFFT_CASE(11) NUFFT_CASE(12)
#undef NUFFT_CASE
        default: return 1;
    }
}

hipError_t launch_spread(int prec, int method, const GeomArgs& g_in, const void* c_in, void* grid,
                         hipStream_t st, bool columns, void* c_scratch) {
    // fp64 plans in 2D and 3D put the strengths in sorted order first, with a streaming gather:
    // their spreading kernels run two wavefronts per SIMD and cannot hide the dependent
    // perm -> c loads of large point sets.  fp32 plans and the 1D kernel (one lane per point,
    // its next point requested one iteration ahead) hide them, and the extra pass would cost
    // more (1D fp64, N = 2^20, M = 2^24: spread 0.65 ms with the pass, 0.39 ms without).
    GeomArgs g = g_in;
    const void* c = c_in;
    if (method == NUFFT_METHOD_GM) {
        g.cperm = nullptr;   // the points are in the caller's order
    } else if (prec == 1 && g.M > 0 && g.dim >= 2) {
        k_gather_c<<<dim3((unsigned)((g.M + 255) / 256), (unsigned)g.nv), 256, 0, st>>>(g.perm, (const cplx<double>*)c_in,
                                                                   (cplx<double>*)c_scratch, g.M);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        g.cperm = nullptr;
        c = c_scratch;
    }
    if (columns && method == NUFFT_METHOD_SM)
        return prec == 0 ? spread_col<float>(g, c, grid, st) : spread_col<double>(g, c, grid, st);
    if (prec == 0) return g.dim == 1 ? spread_dim<float, 1>(method, g, c, grid, st)
                          : g.dim == 2 ? spread_dim<float, 2>(method, g, c, grid, st)
                                       : spread_dim<float, 3>(method, g, c, grid, st);
    return g.dim == 1 ? spread_dim<double, 1>(method, g, c, grid, st)
           : g.dim == 2 ? spread_dim<double, 2>(method, g, c, grid, st)
                        : spread_dim<double, 3>(method, g, c, grid, st);
}

}  // namespace nufft
