// Bin-sort of the nonuniform points (cuFINUFFT paper, Sec. III-A: bins of m1 x m2 (x m3)
// fine cells ordered x-fastest, a point belongs to the bin holding its cell
// floor((x + pi)/h), and the permutation lists bin 1's points, then bin 2's, ...), followed
// by the subproblem split of SM spreading (Sec. III-A "Step 1", chunks of at most `cap`
// consecutive sorted points of one bin).
//
// gfx950 design: the permutation is a least-significant-digit radix sort on the bin key, at
// most 8 bits per pass, the key's bits spread evenly over the passes (fewer digits per pass
// give longer runs per digit in the scatter, so fuller memory transactions).  Each pass is
// (1) a per-workgroup digit histogram in LDS (integer LDS atomics), (2) an exclusive scan over
// digit-major histograms, (3) a stable scatter that ranks equal digits inside a wavefront with
// 64-bit ballots and across the sixteen wavefronts of a workgroup through LDS counters, then
// reorders the tile by digit one array at a time through a single LDS buffer (so two
// workgroups fit per CU) and writes each digit's run to consecutive addresses, with
// neighbouring tiles kept on one XCD.  Every pass is stable, so points keep their original
// order inside a bin and the permutation is deterministic.
#include "nufft_internal.h"

namespace nufft {
namespace {

constexpr int kBlock = 256;                 // threads per workgroup (4 wavefronts)
constexpr int kItems = 16;                  // keys per thread per sort tile
constexpr int kTile = kBlock * kItems;      // keys per sort tile
constexpr int kScatBlock = 1024;           // threads per scatter workgroup (16 wavefronts)
constexpr int kScatItems = kTile / kScatBlock;  // keys per thread in the scatter
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kScanItems = 8;               // elements per thread in the scan
constexpr int kScanTile = kBlock * kScanItems;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------------------------------------
// Bin keys
// ------------------------------------------------------------------------------------------
template <typename T, int DIM>
__device__ __forceinline__ int32_t bin_key(const SortArgs& a, int64_t j, int* __restrict__ bad) {
    int bidx[3] = {0, 0, 0};
    double tf[DIM];
    bool ok = true;
#pragma unroll
    for (int i = 0; i < DIM; ++i) {
        double x = (double)((const T*)a.x[i])[j];
        double t = grid_t(x, a.s[i]);
        int l = 0;
        if (!fold_t(t, a.n[i], l)) { ok = false; l = 0; }
        tf[i] = t;   // folded
        bidx[i] = fast_div(l, a.fdm[i]);
    }
    int key = bidx[0] + a.nb[0] * (bidx[1] + a.nb[1] * bidx[2]);
    if (DIM == 3 && a.colw > 0) {
        // column of the kernel support inside the bin's padded tile (see SortArgs::colw)
        int lo[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            lo[i] = (int)ceil(__dsub_rn(tf[i], 0.5 * (double)a.colw)) - (bidx[i] * a.m[i] - a.colw / 2);
            lo[i] = min(max(lo[i], 0), a.m[i]);
        }
        const int ncx = fast_div(a.m[0] + a.colstep, a.fdc);
        key = key * a.ncol + (fast_div(lo[1], a.fdc) * ncx + fast_div(lo[0], a.fdc)) * (a.m[2] + 1) + lo[2];
    }
    if (!ok) {
        key = 0;
        atomicOr(bad, 1);
    }
    return key;
}

// The keys of one sort tile (kTile points, kItems per thread, the loads of several points in
// flight per thread), and, when hist is given, the tile's histogram of the first radix digit
// (the low bits0 bits), in the digit-major layout the scan and the scatter read
// (hist[d * ntiles + tile]), so the first pass needs no histogram kernel of its own.
template <typename T, int DIM>
__global__ void __launch_bounds__(kBlock) k_bin_keys(SortArgs a, int32_t* __restrict__ keys,
                                                      int* __restrict__ bad, int bits0, int64_t ntiles,
                                                      int32_t* __restrict__ hist) {
    __shared__ int32_t h[kBlock / 64][kRadix];   // one copy per wavefront
    const int mask = (1 << bits0) - 1;
    const int wv = threadIdx.x >> 6;
    if (hist)
        for (int i = threadIdx.x; i < kRadix * (kBlock / 64); i += kBlock) (&h[0][0])[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTile;
#pragma unroll 4
    for (int r = 0; r < kItems; ++r) {
        const int64_t j = base + (int64_t)r * kBlock + threadIdx.x;
        if (j < a.M) {
            const int32_t key = bin_key<T, DIM>(a, j, bad);
            keys[j] = key;
            if (hist) atomicAdd(&h[wv][key & mask], 1);
        }
    }
    if (hist) {
        __syncthreads();
        for (int d = threadIdx.x; d <= mask; d += kBlock) {
            int32_t t = 0;
#pragma unroll
            for (int w = 0; w < kBlock / 64; ++w) t += h[w][d];
            hist[(int64_t)d * ntiles + blockIdx.x] = t;
        }
    }
}

// Points in the caller's order (the GM method, Sec. III-A): the same inside-bin rule and point
// check as the keys above, a copy of the coordinates, the identity permutation and bin counts.
template <typename T, int DIM>
__global__ void __launch_bounds__(kBlock) k_identity_order(SortArgs a, int32_t* __restrict__ perm,
                                                            T* __restrict__ xs_out, int* __restrict__ bad) {
    const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (j >= a.M) return;
    bool ok = true;
#pragma unroll
    for (int i = 0; i < DIM; ++i) {
        const T xv = ((const T*)a.x[i])[j];
        xs_out[(int64_t)i * a.M + j] = xv;
        double t = grid_t((double)xv, a.s[i]);
        int l = 0;
        if (!fold_t(t, a.n[i], l)) ok = false;
    }
    perm[j] = (int32_t)j;
    if (!ok) atomicOr(bad, 1);
}

// ------------------------------------------------------------------------------------------
// Exclusive scan of int32 arrays (multi-level, wave64 shuffles)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int32_t u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}

// Exclusive scan of this thread's value across the workgroup; returns the workgroup total in *total.
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t* total) {
    __shared__ int32_t wsum[kBlock / 64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int32_t inc = wave_incl_scan(v);
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    int32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i) {
        if (i < wv) base += wsum[i];
        tot += wsum[i];
    }
    __syncthreads();
    *total = tot;
    return base + inc - v;
}

__global__ void __launch_bounds__(kBlock) k_scan_tiles(const int32_t* __restrict__ in,
                                                        int32_t* __restrict__ out, int64_t n,
                                                        int32_t* __restrict__ tile_sums) {
    int64_t base = (int64_t)blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    int32_t v[kScanItems];
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = (base + i < n) ? in[base + i] : 0;
        s += v[i];
    }
    int32_t tot;
    int32_t run = block_excl_scan(s, &tot);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        if (base + i < n) out[base + i] = run;
        run += v[i];
    }
    if (threadIdx.x == 0) {
        tile_sums[blockIdx.x] = tot;
        if (gridDim.x == 1) out[n] = tot;   // a one-tile scan writes its total here
    }
}

__global__ void __launch_bounds__(kBlock) k_scan_add(int32_t* __restrict__ out, int64_t n,
                                                      const int32_t* __restrict__ tile_pref) {
    int64_t base = (int64_t)blockIdx.x * kScanTile;
    int32_t add = tile_pref[blockIdx.x];
    for (int i = threadIdx.x; i < kScanTile; i += kBlock) {
        if (base + i < n) out[base + i] += add;
    }
    // the scan of the tile sums ends with their total
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) out[n] = tile_pref[gridDim.x];
}

// Writes total of a scanned array: out[n] = out[n-1] + in[n-1] (or 0 for n == 0).
__global__ void k_scan_total(const int32_t* __restrict__ in, int32_t* __restrict__ out, int64_t n) {
    if (threadIdx.x == 0 && blockIdx.x == 0) out[n] = (n > 0) ? out[n - 1] + in[n - 1] : 0;
}

// Per-digit scan of a radix pass's tile histograms, one workgroup per digit: offs[d * ntiles + t]
// = the digit's count in tiles before t, totals[d] = the digit's count.  The scatter adds the
// exclusive scan of the totals (digits before d), so one launch replaces a scan of the whole
// digit-major array.
__global__ void __launch_bounds__(kBlock) k_digit_scan(const int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ offs, int64_t ntiles,
                                                        int32_t* __restrict__ totals) {
    const int64_t row = (int64_t)blockIdx.x * ntiles;
    int32_t carry = 0;
    for (int64_t b = 0; b < ntiles; b += kScanTile) {
        const int64_t base = b + (int64_t)threadIdx.x * kScanItems;
        int32_t v[kScanItems];
        int32_t sum = 0;
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            v[i] = (base + i < ntiles) ? hist[row + base + i] : 0;
            sum += v[i];
        }
        int32_t tot;
        int32_t run = carry + block_excl_scan(sum, &tot);
#pragma unroll
        for (int i = 0; i < kScanItems; ++i) {
            if (base + i < ntiles) offs[row + base + i] = run;
            run += v[i];
        }
        carry += tot;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = carry;
}

// dbase[d] = the counts of the digits below d (nd <= kBlock digit totals, one workgroup).
__global__ void __launch_bounds__(kBlock) k_digit_base(const int32_t* __restrict__ totals, int nd,
                                                        int32_t* __restrict__ dbase) {
    const int d = threadIdx.x;
    const int32_t v = d < nd ? totals[d] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan(v, &tot);
    if (d < nd) dbase[d] = ex;
}

// Upper bound on the scratch exclusive_scan uses for n elements: per level, the tile sums and
// their scanned copy (t + 1 entries each).
size_t scan_scratch_elems(int64_t n) {
    size_t tot = 0;
    while (n > 0) {
        int64_t t = cdiv(n, kScanTile);
        tot += 2 * (size_t)t + 2;
        if (t <= 1) break;
        n = t;
    }
    return tot;
}

// Exclusive scan in -> out (n elements), and out[n] = total.  `scratch` must hold
// scan_scratch_elems(n) int32.
hipError_t exclusive_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* scratch,
                          hipStream_t st) {
    if (n > 0) {
        int64_t tiles = cdiv(n, kScanTile);
        int32_t* sums = scratch;
        k_scan_tiles<<<dim3((unsigned)tiles), dim3(kBlock), 0, st>>>(in, out, n, sums);
        if (tiles > 1) {
            int32_t* pref = scratch + tiles + 1;
            hipError_t e = exclusive_scan(sums, pref, tiles, pref + tiles + 1, st);
            if (e != hipSuccess) return e;
            k_scan_add<<<dim3((unsigned)tiles), dim3(kBlock), 0, st>>>(out, n, pref);
        }
    } else {
        k_scan_total<<<1, 64, 0, st>>>(in, out, n);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Radix sort passes
// ------------------------------------------------------------------------------------------
// Tile handled by this workgroup.  Workgroups are dispatched to the 8 XCDs round-robin by
// index; mapping index b to tile start(b % 8) + b / 8, with each XCD owning a contiguous range
// of tiles, puts neighbouring tiles -- whose runs of one digit are adjacent in the output --
// behind the same L2, so their partial lines merge before they are written back.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t nt) {
    const int64_t q = nt / 8, r = nt % 8, x = b % 8;
    return x * q + (x < r ? x : r) + b / 8;
}

__global__ void __launch_bounds__(kBlock) k_radix_hist(const int32_t* __restrict__ keys, int64_t M,
                                                        int shift, int bits, int64_t ntiles,
                                                        int32_t* __restrict__ hist) {
    const int mask = (1 << bits) - 1;
    // one copy of the counters per wavefront (fewer colliding LDS atomics), summed at the end
    __shared__ int32_t h[kBlock / 64][kRadix];
    const int wv = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kRadix * (kBlock / 64); i += kBlock) (&h[0][0])[i] = 0;
    __syncthreads();
    int64_t base = (int64_t)blockIdx.x * kTile;
    int32_t kv[kItems];   // (keys are non-negative; -1 marks a slot past the end)
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        int64_t idx = base + (int64_t)r * kBlock + threadIdx.x;
        kv[r] = (idx < M) ? keys[idx] : -1;
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r)
        if (kv[r] >= 0) atomicAdd(&h[wv][(kv[r] >> shift) & mask], 1);
    __syncthreads();
    for (int d = threadIdx.x; d <= mask; d += kBlock) {
        int32_t t = 0;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) t += h[w][d];
        hist[(int64_t)d * ntiles + blockIdx.x] = t;
    }
}

template <typename T, int NP>
struct Payload {
    const T* in[3];
    T* out[3];
};

// Stable scatter of one radix pass.  Besides (key, original index), the NP coordinate arrays
// travel with the keys, so the last pass leaves the coordinates in sorted order without a
// random gather (the first pass reads them in the caller's order, coalesced).
//
// Each wavefront ranks its own contiguous chunk of the tile (kScatItems rounds of 64 keys) with
// ballots and wavefront-private digit counters, so ranking needs no workgroup barrier; the
// per-digit counts of the chunks are then combined into tile offsets, and keys, values
// and coordinates are reordered by digit through one LDS buffer in turn, each digit's run
// written to consecutive addresses.
// IDV: the values are the keys' positions (the first pass), so none are read.
// fp32 tiles are built for 64 VGPRs, so that two workgroups (32 wavefronts) share a CU.
template <typename T, int NP, bool IDV>
__global__ void __launch_bounds__(kScatBlock) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 8 : 1)))
k_radix_scatter(const int32_t* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
                int32_t* __restrict__ keys_out, int32_t* __restrict__ vals_out, int64_t M, int shift,
                int bits, int64_t ntiles, const int32_t* __restrict__ offs,
                const int32_t* __restrict__ dbase, Payload<T, NP> pl) {
    const int mask = (1 << bits) - 1;
    constexpr int kWaves = kScatBlock / 64;
    constexpr int kChunk = kScatItems * 64;              // keys per wavefront
    __shared__ int32_t cnt[kWaves][kRadix];             // per-wavefront digit counts, then offsets
    __shared__ int32_t gbase[kRadix];                   // global start of each digit's run of this tile
    __shared__ int32_t tbase[kRadix];                   // start of each digit's run inside the tile
    __shared__ int32_t wsum[kWaves];
    __shared__ uint32_t sbuf[kTile * (sizeof(T) > 4 ? 2 : 1)];   // one reordered array at a time
    __shared__ uint8_t sdig[kTile];                              // digit of each reordered slot
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t tile = xcd_tile(blockIdx.x, ntiles);
    const int64_t base = tile * kTile;
    const int count = (int)min<int64_t>(kTile, M - base);

    // load this wavefront's chunk (coalesced per round)
    int32_t keys[kScatItems], vals[kScatItems];
    T cvs[kScatItems][NP > 0 ? NP : 1];
#pragma unroll
    for (int r = 0; r < kScatItems; ++r) {
        const int li = wv * kChunk + r * 64 + lane;
        const bool valid = li < count;
        keys[r] = valid ? keys_in[base + li] : 0;
        if constexpr (IDV)
            vals[r] = (int32_t)(base + li);
        else
            vals[r] = valid ? vals_in[base + li] : 0;
#pragma unroll
        for (int d = 0; d < NP; ++d) cvs[r][d] = valid ? pl.in[d][base + li] : (T)0;
    }
    for (int d = lane; d < kRadix; d += 64) cnt[wv][d] = 0;

    // rank inside the wavefront's chunk: rounds in order, lanes in order
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t rank[kScatItems];
#pragma unroll
    for (int r = 0; r < kScatItems; ++r) {
        const bool valid = wv * kChunk + r * 64 + lane < count;
        const int digit = (keys[r] >> shift) & mask;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kRadixBits; ++b) {
            if (b >= bits) break;
            const bool bit = (digit >> b) & 1;
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int32_t before = valid ? cnt[wv][digit] : 0;
        rank[r] = before + __popcll(peers & lt_mask);
        const int leader = peers ? (__ffsll((unsigned long long)peers) - 1) : 64;
        // the counter read above and this update are ordered within the wavefront
        if (valid && lane == leader) cnt[wv][digit] = before + __popcll(peers);
    }
    __syncthreads();

    // tile offsets: digit-major exclusive scan of the tile counts (one thread per digit, the
    // first kRadix threads), then per-wavefront offsets; and the run's global start: the counts
    // of the smaller digits (scan of the digit totals) plus this digit's count in earlier tiles
    {
        static_assert(kRadix % 64 == 0 && kRadix <= kScatBlock, "one thread per digit");
        const int d = tid;
        const bool dt = tid < kRadix;
        int32_t c[kWaves], tot = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            c[i] = dt ? cnt[i][d] : 0;
            tot += c[i];
        }
        int32_t inc = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t u = __shfl_up(inc, off, 64);
            if (lane >= off) inc += u;
        }
        if (dt && lane == 63) wsum[wv] = inc;
        __syncthreads();
        if (dt) {
            int32_t run = inc - tot;
            for (int i = 0; i < wv; ++i) run += wsum[i];
            tbase[d] = run;
            // the counts of the smaller digits plus this digit's count in earlier tiles
            gbase[d] = (d <= mask) ? dbase[d] + offs[(int64_t)d * ntiles + tile] : 0;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                cnt[i][d] = run;
                run += c[i];
            }
        }
    }
    __syncthreads();
    // slot of each item in the digit-ordered tile (-1: past the end of the input)
    int pos[kScatItems];
#pragma unroll
    for (int r = 0; r < kScatItems; ++r) {
        pos[r] = -1;
        if (wv * kChunk + r * 64 + lane < count) {
            const int digit = (keys[r] >> shift) & mask;
            pos[r] = cnt[wv][digit] + rank[r];
            sdig[pos[r]] = (uint8_t)digit;
        }
    }
    // the arrays are reordered through one LDS buffer in turn: keys, values, then coordinates;
    // slot i goes to gbase[digit] + (i - tbase[digit])
    auto emit = [&](auto get, auto put) {
#pragma unroll
        for (int r = 0; r < kScatItems; ++r)
            if (pos[r] >= 0) get(r, pos[r]);
        __syncthreads();
        for (int i = tid; i < count; i += kScatBlock) {
            const int digit = sdig[i];
            put((int64_t)gbase[digit] + (i - tbase[digit]), i);
        }
        __syncthreads();
    };
    int32_t* bi = (int32_t*)sbuf;
    emit([&](int r, int p) { bi[p] = keys[r]; }, [&](int64_t o, int i) { keys_out[o] = bi[i]; });
    emit([&](int r, int p) { bi[p] = vals[r]; }, [&](int64_t o, int i) { vals_out[o] = bi[i]; });
    T* bt = (T*)sbuf;
#pragma unroll
    for (int d = 0; d < NP; ++d)
        emit([&](int r, int p) { bt[p] = cvs[r][d]; }, [&](int64_t o, int i) { pl.out[d][o] = bt[i]; });
}

// Clears n 32-bit words (small flags and counters: a kernel rather than a memset, so that a
// captured stream records no memset node).
__global__ void k_zero_words(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ void k_iota(int32_t* __restrict__ v, int64_t M) {
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j < M) v[j] = (int32_t)j;
}

// offsets[b] = first sorted position whose bin is >= b (offsets[nbins] = M); key = bin * ncol + column,
// so that is the first sorted key >= b * ncol: one binary search per bin.  (Writing the bins between
// consecutive sorted keys from the keys' side makes one thread fill every empty bin of a gap, which
// clustered points turn into a long serial tail.)
__global__ void k_bin_offsets(const int32_t* __restrict__ skeys, int64_t M, int nbins, int ncol,
                              int32_t* __restrict__ offsets) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b > nbins) return;
    const int64_t target = (int64_t)b * ncol;
    int64_t lo = 0, hi = M;   // the answer lies in [lo, hi]
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if ((int64_t)skeys[mid] < target) lo = mid + 1;
        else hi = mid;
    }
    offsets[b] = (int32_t)lo;
}

__global__ void k_counts_nsub(const int32_t* __restrict__ offsets, int nbins, int cap,
                              int32_t* __restrict__ counts, int32_t* __restrict__ nsp) {
    int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nbins) return;
    int32_t c = offsets[b + 1] - offsets[b];
    counts[b] = c;
    nsp[b] = (c + cap - 1) / cap;
}

// One thread per subproblem: its bin is the last bin whose first subproblem index is at or below
// it (a binary search over the scanned per-bin counts; empty bins share their successor's first
// index), and it is that bin's k-th chunk of cap points.  (One thread per bin writing all its
// chunks leaves a serial tail on bins holding many subproblems.)
__global__ void k_build_sub(int nbins, int64_t nsub, int cap, const int32_t* __restrict__ counts,
                            const int32_t* __restrict__ offsets,
                            const int32_t* __restrict__ first, int32_t* __restrict__ sub) {
    const int64_t si = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (si >= nsub) return;
    int lo = 0, hi = nbins - 1;
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (first[mid] <= si) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    const int32_t k = (int32_t)(si - first[b]);
    sub[3 * si + 0] = b;
    sub[3 * si + 1] = offsets[b] + k * cap;
    sub[3 * si + 2] = min(cap, counts[b] - k * cap);
}

struct SortLayout {
    int64_t ntiles;
    size_t keysA, valsA, keysB, valsB, coords, hist, hist_scan, totals, dbase, scan_tmp, nsp, first, end;
};

SortLayout layout(int64_t M, int nbins, int dim, int prec) {
    SortLayout L{};
    L.ntiles = std::max<int64_t>(1, cdiv(M, kTile));
    size_t off = 0;
    auto take = [&](size_t elems) {
        size_t o = off;
        off += ((elems * 4 + 255) / 256) * 256;
        return o;
    };
    size_t Mm = (size_t)std::max<int64_t>(M, 1);
    L.keysA = take(Mm);
    L.valsA = take(Mm);
    L.keysB = take(Mm);
    L.valsB = take(Mm);
    L.coords = take(Mm * (size_t)dim * (prec == 0 ? 1 : 2));
    size_t nh = (size_t)kRadix * L.ntiles;
    L.hist = take(nh);
    L.hist_scan = take(nh);
    L.totals = take(kRadix);
    L.dbase = take(kRadix);
    // (the one multi-level scan left is over the bins' subproblem counts)
    L.scan_tmp = take(scan_scratch_elems((int64_t)nbins + 1) + 16);
    L.nsp = take((size_t)nbins + 1);
    L.first = take((size_t)nbins + 2);
    L.end = off;
    return L;
}

// fn(T{}, std::integral_constant<int, DIM>{}) for the plan's precision (0 = fp32) and dimension.
template <typename F>
void with_type_dim(int prec, int dim, F&& fn) {
    auto by_dim = [&](auto tag) {
        if (dim == 1) fn(tag, std::integral_constant<int, 1>{});
        else if (dim == 2) fn(tag, std::integral_constant<int, 2>{});
        else fn(tag, std::integral_constant<int, 3>{});
    };
    if (prec == 0) by_dim(float{});
    else by_dim(double{});
}

// One radix scatter pass with the dim coordinate arrays cin[] -> cout[] as payload; vi == null
// marks the first pass (values = identity).
template <typename T>
hipError_t scatter_dim(int dim, const int32_t* ki, const int32_t* vi, int32_t* ko, int32_t* vo, int64_t M,
                       int shift, int bits, int ntiles, const int32_t* hscan, const int32_t* dbase,
                       const void* const* cin, void* const* cout, hipStream_t st) {
    auto go = [&](auto dtag) {
        constexpr int D = decltype(dtag)::value;
        Payload<T, D> pl{};
        for (int d = 0; d < D; ++d) { pl.in[d] = (const T*)cin[d]; pl.out[d] = (T*)cout[d]; }
        const dim3 gt((unsigned)ntiles);
        if (vi) k_radix_scatter<T, D, false><<<gt, kScatBlock, 0, st>>>(ki, vi, ko, vo, M, shift, bits, ntiles, hscan, dbase, pl);
        else k_radix_scatter<T, D, true><<<gt, kScatBlock, 0, st>>>(ki, vi, ko, vo, M, shift, bits, ntiles, hscan, dbase, pl);
    };
    if (dim == 1) go(std::integral_constant<int, 1>{});
    else if (dim == 2) go(std::integral_constant<int, 2>{});
    else go(std::integral_constant<int, 3>{});
    return hipGetLastError();
}

}  // namespace

size_t sort_scratch_bytes(int64_t M, int nbins, int dim, int prec) { return layout(M, nbins, dim, prec).end; }

hipError_t launch_zero_words(void* p, int64_t nwords, hipStream_t st) {
    if (nwords <= 0) return hipSuccess;
    k_zero_words<<<dim3((unsigned)cdiv(nwords, kBlock)), kBlock, 0, st>>>((uint32_t*)p, nwords);
    return hipGetLastError();
}

hipError_t launch_sort(const SortArgs& a_in, int32_t* perm, int32_t* counts, int32_t* offsets,
                       void* xs_out, void* scratch, size_t scratch_bytes, int64_t* nsub_dev,
                       int* bad_dev, hipStream_t st) {
    SortArgs a = a_in;
    for (int i = 0; i < 3; ++i) a.fdm[i] = make_fastdiv(std::max(a.m[i], 1));
    a.fdc = make_fastdiv(std::max(a.colstep, 1));
    SortLayout L = layout(a.M, a.nbins, a.dim, a.prec);
    if (scratch_bytes < L.end) return hipErrorInvalidValue;
    char* base = (char*)scratch;
    int32_t* keysA = (int32_t*)(base + L.keysA);
    int32_t* valsA = (int32_t*)(base + L.valsA);
    int32_t* keysB = (int32_t*)(base + L.keysB);
    int32_t* valsB = (int32_t*)(base + L.valsB);
    int32_t* hist = (int32_t*)(base + L.hist);
    int32_t* hscan = (int32_t*)(base + L.hist_scan);
    int32_t* totals = (int32_t*)(base + L.totals);
    int32_t* dbase = (int32_t*)(base + L.dbase);
    int32_t* stmp = (int32_t*)(base + L.scan_tmp);
    int32_t* nsp = (int32_t*)(base + L.nsp);
    int32_t* first = (int32_t*)(base + L.first);
    hipError_t e;
    const int64_t M = a.M;
    if (M > 0) {
        const int passes = (a.nbits + kRadixBits - 1) / kRadixBits;
        // the first pass's digit width (the remaining bits spread evenly over the passes, below)
        const int bits0 = passes > 0 ? (a.nbits + passes - 1) / passes : 0;
        auto keys_kernel = [&](auto tag, auto dtag) {
            using T = decltype(tag);
            k_bin_keys<T, decltype(dtag)::value><<<dim3((unsigned)L.ntiles), kBlock, 0, st>>>(
                a, keysA, bad_dev, bits0, L.ntiles, passes > 0 ? hist : nullptr);
        };
        with_type_dim(a.prec, a.dim, keys_kernel);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        int shift = 0;
        // values: the first pass generates the identity, the last writes the caller's perm, and
        // the passes between alternate valsA / valsB
        int32_t *ki = keysA, *ko = keysB;
        int32_t* vbuf[2] = {valsA, valsB};
        const size_t rs = a.prec == 0 ? 4 : 8;
        char* ctmp = base + L.coords;
        for (int p = 0; p < passes; ++p) {
            // the remaining bits spread evenly over the remaining passes
            const int bits = (a.nbits - shift + (passes - p) - 1) / (passes - p);
            dim3 gt((unsigned)L.ntiles);
            // (the keys kernel wrote the first pass's histogram)
            if (p > 0) k_radix_hist<<<gt, kBlock, 0, st>>>(ki, M, shift, bits, L.ntiles, hist);
            k_digit_scan<<<dim3(1u << bits), kBlock, 0, st>>>(hist, hscan, L.ntiles, totals);
            k_digit_base<<<1, kBlock, 0, st>>>(totals, 1 << bits, dbase);
            // coordinates: caller's arrays -> ... -> sorted output; the last pass writes xs_out
            const bool last = (p == passes - 1);
            const int32_t* vi = (p == 0) ? nullptr : vbuf[(p - 1) & 1];
            int32_t* vo = last ? perm : vbuf[p & 1];
            const bool to_tmp = ((passes - 1 - p) % 2) == 1;
            const void* cin[3];
            void* cout[3];
            for (int d = 0; d < 3; ++d) {
                cin[d] = (p == 0) ? a.x[d] : ((passes - p) % 2 == 1 ? (const void*)(ctmp + (size_t)d * M * rs)
                                                                     : (const void*)((char*)xs_out + (size_t)d * M * rs));
                cout[d] = to_tmp ? (void*)(ctmp + (size_t)d * M * rs) : (void*)((char*)xs_out + (size_t)d * M * rs);
            }
            e = a.prec == 0 ? scatter_dim<float>(a.dim, ki, vi, ko, vo, M, shift, bits, L.ntiles, hscan, dbase, cin, cout, st)
                            : scatter_dim<double>(a.dim, ki, vi, ko, vo, M, shift, bits, L.ntiles, hscan, dbase, cin, cout, st);
            if (e != hipSuccess) return e;
            std::swap(ki, ko);
            shift += bits;
        }
        if (passes == 0) {
            // a single bin: the order is unchanged
            for (int d = 0; d < a.dim; ++d)
                if ((e = hipMemcpyAsync((char*)xs_out + (size_t)d * M * rs, a.x[d], M * rs, hipMemcpyDeviceToDevice,
                                        st)) != hipSuccess)
                    return e;
            k_iota<<<dim3((unsigned)cdiv(M, kBlock)), kBlock, 0, st>>>(perm, M);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        k_bin_offsets<<<dim3((unsigned)cdiv((int64_t)a.nbins + 1, kBlock)), kBlock, 0, st>>>(
            ki, M, a.nbins, std::max(a.ncol, 1), offsets);
    } else {
        if ((e = launch_zero_words(offsets, (int64_t)a.nbins + 1, st)) != hipSuccess) return e;
    }
    k_counts_nsub<<<dim3((unsigned)cdiv(a.nbins, kBlock)), kBlock, 0, st>>>(offsets, a.nbins, a.cap,
                                                                          counts, nsp);
    if ((e = exclusive_scan(nsp, first, a.nbins, stmp, st)) != hipSuccess) return e;
    // total number of subproblems = first[nbins]; widen to int64 for the host read-back
    if ((e = launch_zero_words(nsub_dev, 2, st)) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(nsub_dev, first + a.nbins, sizeof(int32_t), hipMemcpyDeviceToDevice,
                            st)) != hipSuccess)
        return e;
    return hipGetLastError();
}

// Subproblem list from the scratch of the last launch_sort (bins, cap, counts, offsets as there).
hipError_t launch_identity_order(const SortArgs& a, int32_t* perm, void* xs_out, int* bad_dev, hipStream_t st) {
    if (a.M <= 0) return hipSuccess;
    dim3 g((unsigned)cdiv(a.M, kBlock));
    with_type_dim(a.prec, a.dim, [&](auto tag, auto dtag) {
        using T = decltype(tag);
        k_identity_order<T, decltype(dtag)::value><<<g, kBlock, 0, st>>>(a, perm, (T*)xs_out, bad_dev);
    });
    return hipGetLastError();
}

hipError_t launch_build_subproblems_from(int64_t M, int nbins, int dim, int prec, int cap, int64_t nsub,
                                         const int32_t* counts, const int32_t* offsets,
                                         const void* scratch, int32_t* sub, hipStream_t st) {
    if (nsub <= 0 || nbins <= 0) return hipSuccess;
    SortLayout L = layout(M, nbins, dim, prec);
    const int32_t* first = (const int32_t*)((const char*)scratch + L.first);
    k_build_sub<<<dim3((unsigned)cdiv(nsub, kBlock)), kBlock, 0, st>>>(nbins, nsub, cap, counts, offsets,
                                                                      first, sub);
    return hipGetLastError();
}

}  // namespace nufft
