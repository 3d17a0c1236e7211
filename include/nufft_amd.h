/*
 * nufft_amd.h -- C ABI of the MI355X (gfx950) 1D/2D/3D type 1 / type 2 NUFFT library.
 *
 * The transforms (cuFINUFFT paper, "cuFINUFFT: a load-balanced GPU library for
 * general-purpose nonuniform FFTs", Sec. I):
 *   type 1, eq. (1):  f_k = sum_{j=1..M} c_j exp(-i k.x_j),  k in I_N1 x I_N2 (x I_N3),
 *   type 2, eq. (3):  c_j = sum_k f_k exp(+i k.x_j),          j = 1..M,
 * with I_N = {k integer : -N/2 <= k < N/2} (eq. (2)) and points x_j in [-pi, pi)^d, d = 1, 2, 3.
 * (The paper's library lists 1D as not yet provided, Sec. I-B item (4); the scheme of Sec. II
 * applies unchanged with d = 1, as in the FINUFFT discussion page "CUFINUFFT binsize and
 * performance", which reports 1D throughputs.)
 * Both are approximated to a requested tolerance eps by the three-step scheme of
 * Sec. II (ES-kernel spreading / interpolation on a 2x upsampled grid, a plain
 * FFT, and a diagonal correction).  The library follows the paper's "plan,
 * setup, execute, destroy" interface (Sec. I-A): points are bin-sorted once by
 * nufft_setpts and reused by every nufft_execute.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers on the plan's device, in the plan's
 *    precision: `float` / `double` coordinates, interleaved complex (re, im)
 *    `float` / `double` strengths and coefficients.  The caller owns them.
 *  - Coefficient arrays f hold N1*N2(*N3) complex values with k1 varying
 *    fastest; along each dimension k_i runs upward from -floor(N_i/2).  (A
 *    C-contiguous torch tensor of shape (N3, N2, N1).)
 *  - Fine grids hold n1*n2(*n3) complex values, first index fastest; cell l
 *    sits at position l*2pi/n - pi.
 *  - Work is enqueued on the stream given at plan creation and is asynchronous
 *    unless stated otherwise.  A plan is not thread-safe; distinct plans are
 *    independent.
 *  - Return values: 0 = success; >0 = success with a warning; <0 = error
 *    (see nufft_status).  nufft_strerror() names a code; nufft_last_error()
 *    gives the detail of the last error on a plan.  On error, output arrays
 *    are unspecified and the plan stays valid unless it was never created.
 */
#ifndef NUFFT_AMD_H
#define NUFFT_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct nufft_plan_s* nufft_plan;

enum nufft_status {
    NUFFT_OK = 0,
    NUFFT_WARN_EPS_CLAMPED = 1,   /* eps asked for a kernel width outside [2, 16]; w was clamped */
    NUFFT_ERR_BAD_ARG = -1,       /* invalid type, dim, N, eps, precision, pointer or size */
    NUFFT_ERR_BAD_STATE = -2,     /* e.g. execute before setpts */
    NUFFT_ERR_ALLOC = -3,         /* device allocation failed or exceeded opts.max_device_bytes */
    NUFFT_ERR_HIP = -4,           /* a HIP runtime call failed */
    NUFFT_ERR_FFT = -5,           /* a rocFFT call failed */
    NUFFT_ERR_POINTS = -6,        /* a coordinate is NaN/Inf or outside [-3pi, 3pi) */
    NUFFT_ERR_UNSUPPORTED = -7    /* a valid request this build does not implement */
};

enum nufft_spread_method {
    NUFFT_METHOD_AUTO = 0,
    NUFFT_METHOD_GM_SORT = 1,     /* one thread per sorted point, global atomics (Sec. III-A "GM-sort") */
    NUFFT_METHOD_SM = 2,          /* subproblems spread into LDS tiles, then flushed (Sec. III-A "SM") */
    NUFFT_METHOD_GM = 3           /* one thread per point in the caller's order, global atomics
                                     (Sec. III-A "GM"); setpts only checks and copies the points:
                                     the permutation is the identity, there are no subproblems and
                                     the bin counts read zero (no binning) */
};

typedef struct {
    int method;               /* nufft_spread_method for type 1 spreading; 0 = auto */
    int bin[3];               /* bin (tile) size in fine cells per dimension; 0 = tuned default */
    int subproblem_cap;       /* max points per subproblem; 0 = default */
    size_t max_device_bytes;  /* 0 = no limit; otherwise plan-owned device memory above this fails */
    int timing;               /* 1 = record per-stage HIP-event times (see nufft_get_stage_times) */
    int max_batch;            /* vectors per batch in nufft_execute_many; 0 = automatic */
    double upsampfac;         /* fine-grid upsampling factor sigma in [1.25, 2]; 0 = 2 (the paper's) */
} nufft_opts;

/* Fill *opts with defaults (all zero = automatic choices).  NUFFT_ERR_BAD_ARG if opts is NULL. */
int nufft_default_opts(nufft_opts* opts);

/*
 * Create a plan.
 *   type      1 (nonuniform -> uniform, eq. (1)), 2 (uniform -> nonuniform, eq. (3)) or
 *             3 (nonuniform -> nonuniform, f_k = sum_j c_j exp(+i s_k.x_j); see
 *             nufft_setpts_type3; N is not used and may be NULL; sigma must be 2, else
 *             NUFFT_ERR_UNSUPPORTED).
 *   dim       1, 2 or 3.
 *   N         host array of dim mode counts (N1[, N2[, N3]]), each >= 1.
 *   eps       requested relative tolerance > 0.  Kernel width w = ceil(log10(1/eps)) + 1
 *             and shape beta = 2.30 w (eq. (6)); w is clamped to [2, 16] with
 *             NUFFT_WARN_EPS_CLAMPED.  With opts->upsampfac = sigma < 2 (the paper fixes
 *             sigma = 2 and names smaller factors as future work, Sec. I-B item (3)):
 *             w = ceil(ln(1/eps) / (pi sqrt(1 - 1/sigma))) and
 *             beta = gamma pi (1 - 1/(2 sigma)) w, gamma = 2.30 / (0.75 pi), so that the
 *             kernel transform has decayed where the first alias of the band starts; at
 *             sigma = 2 these reduce to the paper's values.  sigma outside [1.25, 2] is
 *             NUFFT_ERR_BAD_ARG.
 *   precision 0 = single (float / complex<float>), 1 = double.
 *   stream    hipStream_t on the current device, or NULL for the null stream.
 *   opts      NULL or tuning/test options.
 *   out       receives the plan.  Nothing is allocated on error.
 * Allocates the fine grid (n_i = smallest 2^a 3^b 5^c >= max(ceil(sigma N_i), w)), the
 * correction factors (eq. (10), computed on the host in fp64) and the rocFFT plan.  Each N_i is
 * at most 2^28 and the fine grid has fewer than 2^32 cells (NUFFT_ERR_BAD_ARG otherwise: rocFFT
 * transforms of 2^32 elements or more gave wrong values on this software stack); the grid is
 * held twice (spreading output and FFT output), so a 2048 x 2048 x 1000 fp32 grid takes 62.5 GiB,
 * and a grid the device cannot hold fails with NUFFT_ERR_ALLOC.
 */
int nufft_plan_create(int type, int dim, const int64_t* N, double eps, int precision,
                      void* stream, const nufft_opts* opts, nufft_plan* out);

/*
 * Set the nonuniform points (Sec. III-A bin-sort and subproblems).
 *   M        number of points, 0 <= M <= 2^31 - 1.
 *   x, y, z  device arrays of M coordinates (z is NULL for dim 2; y and z for dim 1).  Values must be
 *            finite and within one period of [-pi, pi), i.e. about [-3pi, 3pi) (one periodic
 *            fold is applied); exactly, t = (x + pi) n / (2 pi) (two rounded fp64 operations)
 *            must satisfy -n <= floor(t) < 2n, so values at the very ends of that range may be
 *            rejected by rounding.  Otherwise NUFFT_ERR_POINTS and the plan keeps no points.
 * The library copies what it needs (sorted coordinates, permutation); the caller
 * may reuse x, y, z once the stream has passed this call.  Blocks the host until
 * the sort is done (one small device-to-host read of the subproblem count).
 * Replaces any previous points.
 */
int nufft_setpts(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z);

/*
 * nufft_setpts without allocating anything, for callers that cannot allocate memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  No hipMalloc, hipFree
 * or pinned-host allocation happens in this call.  (It still reads the subproblem count back to
 * the host and waits for the plan's stream, as nufft_setpts does.)  Results are those of
 * nufft_setpts on the same points.
 *   Scratch: the sort's temporaries (key and value ping-pong buffers, digit histograms, scans and
 *   two result slots: about 16 + dim * sizeof(real) bytes per point plus a little per bin, e.g.
 *   29 bytes per point in 3D fp32) live in one file-scope device array of
 *   NUFFT_NOALLOC_SCRATCH_BYTES bytes per GPU, loaded with the library and held until the process
 *   ends.  A point set that needs more is rejected with NUFFT_ERR_ALLOC (3D fp32: up to about
 *   2.2 million points; 3D fp64: about 1.6 million).
 *   Plan buffers: the sorted coordinates, permutation, bin counts and offsets and the subproblem
 *   list are the plan's own and are not grown here: an earlier nufft_setpts on this plan with at
 *   least M points (and at least as many subproblems) must have sized them, else NUFFT_ERR_ALLOC.
 *   Concurrency: every call on one GPU uses that GPU's one scratch array, which keeps the last
 *   call's contents; calls that overlap in time on one GPU (from other threads or on other
 *   streams) race, and the caller must serialise them.
 * Errors: those of nufft_setpts, plus NUFFT_ERR_ALLOC as above (the plan then keeps no points).
 */
#define NUFFT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int nufft_setpts_noalloc(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z);

/*
 * Type 3 points: M sources (x, y, z: device arrays, any finite values) and K targets (s, t, u:
 * device arrays of K frequencies, any finite values); unused dimensions NULL.  nufft_execute
 * then maps c (M complex) to f (K complex), f_k ~ sum_j c_j exp(+i (s_k x_j + t_k y_j + u_k z_j)).
 * Type 3 is not on the cuFINUFFT paper's pages (Sec. I-B, item (4), lists it as not provided);
 * the steps are built from those of Sec. II: per dimension the sources are centred and scaled
 * into [-pi, pi) and spread (eq. (7)) onto a fine grid of n = smallest even 5-smooth >=
 * max(2 sigma X S / pi + w, 2 w) cells (X, S: half-widths of the sources and targets), the
 * grid's Fourier sum is evaluated at the scaled targets by a type 2 NUFFT with N = n modes, and
 * each target is divided by the kernel transform phihat (eq. (4)) with the centring phases
 * restored.  The accuracy is about that of the tolerance, as for types 1 and 2.  Errors:
 * NUFFT_ERR_BAD_ARG (not a type 3 plan, M or K out of range, null array, fine grid above
 * 2^31 - 1 cells), NUFFT_ERR_POINTS (a non-finite coordinate).  Blocks the host (reads back the
 * coordinate ranges, then the inner sorts).  nufft_execute_adjoint, the many-vector calls and
 * the single-step calls return NUFFT_ERR_UNSUPPORTED on a type 3 plan.
 */
int nufft_setpts_type3(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z, int64_t K,
                       const void* s, const void* t, const void* u);

/*
 * Run the transform on the points of the last setpts.
 *   type 1: reads c (M complex), writes f (prod N complex).
 *   type 2: reads f, writes c.
 *   type 3: reads c (M complex), writes f (K complex).
 * Asynchronous on the plan's stream.  NUFFT_ERR_BAD_STATE before a successful setpts.  The
 * first call allocates a second fine grid, the output of the out-of-place FFT.
 */
int nufft_execute(nufft_plan plan, void* c, void* f);

/*
 * Run the adjoint transform on the same sorted points: type 2 (f -> c) on a type 1 plan,
 * type 1 (c -> f) on a type 2 plan.  Type 2 is the adjoint of type 1 (cuFINUFFT paper,
 * Sec. I), and iterative solvers apply both to one point set; the bin-sort of setpts is
 * reused.  The first call creates the rocFFT plan of the other direction.  Same argument
 * conventions and errors as nufft_execute.
 */
int nufft_execute_adjoint(nufft_plan plan, void* c, void* f);

/*
 * Many-vector execution on the points of the last setpts (the paper's use case of new
 * strength vectors on the same sorted points, Sec. I-A): nvec >= 1 transforms of the plan's
 * type, vector v reading c + v*M / f + v*prod(N) and writing the other (c holds nvec*M complex
 * values, f nvec*prod(N), both vector-major).  Vectors run in batches: every step of a batch is
 * one launch over all its vectors (blockIdx.y = vector) into a batch of fine grids, and the FFT
 * is one batched rocFFT call.  The batch size is opts.max_batch, or automatic (at most 16
 * vectors and about 2 GiB of batch grids, two per vector); batch grids are plan-owned and kept
 * for later calls.
 * Per-stage times (opts.timing) count each batch as one call.  Errors as nufft_execute, plus
 * NUFFT_ERR_BAD_ARG for nvec < 1.
 */
int nufft_execute_many(nufft_plan plan, int nvec, void* c, void* f);

/* The adjoint transform of nufft_execute_adjoint for nvec vectors, as nufft_execute_many. */
int nufft_execute_adjoint_many(nufft_plan plan, int nvec, void* c, void* f);

/* Free everything the plan owns (waits for its stream first).  NULL is accepted. */
int nufft_destroy(nufft_plan plan);

/* Static string naming a status code. */
const char* nufft_strerror(int status);

/* Detail text of the last error on this plan ("" if none).  Valid until the next call on it. */
const char* nufft_last_error(nufft_plan plan);

/*
 * Plan facts, written to host memory:
 *   info_i[0..19]: type, dim, precision, w, n1, n2, n3, N1, N2, N3, m1, m2, m3,
 *                  nbins, nsubproblems (after setpts, else 0), M (after setpts, else -1),
 *                  subproblem cap, spreading method (nufft_spread_method),
 *                  column order (kernel width w when the points of a 3D bin are ordered by the
 *                  x-y column block where their kernel support starts, see nufft_get_sort;
 *                  else 0), column block edge s (1 when there is no column order)
 *   info_d[0..2]:  beta, eps, sigma
 * For a type 3 plan n1..n3 is the transform's fine grid (after setpts_type3), N1..N3 are 1 and
 * the bin fields are those of the plan itself (0 / 1).
 * Either pointer may be NULL.
 */
int nufft_get_info(nufft_plan plan, int64_t* info_i, double* info_d);

/*
 * Per-step times (ms) when opts.timing = 1, written to ms[0..7] in host memory:
 *   ms[0] sort (setpts),
 *   ms[1] spread, ms[2] type 1 FFT, ms[3] deconvolve + truncate, ms[4] grid clear
 *         (type 1 executions),
 *   ms[5] interp, ms[6] type 2 FFT, ms[7] precorrect + pad (type 2 executions).
 * Each is the average over the calls recorded since the previous nufft_get_stage_times (the
 * last 16 when there were more; each batch of a many-vector call counts as one); a stage not
 * run since then keeps its previous value, zero if never run.  The plan records events on its
 * stream and never waits for them except here: this call synchronises the plan's stream.
 */
int nufft_get_stage_times(nufft_plan plan, double* ms);

/* --------------------------------------------------------------------------------------------
 * Single steps of the method, for testing and per-step timing.  Same argument
 * conventions; all asynchronous on the plan's stream; the plan's own fine grid is
 * not touched unless stated.  Each requires a plan of the matching type.
 * ------------------------------------------------------------------------------------------ */

/* Type 1 step 1 (eq. (7)): spread c onto the caller's fine grid `grid` (overwritten). Needs setpts. */
int nufft_spread(nufft_plan plan, const void* c, void* grid);

/* Type 2 step 3 (interpolation after eq. (12)): c_j from the caller's fine grid. Needs setpts. */
int nufft_interp(nufft_plan plan, const void* grid, void* c);

/* Type 1 step 3 (eq. (10)): f_k = p_k * fhat[k mod n] from a transformed fine grid. */
int nufft_deconvolve(nufft_plan plan, const void* fhat, void* f);

/* Type 2 step 1 (eq. (11)): fhat[k mod n] = p_k f_k on I_N, zero elsewhere (all n^d cells written). */
int nufft_precorrect_pad(nufft_plan plan, const void* f, void* fhat);

/*
 * Copy the bin-sort of the last setpts into caller device buffers (int32):
 *   perm[M]           original index of the i-th point in sorted order
 *                     (bins in order, increasing original index within a bin),
 *   counts[nbins]     points per bin,
 *   subproblems[3*S]  (bin, start, length) per subproblem, S = nsubproblems.
 * Any pointer may be NULL.  Bins are numbered b1 + nb1*(b2 + nb2*b3) with
 * b_i = floor(l_i / m_i), l_i = floor((x_i + pi) n_i / (2 pi)) folded into [0, n_i).
 * Inside a bin the order is the original index; for plans that report a column order w and a
 * column block edge s (nufft_get_info), the points of a bin are first ordered by the block
 * (c2 / s) ceil((m1 + 1) / s) + c1 / s of the column where their kernel support starts, then by
 * the z start c3, with c_i = ceil(t_i - w/2) - (b_i m_i - floor(w/2)) and
 * t_i = (x_i + pi) n_i / (2 pi) folded, and by original index last.
 * With the GM method there is no sort: perm is the identity and counts are all zero.
 */
int nufft_get_sort(nufft_plan plan, int32_t* perm, int32_t* counts, int32_t* subproblems);

/*
 * Number of kernel-support starts that any spreading or interpolation launch on this plan (or,
 * for a type 3 plan, its inner plans) found outside the padded tile of the point's subproblem
 * since the plan was created, written to *count (host).  The bin-sort places every point so
 * that its support starts inside its bin's padded tile (the bin holds floor(t) and the support
 * starts at ceil(t - w/2), Sec. III-A with the kernel of eq. (8)); the kernels check this and
 * clamp a start that is outside, counting it here instead of accessing memory out of bounds.
 * A nonzero count means results are wrong.  Synchronises the plan's stream.
 * NUFFT_ERR_BAD_ARG for a NULL plan or count.
 */
int nufft_get_range_errors(nufft_plan plan, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* NUFFT_AMD_H */
