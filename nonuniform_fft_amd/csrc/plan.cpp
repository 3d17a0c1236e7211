// Host side of the gfx950 NUFFT library: the C ABI of include/nufft_amd.h.
//
// Planning follows the cuFINUFFT paper ("cuFINUFFT: a load-balanced GPU library for
// general-purpose nonuniform FFTs"), Sec. II: kernel width and shape from the tolerance
// (eq. (6)), fine grid sizes, and correction factors from the Fourier transform of the ES
// kernel (eqs. (4), (5), (10)).  Execution chains the device kernels of Sec. III with rocFFT
// for the plain FFT of eqs. (9) and (12).
#include <hip/hip_runtime.h>
#include <rocfft/rocfft.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "nufft_internal.h"

using nufft::DevBuf;

namespace {

// ------------------------------------------------------------------------------------------------
// Kernel Fourier transform by quadrature (host, fp64)
// ------------------------------------------------------------------------------------------------

// Gauss-Legendre nodes/weights on [-1, 1] by Newton iteration on the Legendre polynomial.
void gauss_legendre(int q, std::vector<double>& x, std::vector<double>& wts) {
    x.assign(q, 0.0);
    wts.assign(q, 0.0);
    for (int i = 0; i < (q + 1) / 2; ++i) {
        double z = std::cos(nufft::kPi * (i + 0.75) / (q + 0.5));
        double dp = 0.0;
        for (int it = 0; it < 100; ++it) {
            double p0 = 1.0, p1 = z;
            for (int k = 2; k <= q; ++k) {
                double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                p0 = p1;
                p1 = p2;
            }
            dp = q * (z * p1 - p0) / (z * z - 1.0);
            double dz = p1 / dp;
            z -= dz;
            if (std::fabs(dz) < 1e-16) break;
        }
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= q; ++k) {
            double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
            p0 = p1;
            p1 = p2;
        }
        dp = q * (z * p1 - p0) / (z * z - 1.0);
        x[i] = -z;
        x[q - 1 - i] = z;
        wts[i] = wts[q - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
}

// phihat(xi) = int_{-1}^{1} exp(beta (sqrt(1 - z^2) - 1)) cos(xi z) dz  (eq. (4) applied to the
// even kernel of eq. (5)).  With z = sin(theta) the integrand is smooth on [0, pi/2]:
//   phihat(xi) = 2 int_0^{pi/2} exp(beta (cos(theta) - 1)) cos(xi sin(theta)) cos(theta) dtheta,
// integrated here by composite Gauss-Legendre (16 panels of 24 nodes).
struct PhiHat {
    std::vector<double> th, wt;
    PhiHat() {
        std::vector<double> g, gw;
        gauss_legendre(24, g, gw);
        const int panels = 16;
        const double a = 0.0, b = 0.5 * nufft::kPi, h = (b - a) / panels;
        for (int p = 0; p < panels; ++p) {
            for (size_t i = 0; i < g.size(); ++i) {
                th.push_back(a + h * (p + 0.5 * (g[i] + 1.0)));
                wt.push_back(0.5 * h * gw[i]);
            }
        }
    }
    double operator()(double xi, double beta) const {
        double s = 0.0;
        for (size_t i = 0; i < th.size(); ++i)
            s += wt[i] * std::exp(beta * (std::cos(th[i]) - 1.0)) * std::cos(xi * std::sin(th[i])) *
                 std::cos(th[i]);
        return 2.0 * s;
    }
};

bool is_5smooth(int64_t v) {
    for (int p : {2, 3, 5})
        while (v % p == 0) v /= p;
    return v == 1;
}

int64_t next_5smooth(int64_t v) {
    if (v < 1) v = 1;
    while (!is_5smooth(v)) ++v;
    return v;
}

int bit_length(int64_t v) {
    int b = 0;
    while (v > 0) {
        ++b;
        v >>= 1;
    }
    return b;
}

int fail(nufft_plan p, int code, const std::string& msg) {
    if (p) p->last_error = msg;
    return code;
}

int hip_fail(nufft_plan p, hipError_t e, const char* where) {
    return fail(p, NUFFT_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define NUFFT_HIP(call)                                          \
    do {                                                         \
        hipError_t _e = (call);                                  \
        if (_e != hipSuccess) return hip_fail(plan, _e, #call);  \
    } while (0)

int dev_alloc(nufft_plan plan, DevBuf& b, size_t bytes, const char* what) {
    if (b.p && b.bytes >= bytes) return NUFFT_OK;
    size_t old = b.bytes;
    if (plan->opts.max_device_bytes && plan->bytes_in_use - old + bytes > plan->opts.max_device_bytes)
        return fail(plan, NUFFT_ERR_ALLOC, std::string("allocation of ") + what +
                                               " exceeds opts.max_device_bytes");
    if (b.p) {
        hipError_t e = hipFree(b.p);
        b.p = nullptr;
        b.bytes = 0;
        plan->bytes_in_use -= old;
        if (e != hipSuccess) return hip_fail(plan, e, "hipFree");
    }
    if (bytes == 0) return NUFFT_OK;
    hipError_t e = hipMalloc(&b.p, bytes);
    if (e != hipSuccess) {
        b.p = nullptr;
        (void)hipGetLastError();
        return fail(plan, NUFFT_ERR_ALLOC, std::string("hipMalloc of ") + what + " failed: " +
                                               hipGetErrorString(e));
    }
    b.bytes = bytes;
    plan->bytes_in_use += bytes;
    return NUFFT_OK;
}

void dev_free(nufft_plan plan, DevBuf& b) {
    if (b.p) {
        (void)hipFree(b.p);
        plan->bytes_in_use -= b.bytes;
    }
    b.p = nullptr;
    b.bytes = 0;
}

std::once_flag g_rocfft_once;
rocfft_status g_rocfft_setup = rocfft_status_success;

size_t real_size(const nufft_plan p) { return p->prec == 0 ? sizeof(float) : sizeof(double); }

int64_t grid_cells(const nufft_plan p) { return p->n[0] * p->n[1] * p->n[2]; }

int64_t mode_count(const nufft_plan p) { return p->N[0] * p->N[1] * p->N[2]; }

// Default bin (tile) sizes per (dim, precision, w): the largest candidate whose padded fp64 LDS
// tile plus point staging fits the LDS limit.
void default_bins(nufft_plan p, int* m) {
    static const int c2[][2] = {{32, 32}, {32, 16}, {16, 16}, {16, 8}, {8, 8}, {4, 4}, {2, 2}, {1, 1}};
    static const int c3[][3] = {{32, 16, 8}, {16, 16, 8}, {16, 8, 8}, {8, 8, 8}, {8, 8, 4}, {8, 4, 4},
                                {4, 4, 4}, {4, 4, 2}, {2, 2, 2}, {1, 1, 1}};
    if (p->dim == 1) {
        // 1D: 256 cells (a sweep over 128..8192 cells at N = 2^20, M = 2^24 changed the spread
        // and interpolation times by under 15 %, smallest at 128..256)
        for (int c : {256, 128, 64, 32, 16, 8, 4, 2, 1}) {
            int mm[3] = {c, 1, 1};
            if (nufft::spread_tile_bytes(p->prec, 1, p->w, mm) <= nufft::spread_lds_limit()) {
                m[0] = c;
                m[1] = m[2] = 1;
                return;
            }
        }
    } else if (p->dim == 2) {
        for (auto& c : c2) {
            int mm[3] = {c[0], c[1], 1};
            if (nufft::spread_tile_bytes(p->prec, 2, p->w, mm) <= nufft::spread_lds_limit()) {
                m[0] = c[0];
                m[1] = c[1];
                m[2] = 1;
                return;
            }
        }
    } else {
        // the column-run kernel first (it needs m3 = 8), then the plain SM tile.  The column
        // kernel's bins must fit as many times as its workgroups are meant to share a CU (fp32
        // w <= 6: twice, which gives 16 x 16 x 8).  SM point-patch plans first look for a tile
        // small enough for two workgroups per CU: at N = 128^3, M = 2^24 that took 16 x 8 x 8
        // over 16 x 16 x 8 at w = 3 and 4 (fp32 spread 1.29 -> 0.96 ms and 1.50 -> 1.15 ms;
        // fp64, with its two-workgroup build, 1.94 -> 1.72 ms and 2.26 -> 2.13 ms); w = 2 keeps
        // 16 x 16 x 8, which already fits twice.
        const bool col = nufft::spread_uses_columns(3, p->w) && p->method == NUFFT_METHOD_SM;
        const size_t full = nufft::spread_lds_limit();
        for (int pass = col ? 0 : 1; pass < 3; ++pass) {
            if (pass == 1 && p->method != NUFFT_METHOD_SM) continue;
            const size_t limit = (pass == 1) ? full / 2
                                 : (pass == 0) ? full / (size_t)nufft::spread_col_per_cu(p->prec, p->w)
                                               : full;
            for (auto& c : c3) {
                if (pass >= 1 && c[0] > 16) continue;   // the point-patch kernel keeps at most 16 x 16 x 8
                int mm[3] = {c[0], c[1], c[2]};
                // the column kernel's fp64 bin (z pitch >= depth) also covers the interpolation tile
                const size_t need = (pass == 0) ? nufft::spread_col_lds_bytes(p->prec, p->w, mm)
                                                : nufft::spread_tile_bytes(p->prec, 3, p->w, mm);
                if (need > 0 && need <= limit) {
                    m[0] = c[0];
                    m[1] = c[1];
                    m[2] = c[2];
                    return;
                }
            }
        }
    }
    m[0] = m[1] = m[2] = 1;
}

nufft::GeomArgs geom(const nufft_plan p) {
    nufft::GeomArgs g{};
    g.dim = p->dim;
    g.w = p->w;
    for (int i = 0; i < 3; ++i) {
        g.n[i] = (int)p->n[i];
        g.s[i] = p->s[i];
        g.m[i] = p->m[i];
        g.nb[i] = p->nb[i];
        g.xs[i] = nullptr;
    }
    g.beta = p->beta;
    g.M = p->M;
    for (int i = 0; i < p->dim; ++i)
        g.xs[i] = (const char*)p->xs.p + (size_t)i * (size_t)std::max<int64_t>(p->M, 0) * real_size(p);
    g.perm = (const int32_t*)p->perm.p;
    g.cperm = g.perm;
    g.sub = (const int32_t*)p->sub.p;
    g.nsub = p->nsub;
    g.nv = 1;
    g.cvs = std::max<int64_t>(p->M, 0);
    g.gvs = grid_cells(p);
    g.range_err = (unsigned int*)p->range_err.p;
    return g;
}

void record(nufft_plan p, int i) {
    if (p->opts.timing && p->ev_ok) (void)hipEventRecord(p->ev[p->ev_cur][i], p->stream);
}

// Opens the event set for a stage group (bit: 1 type 1, 2 type 2, 4 sort): a new set when the
// group starts a step (the sort) or when the current set already holds this group.
void begin_group(nufft_plan p, unsigned char bit) {
    if (!p->opts.timing || !p->ev_ok) return;
    if (p->ev_n == 0 || bit == 4 || (p->ev_rec[p->ev_cur] & bit)) {
        p->ev_cur = (p->ev_cur + 1) % nufft_plan_s::kEvRing;
        p->ev_rec[p->ev_cur] = 0;
        p->ev_n = std::min(p->ev_n + 1, nufft_plan_s::kEvRing);
    }
}

void end_group(nufft_plan p, unsigned char bit) {
    if (p->opts.timing && p->ev_ok) p->ev_rec[p->ev_cur] |= bit;
}

int fft_exec(nufft_plan plan, rocfft_plan fp, void* src, void* dst) {
    void* in[1] = {src};
    void* out[1] = {dst};
    rocfft_status s = rocfft_execute(fp, in, out, plan->fft_info);
    if (s != rocfft_status_success) return fail(plan, NUFFT_ERR_FFT, "rocfft_execute failed");
    return NUFFT_OK;
}

// rocFFT plan for one direction (forward for type 1, backward for type 2), unnormalised, over
// nv contiguous fine grids, out of place into a second grid buffer (the input grid is scratch;
// 256^3 fp32: 0.164 ms against 0.193 in place, 512^3 fp64: 3.38 against 3.83 ms); the work
// buffer is shared by all plans and grown when needed.
int make_fft_plan(nufft_plan plan, int direction, int nv = 1) {
    rocfft_plan& slot = (nv == 1) ? ((direction == 1) ? plan->fft_fwd : plan->fft_bwd)
                                  : plan->fft_many[direction - 1];
    if (nv > 1 && plan->fft_many_nv[direction - 1] != nv && slot) {
        rocfft_plan_destroy(slot);
        slot = nullptr;
    }
    if (slot) return NUFFT_OK;
    std::call_once(g_rocfft_once, [] { g_rocfft_setup = rocfft_setup(); });
    if (g_rocfft_setup != rocfft_status_success) return fail(plan, NUFFT_ERR_FFT, "rocfft_setup failed");
    size_t lengths[3] = {(size_t)plan->n[0], (size_t)plan->n[1], (size_t)plan->n[2]};
    rocfft_precision fprec = plan->prec == 0 ? rocfft_precision_single : rocfft_precision_double;
    rocfft_transform_type tt = (direction == 1) ? rocfft_transform_type_complex_forward
                                                : rocfft_transform_type_complex_inverse;
    rocfft_plan fp = nullptr;
    if (rocfft_plan_create(&fp, rocfft_placement_notinplace, tt, fprec, (size_t)plan->dim, lengths, (size_t)nv,
                           nullptr) != rocfft_status_success)
        return fail(plan, NUFFT_ERR_FFT, "rocfft_plan_create failed");
    slot = fp;
    if (nv > 1) plan->fft_many_nv[direction - 1] = nv;
    if (!plan->fft_info) {
        if (rocfft_execution_info_create(&plan->fft_info) != rocfft_status_success)
            return fail(plan, NUFFT_ERR_FFT, "rocfft_execution_info_create failed");
        if (rocfft_execution_info_set_stream(plan->fft_info, plan->stream) != rocfft_status_success)
            return fail(plan, NUFFT_ERR_FFT, "rocfft_execution_info_set_stream failed");
    }
    size_t work = 0;
    if (rocfft_plan_get_work_buffer_size(fp, &work) != rocfft_status_success)
        return fail(plan, NUFFT_ERR_FFT, "rocfft_plan_get_work_buffer_size failed");
    if (work > plan->fft_work.bytes) {
        int rc = dev_alloc(plan, plan->fft_work, work, "FFT work buffer");
        if (rc != NUFFT_OK) return rc;
        if (rocfft_execution_info_set_work_buffer(plan->fft_info, plan->fft_work.p, work) != rocfft_status_success)
            return fail(plan, NUFFT_ERR_FFT, "rocfft_execution_info_set_work_buffer failed");
    }
    return NUFFT_OK;
}

// Timing slots: events [0..4] bracket the type 1 steps (clear, spread, FFT, deconvolve),
// [8..11] the type 2 steps (pad, FFT, interp), [5..6] the sort.
enum { EV_T1 = 0, EV_SORT0 = 5, EV_SORT1 = 6, EV_T2 = 8 };

// Fine grids (spreading / FFT input and FFT output) and fp64 gather scratch for one batch of nv
// vectors: the plan's own buffers for nv = 1, the many-vector buffers otherwise.
int batch_buffers(nufft_plan plan, int nv, void** grid, void** grid2, void** cscratch) {
    const size_t gbytes = (size_t)grid_cells(plan) * 2 * real_size(plan);
    int rc;
    if (nv == 1) {
        if ((rc = dev_alloc(plan, plan->grid2, gbytes, "FFT output grid")) != NUFFT_OK) return rc;
        *grid = plan->grid.p;
        *grid2 = plan->grid2.p;
        *cscratch = plan->sort_tmp.p;
        return NUFFT_OK;
    }
    if ((rc = dev_alloc(plan, plan->grid_many, gbytes * nv, "many-vector fine grids")) != NUFFT_OK) return rc;
    if ((rc = dev_alloc(plan, plan->grid_many2, gbytes * nv, "many-vector FFT output grids")) != NUFFT_OK) return rc;
    // (1D fp64 spreading reads the strengths through the permutation and needs no gather scratch)
    if (plan->prec == 1 && plan->dim >= 2 && plan->M > 0 &&
        (rc = dev_alloc(plan, plan->c_many, (size_t)plan->M * 16 * nv, "many-vector strengths")) != NUFFT_OK)
        return rc;
    *grid = plan->grid_many.p;
    *grid2 = plan->grid_many2.p;
    *cscratch = (plan->prec == 1 && plan->dim >= 2) ? plan->c_many.p : plan->sort_tmp.p;
    return NUFFT_OK;
}

// Type 1 on the plan's points for nv vectors: c (nv x M) -> f (nv x N^d).
int run_type1(nufft_plan plan, const void* c, void* f, int nv = 1) {
    int rc;
    if ((rc = make_fft_plan(plan, 1, nv)) != NUFFT_OK) return rc;
    void *grid, *grid2, *cs;
    if ((rc = batch_buffers(plan, nv, &grid, &grid2, &cs)) != NUFFT_OK) return rc;
    nufft::GeomArgs g = geom(plan);
    g.nv = nv;
    const size_t gbytes = (size_t)grid_cells(plan) * 2 * real_size(plan) * nv;
    begin_group(plan, 1);
    record(plan, EV_T1 + 0);
    NUFFT_HIP(nufft::launch_fill_zero(grid, gbytes, plan->stream));
    record(plan, EV_T1 + 1);
    NUFFT_HIP(nufft::launch_spread(plan->prec, plan->method, g, c, grid, plan->stream, plan->colw > 0, cs));
    record(plan, EV_T1 + 2);
    if ((rc = fft_exec(plan, nv == 1 ? plan->fft_fwd : plan->fft_many[0], grid, grid2)) != NUFFT_OK) return rc;
    record(plan, EV_T1 + 3);
    NUFFT_HIP(nufft::launch_deconvolve(plan->prec, plan->dim, plan->N, plan->n, plan->pcorr.p, grid2, f,
                                       plan->stream, nv));
    record(plan, EV_T1 + 4);
    end_group(plan, 1);
    return NUFFT_OK;
}

// Type 2 on the plan's points for nv vectors: f (nv x N^d) -> c (nv x M).
int run_type2(nufft_plan plan, void* c, const void* f, int nv = 1) {
    int rc;
    if ((rc = make_fft_plan(plan, 2, nv)) != NUFFT_OK) return rc;
    void *grid, *grid2, *cs;
    if ((rc = batch_buffers(plan, nv, &grid, &grid2, &cs)) != NUFFT_OK) return rc;
    nufft::GeomArgs g = geom(plan);
    g.nv = nv;
    begin_group(plan, 2);
    record(plan, EV_T2 + 0);
    NUFFT_HIP(nufft::launch_precorrect_pad(plan->prec, plan->dim, plan->N, plan->n, plan->pcorr.p, f, grid,
                                           plan->stream, nv));
    record(plan, EV_T2 + 1);
    if ((rc = fft_exec(plan, nv == 1 ? plan->fft_bwd : plan->fft_many[1], grid, grid2)) != NUFFT_OK) return rc;
    record(plan, EV_T2 + 2);
    NUFFT_HIP(nufft::launch_interp(plan->prec, plan->method, g, grid2, c, plan->stream));
    record(plan, EV_T2 + 3);
    end_group(plan, 2);
    return NUFFT_OK;
}

// nvec transforms of the given type in batches (see nufft_execute_many).
int run_many(nufft_plan plan, int type, int nvec, void* c, void* f) {
    const size_t cbytes = (size_t)std::max<int64_t>(plan->M, 0) * 2 * real_size(plan);
    const size_t fbytes = (size_t)mode_count(plan) * 2 * real_size(plan);
    int b = plan->opts.max_batch > 0 ? plan->opts.max_batch : 16;
    if (plan->opts.max_batch <= 0) {
        const size_t per = (size_t)grid_cells(plan) * 4 * real_size(plan) + (plan->prec == 1 ? cbytes : 0);
        while (b > 1 && (size_t)b * per > (size_t(2) << 30)) --b;
    }
    for (int v0 = 0; v0 < nvec; v0 += b) {
        const int nv = std::min(b, nvec - v0);
        char* cv = (char*)c + (size_t)v0 * cbytes;
        char* fv = (char*)f + (size_t)v0 * fbytes;
        int rc = type == 1 ? run_type1(plan, cv, fv, nv) : run_type2(plan, cv, fv, nv);
        if (rc != NUFFT_OK) return rc;
    }
    return NUFFT_OK;
}

int check_plan(nufft_plan p) {
    if (!p) return NUFFT_ERR_BAD_ARG;
    return NUFFT_OK;
}

// Entry points that act on the fine grid of a type 1 / type 2 plan.
int check_not_type3(nufft_plan p) {
    if (p->type == 3) return fail(p, NUFFT_ERR_UNSUPPORTED, "not available on a type 3 plan");
    return NUFFT_OK;
}

// Type 3 (see nufft_setpts_type3): f = post * T2(spread(pre * c)).
int run_type3(nufft_plan plan, const void* c, void* f) {
    if (plan->M > 0) NUFFT_HIP(nufft::launch_t3_cmul(plan->prec, c, plan->t3_pre.p, plan->M, plan->t3_cp.p, plan->stream));
    int rc = nufft_spread(plan->t3_spread, plan->t3_cp.p, plan->t3_spread->grid.p);
    if (rc != NUFFT_OK) return fail(plan, rc, std::string("type 3 spreading: ") + plan->t3_spread->last_error);
    rc = nufft_execute(plan->t3_eval, plan->t3_cin.p, plan->t3_spread->grid.p);
    if (rc != NUFFT_OK) return fail(plan, rc, std::string("type 3 evaluation: ") + plan->t3_eval->last_error);
    if (plan->K > 0) NUFFT_HIP(nufft::launch_t3_cmul(plan->prec, plan->t3_cin.p, plan->t3_post.p, plan->K, f, plan->stream));
    return NUFFT_OK;
}

int check_points(nufft_plan p) {
    if (p->M < 0) return fail(p, NUFFT_ERR_BAD_STATE, "no points: call nufft_setpts first");
    return NUFFT_OK;
}

// ------------------------------------------------------------------------------------------------
// setpts (bin-sort and subproblems) with the plan's own scratch, or without allocating
// ------------------------------------------------------------------------------------------------

// Device scratch of nufft_setpts_noalloc: the sort's temporaries (key / value ping-pong buffers,
// digit histograms, scans and the two result slots).  One array per GPU, loaded with the library's
// code and held until the process ends.  In host code `scratch` is only a handle for
// hipGetSymbolAddress: the device address of each GPU's copy is looked up once per device, with
// that device current, and kept in g_scratch_ptr.
constexpr size_t kNoallocScratchBytes = NUFFT_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(int device, void** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != device) (void)hipSetDevice(cur);
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

// noalloc: sort in the device array above, read the result slots into host stack memory, and
// require the plan's point buffers (sized by an earlier nufft_setpts) to be large enough.
int setpts_impl(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z, bool noalloc) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (plan->type == 3) return fail(plan, NUFFT_ERR_BAD_ARG, "a type 3 plan takes nufft_setpts_type3");
    if (M < 0 || M > INT32_MAX) return fail(plan, NUFFT_ERR_BAD_ARG, "M out of range [0, 2^31-1]");
    const void* X[3] = {x, y, z};
    if (M > 0)
        for (int i = 0; i < plan->dim; ++i)
            if (!X[i]) return fail(plan, NUFFT_ERR_BAD_ARG, "null coordinate array");
    plan->M = -1;
    plan->nsub = 0;
    const size_t rs = real_size(plan);
    const size_t Mm = (size_t)std::max<int64_t>(M, 1);
    int rc;
    const size_t sort_bytes = nufft::sort_scratch_bytes(M, (int)plan->nbins, plan->dim, plan->prec) + 256;
    char* scr = nullptr;        // sort scratch: the plan's, or the device array
    size_t scr_bytes = 0;
    if (noalloc) {
        if (sort_bytes > kNoallocScratchBytes)
            return fail(plan, NUFFT_ERR_ALLOC, "nufft_setpts_noalloc: sorting " + std::to_string(M) + " points needs " +
                                                   std::to_string(sort_bytes) + " bytes of scratch, more than the " +
                                                   std::to_string(kNoallocScratchBytes) + "-byte no-allocation scratch");
        if ((size_t)M > plan->pts_cap || plan->counts.bytes < (size_t)plan->nbins * sizeof(int32_t) ||
            plan->offsets.bytes < (size_t)(plan->nbins + 1) * sizeof(int32_t) || !plan->sort_tmp.p)
            return fail(plan, NUFFT_ERR_ALLOC, "nufft_setpts_noalloc: the plan's point buffers hold fewer than " +
                                                   std::to_string(M) +
                                                   " points; size them with nufft_setpts on at least as many points");
        void* p = nullptr;
        NUFFT_HIP(noalloc_scratch(plan->device, &p));
        scr = (char*)p;
        scr_bytes = sort_bytes;
    } else {
        if ((rc = dev_alloc(plan, plan->xs, Mm * plan->dim * rs, "sorted coordinates")) != NUFFT_OK ||
            (rc = dev_alloc(plan, plan->perm, Mm * sizeof(int32_t), "permutation")) != NUFFT_OK ||
            (rc = dev_alloc(plan, plan->counts, (size_t)plan->nbins * sizeof(int32_t), "bin counts")) != NUFFT_OK ||
            (rc = dev_alloc(plan, plan->offsets, (size_t)(plan->nbins + 1) * sizeof(int32_t), "bin offsets")) != NUFFT_OK ||
            (rc = dev_alloc(plan, plan->sort_tmp, sort_bytes, "sort scratch")) != NUFFT_OK)
            return rc;
        // points the buffers hold (they only grow); the sort scratch also holds the gathered
        // strengths of fp64 executes, at least M complex values
        plan->pts_cap = std::min(plan->xs.bytes / (plan->dim * rs), plan->perm.bytes / sizeof(int32_t));
        if (!plan->host_tail) NUFFT_HIP(hipHostMalloc(&plan->host_tail, 128, hipHostMallocDefault));
        scr = (char*)plan->sort_tmp.p;
        scr_bytes = plan->sort_tmp.bytes;
    }
    // two small result slots at the end of the scratch: int64 subproblem count, int bad-point flag,
    // read back into pinned memory (or, without allocation, into host stack memory)
    char* tail = scr + (scr_bytes - 256);
    int64_t* nsub_dev = (int64_t*)tail;
    int* bad_dev = (int*)(tail + 64);
    alignas(64) unsigned char stack_tail[128];
    unsigned char* host_tail = noalloc ? stack_tail : (unsigned char*)plan->host_tail;

    begin_group(plan, 4);
    record(plan, EV_SORT0);
    NUFFT_HIP(nufft::launch_zero_words(bad_dev, 1, plan->stream));
    nufft::SortArgs a{};
    a.dim = plan->dim;
    a.prec = plan->prec;
    a.M = M;
    for (int i = 0; i < 3; ++i) {
        a.x[i] = i < plan->dim ? X[i] : nullptr;
        a.n[i] = (int)plan->n[i];
        a.s[i] = plan->s[i];
        a.m[i] = plan->m[i];
        a.nb[i] = plan->nb[i];
    }
    a.nbins = (int)plan->nbins;
    a.nbits = plan->nbits;
    a.cap = plan->cap;
    a.colw = plan->colw;
    a.colstep = plan->colstep;
    a.ncol = plan->ncol;
    if (plan->method == NUFFT_METHOD_GM) {
        // no sort and no binning: the points stay in the caller's order and the bin counts read zero
        NUFFT_HIP(nufft::launch_fill_zero(plan->counts.p, (size_t)plan->nbins * sizeof(int32_t), plan->stream));
        NUFFT_HIP(nufft::launch_identity_order(a, (int32_t*)plan->perm.p, plan->xs.p, bad_dev, plan->stream));
        NUFFT_HIP(hipMemcpyAsync(host_tail, tail, 128, hipMemcpyDeviceToHost, plan->stream));
        NUFFT_HIP(hipStreamSynchronize(plan->stream));
        const int host_bad = *(const int*)(host_tail + 64);
        if (host_bad) return fail(plan, NUFFT_ERR_POINTS, "a coordinate is not finite or outside [-3pi, 3pi)");
        record(plan, EV_SORT1);
        end_group(plan, 4);
        plan->M = M;
        plan->nsub = 0;
        return NUFFT_OK;
    }
    NUFFT_HIP(nufft::launch_sort(a, (int32_t*)plan->perm.p, (int32_t*)plan->counts.p, (int32_t*)plan->offsets.p,
                                 plan->xs.p, scr, scr_bytes - 256, nsub_dev, bad_dev, plan->stream));
    // one read of both result slots
    NUFFT_HIP(hipMemcpyAsync(host_tail, tail, 128, hipMemcpyDeviceToHost, plan->stream));
    NUFFT_HIP(hipStreamSynchronize(plan->stream));
    const int64_t host_nsub = *(const int64_t*)host_tail;
    const int host_bad = *(const int*)(host_tail + 64);
    if (host_bad) return fail(plan, NUFFT_ERR_POINTS, "a coordinate is not finite or outside [-3pi, 3pi)");
    const size_t sub_bytes = (size_t)std::max<int64_t>(host_nsub, 1) * 3 * sizeof(int32_t);
    if (noalloc) {
        if (plan->sub.bytes < sub_bytes)
            return fail(plan, NUFFT_ERR_ALLOC, "nufft_setpts_noalloc: the plan's subproblem list holds fewer than " +
                                                   std::to_string(host_nsub) +
                                                   " subproblems; size it with nufft_setpts on a point set with as many");
    } else if ((rc = dev_alloc(plan, plan->sub, sub_bytes, "subproblem list")) != NUFFT_OK) {
        return rc;
    }
    NUFFT_HIP(nufft::launch_build_subproblems_from(M, (int)plan->nbins, plan->dim, plan->prec, plan->cap, host_nsub,
                                                   (const int32_t*)plan->counts.p, (const int32_t*)plan->offsets.p,
                                                   scr, (int32_t*)plan->sub.p, plan->stream));
    record(plan, EV_SORT1);
    end_group(plan, 4);
    plan->M = M;
    plan->nsub = host_nsub;
    return NUFFT_OK;
}

}  // namespace

extern "C" {

int nufft_default_opts(nufft_opts* opts) {
    if (!opts) return NUFFT_ERR_BAD_ARG;
    std::memset(opts, 0, sizeof(*opts));
    return NUFFT_OK;
}

const char* nufft_strerror(int status) {
    switch (status) {
        case NUFFT_OK: return "success";
        case NUFFT_WARN_EPS_CLAMPED: return "warning: tolerance outside the supported range; kernel width clamped";
        case NUFFT_ERR_BAD_ARG: return "invalid argument";
        case NUFFT_ERR_BAD_STATE: return "invalid plan state (e.g. execute before setpts)";
        case NUFFT_ERR_ALLOC: return "device allocation failed or exceeded the configured limit";
        case NUFFT_ERR_HIP: return "HIP runtime error";
        case NUFFT_ERR_FFT: return "rocFFT error";
        case NUFFT_ERR_POINTS: return "nonuniform point is not finite or outside [-3pi, 3pi)";
        case NUFFT_ERR_UNSUPPORTED: return "unsupported request";
        default: return "unknown status";
    }
}

const char* nufft_last_error(nufft_plan plan) { return plan ? plan->last_error.c_str() : ""; }

int nufft_destroy(nufft_plan plan) {
    if (!plan) return NUFFT_OK;
    (void)hipStreamSynchronize(plan->stream);
    if (plan->fft_fwd) rocfft_plan_destroy(plan->fft_fwd);
    if (plan->fft_bwd) rocfft_plan_destroy(plan->fft_bwd);
    for (rocfft_plan fp : plan->fft_many)
        if (fp) rocfft_plan_destroy(fp);
    if (plan->fft_info) rocfft_execution_info_destroy(plan->fft_info);
    if (plan->t3_spread) nufft_destroy(plan->t3_spread);
    if (plan->t3_eval) nufft_destroy(plan->t3_eval);
    for (DevBuf* b : {&plan->grid, &plan->grid2, &plan->grid_many2, &plan->pcorr, &plan->fft_work, &plan->xs, &plan->perm, &plan->counts,
                      &plan->offsets, &plan->sub, &plan->range_err, &plan->sort_tmp, &plan->grid_many, &plan->c_many,
                      &plan->t3_part,
                      &plan->t3_y, &plan->t3_theta, &plan->t3_pre, &plan->t3_post, &plan->t3_cp, &plan->t3_cin,
                      &plan->t3_tab})
        dev_free(plan, *b);
    if (plan->host_tail) (void)hipHostFree(plan->host_tail);
    if (plan->ev_ok)
        for (auto& set : plan->ev)
            for (auto& e : set) (void)hipEventDestroy(e);
    delete plan;
    return NUFFT_OK;
}

int nufft_plan_create(int type, int dim, const int64_t* N, double eps, int precision, void* stream,
                      const nufft_opts* opts, nufft_plan* out) {
    if (!out) return NUFFT_ERR_BAD_ARG;
    *out = nullptr;
    if (type < 1 || type > 3 || dim < 1 || dim > 3 || (!N && type != 3) || (precision != 0 && precision != 1))
        return NUFFT_ERR_BAD_ARG;
    if (!(eps > 0.0) || !std::isfinite(eps)) return NUFFT_ERR_BAD_ARG;
    for (int i = 0; type != 3 && i < dim; ++i)
        if (N[i] < 1 || N[i] > (int64_t(1) << 28)) return NUFFT_ERR_BAD_ARG;

    nufft_plan plan = new (std::nothrow) nufft_plan_s();
    if (!plan) return NUFFT_ERR_ALLOC;
    plan->type = type;
    plan->dim = dim;
    plan->prec = precision;
    plan->eps = eps;
    plan->stream = (hipStream_t)stream;
    if (opts) plan->opts = *opts;
    int status = NUFFT_OK;

    // eq. (6): w = ceil(log10(1/eps)) + 1 (an exact power of ten counts as its integer log), beta = 2.30 w.
    // sigma < 2 (not on the page): the kernel transform must have decayed at the first alias of the
    // band, xi = w pi (1 - 1/(2 sigma)), and the truncation error falls like exp(-pi w sqrt(1 - 1/sigma))
    const double sigma = plan->opts.upsampfac == 0.0 ? 2.0 : plan->opts.upsampfac;
    if (!(sigma >= 1.25 && sigma <= 2.0)) {
        delete plan;
        return NUFFT_ERR_BAD_ARG;
    }
    plan->sigma = sigma;
    int w = (sigma == 2.0) ? (int)std::ceil(std::log10(1.0 / eps) - 1e-9) + 1
                           : (int)std::ceil(std::log(1.0 / eps) / (nufft::kPi * std::sqrt(1.0 - 1.0 / sigma)) - 1e-9);
    if (w < nufft::kMinW || w > nufft::kMaxW) {
        w = std::min(std::max(w, nufft::kMinW), nufft::kMaxW);
        status = NUFFT_WARN_EPS_CLAMPED;
    }
    plan->w = w;
    plan->beta = (sigma == 2.0) ? 2.30 * w : (2.30 / (0.75 * nufft::kPi)) * nufft::kPi * (1.0 - 0.5 / sigma) * w;
    if (type == 3) {
        // the fine grid, the inner plans and everything else depend on the points (setpts_type3)
        if (sigma != 2.0) {
            delete plan;
            return NUFFT_ERR_UNSUPPORTED;
        }
        hipError_t he3 = hipGetDevice(&plan->device);
        if (he3 != hipSuccess) {
            delete plan;
            return NUFFT_ERR_HIP;
        }
        *out = plan;
        return status;
    }
    for (int i = 0; i < 3; ++i) {
        plan->N[i] = i < dim ? N[i] : 1;
        plan->n[i] = i < dim ? next_5smooth(std::max<int64_t>((int64_t)std::ceil(sigma * (double)N[i] - 1e-9), w)) : 1;
        plan->s[i] = (double)plan->n[i] / (2.0 * nufft::kPi);
    }
    // fewer than 2^32 cells: rocFFT's 3D transforms of 2^32 elements returned wrong values here
    // (a delta function's transform, 2048 x 2048 x 1024), while 2048 x 2048 x 1000 was exact
    if (grid_cells(plan) >= (int64_t(1) << 32)) {
        nufft_destroy(plan);
        return NUFFT_ERR_BAD_ARG;
    }
    hipError_t he = hipGetDevice(&plan->device);
    if (he != hipSuccess) {
        nufft_destroy(plan);
        return NUFFT_ERR_HIP;
    }

    // method, bins and subproblem cap
    plan->method = (plan->opts.method == NUFFT_METHOD_GM_SORT || plan->opts.method == NUFFT_METHOD_GM)
                       ? plan->opts.method
                       : NUFFT_METHOD_SM;
    int m[3] = {1, 1, 1};
    if (plan->opts.bin[0] > 0) {
        for (int i = 0; i < dim; ++i) m[i] = std::max(1, plan->opts.bin[i]);
    } else {
        default_bins(plan, m);
    }
    for (int i = 0; i < 3; ++i) {
        plan->m[i] = i < dim ? (int)std::min<int64_t>(m[i], plan->n[i]) : 1;
        plan->nb[i] = (int)((plan->n[i] + plan->m[i] - 1) / plan->m[i]);
    }
    plan->nbins = (int64_t)plan->nb[0] * plan->nb[1] * plan->nb[2];
    // 3D spreading by column runs needs the points of a bin ordered by support column
    plan->colw = 0;
    plan->colstep = 1;
    plan->ncol = 1;
    // (the column step is positive only at the widths the column kernels serve, w <= 12)
    const bool col_width = plan->method == NUFFT_METHOD_SM && nufft::spread_uses_columns(dim, w);
    const size_t col_lds = col_width ? nufft::spread_col_lds_bytes(plan->prec, w, plan->m) : 0;
    const int step = col_width ? nufft::spread_col_step(w) : 1;
    const int64_t ncol = (int64_t)((plan->m[0] + step) / step) * ((plan->m[1] + step) / step) *
                         (plan->m[2] + 1);
    const bool col_fits = col_width && plan->m[2] == 8 && col_lds > 0 && col_lds <= nufft::spread_lds_limit() &&
                          plan->nbins * ncol < (int64_t(1) << 31);
    // the bins must fit the spreader this plan will run, and the interpolation tile
    if ((!col_fits && plan->method == NUFFT_METHOD_SM &&
         nufft::spread_tile_bytes(plan->prec, dim, w, plan->m) > nufft::spread_lds_limit()) ||
        nufft::interp_tile_bytes(plan->prec, dim, w, plan->m) > nufft::spread_lds_limit()) {
        plan->last_error = "bin size too large for LDS";
        nufft_destroy(plan);
        return NUFFT_ERR_BAD_ARG;
    }
    if (col_fits) {
        plan->colw = w;
        plan->colstep = step;
        plan->ncol = (int)ncol;
    }
    plan->nbits = bit_length(plan->nbins * plan->ncol - 1);
    int64_t vol = (int64_t)plan->m[0] * plan->m[1] * plan->m[2];
    plan->cap = plan->opts.subproblem_cap > 0 ? plan->opts.subproblem_cap
                                              : (int)std::max<int64_t>(1024, 2 * vol);

    // fine grid and correction factors (eq. (10)): p_i(k) = (2/w) (-1)^k / phihat(alpha_i k),
    // alpha_i = w pi / n_i; (-1)^k is the phase of the grid origin at -pi.
    const size_t rs = real_size(plan);
    int rc;
    if ((rc = dev_alloc(plan, plan->grid, (size_t)grid_cells(plan) * 2 * rs, "fine grid")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->pcorr, (size_t)(plan->N[0] + plan->N[1] + plan->N[2]) * rs,
                        "correction factors")) != NUFFT_OK) {
        nufft_destroy(plan);
        return rc;
    }
    {
        PhiHat ph;
        std::vector<double> p;
        for (int i = 0; i < 3; ++i) {
            const int64_t Ni = plan->N[i];
            const double alpha = w * nufft::kPi / (double)plan->n[i];
            for (int64_t idx = 0; idx < Ni; ++idx) {
                int64_t k = idx - Ni / 2;
                double v = (i < dim) ? (2.0 / w) * ((k % 2 == 0) ? 1.0 : -1.0) / ph(alpha * (double)k, plan->beta)
                                     : 1.0;
                p.push_back(v);
            }
        }
        hipError_t e;
        if (plan->prec == 0) {
            std::vector<float> pf(p.begin(), p.end());
            e = hipMemcpy(plan->pcorr.p, pf.data(), pf.size() * sizeof(float), hipMemcpyHostToDevice);
        } else {
            e = hipMemcpy(plan->pcorr.p, p.data(), p.size() * sizeof(double), hipMemcpyHostToDevice);
        }
        if (e != hipSuccess) {
            hip_fail(plan, e, "hipMemcpy correction factors");
            nufft_destroy(plan);
            return NUFFT_ERR_HIP;
        }
    }

    // counter of kernel-support starts found outside their padded tile (nufft_get_range_errors)
    if ((rc = dev_alloc(plan, plan->range_err, 256, "range-error counter")) != NUFFT_OK) {
        nufft_destroy(plan);
        return rc;
    }
    {
        hipError_t e = hipMemset(plan->range_err.p, 0, 256);
        if (e != hipSuccess) {
            hip_fail(plan, e, "hipMemset range-error counter");
            nufft_destroy(plan);
            return NUFFT_ERR_HIP;
        }
    }

    // rocFFT plan of the plan's own direction (the adjoint direction is made on first use)
    if ((rc = make_fft_plan(plan, type)) != NUFFT_OK) {
        nufft_destroy(plan);
        return rc;
    }
    if (plan->opts.timing) {
        plan->ev_ok = true;
        for (auto& set : plan->ev)
            for (auto& e : set)
                if (hipEventCreate(&e) != hipSuccess) plan->ev_ok = false;
    }
    *out = plan;
    return status;
}

int nufft_setpts(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z) {
    return setpts_impl(plan, M, x, y, z, false);
}

int nufft_setpts_noalloc(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z) {
    return setpts_impl(plan, M, x, y, z, true);
}

int nufft_setpts_type3(nufft_plan plan, int64_t M, const void* x, const void* y, const void* z, int64_t K,
                       const void* s, const void* t, const void* u) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (plan->type != 3) return fail(plan, NUFFT_ERR_BAD_ARG, "nufft_setpts_type3 needs a type 3 plan");
    if (M < 0 || M > INT32_MAX || K < 0 || K > INT32_MAX)
        return fail(plan, NUFFT_ERR_BAD_ARG, "M or K out of range [0, 2^31-1]");
    const void* X[3] = {x, y, z};
    const void* S[3] = {s, t, u};
    const int dim = plan->dim;
    for (int i = 0; i < dim; ++i)
        if ((M > 0 && !X[i]) || (K > 0 && !S[i])) return fail(plan, NUFFT_ERR_BAD_ARG, "null coordinate array");
    plan->M = -1;
    plan->K = -1;
    const size_t rs = real_size(plan);
    int rc;

    // centres and half-widths of sources and targets
    const int nb = nufft::t3_minmax_blocks();
    if ((rc = dev_alloc(plan, plan->t3_part, (size_t)2 * dim * nb * 2 * sizeof(double), "type 3 partials")) != NUFFT_OK)
        return rc;
    double* part = (double*)plan->t3_part.p;
    for (int i = 0; i < dim; ++i) {
        NUFFT_HIP(nufft::launch_t3_minmax(plan->prec, X[i], M, part + (size_t)(2 * i) * nb * 2, plan->stream));
        NUFFT_HIP(nufft::launch_t3_minmax(plan->prec, S[i], K, part + (size_t)(2 * i + 1) * nb * 2, plan->stream));
    }
    std::vector<double> hp((size_t)2 * dim * nb * 2);
    NUFFT_HIP(hipMemcpyAsync(hp.data(), part, hp.size() * sizeof(double), hipMemcpyDeviceToHost, plan->stream));
    NUFFT_HIP(hipStreamSynchronize(plan->stream));
    double C[3] = {0, 0, 0}, Xh[3] = {0, 0, 0}, D[3] = {0, 0, 0}, Sh[3] = {0, 0, 0};
    for (int a = 0; a < 2 * dim; ++a) {
        double lo = INFINITY, hi = -INFINITY;
        for (int b = 0; b < nb; ++b) {
            const double l = hp[((size_t)a * nb + b) * 2], h = hp[((size_t)a * nb + b) * 2 + 1];
            if (std::isnan(l)) return fail(plan, NUFFT_ERR_POINTS, "a type 3 coordinate is not finite");
            lo = std::min(lo, l);
            hi = std::max(hi, h);
        }
        const bool any = (a % 2 == 0) ? M > 0 : K > 0;
        const double ctr = any ? 0.5 * (hi + lo) : 0.0, half = any ? 0.5 * (hi - lo) : 0.0;
        if (a % 2 == 0) {
            C[a / 2] = ctr;
            Xh[a / 2] = half;
        } else {
            D[a / 2] = ctr;
            Sh[a / 2] = half;
        }
    }

    // fine grid n (smallest even 5-smooth >= max(2 sigma X S / pi + w, 2 w)), h = 2 pi / n and
    // scale gamma: n / (2 sigma S) keeps the scaled targets in the kernel's band and, by the
    // choice of n, the scaled sources (x - C) / gamma inside [-pi, pi) with the kernel's reach
    const int w = plan->w;
    const double sigma = plan->sigma;
    int64_t n[3] = {1, 1, 1};
    double h[3] = {1, 1, 1}, gam[3] = {1, 1, 1}, alpha[3] = {0, 0, 0}, off[3] = {0, 0, 0};
    int64_t cells = 1;
    for (int i = 0; i < dim; ++i) {
        const double v = std::max(2.0 * sigma * Xh[i] * Sh[i] / nufft::kPi + w, 2.0 * w);
        if (!(v < (double)(int64_t(1) << 30))) return fail(plan, NUFFT_ERR_BAD_ARG, "type 3 fine grid too large");
        int64_t ni = std::max<int64_t>((int64_t)std::ceil(v - 1e-9), 2);
        while (ni % 2 || !is_5smooth(ni)) ++ni;
        n[i] = ni;
        h[i] = 2.0 * nufft::kPi / (double)ni;
        if (Sh[i] > 0) gam[i] = (double)ni / (2.0 * sigma * Sh[i]);
        else if (Xh[i] > 0) gam[i] = Xh[i] * (double)ni / (nufft::kPi * (double)(ni - w));
        else gam[i] = 1.0;
        alpha[i] = w * h[i] / 2.0;
        off[i] = h[i] * (double)(ni / 2) - nufft::kPi;
        cells *= ni;
        if (cells > (int64_t(1) << 31) - 1) return fail(plan, NUFFT_ERR_BAD_ARG, "type 3 fine grid too large");
    }

    // inner plans: a type 1 plan whose fine grid is n (N = n / 2) and a type 2 plan with N = n modes
    bool same = plan->t3_spread != nullptr;
    for (int i = 0; i < dim; ++i) same = same && plan->t3_n[i] == n[i];
    if (!same) {
        if (plan->t3_spread) nufft_destroy(plan->t3_spread);
        if (plan->t3_eval) nufft_destroy(plan->t3_eval);
        plan->t3_spread = plan->t3_eval = nullptr;
        nufft_opts o = plan->opts;
        o.upsampfac = 0.0;
        o.timing = 0;
        o.max_device_bytes = 0;
        int64_t Nh[3], Nf[3];
        for (int i = 0; i < dim; ++i) {
            Nh[i] = n[i] / 2;
            Nf[i] = n[i];
        }
        rc = nufft_plan_create(1, dim, Nh, plan->eps, plan->prec, plan->stream, &o, &plan->t3_spread);
        if (rc < 0) return fail(plan, rc, "type 3: inner spreading plan");
        rc = nufft_plan_create(2, dim, Nf, plan->eps, plan->prec, plan->stream, &o, &plan->t3_eval);
        if (rc < 0) return fail(plan, rc, std::string("type 3: inner evaluation plan: ") + nufft_strerror(rc));
        for (int i = 0; i < dim; ++i) {
            if (plan->t3_spread->n[i] != n[i]) return fail(plan, NUFFT_ERR_BAD_ARG, "type 3: inner fine grid mismatch");
            plan->t3_n[i] = n[i];
            plan->n[i] = n[i];
        }
    }

    // scaled sources and targets, sorted by the inner plans
    const size_t Mm = (size_t)std::max<int64_t>(M, 1), Km = (size_t)std::max<int64_t>(K, 1);
    if ((rc = dev_alloc(plan, plan->t3_y, Mm * dim * rs, "type 3 scaled sources")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->t3_theta, Km * dim * rs, "type 3 scaled targets")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->t3_pre, Mm * 2 * rs, "type 3 source phases")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->t3_cp, Mm * 2 * rs, "type 3 phased strengths")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->t3_post, Km * 2 * rs, "type 3 target factors")) != NUFFT_OK ||
        (rc = dev_alloc(plan, plan->t3_cin, Km * 2 * rs, "type 3 inner output")) != NUFFT_OK)
        return rc;
    const void* yv[3] = {nullptr, nullptr, nullptr};
    const void* tv[3] = {nullptr, nullptr, nullptr};
    for (int i = 0; i < dim; ++i) {
        void* yi = (char*)plan->t3_y.p + (size_t)i * Mm * rs;
        void* ti = (char*)plan->t3_theta.p + (size_t)i * Km * rs;
        NUFFT_HIP(nufft::launch_t3_scale(plan->prec, X[i], M, C[i], gam[i], 1.0, 1.0, yi, plan->stream));
        NUFFT_HIP(nufft::launch_t3_scale(plan->prec, S[i], K, D[i], 1.0, gam[i], h[i], ti, plan->stream));
        yv[i] = yi;
        tv[i] = ti;
    }
    rc = nufft_setpts(plan->t3_spread, M, yv[0], yv[1], yv[2]);
    if (rc != NUFFT_OK) return fail(plan, rc, std::string("type 3 sources: ") + plan->t3_spread->last_error);
    rc = nufft_setpts(plan->t3_eval, K, tv[0], tv[1], tv[2]);
    if (rc != NUFFT_OK) return fail(plan, rc, std::string("type 3 targets: ") + plan->t3_eval->last_error);

    // per-source phases and per-target factors; phihat by Gauss-Legendre in theta (z = sin theta),
    // 64 nodes on [-pi/2, pi/2] folded to the 32 positive ones (the integrand is even)
    const int nq = 32;
    std::vector<double> g64, w64, tab(2 * nq);
    gauss_legendre(2 * nq, g64, w64);
    int q = 0;
    for (int i = 0; i < 2 * nq; ++i) {
        if (g64[i] <= 0) continue;
        const double th = 0.5 * nufft::kPi * g64[i];
        tab[q] = std::sin(th);
        tab[nq + q] = 2.0 * 0.5 * nufft::kPi * w64[i] * std::exp(plan->beta * (std::cos(th) - 1.0)) * std::cos(th);
        ++q;
    }
    if (q != nq) return fail(plan, NUFFT_ERR_BAD_ARG, "type 3: quadrature table");
    if ((rc = dev_alloc(plan, plan->t3_tab, tab.size() * sizeof(double), "type 3 quadrature table")) != NUFFT_OK)
        return rc;
    NUFFT_HIP(hipMemcpyAsync(plan->t3_tab.p, tab.data(), tab.size() * sizeof(double), hipMemcpyHostToDevice,
                             plan->stream));
    NUFFT_HIP(nufft::launch_t3_factors(plan->prec, dim, C, D, gam, alpha, off, 2.0 / w, X, M, plan->t3_pre.p, S, K,
                                       (const double*)plan->t3_tab.p, nq, plan->t3_post.p, plan->stream));
    // the host table must outlive the copy
    NUFFT_HIP(hipStreamSynchronize(plan->stream));
    plan->M = M;
    plan->K = K;
    return NUFFT_OK;
}

int nufft_execute(nufft_plan plan, void* c, void* f) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (plan->type == 3) {
        if ((plan->M > 0 && !c) || (plan->K > 0 && !f)) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
        return run_type3(plan, c, f);
    }
    if ((plan->M > 0 && !c) || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    return plan->type == 1 ? run_type1(plan, c, f) : run_type2(plan, c, f);
}

int nufft_execute_adjoint(nufft_plan plan, void* c, void* f) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if ((plan->M > 0 && !c) || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    return plan->type == 1 ? run_type2(plan, c, f) : run_type1(plan, c, f);
}

int nufft_execute_many(nufft_plan plan, int nvec, void* c, void* f) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (nvec < 1) return fail(plan, NUFFT_ERR_BAD_ARG, "nvec must be >= 1");
    if ((plan->M > 0 && !c) || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    return run_many(plan, plan->type, nvec, c, f);
}

int nufft_execute_adjoint_many(nufft_plan plan, int nvec, void* c, void* f) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (nvec < 1) return fail(plan, NUFFT_ERR_BAD_ARG, "nvec must be >= 1");
    if ((plan->M > 0 && !c) || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    return run_many(plan, plan->type == 1 ? 2 : 1, nvec, c, f);
}

int nufft_get_stage_times(nufft_plan plan, double* ms) {
    if (!plan || !ms) return NUFFT_ERR_BAD_ARG;
    if (!plan->opts.timing || !plan->ev_ok) return fail(plan, NUFFT_ERR_BAD_STATE, "timing not enabled");
    NUFFT_HIP(hipStreamSynchronize(plan->stream));
    // average each stage over the event sets recorded since the last readout
    double sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < plan->ev_n; ++k) {
        const int set = (plan->ev_cur - k + nufft_plan_s::kEvRing) % nufft_plan_s::kEvRing;
        const unsigned char rec = plan->ev_rec[set];
        auto add = [&](int stage, int a, int b) {
            float t = 0;
            if (hipEventElapsedTime(&t, plan->ev[set][a], plan->ev[set][b]) == hipSuccess) {
                sum[stage] += t;
                ++cnt[stage];
            }
        };
        if (rec & 4) add(0, EV_SORT0, EV_SORT1);
        if (rec & 1) {
            add(4, EV_T1 + 0, EV_T1 + 1);
            add(1, EV_T1 + 1, EV_T1 + 2);
            add(2, EV_T1 + 2, EV_T1 + 3);
            add(3, EV_T1 + 3, EV_T1 + 4);
        }
        if (rec & 2) {
            add(7, EV_T2 + 0, EV_T2 + 1);
            add(6, EV_T2 + 1, EV_T2 + 2);
            add(5, EV_T2 + 2, EV_T2 + 3);
        }
    }
    for (int i = 0; i < 8; ++i)
        if (cnt[i] > 0) plan->stage_ms[i] = sum[i] / cnt[i];
    plan->ev_n = 0;   // the next stage group opens a new set
    for (int i = 0; i < 8; ++i) ms[i] = plan->stage_ms[i];
    return NUFFT_OK;
}

int nufft_get_info(nufft_plan plan, int64_t* info_i, double* info_d) {
    if (!plan) return NUFFT_ERR_BAD_ARG;
    if (info_i) {
        int64_t v[20] = {plan->type, plan->dim, plan->prec, plan->w, plan->n[0], plan->n[1], plan->n[2],
                         plan->N[0], plan->N[1], plan->N[2], plan->m[0], plan->m[1], plan->m[2],
                         plan->nbins, plan->M >= 0 ? plan->nsub : 0, plan->M, plan->cap, plan->method,
                         plan->colw, plan->colstep};
        std::memcpy(info_i, v, sizeof(v));
    }
    if (info_d) {
        info_d[0] = plan->beta;
        info_d[1] = plan->eps;
        info_d[2] = plan->sigma;
    }
    return NUFFT_OK;
}

int nufft_spread(nufft_plan plan, const void* c, void* grid) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (!grid || (plan->M > 0 && !c)) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    nufft::GeomArgs g = geom(plan);
    NUFFT_HIP(nufft::launch_fill_zero(grid, (size_t)grid_cells(plan) * 2 * real_size(plan), plan->stream));
    NUFFT_HIP(nufft::launch_spread(plan->prec, plan->method, g, c, grid, plan->stream, plan->colw > 0,
                                   plan->sort_tmp.p));
    return NUFFT_OK;
}

int nufft_interp(nufft_plan plan, const void* grid, void* c) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (!grid || (plan->M > 0 && !c)) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    nufft::GeomArgs g = geom(plan);
    NUFFT_HIP(nufft::launch_interp(plan->prec, plan->method, g, grid, c, plan->stream));
    return NUFFT_OK;
}

int nufft_deconvolve(nufft_plan plan, const void* fhat, void* f) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    if (!fhat || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    NUFFT_HIP(nufft::launch_deconvolve(plan->prec, plan->dim, plan->N, plan->n, plan->pcorr.p, fhat, f,
                                       plan->stream));
    return NUFFT_OK;
}

int nufft_precorrect_pad(nufft_plan plan, const void* f, void* fhat) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    if (!fhat || !f) return fail(plan, NUFFT_ERR_BAD_ARG, "null data pointer");
    NUFFT_HIP(nufft::launch_precorrect_pad(plan->prec, plan->dim, plan->N, plan->n, plan->pcorr.p, f, fhat,
                                           plan->stream));
    return NUFFT_OK;
}

int nufft_get_sort(nufft_plan plan, int32_t* perm, int32_t* counts, int32_t* subproblems) {
    if (check_plan(plan) != NUFFT_OK) return NUFFT_ERR_BAD_ARG;
    if (check_not_type3(plan) != NUFFT_OK) return NUFFT_ERR_UNSUPPORTED;
    int rc;
    if ((rc = check_points(plan)) != NUFFT_OK) return rc;
    if (perm && plan->M > 0)
        NUFFT_HIP(hipMemcpyAsync(perm, plan->perm.p, sizeof(int32_t) * plan->M, hipMemcpyDeviceToDevice,
                                 plan->stream));
    if (counts)
        NUFFT_HIP(hipMemcpyAsync(counts, plan->counts.p, sizeof(int32_t) * plan->nbins,
                                 hipMemcpyDeviceToDevice, plan->stream));
    if (subproblems && plan->nsub > 0)
        NUFFT_HIP(hipMemcpyAsync(subproblems, plan->sub.p, sizeof(int32_t) * 3 * plan->nsub,
                                 hipMemcpyDeviceToDevice, plan->stream));
    return NUFFT_OK;
}

int nufft_get_range_errors(nufft_plan plan, int64_t* count) {
    if (!plan || !count) return NUFFT_ERR_BAD_ARG;
    *count = 0;
    if (plan->type == 3) {
        // the transform's spreading and evaluation run in its inner plans
        for (nufft_plan q : {plan->t3_spread, plan->t3_eval}) {
            int64_t v = 0;
            if (q) {
                int rc = nufft_get_range_errors(q, &v);
                if (rc != NUFFT_OK) return fail(plan, rc, q->last_error);
            }
            *count += v;
        }
        return NUFFT_OK;
    }
    unsigned int v = 0;
    if (plan->range_err.p) {
        NUFFT_HIP(hipMemcpyAsync(&v, plan->range_err.p, sizeof(v), hipMemcpyDeviceToHost, plan->stream));
        NUFFT_HIP(hipStreamSynchronize(plan->stream));
    }
    *count = (int64_t)v;
    return NUFFT_OK;
}

}  // extern "C"
