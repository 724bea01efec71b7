// api.cpp -- the extern "C" entry points of libbps: argument validation on
// the host, then kernel launches on the caller's stream.
#include <cmath>
#include <cstring>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace bps {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

// Work memory of hyperdiffusion_step_noalloc: one array per GPU (each device
// that loads the library holds its own copy until the process ends).  In host
// code the name `scratch` is only a host-side stand-in: the device address is
// taken with hipGetSymbolAddress, once per device, and used everywhere the
// host needs the array.
static __device__ __align__(256) unsigned char scratch[BPS_NOALLOC_SCRATCH_BYTES];

bps_status prepare_device(void **scratch_dev)
{
    // after a device's first call: one atomic load, no lock (devices past
    // kFastDevices take the locked path every time)
    constexpr int kFastDevices = 64;
    static std::atomic<void *> ready[kFastDevices];
    static std::mutex mu;
    static std::map<int, void *> done;     // device -> address of its scratch
    int dev = 0;
    BPS_HIP(hipGetDevice(&dev));
    if (dev >= 0 && dev < kFastDevices) {
        void *ptr = ready[dev].load(std::memory_order_acquire);
        if (ptr) {
            if (scratch_dev) *scratch_dev = ptr;
            return BPS_OK;
        }
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = done.find(dev);
    if (it == done.end()) {
        BPS_HIP(spike_prepare_device());
        BPS_HIP(hines_prepare_device());
        void *ptr = nullptr;
        BPS_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        if (!ptr) BPS_FAIL(BPS_EHIP, "hipGetSymbolAddress gave no address for the scratch array");
        it = done.emplace(dev, ptr).first;
        if (dev >= 0 && dev < kFastDevices) ready[dev].store(ptr, std::memory_order_release);
    }
    if (scratch_dev) *scratch_dev = it->second;
    return BPS_OK;
}

// from hines.hip
bps_status hines_plan_build(bps_hines_plan **out, int64_t batch, const int32_t *sizes,
                            const int32_t *parent, int mono, int64_t ld, int sched);
bps_status hines_plan_free(bps_hines_plan *p);
bool hines_plan_general(const bps_hines_plan *p);
bool hines_plan_levels(const bps_hines_plan *p);
size_t hines_plan_work_bytes(const bps_hines_plan *p);
template <typename T>
bps_status hines_transform(const bps_hines_plan *P, bool pack, const void *src, void *dst,
                           hipStream_t st);
bps_status hines_launch(const bps_hines_plan *P, const void *u, const void *l, const void *d,
                        void *rhs, void *work, int32_t *info, hipStream_t st);

// Shape of a plan, read from the opaque struct defined in hines.hip.
int64_t hines_plan_elems_of(const bps_hines_plan *p);
int64_t hines_plan_unknowns_of(const bps_hines_plan *p);
int64_t hines_plan_batch_of(const bps_hines_plan *p);
int64_t hines_plan_split_of(const bps_hines_plan *p);
int32_t hines_split_rows(int32_t n, const int32_t *parent, int32_t *node, uint16_t *code, int32_t cap);
bool hines_plan_sep(const bps_hines_plan *p);
int32_t hines_sep_blob(int32_t n, const int32_t *parent, int32_t *out, int32_t cap, std::string &why);

static const int64_t kMaxDim = int64_t(1) << 40;

static bps_status check_desc(const bps_penta_desc *dsc)
{
    if (!dsc) BPS_FAIL(BPS_EINVAL, "desc is NULL");
    if (dtype_size(dsc->dtype) == 0) BPS_FAIL(BPS_EINVAL, "unknown dtype %d", dsc->dtype);
    if (dsc->flags & ~(BPS_CYCLIC | BPS_SHARED_COEF))
        BPS_FAIL(BPS_EINVAL, "unknown flags 0x%x", dsc->flags);
    const int64_t nmin = (dsc->flags & BPS_CYCLIC) ? 6 : 4;
    if (dsc->n < nmin || dsc->n > kMaxDim)
        BPS_FAIL(BPS_EINVAL, "n = %lld must be in [%lld, 2^40]", (long long)dsc->n, (long long)nmin);
    if (dsc->batch < 1 || dsc->batch > (int64_t(1) << 31) - kWave)
        BPS_FAIL(BPS_EINVAL, "batch = %lld must be in [1, 2^31 - 64]", (long long)dsc->batch);
    if (dsc->ld < dsc->batch) BPS_FAIL(BPS_EINVAL, "ld = %lld < batch = %lld", (long long)dsc->ld,
                                       (long long)dsc->batch);
    // element offsets (and their byte sizes) stay far inside int64
    if (dsc->n > kMaxDim / dsc->ld) BPS_FAIL(BPS_EINVAL, "n * ld exceeds 2^40 elements");
    return BPS_OK;
}

static bps_status check_ptr(const void *p, const char *name, int dtype)
{
    if (!p) BPS_FAIL(BPS_EINVAL, "%s is NULL", name);
    if (!aligned(p, dtype_size(dtype))) BPS_FAIL(BPS_EINVAL, "%s is not %zu-byte aligned", name,
                                                 dtype_size(dtype));
    return BPS_OK;
}

#define CHECK(x)                         \
    do {                                 \
        bps_status s_ = (x);             \
        if (s_ != BPS_OK) return s_;     \
    } while (0)

}  // namespace bps

using namespace bps;

extern "C" {

const char *bps_status_str(int status)
{
    switch (status) {
    case BPS_OK: return "BPS_OK";
    case BPS_EINVAL: return "BPS_EINVAL: invalid argument";
    case BPS_ENOTSUP: return "BPS_ENOTSUP: unsupported combination";
    case BPS_EHIP: return "BPS_EHIP: HIP runtime error";
    case BPS_ENOMEM: return "BPS_ENOMEM: device allocation failed";
    default: return "unknown bps_status";
    }
}

const char *bps_last_error(void) { return g_err; }

int bps_version(void) { return 101; }

bps_status bps_init(void)
{
    clear_error();
    return prepare_device();
}

size_t bps_penta_factor_bytes(const bps_penta_desc *dsc)
{
    if (check_desc(dsc) != BPS_OK) return 0;
    const bool shared = dsc->flags & BPS_SHARED_COEF;
    const int64_t ldf = shared ? 1 : dsc->ld;
    return size_t(penta_factor_elems(dsc->n, ldf, dsc->flags & BPS_CYCLIC)) * dtype_size(dsc->dtype);
}

bps_status penta_factor_batch(const bps_penta_desc *dsc, const void *a, const void *b,
                              const void *c, const void *d, const void *e, void *factors,
                              int32_t *info, void *stream)
{
    clear_error();
    CHECK(check_desc(dsc));
    CHECK(check_ptr(a, "a", dsc->dtype)); CHECK(check_ptr(b, "b", dsc->dtype));
    CHECK(check_ptr(c, "c", dsc->dtype)); CHECK(check_ptr(d, "d", dsc->dtype));
    CHECK(check_ptr(e, "e", dsc->dtype)); CHECK(check_ptr(factors, "factors", dsc->dtype));
    if (info && !aligned(info, 4)) BPS_FAIL(BPS_EINVAL, "info is not 4-byte aligned");
    const bool cyc = dsc->flags & BPS_CYCLIC, sh = dsc->flags & BPS_SHARED_COEF;
    if (dsc->dtype == BPS_F64)
        return launch_penta_factor<double>(dsc->n, dsc->batch, dsc->ld, cyc, sh, a, b, c, d, e,
                                           factors, info, as_stream(stream));
    return launch_penta_factor<float>(dsc->n, dsc->batch, dsc->ld, cyc, sh, a, b, c, d, e,
                                      factors, info, as_stream(stream));
}

bps_status penta_solve_batch(const bps_penta_desc *dsc, const void *factors, void *x, void *stream)
{
    clear_error();
    CHECK(check_desc(dsc));
    if (dsc->flags & BPS_CYCLIC)
        BPS_FAIL(BPS_EINVAL, "penta_solve_batch: periodic desc; use penta_cyclic_solve_batch");
    CHECK(check_ptr(factors, "factors", dsc->dtype)); CHECK(check_ptr(x, "x", dsc->dtype));
    const bool sh = dsc->flags & BPS_SHARED_COEF;
    if (dsc->dtype == BPS_F64)
        return launch_penta_solve<double>(dsc->n, dsc->batch, dsc->ld, sh, factors, x, as_stream(stream));
    return launch_penta_solve<float>(dsc->n, dsc->batch, dsc->ld, sh, factors, x, as_stream(stream));
}

bps_status penta_cyclic_solve_batch(const bps_penta_desc *dsc, const void *factors, void *x,
                                    void *stream)
{
    clear_error();
    CHECK(check_desc(dsc));
    if (!(dsc->flags & BPS_CYCLIC))
        BPS_FAIL(BPS_EINVAL, "penta_cyclic_solve_batch: desc lacks BPS_CYCLIC");
    CHECK(check_ptr(factors, "factors", dsc->dtype)); CHECK(check_ptr(x, "x", dsc->dtype));
    const bool sh = dsc->flags & BPS_SHARED_COEF;
    if (dsc->dtype == BPS_F64)
        return launch_penta_cyclic_solve<double>(dsc->n, dsc->batch, dsc->ld, 1, sh, factors, x,
                                                 as_stream(stream));
    return launch_penta_cyclic_solve<float>(dsc->n, dsc->batch, dsc->ld, 1, sh, factors, x,
                                            as_stream(stream));
}

size_t bps_penta_work_bytes(const bps_penta_desc *dsc)
{
    if (check_desc(dsc) != BPS_OK) return 0;
    const size_t es = dtype_size(dsc->dtype);
    if (dsc->flags & BPS_CYCLIC)     // periodic factors, then a mask of int32[ld]
        return size_t(penta_factor_elems(dsc->n, dsc->ld, true)) * es + size_t(dsc->ld) * 4;
    return size_t(2 * dsc->n * dsc->ld) * es;
}

bps_status penta_factor_solve_batch(const bps_penta_desc *dsc, const void *a, const void *b,
                                    const void *c, const void *d, const void *e, void *x,
                                    void *work, int32_t *info, void *stream)
{
    clear_error();
    CHECK(check_desc(dsc));
    if (dsc->flags & BPS_SHARED_COEF)
        BPS_FAIL(BPS_ENOTSUP, "penta_factor_solve_batch takes per-system coefficients only");
    CHECK(check_ptr(a, "a", dsc->dtype)); CHECK(check_ptr(b, "b", dsc->dtype));
    CHECK(check_ptr(c, "c", dsc->dtype)); CHECK(check_ptr(d, "d", dsc->dtype));
    CHECK(check_ptr(e, "e", dsc->dtype)); CHECK(check_ptr(x, "x", dsc->dtype));
    CHECK(check_ptr(work, "work", dsc->dtype));
    if (info && !aligned(info, 4)) BPS_FAIL(BPS_EINVAL, "info is not 4-byte aligned");
    CHECK(prepare_device());
    hipStream_t st = as_stream(stream);
    const int64_t n = dsc->n, batch = dsc->batch, ld = dsc->ld;
    if (dsc->flags & BPS_CYCLIC) {
        // periodic, per system: the chunked kernel where it applies; systems
        // it leaves (breakdown) and other n take the periodic factor + solve
        const bool f64 = dsc->dtype == BPS_F64;
        void *fac = work;
        int32_t *mask = reinterpret_cast<int32_t *>(
            static_cast<char *>(work) + size_t(penta_factor_elems(n, ld, true)) * dtype_size(dsc->dtype));
        if (spike_rows(n, true)) {
            CHECK(f64 ? launch_penta_spike<double>(n, batch, ld, true, a, b, c, d, e, x, fac, info, mask, st)
                      : launch_penta_spike<float>(n, batch, ld, true, a, b, c, d, e, x, fac, info, mask, st));
        } else {
            mask = nullptr;
        }
        CHECK(f64 ? launch_penta_factor<double>(n, batch, ld, true, false, a, b, c, d, e, fac, info, st, mask)
                  : launch_penta_factor<float>(n, batch, ld, true, false, a, b, c, d, e, fac, info, st, mask));
        return f64 ? launch_penta_cyclic_solve<double>(n, batch, ld, 1, false, fac, x, st, mask)
                   : launch_penta_cyclic_solve<float>(n, batch, ld, 1, false, fac, x, st, mask);
    }
    if (spike_rows(n, false)) {
        if (dsc->dtype == BPS_F64)
            return launch_penta_spike<double>(n, batch, ld, false, a, b, c, d, e, x, work, info,
                                              nullptr, st);
        return launch_penta_spike<float>(n, batch, ld, false, a, b, c, d, e, x, work, info, nullptr,
                                         st);
    }
    if (dsc->dtype == BPS_F64)
        return launch_penta_fused<double>(dsc->n, dsc->batch, dsc->ld, a, b, c, d, e, x, work, info,
                                          as_stream(stream));
    return launch_penta_fused<float>(dsc->n, dsc->batch, dsc->ld, a, b, c, d, e, x, work, info,
                                     as_stream(stream));
}

size_t hyperdiffusion_work_bytes(int dtype, int64_t n, int64_t batch)
{
    if (dtype_size(dtype) == 0 || n < 6 || n > kMaxDim || batch < 1) return 0;
    const size_t stream = size_t(5 * n + penta_factor_elems(n, 1, true)) * dtype_size(dtype);
    const size_t res = 5 * n * dtype_size(dtype) + resident_coef_bytes(n);
    return stream > res ? stream : res;
}

// Checks every argument of hyperdiffusion_step but `work`.
static bps_status check_hyper_args(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                                   double dx, const void *diagonals, void *C, int64_t nsteps)
{
    bps_penta_desc dsc{dtype, BPS_CYCLIC | BPS_SHARED_COEF, n, batch, ld};
    CHECK(check_desc(&dsc));
    if (nsteps < 0) BPS_FAIL(BPS_EINVAL, "nsteps = %lld < 0", (long long)nsteps);
    if (!std::isfinite(dt) || !std::isfinite(dx) || dx == 0.0)
        BPS_FAIL(BPS_EINVAL, "dt and dx must be finite and dx nonzero");
    CHECK(check_ptr(C, "C", dtype));
    if (diagonals) CHECK(check_ptr(diagonals, "diagonals", dtype));
    if (!diagonals && !std::isfinite(dt / (dx * dx * dx * dx)))
        BPS_FAIL(BPS_EINVAL, "sigma = dt/dx^4 is not finite");
    return BPS_OK;
}

// The register-resident multi-step kernel applies to the built-in operator
// I + sigma*D4 in fp64 for the chunkable n: every chunk of a system then sees
// the same interior block, and no diagonal arrays are needed.
static bool hyper_resident(int dtype, int64_t n, double dt, double dx, const void *diagonals)
{
    return !diagonals && dtype == BPS_F64 && resident_chunk(n) != 0 && dt / (dx * dx * dx * dx) >= 0.0;
}

// The factor half of hyperdiffusion_step (validated arguments; work of
// hyperdiffusion_work_bytes): the resident kernel's coefficients, or the
// operator's diagonals (built unless given) and their periodic factors.
static bps_status hyper_factor(int dtype, int64_t n, double dt, double dx, const void *diagonals,
                               void *work, hipStream_t st)
{
    const size_t es = dtype_size(dtype);
    char *w = static_cast<char *>(work);
    void *fac = w + 5 * n * es;
    if (hyper_resident(dtype, n, dt, dx, diagonals))
        return launch_hyper_resident(n, 1, 1, 0, dt / (dx * dx * dx * dx), 0, 1.0, 0.0, 0.0, 0.0,
                                     fac, nullptr, st, kResSetup);
    const void *dg = diagonals;
    if (!dg) {
        const double sigma = dt / (dx * dx * dx * dx);
        CHECK(dtype == BPS_F64 ? launch_hyper_diagonals<double>(n, sigma, w, st)
                               : launch_hyper_diagonals<float>(n, sigma, w, st));
        dg = w;
    }
    const char *D = static_cast<const char *>(dg);
    if (dtype == BPS_F64)
        return launch_penta_factor<double>(n, 1, 1, true, true, D, D + n * es, D + 2 * n * es,
                                           D + 3 * n * es, D + 4 * n * es, fac, nullptr, st);
    return launch_penta_factor<float>(n, 1, 1, true, true, D, D + n * es, D + 2 * n * es,
                                      D + 3 * n * es, D + 4 * n * es, fac, nullptr, st);
}

// The solve half: nsteps steps with the factors hyper_factor left in work.
static bps_status hyper_solve(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                              double dx, const void *diagonals, void *C, int64_t nsteps,
                              const void *work, hipStream_t st)
{
    const size_t es = dtype_size(dtype);
    void *fac = const_cast<char *>(static_cast<const char *>(work)) + 5 * n * es;
    if (nsteps == 0) return BPS_OK;
    if (hyper_resident(dtype, n, dt, dx, diagonals))
        return launch_hyper_resident(n, batch, ld, nsteps, dt / (dx * dx * dx * dx), 0, 1.0, 0.0,
                                     0.0, 0.0, fac, C, st, kResSteps);
    return dtype == BPS_F64 ? launch_penta_cyclic_solve<double>(n, batch, ld, nsteps, true, fac, C, st)
                            : launch_penta_cyclic_solve<float>(n, batch, ld, nsteps, true, fac, C, st);
}

static bps_status hyper_steps(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                              double dx, const void *diagonals, void *C, int64_t nsteps,
                              void *work, hipStream_t st)
{
    CHECK(hyper_factor(dtype, n, dt, dx, diagonals, work, st));
    return hyper_solve(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps, work, st);
}

bps_status hyperdiffusion_factor(int dtype, int64_t n, double dt, double dx, const void *diagonals,
                                 void *work, void *stream)
{
    clear_error();
    bps_penta_desc dsc{dtype, BPS_CYCLIC | BPS_SHARED_COEF, n, 1, 1};
    CHECK(check_desc(&dsc));
    if (!std::isfinite(dt) || !std::isfinite(dx) || dx == 0.0)
        BPS_FAIL(BPS_EINVAL, "dt and dx must be finite and dx nonzero");
    if (diagonals) CHECK(check_ptr(diagonals, "diagonals", dtype));
    if (!diagonals && !std::isfinite(dt / (dx * dx * dx * dx)))
        BPS_FAIL(BPS_EINVAL, "sigma = dt/dx^4 is not finite");
    CHECK(check_ptr(work, "work", dtype));
    return hyper_factor(dtype, n, dt, dx, diagonals, work, as_stream(stream));
}

bps_status hyperdiffusion_solve(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                                double dx, const void *diagonals, void *C, int64_t nsteps,
                                const void *work, void *stream)
{
    clear_error();
    CHECK(check_hyper_args(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps));
    CHECK(check_ptr(work, "work", dtype));
    return hyper_solve(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps, work, as_stream(stream));
}

bps_status hyperdiffusion_step(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                               double dx, const void *diagonals, void *C, int64_t nsteps,
                               void *work, void *stream)
{
    clear_error();
    CHECK(check_hyper_args(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps));
    CHECK(check_ptr(work, "work", dtype));
    return hyper_steps(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps, work,
                       as_stream(stream));
}

bps_status hyperdiffusion_step_noalloc(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                                       double dx, const void *diagonals, void *C, int64_t nsteps,
                                       void *stream)
{
    clear_error();
    CHECK(check_hyper_args(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps));
    const size_t need = hyperdiffusion_work_bytes(dtype, n, batch);
    if (need > size_t(BPS_NOALLOC_SCRATCH_BYTES))
        BPS_FAIL(BPS_EINVAL, "hyperdiffusion_step_noalloc: n = %lld needs %zu bytes of work, more "
                 "than the %zu-byte scratch array", (long long)n, need,
                 size_t(BPS_NOALLOC_SCRATCH_BYTES));
    void *work = nullptr;
    CHECK(prepare_device(&work));
    return hyper_steps(dtype, n, batch, ld, dt, dx, diagonals, C, nsteps, work, as_stream(stream));
}

// ---- theta scheme -------------------------------------------------------------------

size_t hyperdiffusion_theta_work_bytes(int dtype, int64_t n, int64_t batch)
{
    const size_t base = hyperdiffusion_work_bytes(dtype, n, batch);
    if (base == 0) return 0;
    return base + size_t(n) * size_t(batch) * dtype_size(dtype);   // + the right-hand sides
}

// Steps (I + si D4) C' = S C (+ rr D2 (C^3 - C) with kResPhase), S the
// stencil (e2, e1, e0, e1, e2) with kResStencil, else the identity;
// arguments already validated.
static bps_status explicit_implicit_steps(int dtype, int64_t n, int64_t batch, int64_t ld, double si,
                                          double e0, double e1, double e2, double rr, int mode,
                                          void *C, int64_t nsteps, void *work, hipStream_t st)
{
    const size_t es = dtype_size(dtype);
    char *w = static_cast<char *>(work);
    void *fac = w + 5 * n * es;
    if (dtype == BPS_F64 && resident_chunk(n) != 0 && si >= 0.0)
        return launch_hyper_resident(n, batch, ld, nsteps, si, mode, e0, e1, e2, rr, fac, C, st);
    // streaming: factor I + si D4 once, then per step the right-hand side
    // into a separate array and a solve in place, alternating between C and
    // that array (the result is copied back when it ends in the array)
    void *R = w + hyperdiffusion_work_bytes(dtype, n, batch);
    if (dtype == BPS_F64) CHECK(launch_hyper_diagonals<double>(n, si, w, st));
    else CHECK(launch_hyper_diagonals<float>(n, si, w, st));
    const char *D = w;
    if (dtype == BPS_F64)
        CHECK(launch_penta_factor<double>(n, 1, 1, true, true, D, D + n * es, D + 2 * n * es,
                                          D + 3 * n * es, D + 4 * n * es, fac, nullptr, st));
    else
        CHECK(launch_penta_factor<float>(n, 1, 1, true, true, D, D + n * es, D + 2 * n * es,
                                         D + 3 * n * es, D + 4 * n * es, fac, nullptr, st));
    if (mode == 0) {
        if (nsteps == 0) return BPS_OK;
        return dtype == BPS_F64 ? launch_penta_cyclic_solve<double>(n, batch, ld, nsteps, true, fac, C, st)
                                : launch_penta_cyclic_solve<float>(n, batch, ld, nsteps, true, fac, C, st);
    }
    const bool ch = (mode & kResPhase) != 0;
    void *cur = C, *nxt = R;
    int64_t lcur = ld, lnxt = batch;
    for (int64_t t = 0; t < nsteps; ++t) {
        if (dtype == BPS_F64) {
            CHECK(launch_hyper_explicit<double>(n, batch, lcur, lnxt, e0, e1, e2, rr, ch, cur, nxt, st));
            CHECK(launch_penta_cyclic_solve<double>(n, batch, lnxt, 1, true, fac, nxt, st));
        } else {
            CHECK(launch_hyper_explicit<float>(n, batch, lcur, lnxt, e0, e1, e2, rr, ch, cur, nxt, st));
            CHECK(launch_penta_cyclic_solve<float>(n, batch, lnxt, 1, true, fac, nxt, st));
        }
        std::swap(cur, nxt);
        std::swap(lcur, lnxt);
    }
    if (cur != C)
        return dtype == BPS_F64 ? launch_copy_interleaved<double>(n, batch, lcur, ld, cur, C, st)
                                : launch_copy_interleaved<float>(n, batch, lcur, ld, cur, C, st);
    return BPS_OK;
}

bps_status hyperdiffusion_theta_step(int dtype, int64_t n, int64_t batch, int64_t ld, double dt,
                                     double dx, double theta, void *C, int64_t nsteps, void *work,
                                     void *stream)
{
    clear_error();
    bps_penta_desc dsc{dtype, BPS_CYCLIC | BPS_SHARED_COEF, n, batch, ld};
    CHECK(check_desc(&dsc));
    if (nsteps < 0) BPS_FAIL(BPS_EINVAL, "nsteps = %lld < 0", (long long)nsteps);
    if (!std::isfinite(dt) || !std::isfinite(dx) || dx == 0.0)
        BPS_FAIL(BPS_EINVAL, "dt and dx must be finite and dx nonzero");
    if (!(theta >= 0.0 && theta <= 1.0)) BPS_FAIL(BPS_EINVAL, "theta = %g not in [0, 1]", theta);
    CHECK(check_ptr(C, "C", dtype));
    CHECK(check_ptr(work, "work", dtype));
    const double sigma = dt / (dx * dx * dx * dx);
    if (!std::isfinite(sigma)) BPS_FAIL(BPS_EINVAL, "sigma = dt/dx^4 is not finite");
    // the two sides, rounded as the operator is defined: implicit
    // I + si D4, explicit stencil (-se, 4 se, 1 - 6 se, 4 se, -se)
    const double si = theta * sigma, se = (1.0 - theta) * sigma;
    const double e2 = -se, e1 = 4.0 * se, e0 = 1.0 - 6.0 * se;
    return explicit_implicit_steps(dtype, n, batch, ld, si, e0, e1, e2, 0.0,
                                   theta != 1.0 ? kResStencil : 0, C, nsteps, work,
                                   as_stream(stream));
}

size_t cahn_hilliard_work_bytes(int dtype, int64_t n, int64_t batch)
{
    return hyperdiffusion_theta_work_bytes(dtype, n, batch);
}

bps_status cahn_hilliard_step(int dtype, int64_t n, int64_t batch, int64_t ld, double dt, double dx,
                              double gamma, double mobility, double theta, void *C, int64_t nsteps,
                              void *work, void *stream)
{
    clear_error();
    bps_penta_desc dsc{dtype, BPS_CYCLIC | BPS_SHARED_COEF, n, batch, ld};
    CHECK(check_desc(&dsc));
    if (nsteps < 0) BPS_FAIL(BPS_EINVAL, "nsteps = %lld < 0", (long long)nsteps);
    if (!std::isfinite(dt) || !std::isfinite(dx) || dx == 0.0)
        BPS_FAIL(BPS_EINVAL, "dt and dx must be finite and dx nonzero");
    if (!(gamma >= 0.0) || !std::isfinite(gamma) || !(mobility >= 0.0) || !std::isfinite(mobility))
        BPS_FAIL(BPS_EINVAL, "gamma and the mobility must be finite and >= 0");
    if (!(theta >= 0.0 && theta <= 1.0)) BPS_FAIL(BPS_EINVAL, "theta = %g not in [0, 1]", theta);
    CHECK(check_ptr(C, "C", dtype));
    CHECK(check_ptr(work, "work", dtype));
    const double r = mobility * dt / (dx * dx);
    const double sigma = gamma * r / (dx * dx);
    if (!std::isfinite(r) || !std::isfinite(sigma))
        BPS_FAIL(BPS_EINVAL, "D dt/dx^2 or gamma D dt/dx^4 is not finite");
    const double si = theta * sigma, se = (1.0 - theta) * sigma;
    const double e2 = -se, e1 = 4.0 * se, e0 = 1.0 - 6.0 * se;
    // theta = 1: the stencil is the identity and is left out
    const int mode = kResPhase | (theta != 1.0 ? kResStencil : 0);
    return explicit_implicit_steps(dtype, n, batch, ld, si, e0, e1, e2, r, mode, C, nsteps, work,
                                   as_stream(stream));
}

// ---- tridiagonal ----------------------------------------------------------------

size_t tri_work_bytes(int dtype, int64_t n, int64_t ld)
{
    if (dtype_size(dtype) == 0 || n < 1 || n > kMaxDim || ld < 1 || ld > kMaxDim) return 0;
    return tri_work_bytes_es(n, ld, dtype_size(dtype));
}

bps_status tri_solve_batch(int dtype, int64_t n, int64_t batch, int64_t ld, const void *a,
                           const void *b, const void *c, void *y, void *work, int32_t *info,
                           void *stream)
{
    clear_error();
    if (dtype_size(dtype) == 0) BPS_FAIL(BPS_EINVAL, "unknown dtype %d", dtype);
    if (n < 1 || n > kMaxDim) BPS_FAIL(BPS_EINVAL, "n = %lld must be in [1, 2^40]", (long long)n);
    if (batch < 1 || batch > (int64_t(1) << 31) - kWave)
        BPS_FAIL(BPS_EINVAL, "batch = %lld must be in [1, 2^31 - 64]", (long long)batch);
    if (ld < batch) BPS_FAIL(BPS_EINVAL, "ld = %lld < batch = %lld", (long long)ld, (long long)batch);
    if (n > kMaxDim / ld) BPS_FAIL(BPS_EINVAL, "n * ld too large");
    CHECK(check_ptr(a, "a", dtype));
    CHECK(check_ptr(b, "b", dtype));
    CHECK(check_ptr(c, "c", dtype));
    CHECK(check_ptr(y, "y", dtype));
    CHECK(check_ptr(work, "work", dtype));
    if (info && !aligned(info, 4)) BPS_FAIL(BPS_EINVAL, "info is not 4-byte aligned");
    hipStream_t st = as_stream(stream);
    return dtype == BPS_F64 ? launch_tri_solve<double>(n, batch, ld, a, b, c, y, work, info, st)
                            : launch_tri_solve<float>(n, batch, ld, a, b, c, y, work, info, st);
}

// ---- Hines ----------------------------------------------------------------------

bps_status hines_plan_create(bps_hines_plan **plan, int64_t batch, const int32_t *sizes,
                             const int32_t *parent, int mono, int64_t ld)
{
    return hines_plan_create_sched(plan, batch, sizes, parent, mono, ld, BPS_HINES_AUTO);
}

int hines_plan_uses_levels(const bps_hines_plan *plan) { return plan && hines_plan_levels(plan); }

int64_t hines_plan_split(const bps_hines_plan *plan) { return plan ? hines_plan_split_of(plan) : 0; }

int hines_plan_uses_sep(const bps_hines_plan *plan) { return plan && hines_plan_sep(plan); }

int32_t hines_sep_multi_layout(int64_t batch, const int32_t *sizes, const int32_t *parent, int64_t *dims,
                               uint16_t *code, int32_t *comp, int32_t *pos, int32_t *lanetab,
                               int64_t *wgoff, int32_t *tabs)
{
    clear_error();
    if (batch < 1 || !sizes || !parent || !dims) {
        set_error("hines_sep_multi_layout: NULL array or batch < 1");
        return -1;
    }
    std::vector<int64_t> off(size_t(batch) + 1, 0);
    for (int64_t s = 0; s < batch; ++s) {
        const int32_t n = sizes[s];
        if (n < 1 || n > (1 << 30)) {
            set_error("hines_sep_multi_layout: sizes[%lld] = %d out of range", (long long)s, n);
            return -1;
        }
        for (int32_t i = 1; i < n; ++i)
            if (parent[off[s] + i] < 0 || parent[off[s] + i] >= i) {
                set_error("hines_sep_multi_layout: neuron %lld: parent[%d] = %d not in [0, %d)",
                          (long long)s, i, parent[off[s] + i], i);
                return -1;
            }
        off[s + 1] = off[s] + n;
    }
    SepMulti M;
    std::string why;
    if (!sep_build_multi(batch, sizes, parent, off.data(), M, why)) {
        set_error("hines_sep_multi_layout: %s", why.c_str());
        return 0;
    }
    dims[0] = M.nwg; dims[1] = M.elems; dims[2] = M.R; dims[3] = int64_t(M.lds);
    dims[4] = int64_t(M.tabs.size());
    dims[5] = M.lanes;
    if (code && comp && pos && lanetab && wgoff && tabs) {
        std::copy(M.code.begin(), M.code.end(), code);
        std::copy(M.comp.begin(), M.comp.end(), comp);
        std::copy(M.pos.begin(), M.pos.end(), pos);
        std::copy(M.lanetab.begin(), M.lanetab.end(), lanetab);
        std::copy(M.wgoff.begin(), M.wgoff.end(), wgoff);
        std::copy(M.tabs.begin(), M.tabs.end(), tabs);
    }
    return 1;
}

int32_t hines_sep_schedule(int32_t n, const int32_t *parent, int32_t *out, int32_t cap)
{
    clear_error();
    if (!parent || !out || cap < 0) {
        set_error("hines_sep_schedule: NULL array or negative cap");
        return -1;
    }
    if (n < 1) {
        set_error("hines_sep_schedule: n = %d out of range", n);
        return -1;
    }
    for (int32_t i = 1; i < n; ++i)
        if (parent[i] < 0 || parent[i] >= i) {
            set_error("hines_sep_schedule: parent[%d] = %d not in [0, %d)", i, parent[i], i);
            return -1;
        }
    std::string why;
    const int32_t m = hines_sep_blob(n, parent, out, cap, why);
    if (m == 0) set_error("hines_sep_schedule: %s", why.c_str());
    if (m < 0) {
        set_error("hines_sep_schedule: %d words do not fit cap = %d", -m, cap);
        return -1;
    }
    return m;
}

int32_t hines_split_schedule(int32_t n, const int32_t *parent, int32_t *node, uint16_t *code,
                             int32_t cap)
{
    clear_error();
    if (!parent || !node || !code || cap < 0) {
        set_error("hines_split_schedule: NULL array or negative cap");
        return -1;
    }
    if (n < 1 || n > (1 << 30)) {
        set_error("hines_split_schedule: n = %d out of range", n);
        return -1;
    }
    for (int32_t i = 1; i < n; ++i)
        if (parent[i] < 0 || parent[i] >= i) {
            set_error("hines_split_schedule: parent[%d] = %d not in [0, %d)", i, parent[i], i);
            return -1;
        }
    const int32_t m = hines_split_rows(n, parent, node, code, cap);
    if (m < 0) {
        set_error("hines_split_schedule: %d rows do not fit cap = %d", -m, cap);
        return -1;
    }
    return m;
}

bps_status hines_plan_create_sched(bps_hines_plan **plan, int64_t batch, const int32_t *sizes,
                                   const int32_t *parent, int mono, int64_t ld, int schedule)
{
    clear_error();
    if (!plan) BPS_FAIL(BPS_EINVAL, "plan is NULL");
    *plan = nullptr;
    if (!sizes || !parent) BPS_FAIL(BPS_EINVAL, "sizes and parent must be host arrays");
    if (batch < 1 || batch > (int64_t(1) << 31) - kWave) BPS_FAIL(BPS_EINVAL, "batch out of range");
    if (mono) {
        const int64_t n = sizes[0];
        if (n < 1 || n > (int64_t(1) << 30)) BPS_FAIL(BPS_EINVAL, "n = %lld out of range", (long long)n);
        if (ld == 0) ld = batch;
        if (ld < batch) BPS_FAIL(BPS_EINVAL, "ld < batch");
        if (n > kMaxDim / ld) BPS_FAIL(BPS_EINVAL, "n * ld exceeds 2^40 elements");
        for (int64_t i = 1; i < n; ++i)
            if (parent[i] < 0 || parent[i] >= i)
                BPS_FAIL(BPS_EINVAL, "parent[%lld] = %d not in [0, %lld)", (long long)i, parent[i],
                         (long long)i);
    } else {
        int64_t off = 0;
        for (int64_t s = 0; s < batch; ++s) {
            const int32_t n = sizes[s];
            if (n < 1 || n > (1 << 30)) BPS_FAIL(BPS_EINVAL, "sizes[%lld] = %d out of range",
                                                 (long long)s, n);
            for (int32_t i = 1; i < n; ++i)
                if (parent[off + i] < 0 || parent[off + i] >= i)
                    BPS_FAIL(BPS_EINVAL, "neuron %lld: parent[%d] = %d not in [0, %d)", (long long)s,
                             i, parent[off + i], i);
            off += n;
        }
    }
    if (schedule != BPS_HINES_AUTO && schedule != BPS_HINES_LANES && schedule != BPS_HINES_LEVELS &&
        schedule != BPS_HINES_SPLIT && schedule != BPS_HINES_SEP)
        BPS_FAIL(BPS_EINVAL, "unknown schedule %d", schedule);
    CHECK(prepare_device());
    return hines_plan_build(plan, batch, sizes, parent, mono, ld, schedule);
}

bps_status hines_plan_destroy(bps_hines_plan *plan)
{
    clear_error();
    if (!plan) return BPS_OK;
    return hines_plan_free(plan);
}

int64_t hines_plan_elems(const bps_hines_plan *plan) { return plan ? hines_plan_elems_of(plan) : 0; }

int64_t hines_plan_unknowns(const bps_hines_plan *plan)
{
    return plan ? hines_plan_unknowns_of(plan) : 0;
}

bps_status hines_pack(const bps_hines_plan *plan, int dtype, const void *flat, void *packed,
                      void *stream)
{
    clear_error();
    if (!plan) BPS_FAIL(BPS_EINVAL, "plan is NULL");
    CHECK(check_ptr(flat, "flat", dtype)); CHECK(check_ptr(packed, "packed", dtype));
    if (dtype == BPS_F64) return hines_transform<double>(plan, true, flat, packed, as_stream(stream));
    return hines_transform<float>(plan, true, flat, packed, as_stream(stream));
}

bps_status hines_unpack(const bps_hines_plan *plan, int dtype, const void *packed, void *flat,
                        void *stream)
{
    clear_error();
    if (!plan) BPS_FAIL(BPS_EINVAL, "plan is NULL");
    CHECK(check_ptr(flat, "flat", dtype)); CHECK(check_ptr(packed, "packed", dtype));
    if (dtype == BPS_F64) return hines_transform<double>(plan, false, packed, flat, as_stream(stream));
    return hines_transform<float>(plan, false, packed, flat, as_stream(stream));
}

size_t hines_work_bytes(const bps_hines_plan *plan, int dtype)
{
    if (!plan || dtype != BPS_F64) return 0;
    return hines_plan_work_bytes(plan);
}

bps_status hines_solve_batch(const bps_hines_plan *plan, int dtype, const void *u, const void *l,
                             const void *d, void *rhs, void *work, int32_t *info, void *stream)
{
    clear_error();
    if (!plan) BPS_FAIL(BPS_EINVAL, "plan is NULL");
    if (dtype != BPS_F64) BPS_FAIL(BPS_ENOTSUP, "hines_solve_batch supports BPS_F64 only");
    CHECK(check_ptr(u, "u", dtype)); CHECK(check_ptr(l, "l", dtype));
    CHECK(check_ptr(d, "d", dtype)); CHECK(check_ptr(rhs, "rhs", dtype));
    CHECK(check_ptr(work, "work", dtype));
    if (info && !aligned(info, 4)) BPS_FAIL(BPS_EINVAL, "info is not 4-byte aligned");
    return hines_launch(plan, u, l, d, rhs, work, info, as_stream(stream));
}

}  // extern "C"
