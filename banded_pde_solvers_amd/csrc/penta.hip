// penta.hip -- batched pentadiagonal kernels for gfx950, one lane per system.
//
// Method: the A = L R factorisation, forward steps (L g = f) and back
// substitution (R x = g) of "cuPentBatch - A batched pentadiagonal solver for
// NVIDIA GPUs", section "Pentadiagonal solver"; periodic matrices by the
// reduction in the hyperdiffusion section of the same page (E, F, G, H
// blocks, eqs. (10)-(12)), evaluated in a fused order described below.
//
// Data layout: interleaved (row i of system s at i*ld + s), so the 64 lanes
// of a wavefront read 64 consecutive systems of one row in one coalesced
// 512-byte (fp64) access per array per elimination step.
//
// Factor buffer (private layout, planar):
//   non-periodic: 5 arrays [n][ldf]:  ralpha = 1/alpha, beta, eps (= a with
//                 eps_0 = eps_1 = 0), gamma (gamma_{n-1} = 0),
//                 delta (delta_{n-2} = delta_{n-1} = 0)
//   periodic:     the same 5 arrays for E (m = n-2 rows), then
//                 V0, V1 = L^{-1} F (the two columns of F pushed through L),
//                 Y0, Y1 = R^{-T} G^T (the two rows of G pushed through R^T),
//                 each [m][ldf], then Sinv = (H - G E^{-1} F)^{-1} as 4 x [ldf].
//   ldf = ld for per-system factors, 1 for shared factors (single column).
//
// Periodic solve in fused order.  With g = L^{-1} f_hat (forward sweep):
//   G E^{-1} f_hat = (R^{-T} G^T)^T g = Y^T g     (accumulated in the sweep),
//   x_t  = Sinv (f_t - Y^T g)                     (eq. (12)),
//   X    = E^{-1}(f_hat - F x_t) = R^{-1}(g - V x_t)   (eq. (11)),
// so one forward sweep, two 2-vector dot products and one backward sweep
// with a rank-2 correction solve the periodic system: the same reads and
// writes as a non-periodic solve.
#include "common.h"
#include "kernels.h"

namespace bps {

// ----------------------------------------------------------------------------
// Factorisation (and the periodic-reduction quantities)
// ----------------------------------------------------------------------------

template <typename T, bool CYC>
__global__ void __launch_bounds__(kWave)
k_penta_factor(int64_t n, int64_t batch, int64_t ld, int64_t ldf,
               const T *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
               const T *__restrict__ D, const T *__restrict__ E, T *__restrict__ fac,
               int32_t *__restrict__ info, const int32_t *__restrict__ mask)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    if (mask && !mask[s]) return;       // only the systems marked in mask
    A += s; B += s; C += s; D += s; E += s;
    const int64_t rows = CYC ? n - 2 : n;     // rows of the factored block
    const int64_t arr = rows * ldf;           // stride between factor arrays
    T *ra = fac + s, *be = ra + arr, *ep = be + arr, *ga = ep + arr, *de = ga + arr;
    T *v0 = de + arr, *v1 = v0 + arr, *y0 = v1 + arr, *y1 = y0 + arr;
    int32_t bad = 0;

    // Periodic coupling entries (only read when CYC).  m = rows.
    //   F column 0 (matrix column n-2): rows 0, m-2, m-1 hold a_0, e_{m-2}, d_{m-1}
    //   F column 1 (matrix column n-1): rows 0, 1, m-1 hold b_0, a_1, e_{m-1}
    //   G row 0 (matrix row n-2): columns 0, m-2, m-1 hold e_m, a_m, b_m
    //   G row 1 (matrix row n-1): columns 0, 1, m-1 hold d_{m+1}, e_{m+1}, a_{m+1}
    //   H = [[c_m, d_m], [b_{m+1}, c_{m+1}]]
    T g0_0 = 0, g0_m2 = 0, g0_m1 = 0, g1_0 = 0, g1_1 = 0, g1_m1 = 0;
    T H00 = 0, H01 = 0, H10 = 0, H11 = 0;
    if (CYC) {
        const int64_t m = rows;
        g0_0 = E[m * ld];  g0_m2 = A[m * ld];  g0_m1 = B[m * ld];
        g1_0 = D[(m + 1) * ld];  g1_1 = E[(m + 1) * ld];  g1_m1 = A[(m + 1) * ld];
        H00 = C[m * ld];  H01 = D[m * ld];  H10 = B[(m + 1) * ld];  H11 = C[(m + 1) * ld];
    }
    // running values of the two previous rows
    T gam1 = 0, gam2 = 0, del1 = 0, del2 = 0;
    T V0a = 0, V0b = 0, V1a = 0, V1b = 0;   // V at rows i-1 (a) and i-2 (b)
    T Y0a = 0, Y0b = 0, Y1a = 0, Y1b = 0;
    T S00 = H00, S01 = H01, S10 = H10, S11 = H11;

    for (int64_t i = 0; i < rows; ++i) {
        const T ci = C[i * ld];
        // entries outside the (sub)matrix are not read: a_0, a_1, b_0, and
        // d_{rows-1}, e_{rows-2}, e_{rows-1}
        const T ai = (i >= 2) ? A[i * ld] : T(0);
        const T bi = (i >= 1) ? B[i * ld] : T(0);
        const T di = (i + 1 < rows) ? D[i * ld] : T(0);
        const T ei = (i + 2 < rows) ? E[i * ld] : T(0);
        const T beta = bi - ai * gam2;
        const T alpha = ci - ai * del2 - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = int32_t(i) + 1;
        const T r = T(1) / alpha;
        const T gam = (di - beta * del1) * r;
        const T del = ei * r;
        ra[i * ldf] = r; be[i * ldf] = beta; ep[i * ldf] = ai;
        ga[i * ldf] = gam; de[i * ldf] = del;
        if (CYC) {
            const int64_t m = rows;
            // F entries of this row
            T f0 = 0, f1 = 0, gg0 = 0, gg1 = 0;
            if (i == 0) { f0 = A[0]; f1 = B[0]; gg0 = g0_0; gg1 = g1_0; }
            if (i == 1) { f1 = A[ld]; gg1 = g1_1; }
            if (i == m - 2) { f0 = E[i * ld]; gg0 = g0_m2; }
            if (i == m - 1) { f0 = D[i * ld]; f1 = E[i * ld]; gg0 = g0_m1; gg1 = g1_m1; }
            const T V0 = (f0 - ai * V0b - beta * V0a) * r;
            const T V1 = (f1 - ai * V1b - beta * V1a) * r;
            const T Y0 = gg0 - gam1 * Y0a - del2 * Y0b;
            const T Y1 = gg1 - gam1 * Y1a - del2 * Y1b;
            v0[i * ldf] = V0; v1[i * ldf] = V1; y0[i * ldf] = Y0; y1[i * ldf] = Y1;
            S00 -= Y0 * V0; S01 -= Y0 * V1; S10 -= Y1 * V0; S11 -= Y1 * V1;
            V0b = V0a; V0a = V0; V1b = V1a; V1a = V1;
            Y0b = Y0a; Y0a = Y0; Y1b = Y1a; Y1a = Y1;
        }
        gam2 = gam1; gam1 = gam; del2 = del1; del1 = del;
    }
    if (CYC) {
        const T det = S00 * S11 - S01 * S10;
        if (!bad && bad_pivot(det)) bad = int32_t(rows) + 1;
        T *si = fac + 9 * arr + s;
        si[0] = S11 / det;
        si[ldf] = -S01 / det;
        si[2 * ldf] = -S10 / det;
        si[3 * ldf] = S00 / det;
    }
    if (info) info[s] = bad;
}

// ----------------------------------------------------------------------------
// Solves with stored factors.  SH = factors shared by all systems (uniform
// addresses, scalar loads); otherwise per-system columns of the same layout.
// ----------------------------------------------------------------------------

template <typename T, bool SH>
__global__ void __launch_bounds__(kWave)
k_penta_solve(int64_t n, int64_t batch, int64_t ld, const T *__restrict__ fac, T *__restrict__ x)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    const int64_t ldf = SH ? 1 : ld;
    const T *f0 = fac + (SH ? 0 : s);
    const int64_t arr = n * ldf;
    const T *ra = f0, *be = f0 + arr, *ep = f0 + 2 * arr, *ga = f0 + 3 * arr, *de = f0 + 4 * arr;
    x += s;
    T g1 = 0, g2 = 0;
#pragma unroll 8
    for (int64_t i = 0; i < n; ++i) {
        const T g = (x[i * ld] - ep[i * ldf] * g2 - be[i * ldf] * g1) * ra[i * ldf];
        x[i * ld] = g;
        g2 = g1; g1 = g;
    }
    T x1 = 0, x2 = 0;
#pragma unroll 8
    for (int64_t i = n - 1; i >= 0; --i) {
        const T xi = x[i * ld] - ga[i * ldf] * x1 - de[i * ldf] * x2;
        x[i * ld] = xi;
        x2 = x1; x1 = xi;
    }
}

// Periodic solve, repeated `nsteps` times (x_{k+1} = A^{-1} x_k).
template <typename T, bool SH>
__global__ void __launch_bounds__(kWave)
k_penta_cyclic_solve(int64_t n, int64_t batch, int64_t ld, int64_t nsteps,
                     const T *__restrict__ fac, T *__restrict__ x, const int32_t *__restrict__ mask)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    if (mask && !mask[s]) return;       // only the systems marked in mask
    const int64_t m = n - 2;
    const int64_t ldf = SH ? 1 : ld;
    const T *f0 = fac + (SH ? 0 : s);
    const int64_t arr = m * ldf;
    const T *ra = f0, *be = f0 + arr, *ep = f0 + 2 * arr, *ga = f0 + 3 * arr, *de = f0 + 4 * arr;
    const T *v0 = f0 + 5 * arr, *v1 = f0 + 6 * arr, *y0 = f0 + 7 * arr, *y1 = f0 + 8 * arr;
    const T *si = f0 + 9 * arr;
    const T S00 = si[0], S01 = si[ldf], S10 = si[2 * ldf], S11 = si[3 * ldf];
    x += s;
    for (int64_t step = 0; step < nsteps; ++step) {
        T g1 = 0, g2 = 0, s0 = 0, s1 = 0;
#pragma unroll 8
        for (int64_t i = 0; i < m; ++i) {
            const T g = (x[i * ld] - ep[i * ldf] * g2 - be[i * ldf] * g1) * ra[i * ldf];
            s0 += y0[i * ldf] * g;
            s1 += y1[i * ldf] * g;
            x[i * ld] = g;
            g2 = g1; g1 = g;
        }
        const T r0 = x[m * ld] - s0, r1 = x[(m + 1) * ld] - s1;
        const T t0 = S00 * r0 + S01 * r1;
        const T t1 = S10 * r0 + S11 * r1;
        x[m * ld] = t0;
        x[(m + 1) * ld] = t1;
        T x1 = 0, x2 = 0;
#pragma unroll 8
        for (int64_t i = m - 1; i >= 0; --i) {
            const T xi = (x[i * ld] - v0[i * ldf] * t0 - v1[i * ldf] * t1)
                         - ga[i * ldf] * x1 - de[i * ldf] * x2;
            x[i * ld] = xi;
            x2 = x1; x1 = xi;
        }
    }
}

// ----------------------------------------------------------------------------
// Fused factor + solve ("rewrite"): one forward pass computes the factors and
// g together; gamma and delta go to `work`, g into x; then back substitution.
// ----------------------------------------------------------------------------

template <typename T, int D>
__global__ void __launch_bounds__(kWave)
k_penta_fused(int64_t n, int64_t batch, int64_t ld,
              const T *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
              const T *__restrict__ D_, const T *__restrict__ E, T *__restrict__ x,
              T *__restrict__ work, int32_t *__restrict__ info)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    A += s; B += s; C += s; D_ += s; E += s; x += s;
    T *ga = work + s, *de = work + n * ld + s;
    int32_t bad = 0;
    T gam1 = 0, gam2 = 0, del1 = 0, del2 = 0, g1 = 0, g2 = 0;
    // rows 0 and 1: a_0, a_1, b_0 are outside the matrix
    {
        const T alpha = C[0];
        if (bad_pivot(alpha)) bad = 1;
        const T r = T(1) / alpha;
        gam1 = D_[0] * r; del1 = E[0] * r; g1 = x[0] * r;
        ga[0] = gam1; de[0] = del1; x[0] = g1;
    }
    {
        const T beta = B[ld];
        const T alpha = C[ld] - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = 2;
        const T r = T(1) / alpha;
        const T gam = (D_[ld] - beta * del1) * r, del = E[ld] * r;
        const T g = (x[ld] - beta * g1) * r;
        ga[ld] = gam; de[ld] = del; x[ld] = g;
        gam2 = gam1; gam1 = gam; del2 = del1; del1 = del; g2 = g1; g1 = g;
    }
    // rows 2 .. n-3 with a prefetch ring: the six inputs of row i + D are
    // loaded while row i is eliminated (one lane per system keeps only one
    // wavefront per SIMD busy, so memory-level parallelism has to come from
    // each lane's own look-ahead).
    const int64_t last = n - 1;
    auto rowp = [&](int64_t r) { return (r < last ? r : last) * ld; };
    T qa[D], qb[D], qc[D], qd[D], qe[D], qf[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
        const int64_t o = rowp(2 + k);
        qa[k] = A[o]; qb[k] = B[o]; qc[k] = C[o]; qd[k] = D_[o]; qe[k] = E[o]; qf[k] = x[o];
    }
    auto fwd_row = [&](int64_t i, T ai, T bi, T ci, T di, T ei, T fi) {
        const int64_t o = i * ld;
        const T beta = bi - ai * gam2;
        const T alpha = ci - ai * del2 - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = int32_t(i) + 1;
        const T r = T(1) / alpha;
        const T gam = (di - beta * del1) * r;
        const T del = ei * r;
        const T g = (fi - ai * g2 - beta * g1) * r;
        ga[o] = gam; de[o] = del; x[o] = g;
        gam2 = gam1; gam1 = gam; del2 = del1; del1 = del; g2 = g1; g1 = g;
    };
    int64_t i = 2;
    for (; i + D <= n - 2; i += D) {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            const T ai = qa[k], bi = qb[k], ci = qc[k], di = qd[k], ei = qe[k], fi = qf[k];
            const int64_t o = rowp(i + k + D);
            qa[k] = A[o]; qb[k] = B[o]; qc[k] = C[o]; qd[k] = D_[o]; qe[k] = E[o]; qf[k] = x[o];
            fwd_row(i + k, ai, bi, ci, di, ei, fi);
        }
    }
#pragma unroll
    for (int k = 0; k < D; ++k)
        if (i + k < n - 2) fwd_row(i + k, qa[k], qb[k], qc[k], qd[k], qe[k], qf[k]);
    // rows n-2 and n-1: d_{n-1}, e_{n-2}, e_{n-1} are outside the matrix
    T gam_n2;
    {
        const int64_t o = (n - 2) * ld;
        const T ai = A[o];
        const T beta = B[o] - ai * gam2;
        const T alpha = C[o] - ai * del2 - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = int32_t(n - 2) + 1;
        const T r = T(1) / alpha;
        gam_n2 = (D_[o] - beta * del1) * r;
        const T g = (x[o] - ai * g2 - beta * g1) * r;
        x[o] = g;
        gam2 = gam1; gam1 = gam_n2; del2 = del1; del1 = 0; g2 = g1; g1 = g;
    }
    T xl;
    {
        const int64_t o = (n - 1) * ld;
        const T ai = A[o];
        const T beta = B[o] - ai * gam2;
        const T alpha = C[o] - ai * del2 - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = int32_t(n - 1) + 1;
        const T r = T(1) / alpha;
        xl = (x[o] - ai * g2 - beta * g1) * r;   // x_{n-1} = g_{n-1}
        x[o] = xl;
    }
    if (info) info[s] = bad;
    // back substitution, rows n-3 .. 0, with the same look-ahead
    T x1 = g1 - gam_n2 * xl;                  // x_{n-2}
    x[(n - 2) * ld] = x1;
    T x2 = xl;
    auto rowb = [&](int64_t r) { return (r > 0 ? r : 0) * ld; };
    T pg[D], pga[D], pde[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
        const int64_t o = rowb(n - 3 - k);
        pg[k] = x[o]; pga[k] = ga[o]; pde[k] = de[o];
    }
    int64_t r = n - 3;
    for (; r - D >= -1; r -= D) {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            const T gi = pg[k], gai = pga[k], dei = pde[k];
            const int64_t o = rowb(r - k - D);
            pg[k] = x[o]; pga[k] = ga[o]; pde[k] = de[o];
            const T xi = gi - gai * x1 - dei * x2;
            x[(r - k) * ld] = xi;
            x2 = x1; x1 = xi;
        }
    }
#pragma unroll
    for (int k = 0; k < D; ++k) {
        if (r - k >= 0) {
            const T xi = pg[k] - pga[k] * x1 - pde[k] * x2;
            x[(r - k) * ld] = xi;
            x2 = x1; x1 = xi;
        }
    }
}

// ----------------------------------------------------------------------------
// Host launchers
// ----------------------------------------------------------------------------

static inline dim3 grid_for(int64_t lanes) { return dim3(unsigned((lanes + kWave - 1) / kWave)); }

template <typename T>
bps_status launch_penta_factor(int64_t n, int64_t batch, int64_t ld, bool cyclic, bool shared,
                               const void *a, const void *b, const void *c, const void *d,
                               const void *e, void *fac, int32_t *info, hipStream_t st,
                               const int32_t *mask)
{
    const int64_t lanes = shared ? 1 : batch;
    const int64_t ldin = shared ? 1 : ld;
    const int64_t ldf = shared ? 1 : ld;
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid_for(lanes), dim3(kWave), 0, st, n, lanes, ldin, ldf,
                           (const T *)a, (const T *)b, (const T *)c, (const T *)d, (const T *)e,
                           (T *)fac, info, mask);
    };
    if (cyclic) args(k_penta_factor<T, true>);
    else args(k_penta_factor<T, false>);
    BPS_LAUNCHED("k_penta_factor");
    return BPS_OK;
}

template <typename T>
bps_status launch_penta_solve(int64_t n, int64_t batch, int64_t ld, bool shared,
                              const void *fac, void *x, hipStream_t st)
{
    if (shared)
        hipLaunchKernelGGL((k_penta_solve<T, true>), grid_for(batch), dim3(kWave), 0, st, n,
                           batch, ld, (const T *)fac, (T *)x);
    else
        hipLaunchKernelGGL((k_penta_solve<T, false>), grid_for(batch), dim3(kWave), 0, st, n,
                           batch, ld, (const T *)fac, (T *)x);
    BPS_LAUNCHED("k_penta_solve");
    return BPS_OK;
}

template <typename T>
bps_status launch_penta_cyclic_solve(int64_t n, int64_t batch, int64_t ld, int64_t nsteps,
                                     bool shared, const void *fac, void *x, hipStream_t st,
                                     const int32_t *mask)
{
    if (shared)
        hipLaunchKernelGGL((k_penta_cyclic_solve<T, true>), grid_for(batch), dim3(kWave), 0, st,
                           n, batch, ld, nsteps, (const T *)fac, (T *)x, mask);
    else
        hipLaunchKernelGGL((k_penta_cyclic_solve<T, false>), grid_for(batch), dim3(kWave), 0, st,
                           n, batch, ld, nsteps, (const T *)fac, (T *)x, mask);
    BPS_LAUNCHED("k_penta_cyclic_solve");
    return BPS_OK;
}

template <typename T>
bps_status launch_penta_fused(int64_t n, int64_t batch, int64_t ld, const void *a, const void *b,
                              const void *c, const void *d, const void *e, void *x, void *work,
                              int32_t *info, hipStream_t st)
{
    hipLaunchKernelGGL((k_penta_fused<T, 8>), grid_for(batch), dim3(kWave), 0, st, n, batch, ld,
                       (const T *)a, (const T *)b, (const T *)c, (const T *)d, (const T *)e,
                       (T *)x, (T *)work, info);
    BPS_LAUNCHED("k_penta_fused");
    return BPS_OK;
}

#define BPS_INST(T)                                                                          \
    template bps_status launch_penta_factor<T>(int64_t, int64_t, int64_t, bool, bool,        \
                                               const void *, const void *, const void *,     \
                                               const void *, const void *, void *, int32_t *, \
                                               hipStream_t, const int32_t *);                \
    template bps_status launch_penta_solve<T>(int64_t, int64_t, int64_t, bool, const void *, \
                                              void *, hipStream_t);                          \
    template bps_status launch_penta_cyclic_solve<T>(int64_t, int64_t, int64_t, int64_t,     \
                                                     bool, const void *, void *, hipStream_t, \
                                                     const int32_t *);                       \
    template bps_status launch_penta_fused<T>(int64_t, int64_t, int64_t, const void *,       \
                                              const void *, const void *, const void *,      \
                                              const void *, void *, void *, int32_t *,       \
                                              hipStream_t);
BPS_INST(float)
BPS_INST(double)
#undef BPS_INST

}  // namespace bps
