// hyper.hip -- periodic hyperdiffusion operator for gfx950.
//
// The implicit step of "cuPentBatch - A batched pentadiagonal solver for
// NVIDIA GPUs" (hyperdiffusion section, eq. (4) discretised with the centred
// fourth difference on a periodic grid): (I + sigma D4) C^{k+1} = C^k with
// D4 = [1, -4, 6, -4, 1] and sigma = dt / dx^4, i.e. the periodic
// pentadiagonal matrix with a = e = sigma, b = d = -4 sigma, c = 1 + 6 sigma.
#include "common.h"
#include "kernels.h"

namespace bps {

// The entries are rounded exactly as written (no fused multiply-add): at
// sigma ~ 1e6 one ulp of c = 1 + 6 sigma shifts the matrix's constant-mode
// eigenvalue (a + b + c + d + e) by ~1e-9 relative, which the solution shows.
template <typename T>
__global__ void k_hyper_diagonals(int64_t n, double sigma, T *__restrict__ diag)
{
#pragma clang fp contract(off)
    const int64_t i = lane_id();
    if (i >= n) return;
    const T sg = T(sigma);
    diag[i] = sg;                          // a
    diag[n + i] = T(-4) * sg;              // b
    diag[2 * n + i] = T(1) + T(6) * sg;    // c
    diag[3 * n + i] = T(-4) * sg;          // d
    diag[4 * n + i] = sg;                  // e
}

template <typename T>
bps_status launch_hyper_diagonals(int64_t n, double sigma, void *diag, hipStream_t st)
{
    hipLaunchKernelGGL((k_hyper_diagonals<T>), dim3(unsigned((n + 255) / 256)), dim3(256), 0, st,
                       n, sigma, (T *)diag);
    BPS_LAUNCHED("k_hyper_diagonals");
    return BPS_OK;
}
template bps_status launch_hyper_diagonals<float>(int64_t, double, void *, hipStream_t);
template bps_status launch_hyper_diagonals<double>(int64_t, double, void *, hipStream_t);

}  // namespace bps
