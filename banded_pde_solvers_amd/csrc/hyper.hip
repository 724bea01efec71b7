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


// ============================================================================
// Register-resident multi-step solver for the constant-coefficient operator
// ============================================================================
//
// Each system of N = P*M unknowns is split into P chunks of M rows.  The last
// two rows of every chunk are "interface" unknowns; the M-2 rows before them
// ("interior") couple only to their own chunk's interface and to the previous
// chunk's interface (the matrix has bandwidth two), so the periodic matrix
// reduces to P independent interior blocks E (all equal, the diagonals being
// constant) plus a 2P x 2P Schur complement S on the interfaces:
//
//   interior j:   E x_j + C_L xI_{j-1} + C_R xI_j = f_j
//   interfaces:   S xI = r,  r_j = fI_j - B_own y_j - B_next y_{j+1},  y = E^{-1} f
//
// One lane owns one chunk of one system and keeps its M values in registers
// for all time steps; the chunks of a system exchange a few numbers per step
// (through LDS, or by DPP row rotations when a system fills a 16-lane row).
// Per step and lane:
//   forward  g = L^{-1} f (E = L R), with y_0, y_1 accumulated as w_k . g,
//            w_k = R^{-T} e_k, and y_{m-1}, y_{m-2} from the last two g;
//   exchange r_j (needs y_0, y_1 of the next chunk), then
//            xI_j = sum_q T_q r_{j+q} with T_q the first block row of S^{-1}
//            (S is block-circulant because every chunk is identical; the
//            set-up gets T by Gauss-Jordan, or for a power-of-two P from the
//            coefficients of periodic block cyclic reduction), or, for 16
//            chunks (one system per 16-lane row), that cyclic reduction
//            itself across the row's lanes;
//   backward x = R^{-1}(g - U_L xI_{j-1} - U_R xI_j), U = L^{-1} C.
// HBM sees the state twice per call (load, store) instead of twice per step.
//
// Accuracy: S is a difference of terms ~1e6 times larger than itself at
// sigma ~ 1e6, so the one-time set-up forms it with compensated dot products
// (the Dot2 algorithm of Ogita, Rump and Oishi, "Accurate sum and dot
// product", 2005) from spikes E^{-1} C refined once with a compensated
// residual; everything used per step is plain fp64.

// --- compensated arithmetic (error-free transformations) -------------------

struct Dot2 {
    double p = 0.0, s = 0.0;
    __device__ void add(double x, double y) {
#pragma clang fp contract(off)
        const double h = x * y;
        const double r = fma(x, y, -h);        // x*y = h + r exactly
        const double t = p + h;                // TwoSum(p, h)
        const double z = t - p;
        const double q = (p - (t - z)) + (h - z);
        p = t;
        s += q + r;
    }
    __device__ double value() const { return p + s; }
};

constexpr int kResMaxP = 16;    // chunks per system supported by the resident kernel (and 32, 64)
#ifndef BPS_RES_BATCH
#define BPS_RES_BATCH 3
#endif
constexpr int kResBatch = BPS_RES_BATCH;   // coefficient rows per scalar-load batch
// A wavefront of the resident kernel holds 64 / P systems times P chunks and
// exchanges interface values only among its own lanes, so the waves never
// wait on one another: the ones sharing a SIMD hide each other's latencies.
// Where the systems of one wavefront fill less than a 128-byte row segment,
// a workgroup gathers the wavefronts of up to 16 neighbouring systems (at
// most 4 wavefronts), so that the state is read and written in whole or
// half cache lines by one CU.
__host__ __device__ constexpr int res_systems(int P) { return kWave / P; }
__host__ __device__ constexpr int res_waves(int P)
{
    // (at most 4 wavefronts: with 32 or 64 chunks a workgroup of 8 or 4
    // systems still leaves room for three per CU)
    return (res_systems(P) * P == kWave && res_systems(P) < 16 && 16 % res_systems(P) == 0)
               ? (16 / res_systems(P) < 4 ? 16 / res_systems(P) : 4) : 1;
}

// coefficient block written by the set-up kernel, read with uniform loads:
//   forward rows i < m:  [ralpha, beta, w0, w1]                  (4 doubles)
//   backward rows i < m: [gamma, delta, UL0, UL1]                (4 doubles)
//   header:     [a, b, c, d, e, URa, URb, URc]                   (8 doubles)
//   P a power of two (after the T blocks): periodic block cyclic
//               reduction on the interface system: per level h = 1, 2, ...,
//               P/2 the 2x2 blocks alpha_h, gamma_h (row-major), then
//               (L + D + U)^{-1} of the last level (8 log2 P + 4 <= 52 doubles);
//               16 chunks use them in the time step, the T blocks of other
//               powers of two are computed from them
//   T blocks:   T_q (2x2, row-major) for q < P                   (4P doubles)
__host__ __device__ constexpr int res_coef_elems(int M, int P) { return 8 * (M - 2) + 8 + 4 * P + 52; }
__host__ __device__ constexpr bool res_pow2(int P) { return (P & (P - 1)) == 0; }
// 16 chunks: one system per 16-lane row, interface step by PCR (see below)
__host__ __device__ constexpr bool res_row(int P) { return P == 16; }

// 64-bit value of lane `lane` (uniform) of the wavefront
__device__ __forceinline__ double read_lane(double v, int lane)
{
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(int(b & 0xffffffffll), lane);
    const int hi = __builtin_amdgcn_readlane(int(b >> 32), lane);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}

// 64-bit value of another lane of the same 16-lane row (DPP row rotation, a
// VALU move: no LDS round trip).  ROR = 1: the lane before (lane 0 of the
// row takes lane 15); ROR = 15: the lane after (lane 15 takes lane 0).
template <int ROR>
__device__ __forceinline__ double row_rotate(double v)
{
    static_assert(ROR >= 1 && ROR <= 15, "row rotation by 1 .. 15 lanes");
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp(int(b & 0xffffffffll), 0x120 + ROR, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(int(b >> 32), 0x120 + ROR, 0xF, 0xF, false);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}

// Backward sweep x = R^{-1} src of the set-up (R unit upper with gamma,
// delta), into dst; the arrays are distinct, so the LDS reads of later rows
// may be issued ahead of the stores of earlier ones.
template <int m>
__device__ __forceinline__ void setup_back_sweep(const double *__restrict__ src,
                                                 const double *__restrict__ ga,
                                                 const double *__restrict__ de,
                                                 double *__restrict__ dst)
{
#pragma clang fp contract(fast)
    double q1 = 0.0, q2 = 0.0;
#pragma unroll
    for (int i = m - 1; i >= 0; --i) {
        const double x = src[i] - ga[i] * q1 - de[i] * q2;
        dst[i] = x;
        q2 = q1; q1 = x;
    }
}

// One wavefront.  The serial recurrences run in every lane at once (lane t
// carries coupling vector t & 7) with the running values in registers, and
// their loops are unrolled so that the LDS reads they need are issued ahead
// of the recurrence: the set-up is then bound by arithmetic latency rather
// than by LDS round trips.
template <int M, int P>
__device__ __forceinline__ void resident_setup(double sigma, double *__restrict__ coef)
{
#pragma clang fp contract(off)
    constexpr int m = M - 2, n2 = 2 * P, w = 4 * P;
    __shared__ double ra[m], be[m], ga[m], de[m];
    __shared__ double vec[8][m];        // UL0, UL1, w0, w1, ZL0, ZL1, ZR0, ZR1
    __shared__ double res[4][m];
    __shared__ double blk[3][2][2];     // blocks of S on interface offsets 0, +1, -1
    const int t = threadIdx.x;
    const double a = sigma, b = -4.0 * sigma, c = 1.0 + 6.0 * sigma, d = -4.0 * sigma, e = sigma;
    auto Ea = [&](int i) { return i >= 2 ? a : 0.0; };
    auto Eb = [&](int i) { return i >= 1 ? b : 0.0; };
    auto Ed = [&](int i) { return i + 1 < m ? d : 0.0; };
    auto Ee = [&](int i) { return i + 2 < m ? e : 0.0; };
    // interior-to-interface couplings: column k of C_L / C_R at row i
    auto CL = [&](int k, int i) { return k == 0 ? (i == 0 ? a : 0.0) : (i == 0 ? b : i == 1 ? a : 0.0); };
    auto CR = [&](int k, int i) { return k == 0 ? (i == m - 2 ? e : i == m - 1 ? d : 0.0)
                                                : (i == m - 1 ? e : 0.0); };
    // lane t builds coupling vector t & 7 (lanes t and t & 7 compute and
    // store equal values):
    //   0,1  U_L = L^{-1} C_L      2,3  w_k = R^{-T} e_k
    //   4,5  Z_L = E^{-1} C_L      6,7  Z_R = E^{-1} C_R
    const int role = t & 7, k = role & 1;
    const bool is_w = (role == 2 || role == 3), is_z = role >= 4, use_cr = role >= 6;
    double *my = vec[role];
    // the forward results of Z_L, Z_R go to `tmpz` (the backward sweep then
    // reads and writes different arrays)
    __shared__ double tmpz[4][m], dump[m];
    double *fw_out = is_z ? tmpz[role - 4] : my;
    // the right-hand side of lane t is nonzero in rows 0, 1, m-2, m-1 only
    const double rh0 = is_w ? (k == 0 ? 1.0 : 0.0) : use_cr ? CR(k, 0) : CL(k, 0);
    const double rh1 = is_w ? (k == 1 ? 1.0 : 0.0) : use_cr ? CR(k, 1) : CL(k, 1);
    const double rhA = is_w ? 0.0 : use_cr ? CR(k, m - 2) : CL(k, m - 2);
    const double rhB = is_w ? 0.0 : use_cr ? CR(k, m - 1) : CL(k, m - 1);
    // ---- factor E = L R (the pentadiagonal steps of the page) and, in the
    // same sweep, the forward recurrence of each lane's vector ----
    {
#pragma clang fp contract(fast)
        double g1 = 0, g2 = 0, d1 = 0, d2 = 0;      // gamma, delta of rows i-1, i-2
        double p1 = 0, p2 = 0;                      // vector values of rows i-1, i-2
#pragma unroll
        for (int i = 0; i < m; ++i) {
            const double beta = Eb(i) - Ea(i) * g2;
            const double alpha = c - Ea(i) * d2 - beta * g1;
            // 1/alpha: hardware estimate and two Newton steps, five
            // instructions on the recurrence's critical path where the
            // correctly rounded quotient takes eleven.  alpha, a pivot of the
            // SPD interior block (not below I), lies in [1, 1 + 6 sigma], so
            // no scaling is needed; the result is within an ulp of 1/alpha
            double r = __builtin_amdgcn_rcp(alpha);
            r = fma(fma(-alpha, r, 1.0), r, r);
            r = fma(fma(-alpha, r, 1.0), r, r);
            const double gam = (Ed(i) - beta * d1) * r, del = Ee(i) * r;
            // every lane stores (the lanes hold equal values): no branch in
            // the unrolled sweep, so its LDS traffic overlaps the recurrence
            ra[i] = r; be[i] = beta; ga[i] = gam; de[i] = del;
            // L^{-1} rhs, or R^{-T} e_k (R^T is unit lower with gamma, delta)
            const double rhs = i == 0 ? rh0 : i == 1 ? rh1 : i == m - 2 ? rhA : i == m - 1 ? rhB : 0.0;
            const double lv = (rhs - Ea(i) * p2 - beta * p1) * r;
            const double wv = rhs - (i >= 1 ? g1 : 0.0) * p1 - (i >= 2 ? d2 : 0.0) * p2;
            const double x = is_w ? wv : lv;
            fw_out[i] = x;                  // lanes t and t & 7 store equal values
            p2 = p1; p1 = x;
            g2 = g1; g1 = gam; d2 = d1; d1 = del;
        }
    }
    __syncthreads();
    // ---- Z = R^{-1} U for lanes 4..7 (the other lanes store into `dump`,
    // so that the unrolled sweep has no branch) ----
    setup_back_sweep<m>(fw_out, ga, de, is_z ? my : dump);
    __syncthreads();
    // ---- one refinement step of Z: residual C - E Z with compensated sums
    // (4m entries over the wavefront's lanes; past the end a lane repeats
    // the last entry and stores it into `dump`) ----
    constexpr int kResid = (4 * m + kWave - 1) / kWave;
#pragma unroll
    for (int it = 0; it < kResid; ++it) {
        const int idx0 = t + kWave * it, idx = idx0 < 4 * m ? idx0 : 4 * m - 1;
        const int kk = idx / m, i = idx % m;
        const double *z = vec[4 + kk];
        // terms outside the block have a zero coefficient (an exact zero
        // product leaves the compensated sum unchanged), their index clamped
        Dot2 acc;
        acc.add(kk < 2 ? CL(kk & 1, i) : CR(kk & 1, i), 1.0);
        acc.add(-Ea(i), z[i >= 2 ? i - 2 : 0]);
        acc.add(-Eb(i), z[i >= 1 ? i - 1 : 0]);
        acc.add(-c, z[i]);
        acc.add(-Ed(i), z[i + 1 < m ? i + 1 : m - 1]);
        acc.add(-Ee(i), z[i + 2 < m ? i + 2 : m - 1]);
        (idx0 < 4 * m ? &res[kk][i] : &dump[0])[0] = acc.value();
    }
    __syncthreads();
    if (t < 4) {
#pragma clang fp contract(fast)
        // lanes 0..3 solve E dz = residual (g in registers) and correct Z
        const double *rv = res[t];
        double gv[m];
        double p1 = 0.0, p2 = 0.0;
#pragma unroll
        for (int i = 0; i < m; ++i) {
            const double g = (rv[i] - Ea(i) * p2 - be[i] * p1) * ra[i];
            gv[i] = g; p2 = p1; p1 = g;
        }
        double q1 = 0.0, q2 = 0.0;
#pragma unroll
        for (int i = m - 1; i >= 0; --i) {
            const double x = gv[i] - ga[i] * q1 - de[i] * q2;
            vec[4 + t][i] += x; q2 = q1; q1 = x;
        }
    }
    __syncthreads();
    // ---- Schur complement S (2P x 2P, block-circulant): the three nonzero
    // 2x2 blocks of block row 0, compensated, by lanes 0..11 ----
    auto ZL = [&](int q) -> const double * { return q ? vec[5] : vec[4]; };
    auto ZR = [&](int q) -> const double * { return q ? vec[7] : vec[6]; };
    if (t < 12) {
        const int bi = t >> 2, r = (t >> 1) & 1, q = t & 1;
        const int K = bi == 0 ? 0 : bi == 1 ? 1 % P : P - 1;   // column block, row block J = 0
        Dot2 acc;
        // rows of B_own (interface j on interior j) and B_next (interface j-1 on interior j)
        auto own = [&](const double *z) {           // B_own[r] . z
            if (r == 0) { acc.add(-a, z[m - 2]); acc.add(-b, z[m - 1]); }
            else acc.add(-a, z[m - 1]);
        };
        auto nxt = [&](const double *z) {           // B_next[r] . z
            if (r == 0) acc.add(-e, z[0]);
            else { acc.add(-d, z[0]); acc.add(-e, z[1]); }
        };
        if (K == 0) {
            acc.add(r == 0 ? (q == 0 ? c : d) : (q == 0 ? b : c), 1.0);
            own(ZR(q)); nxt(ZL(q));
        }
        if (K == P - 1) own(ZL(q));
        if (K == 1) nxt(ZR(q));
        blk[bi][r][q] = acc.value();
    }
    __syncthreads();
    // ---- P a power of two: coefficients of periodic block cyclic reduction on the
    // interface system S xI = r (all block rows alike: L = S_{j,j-1},
    // D = S_{j,j}, U = S_{j,j+1}).  Level h: alpha = -L D^{-1},
    // gamma = -U D^{-1}; r_j += alpha r_{j-h} + gamma r_{j+h}; L, D, U of the
    // next level alpha L, D + alpha U + gamma L, gamma U.  After the level
    // h = P/2, j - P and j + P are j itself: xI_j = (L + D + U)^{-1} r_j.
    // (S is a Schur complement of the SPD I + sigma D4, hence SPD; the
    // reduction is block elimination in another order.)
    __shared__ double pcr[res_pow2(P) ? 52 : 1];
    if constexpr (res_pow2(P)) {
        if (t == 0) {
            struct B2 { double a, b, c, d; };
            auto mul = [](B2 x, B2 y) {
                return B2{x.a * y.a + x.b * y.c, x.a * y.b + x.b * y.d,
                          x.c * y.a + x.d * y.c, x.c * y.b + x.d * y.d};
            };
            auto add = [](B2 x, B2 y) { return B2{x.a + y.a, x.b + y.b, x.c + y.c, x.d + y.d}; };
            auto neg = [](B2 x) { return B2{-x.a, -x.b, -x.c, -x.d}; };
            auto inv = [](B2 x) {
                const double r = 1.0 / (x.a * x.d - x.b * x.c);
                return B2{x.d * r, -x.b * r, -x.c * r, x.a * r};
            };
            B2 L{blk[2][0][0], blk[2][0][1], blk[2][1][0], blk[2][1][1]};
            B2 D{blk[0][0][0], blk[0][0][1], blk[0][1][0], blk[0][1][1]};
            // with 2 chunks both neighbours are the other chunk, and blk[1] and
            // blk[2] each hold its whole coupling: count it once
            B2 U = P == 2 ? B2{0.0, 0.0, 0.0, 0.0}
                          : B2{blk[1][0][0], blk[1][0][1], blk[1][1][0], blk[1][1][1]};
            double *pc = pcr;
            for (int h = 1; h < P; h <<= 1, pc += 8) {
                const B2 Di = inv(D);
                const B2 al = neg(mul(L, Di)), ga = neg(mul(U, Di));
                pc[0] = al.a; pc[1] = al.b; pc[2] = al.c; pc[3] = al.d;
                pc[4] = ga.a; pc[5] = ga.b; pc[6] = ga.c; pc[7] = ga.d;
                const B2 nL = mul(al, L), nU = mul(ga, U);
                D = add(D, add(mul(al, U), mul(ga, L)));
                L = nL; U = nU;
            }
            const B2 Mi = inv(add(L, add(D, U)));
            pc[0] = Mi.a; pc[1] = Mi.b; pc[2] = Mi.c; pc[3] = Mi.d;
        }
        __syncthreads();
        // 8 log2 P + 4 of the 52 entries are set; the rest are written as 0
        constexpr int npcr = 8 * (P >= 64 ? 6 : P >= 32 ? 5 : P >= 16 ? 4 : P >= 8 ? 3 : P >= 4 ? 2 : 1) + 4;
        for (int i = t; i < 52; i += blockDim.x) coef[8 * m + 8 + 4 * P + i] = i < npcr ? pcr[i] : 0.0;
    }
    // ---- other powers of two: T_q, the first block row of S^{-1}, by the
    // same reduction applied to the block column E_0 = [I; 0; ...; 0]
    // (S X = E_0, lane j < P holds the 2x2 block row j of X; S is symmetric,
    // so T_q = X_q^T)
    if constexpr (res_pow2(P) && !res_row(P)) {
        __shared__ double xr[2][P][4];
        double x4[4] = {t == 0 ? 1.0 : 0.0, 0.0, 0.0, t == 0 ? 1.0 : 0.0};
        int cur = 0;
        if (t < P) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xr[0][t][e] = x4[e];
        }
        __syncthreads();
        int lv = 0;
        for (int h = 1; h < P; h <<= 1, ++lv) {
            if (t < P) {
                const double *al = pcr + 8 * lv, *ga = al + 4;
                const double *xm = xr[cur][(t - h + P) % P], *xp = xr[cur][(t + h) % P];
                // x4 += alpha xm + gamma xp (2x2 blocks, row-major)
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        x4[2 * r + c] += al[2 * r] * xm[c] + al[2 * r + 1] * xm[2 + c] +
                                         ga[2 * r] * xp[c] + ga[2 * r + 1] * xp[2 + c];
#pragma unroll
                for (int e = 0; e < 4; ++e) xr[cur ^ 1][t][e] = x4[e];
            }
            cur ^= 1;
            __syncthreads();
        }
        if (t < P) {
            const double *mi = pcr + 8 * lv;
            double xq[4];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c) xq[2 * r + c] = mi[2 * r] * x4[c] + mi[2 * r + 1] * x4[2 + c];
            double *T = coef + 8 * m + 8 + 4 * t;
            T[0] = xq[0]; T[1] = xq[2]; T[2] = xq[1]; T[3] = xq[3];     // X_q^T
        }
    }
    // ---- other chunk counts: Gauss-Jordan on [S | I] without pivoting (S is
    // symmetric positive definite: a Schur complement of I + sigma*D4,
    // sigma >= 0).  Lane t holds column t in registers; pivot column entries
    // are broadcast by readlane.
    if constexpr (!res_pow2(P)) {
    double cv[n2];
#pragma unroll
    for (int i = 0; i < n2; ++i) {
        const int J = i >> 1, r = i & 1;
        double val = 0.0;
        if (t < n2) {
            const int K = t >> 1, q = t & 1, off = (K - J + P) % P;
            if (off == 0) val = blk[0][r][q];
            else if (off == 1) val = blk[1][r][q];
            else if (off == P - 1) val = blk[2][r][q];
        } else if (t < w) {
            val = (i == t - n2) ? 1.0 : 0.0;
        }
        cv[i] = val;
    }
#pragma unroll
    for (int kp = 0; kp < n2; ++kp) {
#pragma clang fp contract(fast)
        double f[n2];
#pragma unroll
        for (int i = 0; i < n2; ++i) f[i] = read_lane(cv[i], kp);
        const double pk = cv[kp] / f[kp];
#pragma unroll
        for (int i = 0; i < n2; ++i) cv[i] = (i == kp) ? pk : cv[i] - f[i] * pk;
    }
    // T_q = rows 0, 1 of S^{-1}, columns 2q, 2q+1 (held by lanes n2 + 2q + c)
    if (t >= n2 && t < w) {
        const int q = (t - n2) >> 1, cc = (t - n2) & 1;
        coef[8 * m + 8 + 4 * q + cc] = cv[0];
        coef[8 * m + 8 + 4 * q + 2 + cc] = cv[1];
    }
    }
    // ---- outputs ----
    for (int idx = t; idx < m; idx += blockDim.x) {
        double *fw = coef + 4 * idx, *bw = coef + 4 * m + 4 * idx;
        fw[0] = ra[idx]; fw[1] = be[idx]; fw[2] = vec[2][idx]; fw[3] = vec[3][idx];
        bw[0] = ga[idx]; bw[1] = de[idx]; bw[2] = vec[0][idx]; bw[3] = vec[1][idx];
    }
    if (t == 0) {
        double *h = coef + 8 * m;
        h[0] = a; h[1] = b; h[2] = c; h[3] = d; h[4] = e;
        const double URa = e * ra[m - 2];              // L^{-1} C_R, last two rows
        const double URb = (d - be[m - 1] * URa) * ra[m - 1];
        const double URc = e * ra[m - 1];
        h[5] = URa; h[6] = URb; h[7] = URc;
    }
}

template <int M, int P>
__global__ void __launch_bounds__(64) k_hyper_resident_setup(double sigma, double *__restrict__ coef)
{
    resident_setup<M, P>(sigma, coef);
}

// The set-ups of two chunk lengths at once, one workgroup each (they run on
// different CUs, so the call costs the longer of the two).
template <int M1, int P1, int M2, int P2>
__global__ void __launch_bounds__(64) k_hyper_resident_setup2(double sigma, double *__restrict__ coef1,
                                                              double *__restrict__ coef2)
{
    if (blockIdx.x == 0) resident_setup<M1, P1>(sigma, coef1);
    else resident_setup<M2, P2>(sigma, coef2);
}

// Right-hand side of each step, by the bits of EX:
//   kResStencil  the explicit five-point stencil (ex2, ex1, ex0, ex1, ex2)
//                of the state, (I - (1 - theta) sigma D4) C, instead of C;
//   kResPhase    plus rr D2 (C^3 - C), the phase-separation term of the
//                Cahn-Hilliard equation at the old time level.
// With either bit the chunks exchange their first and last two rows.
template <int M, int P, int EX>
__global__ void __launch_bounds__(kWave * res_waves(P)) __attribute__((amdgpu_waves_per_eu(3)))
k_hyper_resident(int64_t batch, int64_t ld, int64_t nsteps, const double *__restrict__ coef,
                 double *__restrict__ C, double ex0, double ex1, double ex2, double rr)
{
    constexpr int m = M - 2;
    constexpr int S = res_systems(P), WS = res_waves(P), SW = S * WS;   // systems per wave, per workgroup
    // 16 chunks: a system is one 16-lane row (lane = chunk), and the values
    // of the neighbouring chunks come by row rotation; otherwise lane =
    // chunk * S + system and every exchange goes through LDS
    constexpr bool ROW = res_row(P);
    constexpr int PL = ROW ? 1 : P;          // LDS slots of the neighbour exchanges
    __shared__ double tbuf[2][PL][SW][2];
    // r_k stored at k and k + P (the dense interface step; ROW uses none)
    __shared__ double rbuf[2][ROW ? 1 : 2 * P][SW][2];
    __shared__ double xbuf[2][PL][SW][2];
    constexpr bool LIN = (EX & kResStencil) != 0, PHI = (EX & kResPhase) != 0;
    __shared__ double hbuf[EX != 0 ? PL : 1][SW][4];  // halo rows of the explicit side
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    // chunk, system slot in the workgroup
    const int j = ROW ? (lane & 15) : lane / S, sl = wv * S + (ROW ? lane >> 4 : lane % S);
    auto R = [&](int b, int k) -> double * { return rbuf[b][k][sl]; };
    // workgroups are dispatched round-robin over the 8 XCDs: the ones one
    // XCD runs back to back take neighbouring systems, so that row segments
    // narrower than a 128-byte line share it through one L2
    const unsigned nb = gridDim.x, bid = blockIdx.x, full = nb & ~7u;
    const unsigned tile = bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
    const int64_t s = int64_t(tile) * SW + sl;
    const bool act = s < batch;
    // lanes past the end of the batch compute on a copy of the last system
    // and store nothing
    double *col = C + (act ? s : batch - 1) + int64_t(j) * M * ld;
    // lanes of one wavefront exchange values through LDS: a fence keeps the
    // compiler from moving the accesses across (the wavefront itself executes
    // them in order), and no workgroup barrier is needed
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    const double *H = coef + 8 * m;
    const double a = H[0], b = H[1], d = H[3], e = H[4];
    const double URa = H[5], URb = H[6], URc = H[7];

    // the state, read in groups of 8 rows through a pointer re-derived per
    // group, so that the compiler does not materialise all M row addresses
    // at once (they would spill)
    double x[M];
#pragma unroll
    for (int g = 0; g < M / 8; ++g) {
        const double *pg = col + int64_t(8 * g) * ld;
        asm volatile("" : "+v"(pg));
#pragma unroll
        for (int r = 0; r < 8; ++r) x[8 * g + r] = pg[int64_t(r) * ld];
    }

    const int jn = (j + 1 == P) ? 0 : j + 1;
    const int jm1 = (j == 0) ? P - 1 : j - 1;
    for (int64_t step = 0; step < nsteps; ++step) {
        const int bf = int(step & 1);
        // explicit half of the theta scheme: rows -2, -1 (previous chunk's
        // last rows) and M, M+1 (next chunk's first rows) of the state
        double xm2 = 0.0, xm1 = 0.0, xp0 = 0.0, xp1 = 0.0;
        if constexpr (EX != 0 && ROW) {
            xm2 = row_rotate<1>(x[m]); xm1 = row_rotate<1>(x[m + 1]);
            xp0 = row_rotate<15>(x[0]); xp1 = row_rotate<15>(x[1]);
        } else if constexpr (EX != 0) {
            double *hb = hbuf[j][sl];
            hb[0] = x[0]; hb[1] = x[1]; hb[2] = x[m]; hb[3] = x[m + 1];
            wave_sync();
            xm2 = hbuf[jm1][sl][2]; xm1 = hbuf[jm1][sl][3];
            xp0 = hbuf[jn][sl][0]; xp1 = hbuf[jn][sl][1];
        }
        double o1 = xm1, o2 = xm2;     // state rows i-1, i-2 before this step
        // phase-separation term phi = C^3 - C of rows i-1 and i before this step
        double qa = 0.0, qb = 0.0;
        if constexpr (PHI) {
            qa = fma(xm1 * xm1, xm1, -xm1);
            qb = fma(x[0] * x[0], x[0], -x[0]);
        }
        // Per-row coefficients come from the scalar cache (uniform loads
        // through a pointer in the constant address space), KB rows at a
        // time, one batch ahead: the loads of batch k+1 are issued right after
        // batch k has arrived and before batch k is used.  Scalar loads
        // complete out of order, so any wait on one is a wait on all; the
        // empty asm statements place that wait (they read batch k) before
        // the next batch is requested, and re-derive the pointer so that the
        // compiler neither hoists the loads out of the step loop nor sinks
        // them to their uses.  Each sweep's rows are stored contiguously,
        // so a batch is one 64-byte request: the number of requests, not
        // their size, is what the waits cost (two 32-byte loads per batch
        // measured 7% slower over the whole solve).
        typedef const __attribute__((address_space(4))) double cdouble;
        // KB rows per batch (the last batch may be shorter): a lone wave per
        // SIMD stalls at every wait, so fewer, larger batches keep it issuing
        constexpr int KB = kResBatch, NB = (m + KB - 1) / KB;
        const double *cg = coef;
        asm volatile("" : "+s"(cg));
        cdouble *cf = (cdouble *)cg;
        double cb[2][KB][4];
#pragma unroll
        for (int r = 0; r < KB; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) cb[0][r][q] = r < m ? cf[4 * r + q] : 0.0;
        // forward: g = L^{-1} f_interior, and y_0, y_1 = w . g
        double t0 = 0.0, t1 = 0.0;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int cur = k & 1;
#pragma unroll
            for (int r = 0; r < KB; ++r)
                if (k * KB + r < m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) asm volatile("" ::"s"(cb[cur][r][q]));
            asm volatile("" : "+s"(cg));
            cf = (cdouble *)cg;
            if (k + 1 < NB) {
#pragma unroll
                for (int r = 0; r < KB; ++r)
                    if ((k + 1) * KB + r < m)
#pragma unroll
                        for (int q = 0; q < 4; ++q) cb[cur ^ 1][r][q] = cf[4 * ((k + 1) * KB + r) + q];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                const int i = k * KB + r;
                if (i >= m) break;
                const double *c4 = cb[cur][r];     // [1/alpha, beta, w0, w1]
                double g = x[i];
                if constexpr (LIN) {
                    const double xi = x[i];
                    g = ex2 * o2;
                    g = fma(ex1, o1, g);
                    g = fma(ex0, xi, g);
                    g = fma(ex1, x[i + 1], g);
                    g = fma(ex2, x[i + 2], g);
                    o2 = o1; o1 = xi;
                }
                if constexpr (PHI) {
                    const double xn = x[i + 1];
                    const double qc = fma(xn * xn, xn, -xn);
                    g = fma(rr, fma(-2.0, qb, qa + qc), g);
                    qa = qb; qb = qc;
                }
                if (i >= 2) g -= a * x[i - 2];
                if (i >= 1) g -= c4[1] * x[i - 1];
                g *= c4[0];
                x[i] = g;
                t0 += c4[2] * g;
                t1 += c4[3] * g;
            }
        }
        const double yR1 = x[m - 1];
        const double yR0 = x[m - 2] - cf[4 * m + 4 * (m - 2)] * yR1;
        // y_0, y_1 of the next chunk
        double yn0, yn1;
        if constexpr (ROW) {
            yn0 = row_rotate<15>(t0); yn1 = row_rotate<15>(t1);
        } else {
            tbuf[bf][j][sl][0] = t0; tbuf[bf][j][sl][1] = t1;
            wave_sync();
            yn0 = tbuf[bf][jn][sl][0]; yn1 = tbuf[bf][jn][sl][1];
        }
        double fI0 = x[m], fI1 = x[m + 1];     // right-hand side on the interface rows
        if constexpr (LIN) {
            fI0 = ex2 * o2;
            fI0 = fma(ex1, o1, fI0);
            fI0 = fma(ex0, x[m], fI0);
            fI0 = fma(ex1, x[m + 1], fI0);
            fI0 = fma(ex2, xp0, fI0);
            fI1 = ex2 * o1;
            fI1 = fma(ex1, x[m], fI1);
            fI1 = fma(ex0, x[m + 1], fI1);
            fI1 = fma(ex1, xp0, fI1);
            fI1 = fma(ex2, xp1, fI1);
        }
        if constexpr (PHI) {
            // qa, qb: phi of rows m-1, m
            const double xn = x[m + 1];
            const double qc = fma(xn * xn, xn, -xn);
            const double qd = fma(xp0 * xp0, xp0, -xp0);
            fI0 = fma(rr, fma(-2.0, qb, qa + qc), fI0);
            fI1 = fma(rr, fma(-2.0, qc, qb + qd), fI1);
        }
        const double rj0 = fI0 - a * yR0 - b * yR1 - e * yn0;
        const double rj1 = fI1 - a * yR1 - d * yn0 - e * yn1;
        double r0 = 0.0, r1 = 0.0;
        if constexpr (ROW) {
            // interface values by periodic block cyclic reduction across the
            // row's 16 lanes: four levels of neighbours 1, 2, 4, 8 lanes away
            // (row rotations), then (L + D + U)^{-1}
            const double *pg = coef + 8 * m + 8 + 4 * P;
            asm volatile("" : "+s"(pg) : "v"(rj1));
            cdouble *pc = (cdouble *)pg;
            double q0 = rj0, q1 = rj1;
            auto level = [&](double m0, double m1, double p0, double p1, int lv) {
                cdouble *c8 = pc + 8 * lv;       // [alpha (2x2), gamma (2x2)]
                double n0 = q0, n1 = q1;
                n0 = fma(c8[0], m0, n0); n0 = fma(c8[1], m1, n0);
                n0 = fma(c8[4], p0, n0); n0 = fma(c8[5], p1, n0);
                n1 = fma(c8[2], m0, n1); n1 = fma(c8[3], m1, n1);
                n1 = fma(c8[6], p0, n1); n1 = fma(c8[7], p1, n1);
                q0 = n0; q1 = n1;
            };
            level(row_rotate<1>(q0), row_rotate<1>(q1), row_rotate<15>(q0), row_rotate<15>(q1), 0);
            level(row_rotate<2>(q0), row_rotate<2>(q1), row_rotate<14>(q0), row_rotate<14>(q1), 1);
            level(row_rotate<4>(q0), row_rotate<4>(q1), row_rotate<12>(q0), row_rotate<12>(q1), 2);
            {
                const double h0 = row_rotate<8>(q0), h1 = row_rotate<8>(q1);   // j - 8 = j + 8
                level(h0, h1, h0, h1, 3);
            }
            cdouble *mi = pc + 32;
            r0 = mi[0] * q0; r0 = fma(mi[1], q1, r0);
            r1 = mi[2] * q0; r1 = fma(mi[3], q1, r1);
        } else {
        R(bf, j)[0] = rj0; R(bf, j)[1] = rj1;
        R(bf, j + P)[0] = rj0; R(bf, j + P)[1] = rj1;
        wave_sync();
        // interface values of this chunk: xI_j = sum_q T_q r_{j+q}
        // (block-circulant S^{-1}: T_q is its first block row)
            const double *tg = coef + 8 * m + 8;
            asm volatile("" : "+s"(tg) : "v"(rj1));
            cdouble *T = (cdouble *)tg;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                if (q >= 4 && q % 4 == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("" : "+s"(tg) : "v"(r1));
                    T = (cdouble *)tg;
                }
                const double R0 = R(bf, j + q)[0], R1 = R(bf, j + q)[1];
                r0 = fma(T[4 * q + 0], R0, r0);
                r0 = fma(T[4 * q + 1], R1, r0);
                r1 = fma(T[4 * q + 2], R0, r1);
                r1 = fma(T[4 * q + 3], R1, r1);
            }
        }
        // ... and of the previous chunk, from its lane
        double l0, l1;
        if constexpr (ROW) {
            l0 = row_rotate<1>(r0); l1 = row_rotate<1>(r1);
        } else {
            xbuf[bf][j][sl][0] = r0; xbuf[bf][j][sl][1] = r1;
            wave_sync();
            l0 = xbuf[bf][jm1][sl][0]; l1 = xbuf[bf][jm1][sl][1];
        }
        asm volatile("" : "+s"(cg) : "v"(l1));
        cf = (cdouble *)cg;
        // backward: x = R^{-1}(g - U_L xI_{j-1} - U_R xI_j), coefficient
        // batches of KB rows from the bottom up, loaded one batch ahead
#pragma unroll
        for (int r = 0; r < KB; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) cb[0][r][q] = r < m ? cf[4 * m + 4 * (m - 1 - r) + q] : 0.0;
        x[m - 2] -= URa * r0;
        x[m - 1] -= URb * r0 + URc * r1;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int cur = k & 1;
#pragma unroll
            for (int r = 0; r < KB; ++r)
                if (k * KB + r < m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) asm volatile("" ::"s"(cb[cur][r][q]));
            asm volatile("" : "+s"(cg));
            cf = (cdouble *)cg;
            if (k + 1 < NB) {
#pragma unroll
                for (int r = 0; r < KB; ++r)
                    if ((k + 1) * KB + r < m)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            cb[cur ^ 1][r][q] = cf[4 * m + 4 * (m - 1 - (k + 1) * KB - r) + q];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                if (k * KB + r >= m) break;
                const int i = m - 1 - (k * KB + r);
                const double *c4 = cb[cur][r];     // [gamma, delta, UL0, UL1]
                double v = x[i] - c4[2] * l0 - c4[3] * l1;
                if (i + 1 < m) v -= c4[0] * x[i + 1];
                if (i + 2 < m) v -= c4[1] * x[i + 2];
                x[i] = v;
            }
        }
        x[m] = r0;
        x[m + 1] = r1;
    }
    // the waves of a workgroup write quarters of the same cache lines: let
    // them store together, so that each line is whole when it leaves L2
    if (WS > 1) __syncthreads();
    if (act) {
#pragma unroll
        for (int g = 0; g < M / 8; ++g) {
            double *outg = col + int64_t(8 * g) * ld;
            asm volatile("" : "+v"(outg));
            __attribute__((address_space(1))) double *out = (__attribute__((address_space(1))) double *)outg;
#pragma unroll
            for (int r = 0; r < 8; ++r) out[int64_t(r) * ld] = x[8 * g + r];
        }
    }
}

// Chunk lengths of the resident path for n: M1 (0 if the shape is not
// supported) with P1 chunks, and for n = 256 a second one (M2 = 16, P2 = 16)
// for batches too small to give every SIMD a wavefront with 64-row chunks.
// Sixteen chunks put one system in a 16-lane row (DPP exchanges, cyclic
// reduction on the interface), which beats a dense interface step, so n =
// 384 .. 896 in steps of 128 take 16 chunks of n/16 rows.  Measured (100
// steps, 64-row / n/16-row chunks): n = 256: 64 systems 0.168 / 0.069 ms,
// 4096 0.181 / 0.078, 16384 0.206 / 0.189, 32768 0.331 / 0.361; n = 512:
// 8192 0.291 / 0.184, 65536 1.18 / 1.12; 65536 systems of n = 384, 640, 768,
// 896: 0.94 / 0.91, 1.52 / 1.36, 1.78 / 1.58, 2.10 / 1.83 ms.
struct ResChunks { int M1, P1, M2, P2; };
static ResChunks resident_chunks(int64_t n)
{
    if (n == 256) return {64, 4, 16, 16};
    if (n == 384 || n == 512 || n == 640 || n == 768 || n == 896) return {int(n / 16), 16, 0, 0};
    constexpr int M = 64;
    if (n % M != 0) return {0, 0, 0, 0};
    const int64_t P = n / M;
    return ((P >= 2 && P <= kResMaxP) || P == 32 || P == 64) ? ResChunks{M, int(P), 0, 0}
                                                            : ResChunks{0, 0, 0, 0};
}

int resident_chunk(int64_t n) { return resident_chunks(n).M1; }

size_t resident_coef_bytes(int64_t n)
{
    const ResChunks rc = resident_chunks(n);
    if (!rc.M1) return 0;
    return (size_t(res_coef_elems(rc.M1, rc.P1)) + (rc.M2 ? size_t(res_coef_elems(rc.M2, rc.P2)) : 0)) *
           sizeof(double);
}

template <int M, int P>
static void launch_res(int64_t batch, int64_t ld, int64_t nsteps, double sigma, int mode,
                       double e0, double e1, double e2, double rr, double *coef, double *C,
                       int parts, hipStream_t st)
{
    if (parts & kResSetup)
        hipLaunchKernelGGL((k_hyper_resident_setup<M, P>), dim3(1), dim3(64), 0, st, sigma, coef);
    if (nsteps == 0 || !(parts & kResSteps)) return;
    constexpr int S = res_systems(P), WS = res_waves(P), SW = S * WS;
    const unsigned grid = unsigned((batch + SW - 1) / SW);
    const unsigned threads = WS > 1 ? unsigned(kWave * WS) : unsigned(S * P);
    const double *cf = coef;
    switch (mode) {
    case kResStencil:
        hipLaunchKernelGGL((k_hyper_resident<M, P, kResStencil>), dim3(grid), dim3(threads), 0, st,
                           batch, ld, nsteps, cf, C, e0, e1, e2, rr);
        break;
    case kResPhase:
        hipLaunchKernelGGL((k_hyper_resident<M, P, kResPhase>), dim3(grid), dim3(threads), 0, st,
                           batch, ld, nsteps, cf, C, e0, e1, e2, rr);
        break;
    case kResStencil | kResPhase:
        hipLaunchKernelGGL((k_hyper_resident<M, P, kResStencil | kResPhase>), dim3(grid),
                           dim3(threads), 0, st, batch, ld, nsteps, cf, C, e0, e1, e2, rr);
        break;
    default:
        hipLaunchKernelGGL((k_hyper_resident<M, P, 0>), dim3(grid), dim3(threads), 0, st, batch, ld,
                           nsteps, cf, C, e0, e1, e2, rr);
    }
}

bps_status launch_hyper_resident(int64_t n, int64_t batch, int64_t ld, int64_t nsteps, double sigma,
                                 int mode, double e0, double e1, double e2, double rr, void *coef,
                                 void *C, hipStream_t st, int parts)
{
    const ResChunks rc = resident_chunks(n);
    if (!rc.M1 || !(sigma >= 0.0))
        BPS_FAIL(BPS_ENOTSUP, "resident path needs n = 64*P, 2 <= P <= 16 or P = 32, 64, sigma >= 0");
    double *cf = (double *)coef, *x = (double *)C;
    double *cf2 = cf + res_coef_elems(rc.M1, rc.P1);
    if ((parts & kResSetup) && rc.M2) {
        // both coefficient sets (n = 256 only), in one launch
        hipLaunchKernelGGL((k_hyper_resident_setup2<64, 4, 16, 16>), dim3(2), dim3(64), 0, st, sigma, cf, cf2);
        parts &= ~kResSetup;
    }
    // the second chunk length while 64-row chunks leave SIMDs without a
    // wavefront (at most one wavefront per SIMD: 1024 of 64 / P1 systems)
    const bool second = rc.M2 && batch <= int64_t(1024) * (kWave / rc.P1);
    if (second) {
        launch_res<16, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf2, x, parts, st);
        BPS_LAUNCHED("k_hyper_resident");
        return BPS_OK;
    }
    if (rc.M1 != 64) {
        switch (rc.M1) {
        case 24: launch_res<24, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
        case 32: launch_res<32, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
        case 40: launch_res<40, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
        case 48: launch_res<48, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
        default: launch_res<56, 16>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
        }
        BPS_LAUNCHED("k_hyper_resident");
        return BPS_OK;
    }
    constexpr int M = 64;
#define BPS_RES_CASE(PP) \
    case PP: launch_res<M, PP>(batch, ld, nsteps, sigma, mode, e0, e1, e2, rr, cf, x, parts, st); break;
    switch (rc.P1) {
    BPS_RES_CASE(2) BPS_RES_CASE(3) BPS_RES_CASE(4) BPS_RES_CASE(5) BPS_RES_CASE(6)
    BPS_RES_CASE(7) BPS_RES_CASE(8) BPS_RES_CASE(9) BPS_RES_CASE(10) BPS_RES_CASE(11)
    BPS_RES_CASE(12) BPS_RES_CASE(13) BPS_RES_CASE(14) BPS_RES_CASE(15) BPS_RES_CASE(16)
    BPS_RES_CASE(32) BPS_RES_CASE(64)
    default: BPS_FAIL(BPS_ENOTSUP, "unsupported chunk count");
    }
#undef BPS_RES_CASE
    BPS_LAUNCHED("k_hyper_resident");
    return BPS_OK;
}

// ---- explicit stencil of the theta scheme (streaming path) ------------------

// out[i] = e2 x[i-2] + e1 x[i-1] + e0 x[i] + e1 x[i+1] + e2 x[i+2]
//          (+ rr (phi[i-1] - 2 phi[i] + phi[i+1]), phi = x^3 - x, when CH),
// periodic in the row index, interleaved [n][ld] arrays (separate input and
// output).
template <typename T, bool CH>
__global__ void k_hyper_explicit(int64_t n, int64_t batch, int64_t ldi, int64_t ldo, T e0, T e1,
                                 T e2, T rr, const T *__restrict__ in, T *__restrict__ out)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    const T *c = in + s;
    T *o = out + s;
    T xm2 = c[(n - 2) * ldi], xm1 = c[(n - 1) * ldi], x0 = c[0], xp1 = c[ldi];
    const T first0 = x0, first1 = xp1;
    T qa = T(0), qb = T(0);     // phi of rows i-1, i
    if constexpr (CH) {
        qa = fma(xm1 * xm1, xm1, -xm1);
        qb = fma(x0 * x0, x0, -x0);
    }
    for (int64_t i = 0; i < n; ++i) {
        const T xp2 = i + 2 < n ? c[(i + 2) * ldi] : (i + 2 == n ? first0 : first1);
        T f = e2 * xm2;
        f = fma(e1, xm1, f);
        f = fma(e0, x0, f);
        f = fma(e1, xp1, f);
        f = fma(e2, xp2, f);
        if constexpr (CH) {
            const T qc = fma(xp1 * xp1, xp1, -xp1);
            f = fma(rr, fma(T(-2), qb, qa + qc), f);
            qa = qb; qb = qc;
        }
        o[i * ldo] = f;
        xm2 = xm1; xm1 = x0; x0 = xp1; xp1 = xp2;
    }
}

template <typename T>
__global__ void k_copy_interleaved(int64_t n, int64_t batch, int64_t ldi, int64_t ldo,
                                   const T *__restrict__ in, T *__restrict__ out)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    for (int64_t i = 0; i < n; ++i) out[i * ldo + s] = in[i * ldi + s];
}

template <typename T>
bps_status launch_hyper_explicit(int64_t n, int64_t batch, int64_t ldi, int64_t ldo, double e0,
                                 double e1, double e2, double rr, bool ch, const void *in,
                                 void *out, hipStream_t st)
{
    const dim3 grid(unsigned((batch + 255) / 256)), block(256);
    if (ch)
        hipLaunchKernelGGL((k_hyper_explicit<T, true>), grid, block, 0, st, n, batch, ldi, ldo,
                           T(e0), T(e1), T(e2), T(rr), (const T *)in, (T *)out);
    else
        hipLaunchKernelGGL((k_hyper_explicit<T, false>), grid, block, 0, st, n, batch, ldi, ldo,
                           T(e0), T(e1), T(e2), T(rr), (const T *)in, (T *)out);
    BPS_LAUNCHED("k_hyper_explicit");
    return BPS_OK;
}

template <typename T>
bps_status launch_copy_interleaved(int64_t n, int64_t batch, int64_t ldi, int64_t ldo,
                                   const void *in, void *out, hipStream_t st)
{
    hipLaunchKernelGGL((k_copy_interleaved<T>), dim3(unsigned((batch + 255) / 256)), dim3(256), 0,
                       st, n, batch, ldi, ldo, (const T *)in, (T *)out);
    BPS_LAUNCHED("k_copy_interleaved");
    return BPS_OK;
}

#define BPS_INST(T)                                                                             \
    template bps_status launch_hyper_explicit<T>(int64_t, int64_t, int64_t, int64_t, double,     \
                                                 double, double, double, bool, const void *,     \
                                                 void *, hipStream_t);                            \
    template bps_status launch_copy_interleaved<T>(int64_t, int64_t, int64_t, int64_t,          \
                                                   const void *, void *, hipStream_t);
BPS_INST(float)
BPS_INST(double)
#undef BPS_INST

}  // namespace bps
