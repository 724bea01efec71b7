// penta_spike.hip -- register-resident factor + solve of batched pentadiagonal
// systems with per-system coefficients (the "Rewrite" use of the cuPentBatch
// page: a new matrix every call), for gfx950.
//
// One lane per system streams every row through global memory twice (the
// back substitution needs gamma, delta and g of every row), so HBM sees the
// six inputs, the result and a 24-byte-per-row round trip.  Here each system
// is split into P chunks of M rows and one lane owns one chunk:
//
//   rows 0 .. M-3 of a chunk ("interior") form a pentadiagonal block E_j
//   that couples only to the last two rows of the previous chunk
//   ("interface" I_{j-1}, through C_L) and to its own last two rows (I_j,
//   through C_R);  eliminating the interiors leaves a block-tridiagonal
//   system with 2x2 blocks on the interfaces:
//
//     L_j xI_{j-1} + D_j xI_j + U_j xI_{j+1} = r_j,
//     D_j = A_II - B_own Z_R,j - B_next Z_L,j+1,   L_j = -B_own Z_L,j,
//     U_j = -B_next Z_R,j+1,   r_j = f_I - B_own y_j - B_next y_{j+1},
//     with y = E^{-1} f and Z = E^{-1} C (only their first / last two rows
//     are needed), and B_own / B_next the interface rows' entries on the
//     own / next interior.
//
// The lane factors E_j = L R with the page's elimination steps while the
// inputs stream in, and keeps gamma, delta, g = L^{-1} f and U_L = L^{-1} C_L
// for its rows in registers; the first two rows of E^{-1} f and E^{-1} C come
// from w_k = R^{-T} e_k dot products accumulated in the same sweep.  The
// interface system is solved by block cyclic reduction (parallel, log2 P
// steps through LDS) across the P lanes of a system, and each lane then
// back-substitutes x = R^{-1}(g - U_L xI_{j-1} - U_R xI_j) and writes it.
// HBM traffic: the 5 diagonals and f read once, x written once.
//
// Chunks are M = 16 rows where n allows, else 12 (template parameter M).
//
// Periodic systems (CYC): the wrap entries of rows 0 and 1 (a_0, b_0, a_1)
// couple chunk 0's interior to the last chunk's interface, and those of rows
// n-2 and n-1 (e_{n-2}, d_{n-1}, e_{n-1}) couple the last interface to chunk
// 0's interior: the same C_L / B_next roles as between neighbouring chunks,
// with chunk indices taken modulo P.  The interface system is then block
// tridiagonal and periodic; block cyclic reduction with indices modulo P
// (P a power of two) leaves after log2 P steps each unknown coupled only to
// itself through L_j, D_j and U_j, so xI_j = (L_j + D_j + U_j)^{-1} r_j.
#include "common.h"
#include "kernels.h"

namespace bps {


template <typename T>
struct M22 {
    T a, b, c, d;   // [[a, b], [c, d]]
};

template <typename T>
__device__ __forceinline__ M22<T> mul(const M22<T> &x, const M22<T> &y)
{
    return {x.a * y.a + x.b * y.c, x.a * y.b + x.b * y.d, x.c * y.a + x.d * y.c, x.c * y.b + x.d * y.d};
}

template <typename T>
__device__ __forceinline__ M22<T> inv(const M22<T> &x, T &det)
{
    det = x.a * x.d - x.b * x.c;
    const T r = T(1) / det;
    return {x.d * r, -x.b * r, -x.c * r, x.a * r};
}

// Sequential factor + solve of one system (the page's algorithm, one lane):
// the fallback for a system whose chunked elimination met a zero or
// non-finite pivot.  gamma and delta go to `work` (column s of two n x ld
// arrays), g overwrites f in x.  Returns the 1-based first row whose pivot
// is zero or non-finite, 0 when there is none.
template <typename T>
__device__ int32_t seq_penta_solve(int64_t n, int64_t ld, const T *A, const T *B, const T *C,
                                   const T *D, const T *E, T *x, T *work)
{
    T *wg = work, *wd = work + n * ld;
    T gam1 = 0, gam2 = 0, del1 = 0, del2 = 0, g1 = 0, g2 = 0;
    int32_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t o = i * ld;
        const T ai = i >= 2 ? A[o] : T(0), bi = i >= 1 ? B[o] : T(0);
        const T di = i + 1 < n ? D[o] : T(0), ei = i + 2 < n ? E[o] : T(0);
        const T beta = bi - ai * gam2;
        const T alpha = C[o] - ai * del2 - beta * gam1;
        if (!bad && bad_pivot(alpha)) bad = int32_t(i) + 1;
        const T r = T(1) / alpha;
        const T gm = (di - beta * del1) * r, dl = ei * r;
        const T g = (x[o] - ai * g2 - beta * g1) * r;
        wg[o] = gm; wd[o] = dl; x[o] = g;
        gam2 = gam1; gam1 = gm; del2 = del1; del1 = dl; g2 = g1; g1 = g;
    }
    T x1 = 0, x2 = 0;
    for (int64_t i = n - 1; i >= 0; --i) {
        const int64_t o = i * ld;
        const T v = x[o] - wg[o] * x1 - wd[o] * x2;
        x[o] = v;
        x2 = x1; x1 = v;
    }
    return bad;
}

// One workgroup holds S systems x P chunks of M rows (lane = chunk j of
// system sl); n = P * M, P * S <= 512.  Dynamic LDS: two buffers of
// kSpikeFields * P * S values of T (successive exchange stages alternate
// between them, so one barrier separates a stage's writes from its reads
// and none is needed after the reads) + S flags.
constexpr int kSpikeFields = 10;

// Two consecutive values of the interleaved layout (two neighbouring
// systems of one row) as one vector access.
template <typename T> struct Pair2;
template <> struct Pair2<double> { using type = double2; };
template <> struct Pair2<float> { using type = float2; };

// Value of the other lane of this lane's pair (lanes 2k and 2k+1; DPP quad
// permutation 1, 0, 3, 2: a VALU move, no LDS).
__device__ __forceinline__ int pair_swap(int v)
{
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float pair_swap(float v)
{
    return __int_as_float(pair_swap(__float_as_int(v)));
}
__device__ __forceinline__ double pair_swap(double v)
{
    const long long b = __double_as_longlong(v);
    const int lo = pair_swap(int(b & 0xffffffffll)), hi = pair_swap(int(b >> 32));
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}

// fp32: registers capped for four waves per SIMD (two 512-lane workgroups
// per CU, so that one workgroup's loads overlap the other's reduction), at
// the cost of a few spilled values; fp64 needs about twice the registers
// and runs two waves per SIMD.
//
// PAIR (ld even, arrays aligned to two values): the two lanes of a pair
// (neighbouring systems, same chunk) read rows r and r + 1 of both their
// systems with one vector access each and swap one value, so a row pair of
// an input costs one wavefront access of 2 x 8 (fp64) bytes per lane
// instead of two of 8: half the accesses through the address units, which
// the 8-byte-per-lane pattern keeps busy.
template <typename T, int M, int S, bool CYC, bool PAIR>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 4 : 2)))
k_penta_spike(int P, int64_t batch, int64_t ld, const T *__restrict__ A, const T *__restrict__ B,
              const T *__restrict__ C, const T *__restrict__ D, const T *__restrict__ E,
              T *__restrict__ x, T *__restrict__ work, int32_t *__restrict__ info,
              int32_t *__restrict__ mask)
{
    constexpr int m = M - 2;            // interior rows of a chunk
    extern __shared__ unsigned char lds_raw[];
    T *buf = reinterpret_cast<T *>(lds_raw);          // [2][field][P][S]
    int32_t *flag = reinterpret_cast<int32_t *>(buf + 2 * kSpikeFields * P * S);
    const int tid = threadIdx.x;
    if (tid < S) flag[tid] = 0;
    const int j = tid / S, sl = tid % S;
    // workgroups are dispatched round-robin over the 8 XCDs: give the ones
    // that one XCD runs back to back neighbouring systems, so that a
    // 128-byte line shared by two workgroups (row segments of 64 bytes or
    // less) is fetched once, through one L2
    const unsigned nb = gridDim.x, bid = blockIdx.x, full = nb & ~7u;
    const unsigned tile = bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
    const int64_t s = int64_t(tile) * S + sl;
    const bool act = s < batch;
    // lanes past the end of the batch shadow the last system (identical
    // values, identical stores, no branches around memory operations)
    const int64_t se = act ? s : batch - 1;
    const int64_t off = se + int64_t(j) * M * ld;
    const T *pa = A + off, *pb = B + off, *pc = C + off, *pd = D + off, *pe = E + off;
    T *px = x + off;
    // pair access: this lane reads row r + (sl & 1) of the column pair that
    // holds its system and keeps the value of its own column (cp) of both
    // rows; a shadow lane keeps the column of the system it shadows
    using T2 = typename Pair2<T>::type;
    const int par = sl & 1, cp = int(se & 1);
    const int cpp = PAIR ? pair_swap(cp) : 0;            // the other lane's column
    const int64_t off2 = (se & ~int64_t(1)) + (int64_t(j) * M + par) * ld;
    auto pair_row = [&](const T *base, int r0, T &v0, T &v1) {
        const T2 v = *reinterpret_cast<const T2 *>(base + off2 + int64_t(r0) * ld);
        const T recv = pair_swap(cpp ? v.y : v.x);
        const T mine = cp ? v.y : v.x;
        v0 = par ? recv : mine;                          // row r0
        v1 = par ? mine : recv;                          // row r0 + 1
    };
    auto F = [&](int bb, int field, int jj) -> T & {
        return buf[((bb * kSpikeFields + field) * P + jj) * S + sl];
    };

    // ---- forward sweep over the interior, inputs streamed LA rows ahead ----
    constexpr int LA = 4;
    T qa[LA], qb[LA], qc[LA], qd[LA], qe[LA], qf[LA];
    // rows r0, r0 + 1 (r0 even) into their ring slots
    auto load_pair = [&](int r0) {
        const int k0 = r0 % LA, k1 = (r0 + 1) % LA;
        pair_row(A, r0, qa[k0], qa[k1]); pair_row(B, r0, qb[k0], qb[k1]);
        pair_row(C, r0, qc[k0], qc[k1]); pair_row(D, r0, qd[k0], qd[k1]);
        pair_row(E, r0, qe[k0], qe[k1]); pair_row(x, r0, qf[k0], qf[k1]);
    };
    if constexpr (PAIR) {
        load_pair(0);
        load_pair(2);
    } else {
#pragma unroll
        for (int k = 0; k < LA; ++k) {
            const int64_t o = int64_t(k) * ld;
            qa[k] = pa[o]; qb[k] = pb[o]; qc[k] = pc[o]; qd[k] = pd[o]; qe[k] = pe[o]; qf[k] = px[o];
        }
    }
    T gam[m], del[m], g[m], u0[m], u1[m];
    T gam1 = 0, gam2 = 0, del1 = 0, del2 = 0;      // factors of the two previous rows
    T w01 = 0, w02 = 0, w11 = 0, w12 = 0;          // w_0, w_1 at rows i-1, i-2
    T t0 = 0, t1 = 0, q00 = 0, q01 = 0, q10 = 0, q11 = 0;
    T aL0 = 0, bL0 = 0, aL1 = 0;                   // C_L entries (rows 0, 1)
    T rcp_m2 = 0, rcp_m1 = 0, beta_m1 = 0;
    T eC0 = 0, dC1 = 0, eC1 = 0;                   // C_R entries (rows m-2, m-1)
    bool bad = false;
    // the chunk before the first one is the last one for a periodic system
    const bool first_chunk = (j == 0) && !CYC;
#pragma unroll
    for (int i = 0; i < m; ++i) {
        const int k = i % LA;
        const T a_i = qa[k], b_i = qb[k], c_i = qc[k], d_i = qd[k], e_i = qe[k], f_i = qf[k];
        if constexpr (PAIR) {
            // both rows of the slot pair consumed: fetch the pair LA rows on
            if ((i & 1) && i - 1 + LA < M) load_pair(i - 1 + LA);
        } else {
            const int64_t o = int64_t(i + LA < M ? i + LA : M - 1) * ld;
            qa[k] = pa[o]; qb[k] = pb[o]; qc[k] = pc[o]; qd[k] = pd[o]; qe[k] = pe[o]; qf[k] = px[o];
        }
        // entries of E_j; the others are couplings to the interfaces
        const T ai = (i >= 2) ? a_i : T(0);
        const T bi = (i >= 1) ? b_i : T(0);
        const T di = (i + 1 < m) ? d_i : T(0);
        const T ei = (i + 2 < m) ? e_i : T(0);
        if (i == 0) { aL0 = first_chunk ? T(0) : a_i; bL0 = first_chunk ? T(0) : b_i; }
        if (i == 1) aL1 = first_chunk ? T(0) : a_i;
        if (i == m - 2) eC0 = e_i;
        if (i == m - 1) { dC1 = d_i; eC1 = e_i; }
        const T beta = bi - ai * gam2;
        const T alpha = c_i - ai * del2 - beta * gam1;
        bad |= bad_pivot(alpha);
        const T r = T(1) / alpha;
        const T gm = (di - beta * del1) * r;
        const T dl = ei * r;
        const T gi = (f_i - ai * (i >= 2 ? g[i - 2] : T(0)) - beta * (i >= 1 ? g[i - 1] : T(0))) * r;
        // U_L = L^{-1} C_L (right-hand sides nonzero in rows 0, 1 only)
        const T cl0 = (i == 0) ? aL0 : T(0);
        const T cl1 = (i == 0) ? bL0 : (i == 1) ? aL1 : T(0);
        const T ui0 = (cl0 - ai * (i >= 2 ? u0[i - 2] : T(0)) - beta * (i >= 1 ? u0[i - 1] : T(0))) * r;
        const T ui1 = (cl1 - ai * (i >= 2 ? u1[i - 2] : T(0)) - beta * (i >= 1 ? u1[i - 1] : T(0))) * r;
        // w_k = R^{-T} e_k: rows 0 and 1 of R^{-1}
        const T w0 = T(i == 0 ? 1 : 0) - gam1 * w01 - del2 * w02;
        const T w1 = T(i == 1 ? 1 : 0) - gam1 * w11 - del2 * w12;
        t0 += w0 * gi; t1 += w1 * gi;
        q00 += w0 * ui0; q01 += w0 * ui1; q10 += w1 * ui0; q11 += w1 * ui1;
        gam[i] = gm; del[i] = dl; g[i] = gi; u0[i] = ui0; u1[i] = ui1;
        if (i == m - 2) rcp_m2 = r;
        if (i == m - 1) { rcp_m1 = r; beta_m1 = beta; }
        gam2 = gam1; gam1 = gm; del2 = del1; del1 = dl;
        w02 = w01; w01 = w0; w12 = w11; w11 = w1;
    }
    // U_R = L^{-1} C_R: nonzero in the last two rows only
    const T urA = eC0 * rcp_m2;                    // row m-2, column 0
    const T urB = (dC1 - beta_m1 * urA) * rcp_m1;  // row m-1, column 0
    const T urC = eC1 * rcp_m1;                    // row m-1, column 1
    // last two rows of y = E^{-1} f, Z_L = E^{-1} C_L, Z_R = E^{-1} C_R
    const T yl1 = g[m - 1], yl0 = g[m - 2] - gam[m - 2] * yl1;
    const T zl01 = u0[m - 1], zl00 = u0[m - 2] - gam[m - 2] * zl01;   // column 0, rows m-2, m-1
    const T zl11 = u1[m - 1], zl10 = u1[m - 2] - gam[m - 2] * zl11;   // column 1
    const T zr01 = urB, zr00 = urA - gam[m - 2] * zr01;
    const T zr11 = urC, zr10 = -gam[m - 2] * zr11;
    // first two rows: y_k = w_k . g, Z_L[k][c] = w_k . U_L[c], Z_R[k][c] = w_k . U_R[c]
    const T fr00 = w02 * urA + w01 * urB, fr01 = w01 * urC;       // w_0 at rows m-2 (w02), m-1 (w01)
    const T fr10 = w12 * urA + w11 * urB, fr11 = w11 * urC;
    // interface rows of this chunk (local rows m, m+1)
    constexpr int kR0 = m % LA, kR1 = (m + 1) % LA;
    const bool last_chunk = (j == P - 1) && !CYC;
    const int jn = (j + 1 == P) ? 0 : j + 1, jp = (j == 0) ? P - 1 : j - 1;
    const T aR0 = qa[kR0], bR0 = qb[kR0], cR0 = qc[kR0], dR0 = qd[kR0];
    const T eR0 = last_chunk ? T(0) : qe[kR0], fR0 = qf[kR0];
    const T aR1 = qa[kR1], bR1 = qb[kR1], cR1 = qc[kR1];
    const T dR1 = last_chunk ? T(0) : qd[kR1], eR1 = last_chunk ? T(0) : qe[kR1], fR1 = qf[kR1];

    // ---- publish first-row quantities; build block row j ----
    F(0, 0, j) = t0; F(0, 1, j) = t1;
    F(0, 2, j) = q00; F(0, 3, j) = q01; F(0, 4, j) = q10; F(0, 5, j) = q11;
    F(0, 6, j) = fr00; F(0, 7, j) = fr01; F(0, 8, j) = fr10; F(0, 9, j) = fr11;
    __syncthreads();
    T ny0 = 0, ny1 = 0, nzl00 = 0, nzl01 = 0, nzl10 = 0, nzl11 = 0, nzr00 = 0, nzr01 = 0, nzr10 = 0, nzr11 = 0;
    if (!last_chunk) {
        ny0 = F(0, 0, jn); ny1 = F(0, 1, jn);
        nzl00 = F(0, 2, jn); nzl01 = F(0, 3, jn); nzl10 = F(0, 4, jn); nzl11 = F(0, 5, jn);
        nzr00 = F(0, 6, jn); nzr01 = F(0, 7, jn); nzr10 = F(0, 8, jn); nzr11 = F(0, 9, jn);
    }
    // B_own = [[aR0, bR0], [0, aR1]] on interior rows (m-2, m-1);
    // B_next = [[eR0, 0], [dR1, eR1]] on the next interior rows (0, 1)
    M22<T> Dj, Lj, Uj;
    T rj0, rj1;
    {
        const M22<T> own{aR0, bR0, T(0), aR1}, nxt{eR0, T(0), dR1, eR1};
        const M22<T> ZRl{zr00, zr10, zr01, zr11};       // rows (m-2, m-1) x columns (0, 1)
        const M22<T> ZLl{zl00, zl10, zl01, zl11};
        const M22<T> ZLn{nzl00, nzl01, nzl10, nzl11};   // next chunk rows (0, 1) x columns
        const M22<T> ZRn{nzr00, nzr01, nzr10, nzr11};
        const M22<T> p1 = mul(own, ZRl), p2 = mul(nxt, ZLn), p3 = mul(own, ZLl), p4 = mul(nxt, ZRn);
        Dj = {cR0 - p1.a - p2.a, dR0 - p1.b - p2.b, bR1 - p1.c - p2.c, cR1 - p1.d - p2.d};
        Lj = {-p3.a, -p3.b, -p3.c, -p3.d};
        Uj = {-p4.a, -p4.b, -p4.c, -p4.d};
        rj0 = fR0 - (aR0 * yl0 + bR0 * yl1) - eR0 * ny0;
        rj1 = fR1 - aR1 * yl1 - (dR1 * ny0 + eR1 * ny1);
    }
    // ---- block cyclic reduction across the P chunks of the system ----
    // Each lane publishes D_j^{-1} L_j, D_j^{-1} U_j and D_j^{-1} r_j; with
    // alpha = -L_j D_q^{-1} from the chunk q = j - h and gamma = -U_j D_q^{-1}
    // from q = j + h the reduced row is
    //   L' = -L_j (D^{-1}L)_{j-h},  U' = -U_j (D^{-1}U)_{j+h},
    //   D' = D_j - L_j (D^{-1}U)_{j-h} - U_j (D^{-1}L)_{j+h},
    //   r' = r_j - L_j (D^{-1}r)_{j-h} - U_j (D^{-1}r)_{j+h}.
    int bb = 1;                                    // stage buffer (0 held the first rows)
    for (int h = 1; h < P; h <<= 1, bb ^= 1) {
        T det;
        const M22<T> Di = inv(Dj, det);
        bad |= bad_pivot(det);
        const M22<T> IL = mul(Di, Lj), IU = mul(Di, Uj);
        F(bb, 0, j) = IL.a; F(bb, 1, j) = IL.b; F(bb, 2, j) = IL.c; F(bb, 3, j) = IL.d;
        F(bb, 4, j) = IU.a; F(bb, 5, j) = IU.b; F(bb, 6, j) = IU.c; F(bb, 7, j) = IU.d;
        F(bb, 8, j) = Di.a * rj0 + Di.b * rj1; F(bb, 9, j) = Di.c * rj0 + Di.d * rj1;
        __syncthreads();
        M22<T> nD = Dj, nL{0, 0, 0, 0}, nU{0, 0, 0, 0};
        T nr0 = rj0, nr1 = rj1;
        if (CYC || j - h >= 0) {
            const int q = (j - h) & (CYC ? P - 1 : -1);
            const M22<T> ILq{F(bb, 0, q), F(bb, 1, q), F(bb, 2, q), F(bb, 3, q)};
            const M22<T> IUq{F(bb, 4, q), F(bb, 5, q), F(bb, 6, q), F(bb, 7, q)};
            const T iq0 = F(bb, 8, q), iq1 = F(bb, 9, q);
            const M22<T> l1 = mul(Lj, ILq), l2 = mul(Lj, IUq);
            nL = {-l1.a, -l1.b, -l1.c, -l1.d};
            nD = {nD.a - l2.a, nD.b - l2.b, nD.c - l2.c, nD.d - l2.d};
            nr0 -= Lj.a * iq0 + Lj.b * iq1;
            nr1 -= Lj.c * iq0 + Lj.d * iq1;
        }
        if (CYC || j + h < P) {
            const int q = (j + h) & (CYC ? P - 1 : -1);
            const M22<T> ILq{F(bb, 0, q), F(bb, 1, q), F(bb, 2, q), F(bb, 3, q)};
            const M22<T> IUq{F(bb, 4, q), F(bb, 5, q), F(bb, 6, q), F(bb, 7, q)};
            const T iq0 = F(bb, 8, q), iq1 = F(bb, 9, q);
            const M22<T> u1 = mul(Uj, IUq), u2 = mul(Uj, ILq);
            nU = {-u1.a, -u1.b, -u1.c, -u1.d};
            nD = {nD.a - u2.a, nD.b - u2.b, nD.c - u2.c, nD.d - u2.d};
            nr0 -= Uj.a * iq0 + Uj.b * iq1;
            nr1 -= Uj.c * iq0 + Uj.d * iq1;
        }
        Dj = nD; Lj = nL; Uj = nU; rj0 = nr0; rj1 = nr1;
    }
    if (CYC) {
        // both remaining couplings refer to this chunk's own interface
        Dj = {Dj.a + Lj.a + Uj.a, Dj.b + Lj.b + Uj.b, Dj.c + Lj.c + Uj.c, Dj.d + Lj.d + Uj.d};
    }
    T det;
    const M22<T> Dinv = inv(Dj, det);
    bad |= bad_pivot(det);
    const T xr0 = Dinv.a * rj0 + Dinv.b * rj1, xr1 = Dinv.c * rj0 + Dinv.d * rj1;
    F(bb, 0, j) = xr0; F(bb, 1, j) = xr1;
    if (bad) atomicOr(&flag[sl], 1);
    __syncthreads();
    const T xl0 = first_chunk ? T(0) : F(bb, 0, jp);
    const T xl1 = first_chunk ? T(0) : F(bb, 1, jp);
    if (CYC) {
        // a breakdown leaves the system to the periodic factor + solve pass
        if (j == 0 && act) mask[s] = flag[sl];
        if (flag[sl]) return;
    } else if (flag[sl]) {
        // a chunk pivot or an interface block broke down: redo this system
        // with the sequential elimination, which also fixes info
        if (first_chunk && act) {
            const int32_t r = seq_penta_solve<T>(int64_t(P) * M, ld, A + s, B + s, C + s, D + s,
                                                 E + s, x + s, work + s);
            if (info) info[s] = r;
        }
        return;
    }
    if (j == 0 && act && info) info[s] = 0;
    // ---- back substitution x = R^{-1}(g - U_L xI_{j-1} - U_R xI_j) ----
    T x1 = 0, x2 = 0;
#pragma unroll
    for (int i = m - 1; i >= 0; --i) {
        T v = g[i] - u0[i] * xl0 - u1[i] * xl1;
        if (i == m - 2) v -= urA * xr0;
        if (i == m - 1) v -= urB * xr0 + urC * xr1;
        if (i + 1 < m) v -= gam[i] * x1;
        if (i + 2 < m) v -= del[i] * x2;
        px[int64_t(i) * ld] = v;
        x2 = x1; x1 = v;
    }
    px[int64_t(m) * ld] = xr0;
    px[int64_t(m + 1) * ld] = xr1;
}

// Rows per chunk of the chunked path, 0 when it does not apply: n = P * M
// with M = 16 (else 12) and 2 <= P <= 64; for periodic systems P must also
// be a power of two.
int spike_rows(int64_t n, bool cyclic)
{
    for (const int M : {16, 12}) {
        if (n % M != 0) continue;
        const int64_t P = n / M;
        if (P >= 2 && P <= 64 && (!cyclic || (P & (P - 1)) == 0)) return M;
    }
    return 0;
}

// Dynamic LDS of one launch: the two exchange buffers of kSpikeFields * P * S
// values each, and S int32 flags.
template <typename T, int S>
constexpr size_t spike_lds(int P)
{
    return size_t(2 * kSpikeFields) * P * S * sizeof(T) + S * sizeof(int32_t);
}
// Largest chunk count launched with S systems per workgroup (launch_spike_m).
constexpr int spike_pmax(int S) { return S == 32 ? 3 : S == 16 ? 32 : 64; }

template <typename T, int M, int S, bool CYC, bool PAIR>
static hipError_t spike_raise()
{
    constexpr size_t lds = spike_lds<T, S>(spike_pmax(S));
    if (lds <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void *)k_penta_spike<T, M, S, CYC, PAIR>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

template <typename T, int M, int S>
static hipError_t spike_raise_s()
{
    hipError_t e;
    if ((e = spike_raise<T, M, S, false, false>()) != hipSuccess) return e;
    if ((e = spike_raise<T, M, S, false, true>()) != hipSuccess) return e;
    if ((e = spike_raise<T, M, S, true, false>()) != hipSuccess) return e;
    return spike_raise<T, M, S, true, true>();
}

template <typename T, int M>
static hipError_t spike_raise_m()
{
    hipError_t e;
    if ((e = spike_raise_s<T, M, 32>()) != hipSuccess) return e;
    if ((e = spike_raise_s<T, M, 16>()) != hipSuccess) return e;
    return spike_raise_s<T, M, 8>();
}

// Every instantiation whose largest launch needs more than the default 64 KiB
// of dynamic LDS is allowed that largest amount on the current device.
hipError_t spike_prepare_device()
{
    hipError_t e;
    if ((e = spike_raise_m<double, 16>()) != hipSuccess) return e;
    if ((e = spike_raise_m<double, 12>()) != hipSuccess) return e;
    if ((e = spike_raise_m<float, 16>()) != hipSuccess) return e;
    return spike_raise_m<float, 12>();
}

template <typename T, int M, int S, bool PAIR>
static hipError_t launch_spike(int P, int64_t batch, int64_t ld, bool cyclic, const void *a,
                         const void *b, const void *c, const void *d, const void *e, void *x,
                         void *work, int32_t *info, int32_t *mask, hipStream_t st)
{
    // within the limit spike_prepare_device set for this instantiation
    const size_t lds = spike_lds<T, S>(P);
    if (P > spike_pmax(S)) return hipErrorInvalidConfiguration;
    const dim3 grid(unsigned((batch + S - 1) / S)), block(unsigned(P * S));
    if (cyclic)
        hipLaunchKernelGGL((k_penta_spike<T, M, S, true, PAIR>), grid, block, lds, st, P, batch, ld,
                           (const T *)a, (const T *)b, (const T *)c, (const T *)d, (const T *)e,
                           (T *)x, (T *)work, info, mask);
    else
        hipLaunchKernelGGL((k_penta_spike<T, M, S, false, PAIR>), grid, block, lds, st, P, batch, ld,
                           (const T *)a, (const T *)b, (const T *)c, (const T *)d, (const T *)e,
                           (T *)x, (T *)work, info, mask);
    return hipSuccess;
}

template <typename T, int M>
static hipError_t launch_spike_m(int P, int64_t batch, int64_t ld, bool cyclic, const void *a,
                           const void *b, const void *c, const void *d, const void *e, void *x,
                           void *work, int32_t *info, int32_t *mask, hipStream_t st)
{
    // 16 systems per workgroup (a 128-byte row segment in fp64, 64 in
    // fp32); 32 when the systems are short so that a workgroup fills a
    // wavefront, 8 when they are long so that it stays within 512 lanes.
    // Pair accesses need ld even and every input aligned to two values.
    const size_t al = 2 * sizeof(T);
    const bool pair = ld % 2 == 0 && aligned(a, al) && aligned(b, al) && aligned(c, al) &&
                      aligned(d, al) && aligned(e, al) && aligned(x, al);
#define BPS_SPIKE_S(SS)                                                                            \
    return pair ? launch_spike<T, M, SS, true>(P, batch, ld, cyclic, a, b, c, d, e, x, work, info,  \
                                               mask, st)                                           \
                : launch_spike<T, M, SS, false>(P, batch, ld, cyclic, a, b, c, d, e, x, work, info, \
                                                mask, st)
    if (P < 4) BPS_SPIKE_S(32);
    if (P <= 32) BPS_SPIKE_S(16);
    BPS_SPIKE_S(8);
#undef BPS_SPIKE_S
}

template <typename T>
bps_status launch_penta_spike(int64_t n, int64_t batch, int64_t ld, bool cyclic, const void *a,
                              const void *b, const void *c, const void *d, const void *e, void *x,
                              void *work, int32_t *info, int32_t *mask, hipStream_t st)
{
    const int M = spike_rows(n, cyclic);
    if (!M)
        BPS_FAIL(BPS_ENOTSUP, "chunked pentadiagonal solve needs n = 16 P or 12 P, 2 <= P <= 64 "
                              "(a power of two for periodic systems)");
    if (cyclic && !mask) BPS_FAIL(BPS_EINVAL, "periodic chunked solve needs a mask array");
    if (batch == 0) return BPS_OK;
    const int P = int(n / M);
    const hipError_t err = M == 16
        ? launch_spike_m<T, 16>(P, batch, ld, cyclic, a, b, c, d, e, x, work, info, mask, st)
        : launch_spike_m<T, 12>(P, batch, ld, cyclic, a, b, c, d, e, x, work, info, mask, st);
    if (err != hipSuccess)
        BPS_FAIL(BPS_EHIP, "k_penta_spike: %s", hipGetErrorString(err));
    BPS_LAUNCHED("k_penta_spike");
    return BPS_OK;
}

template bps_status launch_penta_spike<float>(int64_t, int64_t, int64_t, bool, const void *,
                                              const void *, const void *, const void *,
                                              const void *, void *, void *, int32_t *, int32_t *,
                                              hipStream_t);
template bps_status launch_penta_spike<double>(int64_t, int64_t, int64_t, bool, const void *,
                                               const void *, const void *, const void *,
                                               const void *, void *, void *, int32_t *, int32_t *,
                                               hipStream_t);

}  // namespace bps
