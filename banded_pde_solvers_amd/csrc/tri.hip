// tri.hip -- batched tridiagonal systems with per-system coefficients
// (the Hines page, section 4.1: the Thomas algorithm and cuThomasBatch, one
// system per thread on the interleaved layout), for gfx950.
//
// Thomas on one lane per system must write c' of every row and read it back
// (a 16-byte-per-row round trip in fp64 on top of the 32 bytes in and 8 out),
// and a batch of a few thousand systems fills only a few percent of the
// chip.  For n = 16 P (2 <= P <= 64) each system is instead split into P
// chunks of 16 rows, one lane per chunk:
//
//   rows 0 .. 14 of a chunk ("interior") form a tridiagonal block E_j that
//   couples to the previous chunk's last row (the interface unknown
//   xI_{j-1}, through its row 0 entry a_0) and to its own last row (xI_j,
//   through its row 14 entry c_14).  With the Thomas factors of E_j,
//     y = R^{-1} (g - xI_{j-1} gv) with y_15 = xI_j,   g = L^{-1} f,
//     gv = L^{-1} (a_0 e_0),  R unit upper bidiagonal with c'_i above,
//   the last interior row is y_14 = g_14 - xI_{j-1} gv_14 - c'_14 xI_j and
//   the first is y_0 = z0 - xI_{j-1} p0 - xI_j q0 with z0 = w . g,
//   p0 = w . gv, q0 = w_14 c'_14, w = R^{-T} e_0 (w_0 = 1,
//   w_i = -c'_{i-1} w_{i-1}).  Each interface row then reads
//     L_j xI_{j-1} + D_j xI_j + U_j xI_{j+1} = R_j,
//     L_j = -a gv_14,  D_j = b - a c'_14 - c p0_{j+1},  U_j = -c q0_{j+1},
//     R_j = f - a g_14 - c z0_{j+1}   (a, b, c, f of the interface row),
//   a scalar tridiagonal system over the chunks, solved by parallel cyclic
//   reduction through LDS (ceil(log2 P) steps).  Each lane keeps c', g and
//   gv of its rows in registers and back-substitutes once xI is known: the
//   four inputs are read once and the solution written once.
// A system whose chunked elimination meets a zero or non-finite pivot is
// re-solved in the same launch by the sequential Thomas algorithm, so info
// and the result are those of the page's method.
#include "common.h"
#include "kernels.h"

namespace bps {

// Thomas on one system (column s already applied to the pointers): c' to
// work (n x ld), y' then the solution in place of y.  Returns 1 + the first
// row whose pivot is zero or not finite, 0 when there is none.  a_0 and
// c_{n-1} lie outside the matrix and are not read.
template <typename T>
__device__ int32_t seq_thomas(int64_t n, int64_t ld, const T *A, const T *B, const T *C, T *Y,
                              T *work)
{
    int32_t bad = 0;
    T cpp = 0, yp = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t o = i * ld;
        const T ai = i > 0 ? A[o] : T(0);
        const T ci = i + 1 < n ? C[o] : T(0);
        const T den = B[o] - cpp * ai;
        if (!bad && bad_pivot(den)) bad = int32_t(i) + 1;
        const T r = T(1) / den;
        const T cp = ci * r;
        const T yv = (Y[o] - yp * ai) * r;
        work[o] = cp;
        Y[o] = yv;
        cpp = cp; yp = yv;
    }
    T un = 0;
    for (int64_t i = n - 1; i >= 0; --i) {
        const int64_t o = i * ld;
        const T v = (i + 1 < n) ? Y[o] - work[o] * un : Y[o];
        Y[o] = v;
        un = v;
    }
    return bad;
}

// cuThomasBatch: one lane per system on the interleaved layout.
template <typename T>
__global__ void __launch_bounds__(256)
k_tri_thomas(int64_t n, int64_t batch, int64_t ld, const T *__restrict__ A,
             const T *__restrict__ B, const T *__restrict__ C, T *__restrict__ Y,
             T *__restrict__ work, int32_t *__restrict__ info)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    const int32_t r = seq_thomas<T>(n, ld, A + s, B + s, C + s, Y + s, work + s);
    if (info) info[s] = r;
}

// Rows of an interface system assembled on load (the partitioned path's
// partial interface rows, see k_tri_part_fwd): with Lp, Dp, cI, Rp of row r
// in A, B, C, Y and z0, p0, q0 of the next chunk in Z0, P0, Q0 (row r + 1),
//   a_r = Lp,  b_r = Dp - cI p0,  c_r = -cI q0,  f_r = Rp - cI z0.
template <typename T>
struct TriAssemble {
    const T *Z0, *P0, *Q0;
};

// One workgroup holds S systems x P chunks of M rows (lane = chunk j of
// system sl); n = P * M, P * S <= 512.  Dynamic LDS: 4 * P * S values of T
// + S flags.  ASM: the rows are assembled on load (TriAssemble); a system
// whose chunked elimination breaks down is then only reported (info 1), for
// the caller to re-solve from its own inputs.
template <typename T, int M, int S, bool ASM>
__global__ void __launch_bounds__(512)
k_tri_chunk(int P, int64_t batch, int64_t ld, const T *__restrict__ A, const T *__restrict__ B,
            const T *__restrict__ C, T *__restrict__ Y, T *__restrict__ work,
            int32_t *__restrict__ info, TriAssemble<T> asmb)
{
    constexpr int m = M - 1;            // interior rows of a chunk
    extern __shared__ unsigned char lds_raw[];
    T *buf = reinterpret_cast<T *>(lds_raw);          // [field][P][S]
    int32_t *flag = reinterpret_cast<int32_t *>(buf + 4 * P * S);
    const int tid = threadIdx.x;
    if (tid < S) flag[tid] = 0;
    const int j = tid / S, sl = tid % S;
    // workgroups are dispatched round-robin over the 8 XCDs: the ones one
    // XCD runs back to back take neighbouring systems, so that a 128-byte
    // line shared by two workgroups is fetched once, through one L2
    const unsigned nb = gridDim.x, bid = blockIdx.x, full = nb & ~7u;
    const unsigned tile = bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
    const int64_t s = int64_t(tile) * S + sl;
    const bool act = s < batch;
    // lanes past the end of the batch shadow the last system (identical
    // values, identical stores, no branches around memory operations)
    const int64_t off = (act ? s : batch - 1) + int64_t(j) * M * ld;
    const T *pa = A + off, *pb = B + off, *pc = C + off;
    T *py = Y + off;
    auto F = [&](int field, int jj) -> T & { return buf[(field * P + jj) * S + sl]; };
    const bool first_chunk = (j == 0), last_chunk = (j == P - 1);

    // ---- forward sweep over the interior, inputs streamed LA rows ahead ----
    constexpr int LA = 4;
    T qa[LA], qb[LA], qc[LA], qy[LA];
    // ASM: z0, p0, q0 of the row after each ring row (the last row of the
    // system has none: its cI is zero, and its own values stand in)
    T qz[ASM ? LA : 1], qp[ASM ? LA : 1], qq[ASM ? LA : 1];
    const T *pz = nullptr, *pp = nullptr, *pq = nullptr;
    if constexpr (ASM) {
        const int64_t noff = off + ld;
        pz = asmb.Z0 + noff; pp = asmb.P0 + noff; pq = asmb.Q0 + noff;
    }
    auto load_row = [&](int k, int i) {
        const int64_t o = int64_t(i) * ld;
        qa[k] = pa[o]; qb[k] = pb[o]; qc[k] = pc[o]; qy[k] = py[o];
        if constexpr (ASM) {
            const int64_t on = (last_chunk && i == M - 1) ? o - ld : o;
            qz[k] = pz[on]; qp[k] = pp[on]; qq[k] = pq[on];
        }
    };
    // row entries a, b, c, f of ring slot k
    auto row = [&](int k, T &a, T &b, T &c, T &f) {
        if constexpr (ASM) {
            a = qa[k]; b = qb[k] - qc[k] * qp[k]; c = -qc[k] * qq[k]; f = qy[k] - qc[k] * qz[k];
        } else {
            a = qa[k]; b = qb[k]; c = qc[k]; f = qy[k];
        }
    };
#pragma unroll
    for (int k = 0; k < LA; ++k) load_row(k, k);
    T cp[m], g[m], gv[m];
    T cpp = 0, gp = 0, gvp = 0, w = 1, z0 = 0, p0 = 0;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < m; ++i) {
        const int k = i % LA;
        T a_i, b_i, c_i, f_i;
        row(k, a_i, b_i, c_i, f_i);
        load_row(k, i + LA < M ? i + LA : M - 1);
        const T ai = (i > 0) ? a_i : T(0);                         // entry of E_j
        const T al = (i == 0 && !first_chunk) ? a_i : T(0);         // coupling to xI_{j-1}
        const T den = b_i - cpp * ai;
        bad |= bad_pivot(den);
        const T r = T(1) / den;
        const T cpi = c_i * r;          // row m-1: the coupling to xI_j
        const T gi = (f_i - ai * gp) * r;
        const T gvi = (al - ai * gvp) * r;
        if (i > 0) w = -cpp * w;
        z0 += w * gi;
        p0 += w * gvi;
        cp[i] = cpi; g[i] = gi; gv[i] = gvi;
        cpp = cpi; gp = gi; gvp = gvi;
    }
    const T q0 = w * cp[m - 1];
    constexpr int kI = m % LA;          // the interface row (local row m)
    T aI, bI, cI, fI;
    row(kI, aI, bI, cI, fI);
    if (last_chunk) cI = T(0);

    // ---- publish first-row quantities; build interface row j ----
    F(0, j) = z0; F(1, j) = p0; F(2, j) = q0;
    __syncthreads();
    T nz0 = 0, np0 = 0, nq0 = 0;
    if (!last_chunk) { nz0 = F(0, j + 1); np0 = F(1, j + 1); nq0 = F(2, j + 1); }
    T Lj = -aI * gv[m - 1];
    T Dj = bI - aI * cp[m - 1] - cI * np0;
    T Uj = -cI * nq0;
    T Rj = fI - aI * g[m - 1] - cI * nz0;
    __syncthreads();
    // ---- parallel cyclic reduction across the P chunks of the system ----
    for (int h = 1; h < P; h <<= 1) {
        bad |= bad_pivot(Dj);
        F(0, j) = Lj; F(1, j) = T(1) / Dj; F(2, j) = Uj; F(3, j) = Rj;
        __syncthreads();
        T nL = 0, nU = 0, nD = Dj, nR = Rj;
        if (j - h >= 0) {
            const int q = j - h;
            const T al = -Lj * F(1, q);
            nL = al * F(0, q);
            nD += al * F(2, q);
            nR += al * F(3, q);
        }
        if (j + h < P) {
            const int q = j + h;
            const T be = -Uj * F(1, q);
            nU = be * F(2, q);
            nD += be * F(0, q);
            nR += be * F(3, q);
        }
        Lj = nL; Uj = nU; Dj = nD; Rj = nR;
        __syncthreads();
    }
    bad |= bad_pivot(Dj);
    const T xI = Rj / Dj;
    F(0, j) = xI;
    if (bad) atomicOr(&flag[sl], 1);
    __syncthreads();
    const T xL = first_chunk ? T(0) : F(0, j - 1);
    if (flag[sl]) {
        // an interior pivot or a reduced diagonal broke down: redo this
        // system with the sequential algorithm, which also sets info (ASM:
        // report it; the caller redoes the system it came from)
        if (first_chunk && act) {
            if constexpr (ASM) {
                info[s] = 1;
            } else {
                const int32_t r = seq_thomas<T>(int64_t(P) * M, ld, A + s, B + s, C + s, Y + s, work + s);
                if (info) info[s] = r;
            }
        }
        return;
    }
    if (first_chunk && act && info) info[s] = 0;
    // ---- back substitution y_i = g_i - xI_{j-1} gv_i - c'_i y_{i+1} ----
    T yn = xI;
#pragma unroll
    for (int i = m - 1; i >= 0; --i) {
        const T v = g[i] - gv[i] * xL - cp[i] * yn;
        py[int64_t(i) * ld] = v;
        yn = v;
    }
    py[int64_t(m) * ld] = xI;
}

// Rows per chunk of the chunked path, 0 when it does not apply: n = P * M
// with M = 16 (else 12) and 2 <= P <= 64.
int tri_rows(int64_t n)
{
    for (const int M : {16, 12})
        if (n % M == 0 && n / M >= 2 && n / M <= 64) return M;
    return 0;
}

// ---- partitioned path for long systems (n = 16 P, P > 64) ------------------
//
// The same chunk algebra as k_tri_chunk, with the chunks of a system spread
// over many workgroups (a wavefront holds 64 neighbouring systems at the same
// chunk, so every row access is a contiguous 512-byte segment):
//   1. k_tri_part_fwd: Thomas over each chunk interior, then the chunk's
//      interface row as far as the chunk itself determines it (L_j and the
//      parts of D_j, R_j without the next chunk, and its c), and z0, p0, q0;
//   2. the interface system (P unknowns per system): by k_tri_chunk, which
//      adds the next chunk's terms to each row as it loads it, when P suits
//      it; otherwise k_tri_part_iface completes the rows in place and
//      launch_tri_solve solves them (recursively for long interfaces);
//   3. k_tri_part_back: each chunk's forward sweep again, now with the left
//      interface value known, and its back substitution;
//   4. k_tri_part_rescue: the sequential algorithm for systems whose chunk
//      or interface elimination met a bad pivot (it also writes info).
// HBM: the four inputs twice, the solution once, about 11 values per chunk.
constexpr int kPartM = 16;

int tri_part_chunks(int64_t n)
{
    if (n % kPartM != 0) return 0;
    const int64_t P = n / kPartM;
    return (P > 64 && P <= 65535) ? int(P) : 0;    // the chunk index is blockIdx.y
}

// Per chunk: Thomas over the interior, then the interface row's partial
// entries Lp = -a gv, Dp = b - a c', Rp = f - a g and its c (cI, zero for
// the last chunk) into lo, di, rh, up, and the first-row quantities z0, p0,
// q0 into summ ([3][P][ld]); the next chunk's z0, p0, q0 complete the row.
template <typename T>
__global__ void __launch_bounds__(256)
k_tri_part_fwd(int P, int64_t batch, int64_t ld, const T *__restrict__ A, const T *__restrict__ B,
               const T *__restrict__ C, const T *__restrict__ Y, T *__restrict__ summ,
               T *__restrict__ lo, T *__restrict__ di, T *__restrict__ up, T *__restrict__ rh,
               int32_t *__restrict__ flag)
{
    constexpr int M = kPartM, m = M - 1;
    const int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int j = int(blockIdx.y);
    if (s >= batch) return;
    const int64_t off = s + int64_t(j) * M * ld;
    const T *pa = A + off, *pb = B + off, *pc = C + off, *py = Y + off;
    T cpp = 0, gp = 0, gvp = 0, w = 1, z0 = 0, p0 = 0;
    bool bad = false;
#pragma unroll
    for (int i = 0; i < m; ++i) {
        const int64_t o = int64_t(i) * ld;
        const T a_i = pa[o], b_i = pb[o], c_i = pc[o], f_i = py[o];
        const T ai = (i > 0) ? a_i : T(0);
        const T al = (i == 0 && j > 0) ? a_i : T(0);
        const T den = b_i - cpp * ai;
        bad |= bad_pivot(den);
        const T r = T(1) / den;
        const T cpi = c_i * r;
        const T gi = (f_i - ai * gp) * r;
        const T gvi = (al - ai * gvp) * r;
        if (i > 0) w = -cpp * w;
        z0 += w * gi;
        p0 += w * gvi;
        cpp = cpi; gp = gi; gvp = gvi;
    }
    const int64_t mo = int64_t(m) * ld;
    const T aI = pa[mo], bI = pb[mo], fI = py[mo];
    const T cI = (j == P - 1) ? T(0) : pc[mo];
    const int64_t so = int64_t(P) * ld, o = int64_t(j) * ld + s;
    lo[o] = -aI * gvp;
    di[o] = bI - aI * cpp;
    rh[o] = fI - aI * gp;
    up[o] = cI;
    summ[o] = z0; summ[so + o] = p0; summ[2 * so + o] = w * cpp;
    if (bad) flag[s] = 1;
}

// Completes interface row j in place (when the interface system is not
// solved by the assembling chunk kernel): D_j = Dp - cI p0_{j+1},
// U_j = -cI q0_{j+1}, R_j = Rp - cI z0_{j+1}; L_j = Lp is final already.
template <typename T>
__global__ void __launch_bounds__(256)
k_tri_part_iface(int P, int64_t batch, int64_t ld, const T *__restrict__ summ,
                 T *__restrict__ di, T *__restrict__ up, T *__restrict__ rh)
{
    const int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int j = int(blockIdx.y);
    if (s >= batch) return;
    const int64_t so = int64_t(P) * ld, o = int64_t(j) * ld + s;
    const T cI = up[o];
    T nz0 = 0, np0 = 0, nq0 = 0;
    if (j < P - 1) {
        nz0 = summ[o + ld]; np0 = summ[so + o + ld]; nq0 = summ[2 * so + o + ld];
    }
    di[o] = di[o] - cI * np0;
    up[o] = -cI * nq0;
    rh[o] = rh[o] - cI * nz0;
}

template <typename T>
__global__ void __launch_bounds__(256)
k_tri_part_back(int P, int64_t batch, int64_t ld, const T *__restrict__ A, const T *__restrict__ B,
                const T *__restrict__ C, T *__restrict__ Y, const T *__restrict__ xI,
                const int32_t *__restrict__ flag, const int32_t *__restrict__ info2)
{
    constexpr int M = kPartM, m = M - 1;
    const int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int j = int(blockIdx.y);
    if (s >= batch) return;
    if (flag[s] || info2[s]) return;          // left to the sequential rescue
    const T xL = j > 0 ? xI[int64_t(j - 1) * ld + s] : T(0);
    const T xR = xI[int64_t(j) * ld + s];
    const int64_t off = s + int64_t(j) * M * ld;
    const T *pa = A + off, *pb = B + off, *pc = C + off;
    T *py = Y + off;
    T cp[m], g[m];
    T cpp = 0, gp = 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
        const int64_t o = int64_t(i) * ld;
        const T a_i = pa[o], b_i = pb[o], c_i = pc[o], f_i = py[o];
        const T ai = (i > 0) ? a_i : T(0);
        const T fi = (i == 0 && j > 0) ? f_i - a_i * xL : f_i;
        const T r = T(1) / (b_i - cpp * ai);
        cp[i] = c_i * r;
        g[i] = (fi - ai * gp) * r;
        cpp = cp[i]; gp = g[i];
    }
    T yn = xR;
#pragma unroll
    for (int i = m - 1; i >= 0; --i) {
        yn = g[i] - cp[i] * yn;
        py[int64_t(i) * ld] = yn;
    }
    py[int64_t(m) * ld] = xR;
}

template <typename T>
__global__ void __launch_bounds__(256)
k_tri_part_rescue(int64_t n, int64_t batch, int64_t ld, const T *__restrict__ A,
                  const T *__restrict__ B, const T *__restrict__ C, T *__restrict__ Y,
                  T *__restrict__ work, const int32_t *__restrict__ flag,
                  const int32_t *__restrict__ info2, int32_t *__restrict__ info)
{
    const int64_t s = lane_id();
    if (s >= batch) return;
    int32_t r = 0;
    if (flag[s] || info2[s]) r = seq_thomas<T>(n, ld, A + s, B + s, C + s, Y + s, work + s);
    if (info) info[s] = r;
}

__global__ void k_tri_fill_zero(int64_t count, int32_t *__restrict__ p)
{
    const int64_t i = lane_id();
    if (i < count) p[i] = 0;
}

// Work of a solve of n rows (bytes).  Partitioned path (values of T unless
// noted): [n ld: c' of the rescue] [3 P ld: z0, p0, q0 of the chunks]
// [4 P ld: interface rows] [ld int32: flags] [ld int32: info of the
// interface solve] [the work of the interface solve, P rows]; other paths:
// n ld values.
size_t tri_work_bytes_es(int64_t n, int64_t ld, size_t es)
{
    if (const int P = tri_part_chunks(n))
        return size_t(n + 7 * int64_t(P)) * size_t(ld) * es + 2 * size_t(ld) * sizeof(int32_t) +
               tri_work_bytes_es(P, ld, es);
    return size_t(n) * size_t(ld) * es;
}

template <typename T, int M, int S, bool ASM>
static void launch_chunk(int P, int64_t batch, int64_t ld, const void *a, const void *b,
                         const void *c, void *y, void *work, int32_t *info, TriAssemble<T> asmb,
                         hipStream_t st)
{
    const size_t lds = size_t(4) * P * S * sizeof(T) + S * sizeof(int32_t);
    const dim3 grid(unsigned((batch + S - 1) / S)), block(unsigned(P * S));
    hipLaunchKernelGGL((k_tri_chunk<T, M, S, ASM>), grid, block, lds, st, P, batch, ld,
                       (const T *)a, (const T *)b, (const T *)c, (T *)y, (T *)work, info, asmb);
}

template <typename T, int M, bool ASM = false>
static void launch_chunk_m(int P, int64_t batch, int64_t ld, const void *a, const void *b,
                           const void *c, void *y, void *work, int32_t *info, hipStream_t st,
                           TriAssemble<T> asmb = {})
{
    // 16 systems per workgroup (a 128-byte row segment in fp64), 32 for
    // short systems so that a workgroup fills a wavefront, 8 for long ones
    // so that it stays within 512 lanes.  fp64 at 32 chunks: 8 systems (256
    // lanes, three workgroups per CU at 168 VGPRs instead of one of 512)
    // measured 4% faster; fp32 loses with 32-byte rows.
    if (P < 4) launch_chunk<T, M, 32, ASM>(P, batch, ld, a, b, c, y, work, info, asmb, st);
    else if (P < 32 || (P == 32 && sizeof(T) == 4))
        launch_chunk<T, M, 16, ASM>(P, batch, ld, a, b, c, y, work, info, asmb, st);
    else launch_chunk<T, M, 8, ASM>(P, batch, ld, a, b, c, y, work, info, asmb, st);
}

template <typename T>
static bps_status launch_tri_part(int P, int64_t batch, int64_t ld, const T *a, const T *b,
                                  const T *c, T *y, void *work, int32_t *info, hipStream_t st)
{
    const int64_t n = int64_t(P) * kPartM, pl = int64_t(P) * ld;
    T *w0 = static_cast<T *>(work);
    T *summ = w0 + n * ld;
    T *lo = summ + 3 * pl, *di = lo + pl, *up = di + pl, *rh = up + pl;
    int32_t *flag = reinterpret_cast<int32_t *>(rh + pl);
    int32_t *info2 = flag + ld;
    void *iw = info2 + ld;          // 8-byte aligned: 2 ld int32 above
    const dim3 blk(256), grid2(unsigned((batch + 255) / 256), unsigned(P));
    const dim3 grid1(unsigned((batch + 255) / 256));
    hipLaunchKernelGGL(k_tri_fill_zero, grid1, blk, 0, st, batch, flag);
    hipLaunchKernelGGL((k_tri_part_fwd<T>), grid2, blk, 0, st, P, batch, ld, a, b, c, y, summ, lo,
                       di, up, rh, flag);
    if (const int MI = tri_rows(P)) {
        // the interface system goes to the chunk kernel, which completes its
        // rows as it loads them; a breakdown there re-solves the whole system
        // below (info2 = 1)
        const TriAssemble<T> asmb{summ, summ + pl, summ + 2 * pl};
        if (MI == 16) launch_chunk_m<T, 16, true>(P / 16, batch, ld, lo, di, up, rh, iw, info2, st, asmb);
        else launch_chunk_m<T, 12, true>(P / 12, batch, ld, lo, di, up, rh, iw, info2, st, asmb);
    } else {
        hipLaunchKernelGGL((k_tri_part_iface<T>), grid2, blk, 0, st, P, batch, ld, summ, di, up, rh);
        bps_status r = launch_tri_solve<T>(P, batch, ld, lo, di, up, rh, iw, info2, st);
        if (r != BPS_OK) return r;
    }
    hipLaunchKernelGGL((k_tri_part_back<T>), grid2, blk, 0, st, P, batch, ld, a, b, c, y, rh, flag,
                       info2);
    hipLaunchKernelGGL((k_tri_part_rescue<T>), grid1, blk, 0, st, n, batch, ld, a, b, c, y, w0,
                       flag, info2, info);
    BPS_LAUNCHED("k_tri_part");
    return BPS_OK;
}

template <typename T>
bps_status launch_tri_solve(int64_t n, int64_t batch, int64_t ld, const void *a, const void *b,
                            const void *c, void *y, void *work, int32_t *info, hipStream_t st)
{
    if (batch == 0) return BPS_OK;
    if (const int P = tri_part_chunks(n))
        return launch_tri_part<T>(P, batch, ld, (const T *)a, (const T *)b, (const T *)c, (T *)y,
                                  work, info, st);
    if (const int M = tri_rows(n)) {
        const int P = int(n / M);
        if (M == 16) launch_chunk_m<T, 16>(P, batch, ld, a, b, c, y, work, info, st);
        else launch_chunk_m<T, 12>(P, batch, ld, a, b, c, y, work, info, st);
        BPS_LAUNCHED("k_tri_chunk");
        return BPS_OK;
    }
    hipLaunchKernelGGL((k_tri_thomas<T>), dim3(unsigned((batch + 255) / 256)), dim3(256), 0, st, n,
                       batch, ld, (const T *)a, (const T *)b, (const T *)c, (T *)y, (T *)work, info);
    BPS_LAUNCHED("k_tri_thomas");
    return BPS_OK;
}

template bps_status launch_tri_solve<float>(int64_t, int64_t, int64_t, const void *, const void *,
                                            const void *, void *, void *, int32_t *, hipStream_t);
template bps_status launch_tri_solve<double>(int64_t, int64_t, int64_t, const void *, const void *,
                                             const void *, void *, void *, int32_t *, hipStream_t);

}  // namespace bps
