// hines_sep.hip -- Hines systems of one shared morphology, each neuron
// solved by sixteen, thirty-two or sixty-four lanes, and multi-morphology
// batches with every tree on its own lanes ([H] section 2, Algorithm 1, and the
// per-branch decomposition of section 4).
//
// A set S of single compartments ("separators") cuts the tree into
// components, each with at most one separator below it.  Given the voltages
// of S, the components are independent: every lane eliminates the
// components it was given (leaves to root, Algorithm 1 inside each
// component) and keeps q_i, m_i of its rows in registers, so that they never
// go to memory; the compartments on the path from a component's lower
// separator up to the component's root also carry the coefficient of that
// separator's voltage (the fill-in of the partitioned elimination).  The
// components' Schur complements on S form a smaller tree system (the
// voltages of S), solved by Algorithm 1 in LDS; then each lane substitutes
// its rows from the root of each component down.  Per compartment the
// kernel reads u, l, d, rhs and writes V once: 40 bytes, where one lane per
// neuron also writes and reads q, m.
//
// Workgroup: 16 neurons x 16 lanes, 8 neurons x 32 or 64 lanes, or 4
// neurons x 64 lanes.  Thread (k, j) = lane k of neuron j; a wavefront holds
// 4 lanes of 16 neighbouring neurons (every access four 128-byte row
// segments of the interleaved layout), 8 lanes of 8 (eight 64-byte halves,
// the other halves read by a workgroup on the same XCD) or 16 lanes of 4
// (32-byte quarters, the others read by three workgroups on the same XCD).
// A lane keeps its compartments' pending updates and voltages in 8 ring
// slots that the schedule assigns.
#include <algorithm>
#include <cstring>
#include <string>
#include <thread>
#include <tuple>
#include <utility>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace bps {

namespace {

constexpr int kSepNeurons = 16;     // neurons per workgroup with 16 lanes each (8 with 32, 8 or 4 with 64)
constexpr int kSepSlots = 8;        // ring of pending updates / voltages per lane
constexpr int kSepHeader = 8;

// Row code (one word): compartment (bits 0-10), its ring slot (11-13), its
// parent's slot (14-16), flags.  Components, path rows and components with
// a path are numbered in the order the lanes visit them (lane by lane), so
// a lane finds their numbers by counting from its bases.
constexpr uint32_t kSepLive = 1u << 17;   // a compartment (not padding)
constexpr uint32_t kSepPath = 1u << 18;   // on the path from a separator up to the component root
constexpr uint32_t kSepPath0 = 1u << 19;  // first row of that path (the separator's parent)
constexpr uint32_t kSepTop = 1u << 20;    // root of its component

struct SepArgs {
    int64_t batch;
    uint32_t ld8;       // ld * 8
    uint32_t bytes;     // n * ld * 8
    int32_t n, ns, nc, npc, nh;
    const int32_t *tab;         // codes [lanes][R], bases [lanes][3], separators [ns][5],
                                // components [nc][3], component list [nc]
    const int32_t *parent;      // [n] for Algorithm 1 on a neuron that breaks down
    const double *u, *l, *d;
    double *rhs, *work;
    int32_t *info;
};

struct SepBuf {
    __amdgpu_buffer_rsrc_t r;
    __device__ SepBuf(const void *base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, int(bytes), 0x00020000)) {}
    __device__ double ld(uint32_t off) const {
        return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
    __device__ void st(double v, uint32_t off) const {
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, off, 0, 0);
    }
};

constexpr uint32_t kSepNoStore = 0xFFFFFFF0u;   // beyond every descriptor: dropped

// 1 / x: the hardware estimate refined by two Newton steps (within an ulp
// or two of the quotient; zero and non-finite x give non-finite results).
__device__ __forceinline__ double recip(double x)
{
    double r = __builtin_amdgcn_rcp(x);
    r = fma(fma(-x, r, 1.0), r, r);
    return fma(fma(-x, r, 1.0), r, r);
}

// Words of the schedule's tables after the header (lanes per neuron: 16 or 32).
__host__ __device__ inline int sep_tab_words(int R, int ns, int nc, int lanes)
{
    return lanes * R + lanes * 3 + ns * 5 + nc * 4;
}

// Neuron group of a workgroup.  With NEU < 16 neurons per workgroup a
// 128-byte row segment holds G = 16 / NEU groups' values; workgroups are
// handed to the 8 XCDs in turn (block b to XCD b mod 8), so within each run
// of 8 G blocks, blocks b, b + 8, ..., b + 8 (G - 1) take groups G m, ...,
// G m + G - 1: the parts of each segment are read by one XCD's L2 at about
// the same time.  A last partial run keeps its order.
template <int NEU>
__device__ __forceinline__ int64_t sep_group(int64_t b, int64_t nblk)
{
    constexpr int G = 16 / NEU, RUN = 8 * G;
    if (G == 1 || b >= nblk / RUN * RUN) return b;
    const int64_t r = b % RUN;
    return b - r + G * (r % 8) + r / 8;
}

template <int R, int LANES, int NEU>
__global__ void __launch_bounds__(LANES * NEU) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_hines_sep(SepArgs A)
{
    constexpr int NT = LANES * NEU;   // threads: lane k = tid / NEU of neuron j = tid % NEU
    extern __shared__ __align__(16) unsigned char sep_lds[];
    const int tid = threadIdx.x, k = tid / NEU, j = tid % NEU;
    const int64_t s = sep_group<NEU>(blockIdx.x, gridDim.x) * NEU + j;
    const bool act = s < A.batch;
    // lanes past the batch shadow the last neuron (loads only)
    const uint32_t s8 = uint32_t(uint64_t(act ? s : A.batch - 1) * 8);
    const int ns = A.ns, nc = A.nc, npc = A.npc, nh = A.nh;
    double2 *ring = reinterpret_cast<double2 *>(sep_lds);     // [8][NT]
    double2 *red = ring + kSepSlots * NT;             // [nc][NEU]
    double2 *pdat = red + nc * NEU;                    // [npc][NEU][2]
    double2 *sepv = pdat + npc * 2 * NEU;              // [ns][NEU][2]
    double *su = reinterpret_cast<double *>(sepv + ns * 2 * NEU);   // [ns][NEU]
    double *hbuf = su + ns * NEU;                      // [nh + 2][NEU]
    int *badf = reinterpret_cast<int *>(hbuf + (nh + 2) * NEU);  // [NT]
    int *flag = badf + NT;                            // [NEU]
    int *tab = flag + NEU;                             // the schedule's tables
    const int *codes = tab, *bases = tab + LANES * R, *septab = bases + LANES * 3;
    const int *comptab = septab + ns * 5, *clist = comptab + nc * 3;

    const SepBuf U(A.u, A.bytes), L(A.l, A.bytes), Dg(A.d, A.bytes), Rh(A.rhs, A.bytes);
    const uint32_t ld8 = A.ld8;
    const int ntab = sep_tab_words(R, ns, nc, LANES);
    for (int i = tid; i < ntab; i += NT) tab[i] = A.tab[i];
#pragma unroll
    for (int q = 0; q < kSepSlots; ++q) ring[q * NT + tid] = make_double2(0.0, 0.0);
    if (k == 0) hbuf[nh * NEU + j] = 0.0;              // read by rows off the paths
    // the separators' own rows
    for (int i = k; i < ns; i += LANES) {
        const uint32_t o = uint32_t(A.tab[LANES * R + LANES * 3 + i * 5]) * ld8 + s8;
        const double uu = U.ld(o), ll = L.ld(o), dd = Dg.ld(o), rr = Rh.ld(o);
        su[i * NEU + j] = uu;
        sepv[(i * NEU + j) * 2] = make_double2(dd, rr);
        sepv[(i * NEU + j) * 2 + 1] = make_double2(ll, uu);
    }
    __syncthreads();

    // ---- first sweep: each component from its leaves to its root ----
    const int *code = codes + k * R;
    int ccomp = bases[k * 3], chidx = bases[k * 3 + 1], cpidx = bases[k * 3 + 2];
    double q[R], m[R];
    constexpr int D = 8;                  // rows of look-ahead
    double bu[D], bl[D], bd[D], br[D];
    auto load = [&](int t, double dep) {
        uint32_t o = uint32_t(code[t] & 2047) * ld8 + s8;
        asm volatile("" : "+v"(o) : "v"(dep));   // issue no earlier than this point
        bu[t % D] = U.ld(o); bl[t % D] = L.ld(o); bd[t % D] = Dg.ld(o); br[t % D] = Rh.ld(o);
    };
#pragma unroll
    for (int t = 0; t < D; ++t) load(t, 0.0);
    int bad = 0;
    double g = 0.0, P = 0.0, al = 0.0, ga = 0.0;   // path: spike, product of -m, sums of P q and P h
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const uint32_t w0 = uint32_t(code[t]);
        const double u_ = bu[t % D], l_ = bl[t % D], d_ = bd[t % D], r_ = br[t % D];
        const bool live = w0 & kSepLive, path = w0 & kSepPath, top = w0 & kSepTop;
        const int own = (w0 >> 11) & 7, par = (w0 >> 14) & 7;
        const double2 pd = ring[own * NT + tid];
        const double2 po = ring[par * NT + tid];
        ring[own * NT + tid] = make_double2(0.0, 0.0);
        const double dd = d_ - pd.x, rr = r_ - pd.y;
        bad |= int(live) & int(bad_pivot(dd));
        asm volatile("" : "+v"(bad));   // test each pivot now, not all of them at the end
        const double rcp = recip(dd);
        const double qq = rr * rcp, mm = l_ * rcp, fac = u_ * rcp;
        q[t] = qq;
        m[t] = mm;
        if (w0 & kSepPath0) { g = 1.0; P = 1.0; al = 0.0; ga = 0.0; }
        const double h = g * rcp;
        hbuf[(path ? chidx : nh + 1) * NEU + j] = h;
        if (path) {
            ++chidx;
            al = fma(P, qq, al);
            ga = fma(-P, h, ga);
            P = -mm * P;
            g = -fac * g;
        }
        const double2 cb = make_double2(fac * l_, fac * rr);
        if (top) {
            red[ccomp * NEU + j] = cb;
            ++ccomp;
            if (path) {
                pdat[(cpidx * NEU + j) * 2] = make_double2(g, al);
                pdat[(cpidx * NEU + j) * 2 + 1] = make_double2(P, ga);
                ++cpidx;
            }
        } else {
            const double2 o = par == own ? make_double2(0.0, 0.0) : po;
            ring[par * NT + tid] = make_double2(o.x + cb.x, o.y + cb.y);
        }
        if (t + D < R) load(t + D, qq);
    }
    badf[tid] = bad;
    __syncthreads();

    // ---- the separators' tree system ----
    // (a) every separator's row with its components' terms (all lanes)
    for (int i = k; i < ns; i += LANES) {
        const int rp = septab[i * 5 + 1], pcomp = septab[i * 5 + 2];
        const int cb = septab[i * 5 + 3], ce = septab[i * 5 + 4];
        const double2 dr = sepv[(i * NEU + j) * 2];
        const double2 lu = sepv[(i * NEU + j) * 2 + 1];
        double dh = dr.x, rh = dr.y, lh = 0.0, uh = 0.0;
        for (int c = cb; c < ce; ++c) {
            const double2 v = red[clist[c] * NEU + j];
            dh -= v.x;
            rh -= v.y;
        }
        if (pcomp >= 0) {
            // the separator meets its parent component through the path: the
            // parent compartment's voltage is al + P x_top + ga (u x_sep)
            const int pi = comptab[pcomp * 3 + 2];
            const double2 a = pdat[(pi * NEU + j) * 2];
            const double2 b = pdat[(pi * NEU + j) * 2 + 1];
            dh = fma(lu.x * lu.y, b.y, dh);
            rh = fma(-lu.x, a.y, rh);
            lh = lu.x * b.x;
            uh = lu.y * a.x;
        } else if (rp >= 0) {
            lh = lu.x;
            uh = lu.y;
        }
        sepv[(i * NEU + j) * 2] = make_double2(dh, rh);
        sepv[(i * NEU + j) * 2 + 1] = make_double2(lh, uh);
    }
    __syncthreads();
    // (b) Algorithm 1 on the separators (one lane per neuron), in place
    if (k == 0) {
        // one lane per neuron runs a serial chain while the other waves of
        // the CU run their sweeps: it takes the issue slots first
        __builtin_amdgcn_s_setprio(3);
        int anyb = 0;
        for (int kk = 0; kk < LANES; ++kk) anyb |= badf[kk * NEU + j];
        // the next separator's row is read one step ahead (two register sets
        // in turn); an update for the next separator is carried in registers,
        // others go through LDS (they reach two or more rows ahead, which
        // have not been read yet)
        double cf = 0.0, cl = 0.0, cr = 0.0;
        auto at = [&](int i) { return (i * NEU + j) * 2; };
        auto rd = [&](int i, double2 &a, double2 &b, int &r) {
            const int ii = i < ns ? i : ns - 1;
            a = sepv[at(ii)];
            b = sepv[at(ii) + 1];
            r = septab[ii * 5 + 1];
        };
        auto elim = [&](int i, const double2 dr0, const double2 lu, const int rp) {
            const double2 dr = make_double2(fma(-cf, cl, dr0.x), fma(-cf, cr, dr0.y));
            anyb |= int(bad_pivot(dr.x));
            const double rcp = recip(dr.x);
            sepv[at(i) + 1] = make_double2(dr.y * rcp, lu.x * rcp);
            cf = 0.0;
            if (rp >= 0) {
                const double f = lu.y * rcp;
                if (rp == i + 1) {
                    cf = f; cl = lu.x; cr = dr.y;
                } else {
                    const double2 o = sepv[at(rp)];
                    sepv[at(rp)] = make_double2(fma(-f, lu.x, o.x), fma(-f, dr.y, o.y));
                }
            }
        };
        double xn = 0.0;
        if (ns > 0) {
            double2 a0, b0, a1, b1;
            int r0, r1;
            rd(0, a0, b0, r0);
            for (int i = 0; i < ns; i += 2) {
                rd(i + 1, a1, b1, r1);
                elim(i, a0, b0, r0);
                if (i + 1 >= ns) break;
                rd(i + 2, a0, b0, r0);
                elim(i + 1, a1, b1, r1);
            }
            // substitution from the top: the next row read one step ahead, the
            // parent's voltage from registers when it is the previous row
            auto rq = [&](int i, double2 &q, int &r) {
                const int ii = i >= 0 ? i : 0;
                q = sepv[at(ii) + 1];
                r = septab[ii * 5 + 1];
            };
            auto sub = [&](int i, const double2 qm, const int rp) {
                double xp = xn;
                if (rp != i + 1) xp = rp >= 0 ? sepv[at(rp)].x : 0.0;
                xn = fma(-qm.y, xp, qm.x);
                sepv[at(i)].x = xn;
            };
            double2 q0, q1;
            rq(ns - 1, q0, r0);
            for (int i = ns - 1; i >= 0; i -= 2) {
                rq(i - 1, q1, r1);
                sub(i, q0, r0);
                if (i - 1 < 0) break;
                rq(i - 2, q0, r0);
                sub(i - 1, q1, r1);
            }
        }
        flag[j] = anyb;
        if (!anyb && act && A.info) A.info[s] = 0;
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    // (c) each component's parent voltage and u x of its lower separator
    for (int c = k; c < nc; c += LANES) {
        const int pc = comptab[c * 3], sc = comptab[c * 3 + 1];
        const double xp = pc >= 0 ? sepv[(pc * NEU + j) * 2].x : 0.0;
        const double sg = sc >= 0 ? su[sc * NEU + j] * sepv[(sc * NEU + j) * 2].x : 0.0;
        red[c * NEU + j] = make_double2(xp, sg);
    }
    __syncthreads();

    // ---- second sweep: each component from its root down ----
    const bool ok = flag[j] == 0;
    const SepBuf V(A.rhs, act && ok ? A.bytes : 0u);
    for (int i = k; i < ns; i += LANES)
        V.st(sepv[(i * NEU + j) * 2].x, uint32_t(septab[i * 5]) * ld8 + s8);
    double sg = 0.0;
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
        const uint32_t w0 = uint32_t(code[t]);
        const bool top = w0 & kSepTop, path = w0 & kSepPath;
        const int own = (w0 >> 11) & 7, par = (w0 >> 14) & 7;
        if (top) --ccomp;
        if (path) --chidx;
        const double2 v = top ? red[ccomp * NEU + j] : ring[par * NT + tid];
        sg = top ? v.y : sg;
        const double h = hbuf[(path ? chidx : nh) * NEU + j];
        const double x = q[t] - m[t] * v.x - h * sg;
        reinterpret_cast<double *>(ring)[(own * NT + tid) * 2] = x;
        V.st(x, (w0 & kSepLive) ? uint32_t(w0 & 2047) * ld8 + s8 : kSepNoStore);
    }

    // ---- a neuron whose partitioned elimination met a bad pivot: Algorithm
    // 1 on one lane (in place, pivots in work), which also sets info ----
    if (k == 0 && act && !ok) {
        const int64_t ld = ld8 / 8, n = A.n;
        const double *uu = A.u + s, *ll = A.l + s, *dg = A.d + s;
        double *rh = A.rhs + s, *w = A.work + s;
        for (int64_t i = 0; i < n; ++i) w[i * ld] = 0.0;
        int32_t b = 0;
        for (int64_t i = n - 1; i >= 1; --i) {
            const double dd = dg[i * ld] - w[i * ld];
            const double rr = rh[i * ld];
            if (!b && bad_pivot(dd)) b = int32_t(i + 1);
            const int64_t p = A.parent[i];
            const double fac = uu[i * ld] / dd;
            w[p * ld] += fac * ll[i * ld];
            rh[p * ld] -= fac * rr;
            w[i * ld] = dd;
        }
        const double d0 = dg[0] - w[0];
        if (!b && bad_pivot(d0)) b = 1;
        rh[0] = rh[0] / d0;
        for (int64_t i = 1; i < n; ++i)
            rh[i * ld] = (rh[i * ld] - ll[i * ld] * rh[int64_t(A.parent[i]) * ld]) / w[i * ld];
        if (A.info) A.info[s] = b;
    }
}

// ---- multi-morphology: every tree its own schedule ----------------------
//
// Trees are packed into workgroups of 128 lanes, each tree on as many lanes
// as its components need (at most R rows per lane), the separators' own
// rows among them.  Values are stored in schedule order: element (w, t, k)
// -- workgroup w, step t, lane k -- at ((w R + t) 128 + k), so every step
// of a wavefront is one contiguous 512-byte access; the row codes (16 bits)
// use the same order.  A workgroup's separator and component tables are
// copied into LDS.

// Row code bits of the multi-morphology layout.
constexpr uint32_t kMOwn = 7u, kMLive = 1u << 6, kMPath = 1u << 7, kMPath0 = 1u << 8,
                   kMTop = 1u << 9, kMSep = 1u << 10;
constexpr int kMHeader = 8;     // words of a workgroup's table header
constexpr int kMThreads = 128;  // lanes per workgroup (four workgroups per CU)
constexpr int kMTree = 5;       // words per tree: separator range, lane range, tree number
constexpr int kMJump = 4;       // separators per lane in the substitution (at most 512 per workgroup)

struct SepMArgs {
    uint32_t bytes;             // elems * 8
    const uint16_t *code;       // [elems]
    const int32_t *lanetab;     // [nwg * 128][5]: tree slot, bases (components, path rows,
                                // path components, separators)
    const int64_t *wgoff;       // [nwg + 1] word offsets into tabs
    const int32_t *tabs;        // per workgroup: header, trees, 16-bit tables
    const int32_t *pos;         // flat compartment -> element (Algorithm 1 after a breakdown)
    const int32_t *parent;      // flat parents (local indices)
    const int64_t *src_off;     // [batch + 1]
    const double *u, *l, *d;
    double *rhs, *work;
    int32_t *info;
};

template <int R>
__global__ void __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_hines_sepm(SepMArgs A)
{
    extern __shared__ __align__(16) unsigned char sep_lds[];
    const int tid = threadIdx.x;
    const int64_t w = blockIdx.x;
    const int32_t *wt = A.tabs + A.wgoff[w];
    const int nt = wt[0], ns = wt[1], nc = wt[2], npc = wt[3], nh = wt[4], n16 = wt[5];
    double2 *ring = reinterpret_cast<double2 *>(sep_lds);     // [8][256]
    double2 *red = ring + kSepSlots * kMThreads;             // [nc]
    double2 *pdat = red + nc;                                  // [npc][2]
    double2 *sepv = pdat + 2 * npc;                            // [ns][2]
    double *su = reinterpret_cast<double *>(sepv + 2 * ns);    // [ns]
    double *hbuf = su + ns;                                    // [nh + 2]
    int *badf = reinterpret_cast<int *>(hbuf + nh + 2);        // [256]
    int *tflag = badf + kMThreads;                           // [nt]
    int *trees = tflag + nt;                                   // [nt][5]
    int16_t *t16 = reinterpret_cast<int16_t *>(trees + nt * kMTree);   // septab, comptab, clist
    const int16_t *septab = t16, *comptab = t16 + ns * 4, *clist = comptab + nc * 3;
    for (int i = tid; i < nt * kMTree; i += kMThreads) trees[i] = wt[kMHeader + i];
    for (int i = tid; i < nt; i += kMThreads) tflag[i] = 0;
    {
        const int32_t *src = wt + kMHeader + nt * kMTree;
        int32_t *dst = reinterpret_cast<int32_t *>(t16);
        for (int i = tid; i < (n16 + 1) / 2; i += kMThreads) dst[i] = src[i];
    }
#pragma unroll
    for (int q = 0; q < kSepSlots; ++q) ring[q * kMThreads + tid] = make_double2(0.0, 0.0);
    if (tid == 0) hbuf[nh] = 0.0;
    const int32_t *lt = A.lanetab + (w * kMThreads + tid) * 5;
    const int tslot = lt[0];
    int ccomp = lt[1], chidx = lt[2], cpidx = lt[3], csep = lt[4];
    __syncthreads();

    const SepBuf U(A.u, A.bytes), L(A.l, A.bytes), Dg(A.d, A.bytes), Rh(A.rhs, A.bytes);
    const SepBuf C(A.code, A.bytes / 4);
    const uint32_t lane8 = uint32_t(tid) * 8;
    auto rowoff = [&](int t) { return uint32_t((w * R + t) * kMThreads) * 8u; };   // bytes
    auto code_at = [&](int t) {
        return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(C.r, uint32_t(tid) * 2, rowoff(t) / 4, 0));
    };

    // ---- first sweep ----
    double q[R], m[R];
    constexpr int D = 8, CD = 16;
    double bu[D], bl[D], bd[D], br[D];
    uint32_t cc[CD];
#pragma unroll
    for (int t = 0; t < CD; ++t) cc[t] = t < R ? code_at(t) : 0u;
    auto load = [&](int t, double dep) {
        const uint32_t c = cc[t % CD];
        uint32_t o = (c & (kMLive | kMSep)) ? lane8 : kSepNoStore;
        asm volatile("" : "+v"(o) : "v"(dep));
        const uint32_t so = rowoff(t);
        bu[t % D] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(U.r, o, so, 0));
        bl[t % D] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(L.r, o, so, 0));
        bd[t % D] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(Dg.r, o, so, 0));
        br[t % D] = __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(Rh.r, o, so, 0));
    };
#pragma unroll
    for (int t = 0; t < D; ++t) load(t, 0.0);
    int bad = 0;
    double g = 0.0, P = 0.0, al = 0.0, ga = 0.0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const uint32_t c = cc[t % CD];
        const double u_ = bu[t % D], l_ = bl[t % D], d_ = bd[t % D], r_ = br[t % D];
        const bool live = c & kMLive, path = c & kMPath, top = c & kMTop;
        const int own = int(c & kMOwn), par = int((c >> 3) & kMOwn);
        if (c & kMSep) {
            sepv[csep * 2] = make_double2(d_, r_);
            sepv[csep * 2 + 1] = make_double2(l_, u_);
            su[csep] = u_;
            ++csep;
        }
        const double2 pd = ring[own * kMThreads + tid];
        const double2 po = ring[par * kMThreads + tid];
        ring[own * kMThreads + tid] = make_double2(0.0, 0.0);
        const double dd = d_ - pd.x, rr = r_ - pd.y;
        bad |= int(live) & int(bad_pivot(dd));
        asm volatile("" : "+v"(bad));
        const double rcp = recip(dd);
        const double qq = rr * rcp, mm = l_ * rcp, fac = u_ * rcp;
        q[t] = qq;
        m[t] = mm;
        if (c & kMPath0) { g = 1.0; P = 1.0; al = 0.0; ga = 0.0; }
        const double h = g * rcp;
        hbuf[path ? chidx : nh + 1] = h;
        if (path) {
            ++chidx;
            al = fma(P, qq, al);
            ga = fma(-P, h, ga);
            P = -mm * P;
            g = -fac * g;
        }
        const double2 cb = live ? make_double2(fac * l_, fac * rr) : make_double2(0.0, 0.0);
        if (top) {
            red[ccomp] = cb;
            ++ccomp;
            if (path) {
                pdat[cpidx * 2] = make_double2(g, al);
                pdat[cpidx * 2 + 1] = make_double2(P, ga);
                ++cpidx;
            }
        } else {
            const double2 o = par == own ? make_double2(0.0, 0.0) : po;
            ring[par * kMThreads + tid] = make_double2(o.x + cb.x, o.y + cb.y);
        }
        if (t + CD < R) {
            uint32_t so = rowoff(t + CD) / 4;
            asm volatile("" : "+s"(so) : "v"(qq));
            cc[t % CD] = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(C.r, uint32_t(tid) * 2, so, 0));
        }
        if (t + D < R) load(t + D, qq);
    }
    if (bad && tslot >= 0) atomicOr(&tflag[tslot], 1);
    __syncthreads();

    // ---- the separators' tree systems ----
    for (int i = tid; i < ns; i += kMThreads) {
        const int rp = septab[i * 4], pcomp = septab[i * 4 + 1];
        const int cb = septab[i * 4 + 2], ce = septab[i * 4 + 3];
        const double2 dr = sepv[i * 2], lu = sepv[i * 2 + 1];
        double dh = dr.x, rh = dr.y, lh = 0.0, uh = 0.0;
        for (int c = cb; c < ce; ++c) {
            const double2 v = red[clist[c]];
            dh -= v.x;
            rh -= v.y;
        }
        if (pcomp >= 0) {
            const int pi = comptab[pcomp * 3 + 2];
            const double2 a = pdat[pi * 2], b = pdat[pi * 2 + 1];
            dh = fma(lu.x * lu.y, b.y, dh);
            rh = fma(-lu.x, a.y, rh);
            lh = lu.x * b.x;
            uh = lu.y * a.x;
        } else if (rp >= 0) {
            lh = lu.x;
            uh = lu.y;
        }
        sepv[i * 2] = make_double2(dh, rh);
        sepv[i * 2 + 1] = make_double2(lh, uh);
    }
    __syncthreads();
    if (tid < nt) {
        // one lane per tree runs a serial chain while the other waves of the
        // CU run their sweeps: it takes the issue slots first
        __builtin_amdgcn_s_setprio(3);
        const int *tr = trees + tid * kMTree;
        int anyb = tflag[tid];
        // the next separator's row is read one step ahead (two register sets
        // in turn); an update for the next separator is carried in registers,
        // others are added in LDS by atomics that return nothing (they reach
        // two or more rows ahead, which have not been read yet, and one lane's
        // LDS operations complete in order), so no step waits on them
        const int s0 = tr[0], s1 = tr[1];
        double cf = 0.0, cl = 0.0, cr = 0.0;
        auto rd = [&](int i, double2 &a, double2 &b, int &r) {
            const int ii = i < s1 ? i : s1 - 1;
            r = septab[ii * 4];         // first: the oldest of the three reads
            a = sepv[ii * 2];
            b = sepv[ii * 2 + 1];
        };
        auto elim = [&](int i, const double2 dr0, const double2 lu, const int rp) {
            const double2 dr = make_double2(fma(-cf, cl, dr0.x), fma(-cf, cr, dr0.y));
            anyb |= int(bad_pivot(dr.x));
            const double rcp = recip(dr.x);
            // x_i = q_i + (-m_i) x_rp: the substitution's affine map
            sepv[i * 2 + 1] = make_double2(dr.y * rcp, -(lu.x * rcp));
            const double f = lu.y * rcp;
            const bool next = rp == i + 1;
            cf = next ? f : 0.0;
            cl = next ? lu.x : 0.0;
            cr = next ? dr.y : 0.0;
            if (rp > i + 1) {
                double *o = reinterpret_cast<double *>(sepv + rp * 2);
                __hip_atomic_fetch_add(o, -(f * lu.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(o + 1, -(f * dr.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        };
        if (s0 < s1) {
            double2 a0, b0, a1, b1;
            int r0, r1;
            rd(s0, a0, b0, r0);
            for (int i = s0; i < s1; i += 2) {
                rd(i + 1, a1, b1, r1);
                elim(i, a0, b0, r0);
                if (i + 1 >= s1) break;
                rd(i + 2, a0, b0, r0);
                elim(i + 1, a1, b1, r1);
            }
        }
        tflag[tid] = anyb;
        if (!anyb && A.info) A.info[tr[4]] = 0;
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    // substitution over the separators' forest by pointer jumping, every lane
    // holding up to kMJump separators in registers: x_i = a_i + b_i x_p(i)
    // becomes x_i = (a_i + b_i a_p) + (b_i b_p) x_p(p) each round, until no
    // pointer is left (the table header holds the rounds, from the deepest
    // separator of the workgroup). A round reads the parents' entries from
    // one buffer and publishes its own to the other: (a, b) in the
    // separator's second and first value pairs, p in columns 0 and 2 of its
    // table row (column 2 is read no more by then)
    {
        int16_t *sp = t16;
        const int rounds = wt[6];
        double ja[kMJump], jb[kMJump];
        int jp[kMJump];
#pragma unroll
        for (int j = 0; j < kMJump; ++j) {
            const int i = tid + j * kMThreads;
            if (i < ns) {
                const double2 v = sepv[i * 2 + 1];
                ja[j] = v.x;
                jb[j] = v.y;
                jp[j] = septab[i * 4];
            }
        }
        for (int k = 0; k < rounds; ++k) {
            const int ci = (k & 1) ? 0 : 1, ni = (k & 1) ? 1 : 0;
            const int cp = (k & 1) ? 2 : 0, np = (k & 1) ? 0 : 2;
#pragma unroll
            for (int j = 0; j < kMJump; ++j) {
                const int i = tid + j * kMThreads;
                if (i < ns) {
                    const int p = jp[j];
                    if (p >= 0) {
                        const double2 vp = sepv[p * 2 + ci];
                        jp[j] = sp[p * 4 + cp];
                        ja[j] = fma(jb[j], vp.x, ja[j]);
                        jb[j] *= vp.y;
                    }
                    sepv[i * 2 + ni] = make_double2(ja[j], jb[j]);
                    sp[i * 4 + np] = int16_t(jp[j]);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < kMJump; ++j) {
            const int i = tid + j * kMThreads;
            if (i < ns) sepv[i * 2].x = ja[j];
        }
    }
    __syncthreads();
    for (int c = tid; c < nc; c += kMThreads) {
        const int pc = comptab[c * 3], sc = comptab[c * 3 + 1];
        const double xp = pc >= 0 ? sepv[pc * 2].x : 0.0;
        const double sg = sc >= 0 ? su[sc] * sepv[sc * 2].x : 0.0;
        red[c] = make_double2(xp, sg);
    }
    __syncthreads();

    // ---- second sweep ----
    const bool ok = tslot < 0 || tflag[tslot] == 0;
    const SepBuf V(A.rhs, ok ? A.bytes : 0u);
    double sg = 0.0;
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
        const int ci = (R - 1 - t) % CD;
        if (t == R - 1) {
#pragma unroll
            for (int k = 0; k < CD; ++k) cc[k] = R - 1 - k >= 0 ? code_at(R - 1 - k) : 0u;
        }
        const uint32_t c = cc[ci];
        const bool top = c & kMTop, path = c & kMPath, live = c & kMLive, sepr = c & kMSep;
        const int own = int(c & kMOwn), par = int((c >> 3) & kMOwn);
        if (top) --ccomp;
        if (path) --chidx;
        if (sepr) --csep;
        const double2 v = top ? red[ccomp] : ring[par * kMThreads + tid];
        sg = top ? v.y : sg;
        const double h = hbuf[path ? chidx : nh];
        double x = q[t] - m[t] * v.x - h * sg;
        reinterpret_cast<double *>(ring)[(own * kMThreads + tid) * 2] = x;
        if (sepr) x = sepv[csep * 2].x;
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, x), V.r,
            (live || sepr) ? lane8 : kSepNoStore, rowoff(t), 0);
        if (t - CD >= 0) {
            uint32_t so = rowoff(t - CD) / 4;
            asm volatile("" : "+s"(so) : "v"(x));
            cc[ci] = uint32_t(__builtin_amdgcn_raw_buffer_load_b16(C.r, uint32_t(tid) * 2, so, 0));
        }
    }

    // ---- a tree whose partitioned elimination met a bad pivot: Algorithm 1
    // on one lane through the element map (pivots in work), which sets info ----
    if (tid < nt && tflag[tid]) {
        const int64_t T = trees[tid * kMTree + 4];
        const int64_t o = A.src_off[T];
        const int64_t n = A.src_off[T + 1] - o;
        const int32_t *pos = A.pos + o, *par = A.parent + o;
        double *rh = A.rhs, *wk = A.work;
        for (int64_t i = 0; i < n; ++i) wk[pos[i]] = 0.0;
        int32_t b = 0;
        for (int64_t i = n - 1; i >= 1; --i) {
            const int64_t e = pos[i], pe = pos[par[i]];
            const double dd = A.d[e] - wk[e];
            const double rr = rh[e];
            if (!b && bad_pivot(dd)) b = int32_t(i + 1);
            const double fac = A.u[e] / dd;
            wk[pe] += fac * A.l[e];
            rh[pe] -= fac * rr;
            wk[e] = dd;
        }
        const int64_t e0 = pos[0];
        const double d0 = A.d[e0] - wk[e0];
        if (!b && bad_pivot(d0)) b = 1;
        rh[e0] = rh[e0] / d0;
        for (int64_t i = 1; i < n; ++i) {
            const int64_t e = pos[i];
            rh[e] = (rh[e] - A.l[e] * rh[pos[par[i]]]) / wk[e];
        }
        if (A.info) A.info[T] = b;
    }
}

// flat <-> schedule-ordered layout through the element map
template <typename T, bool PACK>
__global__ void k_sepm_pack(const int32_t *__restrict__ gcomp, int64_t elems, const T *__restrict__ src,
                            T *__restrict__ dst)
{
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < elems;
         e += int64_t(gridDim.x) * blockDim.x) {
        const int32_t c = gcomp[e];
        if (PACK) dst[e] = c >= 0 ? src[c] : T(0);
        else if (c >= 0) dst[c] = src[e];
    }
}

// ---------------------------------------------------------------- host --

struct SepPart {
    std::vector<char> sep;
    std::vector<int32_t> comp;      // component of each non-separator, -1 for separators
    std::vector<int32_t> csize;
};

// Separators bottom-up: a compartment becomes one when the component it
// would close holds more than `target` compartments or two separators below.
SepPart sep_partition(int32_t n, const int32_t *p, int32_t target)
{
    SepPart S;
    S.sep.assign(n, 0);
    std::vector<int32_t> osize(n, 0), osep(n, 0);
    for (int32_t v = n - 1; v >= 0; --v) {
        // children's open parts were accumulated into v below
        const int32_t size = 1 + osize[v];
        const int32_t sc = osep[v];
        if (size > target || sc > 1) {
            S.sep[v] = 1;
            if (v > 0) osep[p[v]] += 1;
        } else if (v > 0) {
            osize[p[v]] += size;
            osep[p[v]] += sc;
        }
    }
    S.comp.assign(n, -1);
    for (int32_t v = 0; v < n; ++v) {
        if (S.sep[v]) continue;
        if (v == 0 || S.sep[p[v]]) {
            S.comp[v] = int32_t(S.csize.size());
            S.csize.push_back(0);
        } else {
            S.comp[v] = S.comp[p[v]];
        }
        S.csize[S.comp[v]] += 1;
    }
    return S;
}

}  // namespace

size_t sep_lds_bytes(const int32_t *blob);

// One tree's schedule over L lanes of at most R rows each (host): each
// lane's rows in first-sweep order, components and path rows numbered in
// the lanes' order (lane by lane, so that a lane counts from its bases),
// the separators in descending compartment order.  With sep_rows the
// separators' own rows are also given to lanes (contiguous numbers per
// lane, at the start of its rows: the multi-morphology kernel reads all
// values through the lanes).
struct SepRow {
    int32_t node;
    uint32_t flags;     // kSepLive, kSepPath, kSepPath0, kSepTop, kSepSepRow
    int own, par;       // ring slots
};
constexpr uint32_t kSepSepRow = 1u << 21;   // a separator's own row (multi-morphology)

struct SepTree {
    int L = 0, R = 0;
    int32_t ns = 0, nc = 0, npc = 0, nh = 0;
    std::vector<std::vector<SepRow>> lanes;
    std::vector<int32_t> snode, rp, pcomp;           // per separator (pcomp: component number)
    std::vector<std::vector<int32_t>> schild;         // per separator: components below it
    std::vector<int32_t> cpar, clow, cpid;            // per component number
    std::vector<int32_t> cbase, hbase, pbase, sbase;  // per lane
};

static bool sep_tree(int32_t n, const int32_t *p, int L, int R, bool sep_rows, SepTree &T,
                     int32_t min_target = 6)
{
    for (int32_t target = std::min(R, 32); target >= min_target; target -= 2) {
        SepPart S = sep_partition(n, p, target);
        const int32_t nc = int32_t(S.csize.size());
        std::vector<int32_t> sidx(n, -1), snode;
        for (int32_t v = n - 1; v >= 0; --v)
            if (S.sep[v]) { sidx[v] = int32_t(snode.size()); snode.push_back(v); }
        const int32_t ns = int32_t(snode.size());
        // lanes: largest component first onto the least loaded lane
        std::vector<int32_t> order(nc), load(L, 0);
        for (int32_t c = 0; c < nc; ++c) order[c] = c;
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t a, int32_t b) { return S.csize[a] > S.csize[b]; });
        std::vector<std::vector<int32_t>> lane(L);
        for (int32_t c : order) {
            const int l = int(std::min_element(load.begin(), load.end()) - load.begin());
            load[l] += S.csize[c];
            lane[l].push_back(c);
        }
        // separators' rows: contiguous numbers, lane by lane, to the lanes
        // with room (fewest rows first)
        std::vector<int32_t> scnt(L, 0);
        if (sep_rows) {
            for (int32_t i = 0; i < ns; ++i) {
                const int l = int(std::min_element(load.begin(), load.end()) - load.begin());
                load[l] += 1;
                scnt[l] += 1;
            }
        }
        if (*std::max_element(load.begin(), load.end()) > R) continue;
        // components: root, parent separator, lower separator, path
        std::vector<int32_t> croot(nc, -1), cpar(nc, -1), clow(nc, -1), cpi(nc, -1);
        for (int32_t v = 0; v < n; ++v)
            if (S.comp[v] >= 0 && croot[S.comp[v]] < 0) croot[S.comp[v]] = v;
        for (int32_t c = 0; c < nc; ++c) cpar[c] = croot[c] == 0 ? -1 : sidx[p[croot[c]]];
        std::vector<char> onpath(n, 0), first(n, 0);
        std::vector<int32_t> rp(ns, -1), pcomp(ns, -1);
        bool okc = true;
        for (int32_t i = 0; i < ns; ++i) {
            const int32_t sv = snode[i];
            if (sv == 0) continue;
            const int32_t pv = p[sv];
            if (S.sep[pv]) { rp[i] = sidx[pv]; continue; }
            const int32_t c = S.comp[pv];
            if (clow[c] >= 0) { okc = false; break; }   // cannot happen by construction
            clow[c] = i;
            cpi[c] = 1;
            pcomp[i] = c;
            rp[i] = cpar[c];
            first[pv] = 1;
            for (int32_t v = pv; v >= 0 && S.comp[v] == c; v = v > 0 ? p[v] : -1) onpath[v] = 1;
        }
        if (!okc) continue;
        // numbering in the lanes' order
        T = SepTree();
        T.L = L; T.R = R; T.ns = ns; T.nc = nc;
        T.lanes.assign(L, {});
        T.cbase.assign(L, 0); T.hbase.assign(L, 0); T.pbase.assign(L, 0); T.sbase.assign(L, 0);
        std::vector<int32_t> cid(nc, -1);
        int32_t nh = 0, ncid = 0, npid = 0, nsid = 0;
        for (int l = 0; l < L; ++l) {
            T.cbase[l] = ncid; T.hbase[l] = nh; T.pbase[l] = npid; T.sbase[l] = nsid;
            for (int32_t q = 0; q < scnt[l]; ++q, ++nsid)
                T.lanes[l].push_back({snode[nsid], kSepSepRow, 0, 0});
            for (int32_t c : lane[l]) {
                cid[c] = ncid++;
                if (cpi[c] >= 0) npid++;
                for (int32_t v = n - 1; v >= 0; --v)
                    if (S.comp[v] == c) {
                        uint32_t f = kSepLive;
                        if (v == croot[c]) f |= kSepTop;
                        if (onpath[v]) { f |= kSepPath; ++nh; }
                        if (first[v]) f |= kSepPath0;
                        T.lanes[l].push_back({v, f, 0, 0});
                    }
            }
        }
        // ring slots, lane by lane in stream order: a compartment's slot holds
        // its children's pending updates (first sweep) and then its voltage for
        // them (second sweep), from its first child's row to its own; the
        // parent's slot opens at its first child's row in the slot that row
        // frees, a leaf takes any free slot for its own row
        bool fits = true;
        std::vector<int8_t> slot(size_t(n), -1);
        for (int l = 0; l < L && fits; ++l) {
            uint32_t busy = 0;
            for (SepRow &r : T.lanes[l]) {
                if (!(r.flags & kSepLive)) continue;
                int sv = slot[size_t(r.node)];
                if (sv < 0) {
                    if (busy == (1u << kSepSlots) - 1) { fits = false; break; }
                    sv = __builtin_ctz(~busy);
                }
                r.own = sv;
                busy &= ~(1u << sv);
                if (r.flags & kSepTop) continue;
                int8_t &sp = slot[size_t(p[r.node])];
                if (sp < 0) { sp = int8_t(sv); busy |= 1u << sv; }
                r.par = sp;
            }
        }
        if (!fits) continue;      // more than 8 pending at once: smaller components
        T.nh = nh;
        T.npc = npid;
        T.snode = snode;
        T.rp = rp;
        T.pcomp.assign(ns, -1);
        T.schild.assign(ns, {});
        T.cpar.assign(nc, -1); T.clow.assign(nc, -1); T.cpid.assign(nc, -1);
        std::vector<int32_t> byid(nc);
        for (int32_t c = 0; c < nc; ++c) byid[cid[c]] = c;
        int32_t q = 0;
        for (int32_t c2 = 0; c2 < nc; ++c2) {
            const int32_t c = byid[c2];
            T.cpar[c2] = cpar[c];
            T.clow[c2] = clow[c];
            if (cpi[c] >= 0) T.cpid[c2] = q++;
            if (cpar[c] >= 0) T.schild[cpar[c]].push_back(c2);
        }
        for (int32_t i = 0; i < ns; ++i) T.pcomp[i] = pcomp[i] >= 0 ? cid[pcomp[i]] : -1;
        // replay the ring traffic of both sweeps: every slot read holds
        // exactly the updates (first sweep) or the voltage (second sweep) of
        // the compartment that reads it
        for (int l = 0; l < L; ++l) {
            int32_t owner[kSepSlots];
            std::fill(owner, owner + kSepSlots, -1);
            for (const SepRow &r : T.lanes[l]) {
                if (!(r.flags & kSepLive)) continue;
                if (owner[r.own] >= 0 && owner[r.own] != r.node) return false;
                owner[r.own] = -1;
                if (!(r.flags & kSepTop)) {
                    if (owner[r.par] < 0) owner[r.par] = p[r.node];
                    else if (owner[r.par] != p[r.node]) return false;
                }
            }
            for (int k = 0; k < kSepSlots; ++k)
                if (owner[k] >= 0) return false;
            std::fill(owner, owner + kSepSlots, -1);
            for (auto it = T.lanes[l].rbegin(); it != T.lanes[l].rend(); ++it) {
                if (!(it->flags & kSepLive)) continue;
                if (!(it->flags & kSepTop) && owner[it->par] != p[it->node]) return false;
                owner[it->own] = it->node;
            }
        }
        return true;
    }
    return false;
}

// The schedule of one tree (host): empty, with the reason, when the tree
// does not qualify (more than 2047 compartments, or no partition whose lanes
// fit R rows with at most 8 compartments pending at once in a lane).
std::vector<int32_t> sep_schedule(int32_t n, const int32_t *p, std::string &why)
{
    if (n < 1 || n > 2047) { why = "tree size outside [1, 2047]"; return {}; }
    // sixteen lanes of 16 or 32 rows, else thirty-two lanes of 24 or 32 rows,
    // else sixty-four of 32; sixteen lanes of 32 rows only with components of
    // at least 16 rows
    // (measured: a tree of 560 squeezed into them by components of ~10
    // rows, 57 separators, took 0.89 ms for 91424 neurons where one lane per
    // neuron takes 0.72)
    for (const auto [lanes, R, tmin] :
         {std::tuple<int, int, int>{16, 16, 6}, {16, 32, 16}, {32, 24, 12}, {32, 32, 6}, {64, 32, 6}}) {
        SepTree T;
        if (!sep_tree(n, p, lanes, R, false, T, tmin)) continue;
        const int32_t ns = T.ns, nc = T.nc;
        if (nc > 255 || ns > 255 || T.nh > 1000) continue;
        std::vector<int32_t> blob(kSepHeader + sep_tab_words(R, ns, nc, lanes), 0);
        blob[0] = R; blob[1] = ns; blob[2] = nc; blob[3] = T.npc; blob[4] = T.nh; blob[5] = n;
        blob[6] = lanes;
        blob[7] = kSepNeurons * 16 / lanes;          // neurons per workgroup
        // 64 lanes: 8 neurons per workgroup (one per CU, 64-byte halves of
        // the row segments per access) when its LDS fits, else 4
        if (lanes == 64) {
            blob[7] = 8;
            if (sep_lds_bytes(blob.data()) > 160 * 1024) blob[7] = 4;
        }
        int32_t *codes = blob.data() + kSepHeader;
        for (int l = 0; l < lanes; ++l) {
            int t = 0;
            for (const SepRow &r : T.lanes[l])
                codes[l * R + t++] = int32_t(uint32_t(r.node) | (uint32_t(r.own) << 11) |
                                             (uint32_t(r.par) << 14) | r.flags);
        }
        int32_t *bt = codes + lanes * R;
        for (int l = 0; l < lanes; ++l) {
            bt[l * 3] = T.cbase[l]; bt[l * 3 + 1] = T.hbase[l]; bt[l * 3 + 2] = T.pbase[l];
        }
        int32_t *st = bt + lanes * 3;
        int32_t *ct = st + ns * 5;
        int32_t *cl = ct + nc * 3;
        int32_t ncl = 0;
        for (int32_t i = 0; i < ns; ++i) {
            st[i * 5] = T.snode[i];
            st[i * 5 + 1] = T.rp[i];
            st[i * 5 + 2] = T.pcomp[i];
            st[i * 5 + 3] = ncl;
            for (int32_t c : T.schild[i]) cl[ncl++] = c;
            st[i * 5 + 4] = ncl;
        }
        for (int32_t c = 0; c < nc; ++c) {
            ct[c * 3] = T.cpar[c];
            ct[c * 3 + 1] = T.clow[c];
            ct[c * 3 + 2] = T.cpid[c];
        }
        if (sep_lds_bytes(blob.data()) > 160 * 1024) continue;
        return blob;
    }
    why = "no partition fits 64 lanes of 32 rows";
    return {};
}

// Multi-morphology schedule (host): every tree its schedule (the fewest
// lanes of at most 32 rows, separators' rows included), trees packed first
// fit, largest first, into workgroups of 128 lanes whose LDS stays within
// 40 KB (four workgroups per CU).  Fails, with the reason, when a tree does
// not qualify.
constexpr int kSepMR = 32;
constexpr size_t kSepMLds = 40 * 1024;

static size_t sepm_tree_lds(const SepTree &T)
{
    return size_t(T.nc) * 16 + size_t(T.npc) * 32 + size_t(T.ns) * 40 + size_t(T.nh) * 8 +
           size_t(T.ns + T.nc) * 8 + 4 + 4 * kMTree;
}
// the kernel's carve-up: the ring, 16 bytes of alignment, the lanes' flags, 8
// bytes of alignment, two spare path entries (16 bytes) and the 16-bit tables'
// rounding (4 bytes); a workgroup needs this plus sepm_tree_lds of its trees
static size_t sepm_fixed_lds() { return size_t(kSepSlots) * kMThreads * 16 + 16 + kMThreads * 4 + 8 + 16 + 4; }

bool sep_build_multi(int64_t batch, const int32_t *sizes, const int32_t *parent, const int64_t *off,
                     SepMulti &M, std::string &why, std::vector<char> *skip)
{
    const int R = kSepMR;
    std::vector<SepTree> tr(static_cast<size_t>(batch));
    std::vector<int> fail(static_cast<size_t>(batch), 0);
    const int nth = int(std::max<int64_t>(1, std::min<int64_t>(16, (batch + 255) / 256)));
    std::vector<std::thread> th;
    for (int k = 0; k < nth; ++k)
        th.emplace_back([&, k] {
            for (int64_t s = k; s < batch; s += nth) {
                const int32_t n = sizes[s];
                const int32_t *p = parent + off[s];
                if (n > 8191) { fail[s] = 1; continue; }
                int L = std::max(1, (n + 29) / 30);
                while (L <= kMThreads && !sep_tree(n, p, L, R, true, tr[s])) ++L;
                if (L > kMThreads || sepm_tree_lds(tr[s]) + sepm_fixed_lds() > kSepMLds) fail[s] = 3;
            }
        });
    for (auto &t : th) t.join();
    // a tree that does not fit fails the batch, or with `skip` is left out
    // (marked) for the caller to solve otherwise
    int64_t nfit = 0;
    if (skip) skip->assign(size_t(batch), 0);
    for (int64_t s = 0; s < batch; ++s) {
        if (!fail[s]) { ++nfit; continue; }
        if (!skip) {
            why = "a tree too large for 128 lanes of 32 rows";
            return false;
        }
        (*skip)[size_t(s)] = 1;
    }
    if (nfit == 0) { why = "no tree fits 128 lanes of 32 rows"; return false; }
    // best fit, largest first: each tree into the workgroup with the fewest
    // free lanes that still holds it (and its LDS), workgroups bucketed by
    // free lanes
    std::vector<int64_t> order;
    order.reserve(size_t(nfit));
    for (int64_t s = 0; s < batch; ++s)
        if (!fail[s]) order.push_back(s);
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return tr[a].L > tr[b].L; });
    struct Bin { int lanes = 0; size_t lds = 0; std::vector<int64_t> trees; };
    std::vector<Bin> bins;
    std::vector<std::vector<int32_t>> bucket(kMThreads + 1);   // by free lanes
    for (int64_t s : order) {
        const int L = tr[s].L;
        const size_t ld = sepm_tree_lds(tr[s]);
        int32_t b = -1;
        for (int f = L; f <= kMThreads && b < 0; ++f) {
            auto &bk = bucket[f];
            for (size_t q = 0; q < bk.size(); ++q)
                if (sepm_fixed_lds() + bins[bk[q]].lds + ld <= kSepMLds) {
                    b = bk[q];
                    bk[q] = bk.back();
                    bk.pop_back();
                    break;
                }
        }
        if (b < 0) {
            b = int32_t(bins.size());
            bins.emplace_back();
        }
        bins[b].lanes += L;
        bins[b].lds += ld;
        bins[b].trees.push_back(s);
        bucket[kMThreads - bins[b].lanes].push_back(b);
    }
    const int64_t nwg = int64_t(bins.size());
    const int64_t elems = nwg * R * kMThreads;
    int64_t total = 0;
    for (int64_t s = 0; s < batch; ++s) total += sizes[s];
    if (elems * 8 > int64_t(0xFFFF0000u)) { why = "more than 4 GiB per array in the schedule-ordered layout"; return false; }
    M = SepMulti();
    M.R = R;
    M.lanes = kMThreads;
    M.nwg = nwg;
    M.elems = elems;
    M.code.assign(size_t(elems), 0);
    M.comp.assign(size_t(elems), -1);
    M.pos.assign(size_t(total), -1);
    M.lanetab.assign(size_t(nwg) * kMThreads * 5, 0);
    M.wgoff.assign(size_t(nwg) + 1, 0);
    M.lds = 0;
    for (int64_t wgi = 0; wgi < nwg; ++wgi) {
        const Bin &B = bins[size_t(wgi)];
        const int nt = int(B.trees.size());
        int32_t ns = 0, nc = 0, npc = 0, nh = 0;
        for (int64_t s : B.trees) { ns += tr[s].ns; nc += tr[s].nc; npc += tr[s].npc; nh += tr[s].nh; }
        const int32_t n16 = ns * 4 + nc * 4;
        std::vector<int32_t> tab(size_t(kMHeader + nt * kMTree + (n16 + 1) / 2), 0);
        tab[0] = nt; tab[1] = ns; tab[2] = nc; tab[3] = npc; tab[4] = nh; tab[5] = n16;
        int32_t depth = 0;                       // most ancestors of a separator
        for (int64_t s : B.trees) {
            const SepTree &T = tr[size_t(s)];
            std::vector<int32_t> dp(size_t(T.ns), 0);
            for (int32_t i = T.ns - 1; i >= 0; --i) {
                dp[size_t(i)] = T.rp[size_t(i)] >= 0 ? dp[size_t(T.rp[size_t(i)])] + 1 : 0;
                depth = std::max(depth, dp[size_t(i)]);
            }
        }
        int32_t rounds = 0;                      // 2^rounds > depth
        while ((int64_t(1) << rounds) <= depth) ++rounds;
        tab[6] = rounds;
        int16_t *t16 = reinterpret_cast<int16_t *>(tab.data() + kMHeader + nt * kMTree);
        int16_t *septab = t16, *comptab = t16 + ns * 4, *clist = comptab + nc * 3;
        int32_t sb = 0, cb = 0, pb = 0, hb = 0, lane0 = 0, ncl = 0;
        for (int ti = 0; ti < nt; ++ti) {
            const int64_t s = B.trees[size_t(ti)];
            const SepTree &T = tr[size_t(s)];
            const int32_t *p = parent + off[s];
            int32_t *trow = tab.data() + kMHeader + ti * kMTree;
            trow[0] = sb; trow[1] = sb + T.ns; trow[2] = lane0; trow[3] = lane0 + T.L; trow[4] = int32_t(s);
            for (int32_t i = 0; i < T.ns; ++i) {
                septab[(sb + i) * 4] = int16_t(T.rp[i] >= 0 ? sb + T.rp[i] : -1);
                septab[(sb + i) * 4 + 1] = int16_t(T.pcomp[i] >= 0 ? cb + T.pcomp[i] : -1);
                septab[(sb + i) * 4 + 2] = int16_t(ncl);
                for (int32_t c : T.schild[i]) clist[ncl++] = int16_t(cb + c);
                septab[(sb + i) * 4 + 3] = int16_t(ncl);
            }
            for (int32_t c = 0; c < T.nc; ++c) {
                comptab[(cb + c) * 3] = int16_t(T.cpar[c] >= 0 ? sb + T.cpar[c] : -1);
                comptab[(cb + c) * 3 + 1] = int16_t(T.clow[c] >= 0 ? sb + T.clow[c] : -1);
                comptab[(cb + c) * 3 + 2] = int16_t(T.cpid[c] >= 0 ? pb + T.cpid[c] : -1);
            }
            for (int l = 0; l < T.L; ++l) {
                const int lane = lane0 + l;
                int32_t *lt = M.lanetab.data() + (wgi * kMThreads + lane) * 5;
                lt[0] = ti; lt[1] = cb + T.cbase[l]; lt[2] = hb + T.hbase[l]; lt[3] = pb + T.pbase[l];
                lt[4] = sb + T.sbase[l];
                int t = 0;
                for (const SepRow &r : T.lanes[l]) {
                    const int64_t e = (wgi * R + t) * kMThreads + lane;
                    uint32_t c = uint32_t(r.own) | (uint32_t(r.par) << 3);
                    if (r.flags & kSepLive) c |= kMLive;
                    if (r.flags & kSepPath) c |= kMPath;
                    if (r.flags & kSepPath0) c |= kMPath0;
                    if (r.flags & kSepTop) c |= kMTop;
                    if (r.flags & kSepSepRow) c |= kMSep;
                    M.code[size_t(e)] = uint16_t(c);
                    M.comp[size_t(e)] = int32_t(off[s] + r.node);
                    M.pos[size_t(off[s] + r.node)] = int32_t(e);
                    ++t;
                }
            }
            (void)p;
            sb += T.ns; cb += T.nc; pb += T.npc; hb += T.nh; lane0 += T.L;
        }
        for (int lane = lane0; lane < kMThreads; ++lane) M.lanetab[size_t((wgi * kMThreads + lane) * 5)] = -1;
        M.wgoff[size_t(wgi) + 1] = M.wgoff[size_t(wgi)] + int64_t(tab.size());
        M.tabs.insert(M.tabs.end(), tab.begin(), tab.end());
        const size_t lds = sepm_fixed_lds() + size_t(nc) * 16 + size_t(npc) * 32 + size_t(ns) * 40 +
                           size_t(nh) * 8 + size_t(nt) * (4 + 4 * kMTree) + size_t(n16) * 2;
        if (lds != sepm_fixed_lds() + B.lds || lds > kSepMLds || ns > kMJump * kMThreads) {
            why = "internal: a workgroup's LDS outside its budget";
            return false;
        }
        M.lds = std::max(M.lds, lds);
    }
    return true;
}

hipError_t sepm_pack(bool pack, bool f64, const int32_t *gcomp, int64_t elems, const void *src, void *dst,
                     hipStream_t st)
{
    const unsigned grid = unsigned(std::min<int64_t>((elems + 255) / 256, 65536));
    if (f64) {
        if (pack) hipLaunchKernelGGL((k_sepm_pack<double, true>), dim3(grid), dim3(256), 0, st, gcomp, elems,
                                     (const double *)src, (double *)dst);
        else hipLaunchKernelGGL((k_sepm_pack<double, false>), dim3(grid), dim3(256), 0, st, gcomp, elems,
                                (const double *)src, (double *)dst);
    } else {
        if (pack) hipLaunchKernelGGL((k_sepm_pack<float, true>), dim3(grid), dim3(256), 0, st, gcomp, elems,
                                     (const float *)src, (float *)dst);
        else hipLaunchKernelGGL((k_sepm_pack<float, false>), dim3(grid), dim3(256), 0, st, gcomp, elems,
                                (const float *)src, (float *)dst);
    }
    return hipGetLastError();
}

bps_status launch_hines_sepm(const SepMultiDev &S, const int32_t *parent_dev, const int64_t *src_off,
                             const void *u, const void *l, const void *d, void *rhs, void *work,
                             int32_t *info, hipStream_t st)
{
    SepMArgs A{};
    A.bytes = uint32_t(S.elems * 8);
    A.code = S.code; A.lanetab = S.lanetab; A.wgoff = S.wgoff; A.tabs = S.tabs; A.pos = S.pos;
    A.parent = parent_dev; A.src_off = src_off;
    A.u = (const double *)u; A.l = (const double *)l; A.d = (const double *)d;
    A.rhs = (double *)rhs; A.work = (double *)work; A.info = info;
    hipLaunchKernelGGL(k_hines_sepm<kSepMR>, dim3(unsigned(S.nwg)), dim3(kMThreads), S.lds, st, A);
    BPS_LAUNCHED("k_hines_sepm");
    return BPS_OK;
}

size_t sep_lds_bytes(const int32_t *blob)
{
    const size_t R = size_t(blob[0]), ns = size_t(blob[1]), nc = size_t(blob[2]);
    const size_t npc = size_t(blob[3]), nh = size_t(blob[4]), neu = size_t(blob[7]), nt = size_t(blob[6]) * neu;
    return size_t(kSepSlots) * nt * 16 + nc * neu * 16 + npc * neu * 32 + ns * neu * 32 + ns * neu * 8 +
           (nh + 2) * neu * 8 + size_t(nt + neu) * 4 + size_t(sep_tab_words(int(R), int(ns), int(nc), blob[6])) * 4;
}

hipError_t sep_prepare_device()
{
    for (const void *f : {reinterpret_cast<const void *>(&k_hines_sep<16, 16, 16>),
                          reinterpret_cast<const void *>(&k_hines_sep<32, 16, 16>),
                          reinterpret_cast<const void *>(&k_hines_sep<24, 32, 8>),
                          reinterpret_cast<const void *>(&k_hines_sep<32, 32, 8>),
                          reinterpret_cast<const void *>(&k_hines_sep<32, 64, 4>),
                          reinterpret_cast<const void *>(&k_hines_sep<32, 64, 8>)}) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_hines_sepm<kSepMR>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
}

bps_status launch_hines_sep(const int32_t *blob_host, const int32_t *blob_dev, int64_t batch, int64_t ld,
                            const int32_t *parent_dev, const void *u, const void *l, const void *d,
                            void *rhs, void *work, int32_t *info, hipStream_t st)
{
    const int R = blob_host[0];
    SepArgs A{};
    A.batch = batch;
    A.ld8 = uint32_t(ld * 8);
    A.n = blob_host[5];
    A.bytes = uint32_t(int64_t(A.n) * ld * 8);
    A.ns = blob_host[1]; A.nc = blob_host[2]; A.npc = blob_host[3]; A.nh = blob_host[4];
    A.tab = blob_dev + kSepHeader;
    A.parent = parent_dev;
    A.u = (const double *)u; A.l = (const double *)l; A.d = (const double *)d;
    A.rhs = (double *)rhs; A.work = (double *)work; A.info = info;
    const size_t lds = sep_lds_bytes(blob_host);
    const int lanes = blob_host[6], neu = blob_host[7];
    const dim3 grid(unsigned((batch + neu - 1) / neu)), block(unsigned(lanes * neu));
    if (lanes == 64 && neu == 8) hipLaunchKernelGGL((k_hines_sep<32, 64, 8>), grid, block, lds, st, A);
    else if (lanes == 64) hipLaunchKernelGGL((k_hines_sep<32, 64, 4>), grid, block, lds, st, A);
    else if (lanes == 32 && R == 24) hipLaunchKernelGGL((k_hines_sep<24, 32, 8>), grid, block, lds, st, A);
    else if (lanes == 32) hipLaunchKernelGGL((k_hines_sep<32, 32, 8>), grid, block, lds, st, A);
    else if (R == 16) hipLaunchKernelGGL((k_hines_sep<16, 16, 16>), grid, block, lds, st, A);
    else hipLaunchKernelGGL((k_hines_sep<32, 16, 16>), grid, block, lds, st, A);
    BPS_LAUNCHED("k_hines_sep");
    return BPS_OK;
}

}  // namespace bps
