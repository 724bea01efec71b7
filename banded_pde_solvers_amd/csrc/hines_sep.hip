// hines_sep.hip -- Hines systems of one shared morphology, each neuron
// solved by sixteen lanes ([H] section 2, Algorithm 1, and the per-branch
// decomposition of section 4).
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
// Workgroup: 16 neurons x 16 lanes.  Thread (k, j) = lane k of neuron j;
// a wavefront holds 4 lanes of 16 neighbouring neurons, so every access is
// four 128-byte row segments of the interleaved layout.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace bps {

namespace {

constexpr int kSepLanes = 16;       // lanes per neuron
constexpr int kSepNeurons = 16;     // neurons per workgroup
constexpr int kSepThreads = kSepLanes * kSepNeurons;
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
    const int32_t *tab;         // codes [16][R], bases [16][3], separators [ns][5],
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

// Words of the schedule's tables after the header.
__host__ __device__ inline int sep_tab_words(int R, int ns, int nc)
{
    return kSepLanes * R + kSepLanes * 3 + ns * 5 + nc * 4;
}

template <int R>
__global__ void __launch_bounds__(kSepThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_hines_sep(SepArgs A)
{
    extern __shared__ __align__(16) unsigned char sep_lds[];
    const int tid = threadIdx.x, k = tid >> 4, j = tid & 15;
    const int64_t s = int64_t(blockIdx.x) * kSepNeurons + j;
    const bool act = s < A.batch;
    // lanes past the batch shadow the last neuron (loads only)
    const uint32_t s8 = uint32_t(uint64_t(act ? s : A.batch - 1) * 8);
    const int ns = A.ns, nc = A.nc, npc = A.npc, nh = A.nh;
    double2 *ring = reinterpret_cast<double2 *>(sep_lds);     // [8][256]
    double2 *red = ring + kSepSlots * kSepThreads;             // [nc][16]
    double2 *pdat = red + nc * kSepNeurons;                    // [npc][16][2]
    double2 *sepv = pdat + npc * 2 * kSepNeurons;              // [ns][16][2]
    double *su = reinterpret_cast<double *>(sepv + ns * 2 * kSepNeurons);   // [ns][16]
    double *hbuf = su + ns * kSepNeurons;                      // [nh + 2][16]
    int *badf = reinterpret_cast<int *>(hbuf + (nh + 2) * kSepNeurons);  // [256]
    int *flag = badf + kSepThreads;                            // [16]
    int *tab = flag + kSepNeurons;                             // the schedule's tables
    const int *codes = tab, *bases = tab + kSepLanes * R, *septab = bases + kSepLanes * 3;
    const int *comptab = septab + ns * 5, *clist = comptab + nc * 3;

    const SepBuf U(A.u, A.bytes), L(A.l, A.bytes), Dg(A.d, A.bytes), Rh(A.rhs, A.bytes);
    const uint32_t ld8 = A.ld8;
    const int ntab = sep_tab_words(R, ns, nc);
    for (int i = tid; i < ntab; i += kSepThreads) tab[i] = A.tab[i];
#pragma unroll
    for (int q = 0; q < kSepSlots; ++q) ring[q * kSepThreads + tid] = make_double2(0.0, 0.0);
    if (k == 0) hbuf[nh * kSepNeurons + j] = 0.0;              // read by rows off the paths
    // the separators' own rows
    for (int i = k; i < ns; i += kSepLanes) {
        const uint32_t o = uint32_t(A.tab[kSepLanes * R + kSepLanes * 3 + i * 5]) * ld8 + s8;
        const double uu = U.ld(o), ll = L.ld(o), dd = Dg.ld(o), rr = Rh.ld(o);
        su[i * kSepNeurons + j] = uu;
        sepv[(i * kSepNeurons + j) * 2] = make_double2(dd, rr);
        sepv[(i * kSepNeurons + j) * 2 + 1] = make_double2(ll, uu);
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
        const double2 pd = ring[own * kSepThreads + tid];
        const double2 po = ring[par * kSepThreads + tid];
        ring[own * kSepThreads + tid] = make_double2(0.0, 0.0);
        const double dd = d_ - pd.x, rr = r_ - pd.y;
        bad |= int(live) & int(bad_pivot(dd));
        asm volatile("" : "+v"(bad));   // test each pivot now, not all of them at the end
        const double rcp = recip(dd);
        const double qq = rr * rcp, mm = l_ * rcp, fac = u_ * rcp;
        q[t] = qq;
        m[t] = mm;
        if (w0 & kSepPath0) { g = 1.0; P = 1.0; al = 0.0; ga = 0.0; }
        const double h = g * rcp;
        hbuf[(path ? chidx : nh + 1) * kSepNeurons + j] = h;
        if (path) {
            ++chidx;
            al = fma(P, qq, al);
            ga = fma(-P, h, ga);
            P = -mm * P;
            g = -fac * g;
        }
        const double2 cb = make_double2(fac * l_, fac * rr);
        if (top) {
            red[ccomp * kSepNeurons + j] = cb;
            ++ccomp;
            if (path) {
                pdat[(cpidx * kSepNeurons + j) * 2] = make_double2(g, al);
                pdat[(cpidx * kSepNeurons + j) * 2 + 1] = make_double2(P, ga);
                ++cpidx;
            }
        } else {
            const double2 o = par == own ? make_double2(0.0, 0.0) : po;
            ring[par * kSepThreads + tid] = make_double2(o.x + cb.x, o.y + cb.y);
        }
        if (t + D < R) load(t + D, qq);
    }
    badf[tid] = bad;
    __syncthreads();

    // ---- the separators' tree system ----
    // (a) every separator's row with its components' terms (all lanes)
    for (int i = k; i < ns; i += kSepLanes) {
        const int rp = septab[i * 5 + 1], pcomp = septab[i * 5 + 2];
        const int cb = septab[i * 5 + 3], ce = septab[i * 5 + 4];
        const double2 dr = sepv[(i * kSepNeurons + j) * 2];
        const double2 lu = sepv[(i * kSepNeurons + j) * 2 + 1];
        double dh = dr.x, rh = dr.y, lh = 0.0, uh = 0.0;
        for (int c = cb; c < ce; ++c) {
            const double2 v = red[clist[c] * kSepNeurons + j];
            dh -= v.x;
            rh -= v.y;
        }
        if (pcomp >= 0) {
            // the separator meets its parent component through the path: the
            // parent compartment's voltage is al + P x_top + ga (u x_sep)
            const int pi = comptab[pcomp * 3 + 2];
            const double2 a = pdat[(pi * kSepNeurons + j) * 2];
            const double2 b = pdat[(pi * kSepNeurons + j) * 2 + 1];
            dh = fma(lu.x * lu.y, b.y, dh);
            rh = fma(-lu.x, a.y, rh);
            lh = lu.x * b.x;
            uh = lu.y * a.x;
        } else if (rp >= 0) {
            lh = lu.x;
            uh = lu.y;
        }
        sepv[(i * kSepNeurons + j) * 2] = make_double2(dh, rh);
        sepv[(i * kSepNeurons + j) * 2 + 1] = make_double2(lh, uh);
    }
    __syncthreads();
    // (b) Algorithm 1 on the separators (one lane per neuron), in place
    if (k == 0) {
        int anyb = 0;
        for (int kk = 0; kk < kSepLanes; ++kk) anyb |= badf[kk * kSepNeurons + j];
        for (int i = 0; i < ns; ++i) {
            const int rp = septab[i * 5 + 1];
            const double2 dr = sepv[(i * kSepNeurons + j) * 2];
            const double2 lu = sepv[(i * kSepNeurons + j) * 2 + 1];
            anyb |= int(bad_pivot(dr.x));
            const double rcp = recip(dr.x);
            sepv[(i * kSepNeurons + j) * 2 + 1] = make_double2(dr.y * rcp, lu.x * rcp);
            if (rp >= 0) {
                const double f = lu.y * rcp;
                double2 &t = sepv[(rp * kSepNeurons + j) * 2];
                const double2 o = t;
                t = make_double2(fma(-f, lu.x, o.x), fma(-f, dr.y, o.y));
            }
        }
        for (int i = ns - 1; i >= 0; --i) {
            const int rp = septab[i * 5 + 1];
            const double2 qm = sepv[(i * kSepNeurons + j) * 2 + 1];
            const double xp = rp >= 0 ? sepv[(rp * kSepNeurons + j) * 2].x : 0.0;
            sepv[(i * kSepNeurons + j) * 2].x = qm.x - qm.y * xp;
        }
        flag[j] = anyb;
        if (!anyb && act && A.info) A.info[s] = 0;
    }
    __syncthreads();
    // (c) each component's parent voltage and u x of its lower separator
    for (int c = k; c < nc; c += kSepLanes) {
        const int pc = comptab[c * 3], sc = comptab[c * 3 + 1];
        const double xp = pc >= 0 ? sepv[(pc * kSepNeurons + j) * 2].x : 0.0;
        const double sg = sc >= 0 ? su[sc * kSepNeurons + j] * sepv[(sc * kSepNeurons + j) * 2].x : 0.0;
        red[c * kSepNeurons + j] = make_double2(xp, sg);
    }
    __syncthreads();

    // ---- second sweep: each component from its root down ----
    const bool ok = flag[j] == 0;
    const SepBuf V(A.rhs, act && ok ? A.bytes : 0u);
    for (int i = k; i < ns; i += kSepLanes)
        V.st(sepv[(i * kSepNeurons + j) * 2].x, uint32_t(septab[i * 5]) * ld8 + s8);
    double sg = 0.0;
#pragma unroll
    for (int t = R - 1; t >= 0; --t) {
        const uint32_t w0 = uint32_t(code[t]);
        const bool top = w0 & kSepTop, path = w0 & kSepPath;
        const int own = (w0 >> 11) & 7, par = (w0 >> 14) & 7;
        if (top) --ccomp;
        if (path) --chidx;
        const double2 v = top ? red[ccomp * kSepNeurons + j] : ring[par * kSepThreads + tid];
        sg = top ? v.y : sg;
        const double h = hbuf[(path ? chidx : nh) * kSepNeurons + j];
        const double x = q[t] - m[t] * v.x - h * sg;
        reinterpret_cast<double *>(ring)[(own * kSepThreads + tid) * 2] = x;
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

// The schedule of one tree (host): empty, with the reason, when the tree
// does not qualify (a parent more than 8 compartments away, more than 2047
// compartments, or no partition whose lanes fit R rows).
std::vector<int32_t> sep_schedule(int32_t n, const int32_t *p, std::string &why)
{
    if (n < 1 || n > 2047) { why = "tree size outside [1, 2047]"; return {}; }
    for (int32_t i = 1; i < n; ++i)
        if (i - p[i] > kSepSlots) { why = "a parent more than 8 compartments away"; return {}; }
    for (int R : {16, 32}) {
        for (int32_t target = std::min(R, 32); target >= 6; target -= 2) {
            SepPart S = sep_partition(n, p, target);
            const int32_t nc = int32_t(S.csize.size());
            std::vector<int32_t> sidx(n, -1), snode;
            for (int32_t v = n - 1; v >= 0; --v)
                if (S.sep[v]) { sidx[v] = int32_t(snode.size()); snode.push_back(v); }
            const int32_t ns = int32_t(snode.size());
            if (nc > 255 || ns > 255) continue;
            // lanes: largest component first onto the least loaded lane
            std::vector<int32_t> order(nc), load(kSepLanes, 0);
            for (int32_t c = 0; c < nc; ++c) order[c] = c;
            std::stable_sort(order.begin(), order.end(),
                             [&](int32_t a, int32_t b) { return S.csize[a] > S.csize[b]; });
            std::vector<std::vector<int32_t>> lane(kSepLanes);
            for (int32_t c : order) {
                const int l = int(std::min_element(load.begin(), load.end()) - load.begin());
                load[l] += S.csize[c];
                lane[l].push_back(c);
            }
            if (*std::max_element(load.begin(), load.end()) > R) continue;
            // components: root, parent separator, lower separator, path
            std::vector<int32_t> croot(nc, -1), cpar(nc, -1), clow(nc, -1), cpi(nc, -1);
            for (int32_t v = 0; v < n; ++v)
                if (S.comp[v] >= 0 && croot[S.comp[v]] < 0) croot[S.comp[v]] = v;
            for (int32_t c = 0; c < nc; ++c) cpar[c] = croot[c] == 0 ? -1 : sidx[p[croot[c]]];
            std::vector<char> onpath(n, 0), first(n, 0);
            std::vector<int32_t> rp(ns, -1), pcomp(ns, -1);
            int32_t npc = 0;
            bool okc = true;
            for (int32_t i = 0; i < ns; ++i) {
                const int32_t sv = snode[i];
                if (sv == 0) continue;
                const int32_t pv = p[sv];
                if (S.sep[pv]) { rp[i] = sidx[pv]; continue; }
                const int32_t c = S.comp[pv];
                if (clow[c] >= 0) { okc = false; break; }   // cannot happen by construction
                clow[c] = i;
                cpi[c] = npc++;
                pcomp[i] = c;
                rp[i] = cpar[c];
                first[pv] = 1;
                for (int32_t v = pv; v >= 0 && S.comp[v] == c; v = v > 0 ? p[v] : -1) onpath[v] = 1;
            }
            if (!okc) continue;
            // numbering in the lanes' order: components, path rows, components
            // with a path; each lane's first numbers are its bases
            std::vector<int32_t> cid(nc, -1);
            std::vector<int32_t> base(kSepLanes * 3, 0);
            int32_t nh = 0, ncid = 0, npid = 0;
            std::vector<std::vector<int32_t>> rows(kSepLanes);
            for (int l = 0; l < kSepLanes; ++l) {
                base[l * 3] = ncid; base[l * 3 + 1] = nh; base[l * 3 + 2] = npid;
                for (int32_t c : lane[l]) {
                    cid[c] = ncid++;
                    if (cpi[c] >= 0) npid++;
                    for (int32_t v = n - 1; v >= 0; --v)
                        if (S.comp[v] == c) {
                            rows[l].push_back(v);
                            if (onpath[v]) ++nh;
                        }
                }
            }
            if (nh > 1000) continue;
            // path data index in the lanes' order
            std::vector<int32_t> pid(nc, -1);
            {
                int32_t q = 0;
                for (int l = 0; l < kSepLanes; ++l)
                    for (int32_t c : lane[l])
                        if (cpi[c] >= 0) pid[c] = q++;
            }
            // blob
            std::vector<int32_t> blob(kSepHeader + sep_tab_words(R, ns, nc), 0);
            blob[0] = R; blob[1] = ns; blob[2] = nc; blob[3] = npc; blob[4] = nh; blob[5] = n;
            blob[6] = kSepLanes;
            int32_t *codes = blob.data() + kSepHeader;
            for (int l = 0; l < kSepLanes; ++l) {
                int t = 0;
                for (int32_t v : rows[l]) {
                    const int32_t c = S.comp[v];
                    uint32_t w0 = uint32_t(v) | (uint32_t(v & 7) << 11) | kSepLive;
                    if (v != croot[c]) w0 |= uint32_t(p[v] & 7) << 14;
                    else w0 |= kSepTop;
                    if (onpath[v]) w0 |= kSepPath;
                    if (first[v]) w0 |= kSepPath0;
                    codes[l * R + t] = int32_t(w0);
                    ++t;
                }
            }
            int32_t *bt = codes + kSepLanes * R;
            std::copy(base.begin(), base.end(), bt);
            int32_t *st = bt + kSepLanes * 3;
            int32_t *ct = st + ns * 5;
            int32_t *cl = ct + nc * 3;
            int32_t ncl = 0;
            std::vector<int32_t> byid(nc);
            for (int32_t c = 0; c < nc; ++c) byid[cid[c]] = c;
            for (int32_t i = 0; i < ns; ++i) {
                st[i * 5] = snode[i];
                st[i * 5 + 1] = rp[i];
                st[i * 5 + 2] = pcomp[i] >= 0 ? cid[pcomp[i]] : -1;
                st[i * 5 + 3] = ncl;
                for (int32_t c2 = 0; c2 < nc; ++c2)
                    if (cpar[byid[c2]] == i) cl[ncl++] = c2;
                st[i * 5 + 4] = ncl;
            }
            for (int32_t c2 = 0; c2 < nc; ++c2) {
                const int32_t c = byid[c2];
                ct[c2 * 3] = cpar[c];
                ct[c2 * 3 + 1] = clow[c];
                ct[c2 * 3 + 2] = pid[c];
            }
            // replay the ring traffic of both sweeps: every slot read holds
            // exactly the updates (first sweep) or the voltage (second sweep)
            // of the compartment that reads it
            bool good = true;
            for (int l = 0; l < kSepLanes && good; ++l) {
                int32_t owner[kSepSlots];
                std::fill(owner, owner + kSepSlots, -1);
                for (int t = 0; t < R && good; ++t) {
                    const uint32_t w0 = uint32_t(codes[l * R + t]);
                    if (!(w0 & kSepLive)) break;
                    const int32_t v = int32_t(w0 & 2047);
                    const int own = (w0 >> 11) & 7, par = (w0 >> 14) & 7;
                    if (owner[own] >= 0 && owner[own] != v) good = false;
                    owner[own] = -1;
                    if (!(w0 & kSepTop)) {
                        if (owner[par] < 0) owner[par] = p[v];
                        else if (owner[par] != p[v]) good = false;
                    }
                }
                for (int q = 0; q < kSepSlots; ++q) good = good && owner[q] < 0;
                std::fill(owner, owner + kSepSlots, -1);
                for (int t = R - 1; t >= 0 && good; --t) {
                    const uint32_t w0 = uint32_t(codes[l * R + t]);
                    if (!(w0 & kSepLive)) continue;
                    const int32_t v = int32_t(w0 & 2047);
                    const int own = (w0 >> 11) & 7, par = (w0 >> 14) & 7;
                    if (!(w0 & kSepTop) && owner[par] != p[v]) good = false;
                    owner[own] = v;
                }
            }
            if (!good) { why = "internal: slot replay failed"; return {}; }
            if (sep_lds_bytes(blob.data()) > 160 * 1024) continue;
            return blob;
        }
    }
    why = "no partition fits 16 lanes of 32 rows";
    return {};
}

size_t sep_lds_bytes(const int32_t *blob)
{
    const size_t R = size_t(blob[0]), ns = size_t(blob[1]), nc = size_t(blob[2]);
    const size_t npc = size_t(blob[3]), nh = size_t(blob[4]);
    return size_t(kSepSlots) * kSepThreads * 16 + nc * kSepNeurons * 16 + npc * kSepNeurons * 32 +
           ns * kSepNeurons * 32 + ns * kSepNeurons * 8 + (nh + 2) * kSepNeurons * 8 +
           size_t(kSepThreads + kSepNeurons) * 4 + size_t(sep_tab_words(int(R), int(ns), int(nc))) * 4;
}

hipError_t sep_prepare_device()
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_hines_sep<16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_hines_sep<32>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
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
    const dim3 grid(unsigned((batch + kSepNeurons - 1) / kSepNeurons));
    if (R == 16) hipLaunchKernelGGL(k_hines_sep<16>, grid, dim3(kSepThreads), lds, st, A);
    else hipLaunchKernelGGL(k_hines_sep<32>, grid, dim3(kSepThreads), lds, st, A);
    BPS_LAUNCHED("k_hines_sep");
    return BPS_OK;
}

}  // namespace bps
