// hines.hip -- batched Hines (tree-tridiagonal) solves for gfx950.
//
// Method: Algorithm 1 of "Simulating the behavior of the human brain on
// GPUs" (section 2): eliminate from the leaves to the root (factor u_i/d_i,
// update the parent's diagonal and right-hand side), divide at the root, then
// substitute from the root to the leaves.  One lane per neuron (section 3);
// in multi-morphology batches the largest trees may take two lanes of their
// wavefront, split into trunk and side branches (section 4's per-branch
// decomposition; k_hines_split, build_split).
//
// Layouts: mono-morphology uses the Full-Interleaved layout [n][ld] with one
// parent vector shared by every lane (wave-uniform, scalar loads).
// Multi-morphology (section 4) uses the Block-Interleaved layout with a block
// of 64 neurons (one wavefront) stored [rows_b][64]; neurons are sorted by
// size so each block's lanes have nearly equal lengths, and each lane reads
// its own parent stream stored in the same layout.
//
// Between the sweeps each compartment keeps q_i = rhs'_i / d'_i (written in
// place into rhs) and m_i = l_i / d'_i (written to work), so the second sweep
// is V_i = q_i - m_i V_{p_i}: algebraically the page's
// (rhs'_i - l_i V_{p_i}) / d'_i with the division done once per compartment.
//
// Pending parent updates (subtractions from d and rhs of the parent) are held
// in a per-lane ring of W slots in LDS, indexed by row mod W; a parent at
// distance <= W from its child is always inside the ring.  Trees with a larger
// parent distance use the general variant, which sends those updates through
// per-lane accumulators in global memory (zeroed before each solve).
#include <algorithm>
#include <numeric>
#include <thread>
#include <vector>

#include "common.h"
#include "kernels.h"

struct bps_hines_plan {
    int mono = 1;
    int64_t batch = 0;
    int64_t n = 0;           // mono: compartments per neuron
    int64_t ld = 0;          // mono: leading dimension
    int64_t elems = 0;       // values per array in the solver layout
    int64_t unknowns = 0;    // real compartments
    int32_t max_dist = 0;    // largest i - p_i
    int64_t nblocks = 0;     // multi: number of 64-neuron blocks
    int32_t max_rows = 0;    // multi: largest block row count
    // device arrays
    int32_t *parent = nullptr;     // mono [n]; multi packed [elems]
    uint8_t *dist8 = nullptr;      // multi packed [elems]: i - p_i (0 for roots and padding,
                                   // kFar for a parent more than kRing rows up)
    int64_t *blk_off = nullptr;    // multi [nblocks]
    int32_t *blk_rows = nullptr;   // multi [nblocks]
    int32_t *lane_n = nullptr;     // multi [nblocks*64]
    int32_t *lane_src = nullptr;   // multi [nblocks*64] original neuron (-1 empty)
    // two lanes per neuron for the largest trees (k_hines_split): built when
    // at least one tree is split; then lane_n holds each lane's branch rows
    int64_t nsplit = 0;            // neurons on two lanes
    uint16_t *code16 = nullptr;    // multi packed [elems]: row codes
    int32_t *comp = nullptr;       // multi packed [elems]: compartment of the row, -1 padding
    int64_t *src_off = nullptr;    // multi [batch+1] offsets in the flat layout
    // level schedule (one wavefront per neuron, sections of each tree by
    // level; see k_hines_levels): built when the plan may use it
    int sched = 0;                 // BPS_HINES_AUTO / _LANES / _LEVELS as created
    bool use_levels = false;       // the schedule hines_launch takes
    int32_t lv_maxn = 0;           // largest tree of the batch
    int32_t *lv_perm = nullptr;    // per tree: new index -> compartment
    int32_t *lv_sec = nullptr;     // per tree: section start (new index), nsec + 1 entries
    int32_t *lv_spar = nullptr;    // per tree: parent (new index) of each section head, -1 root
    int32_t *lv_lev = nullptr;     // per tree: section ranges per level, nlev + 1 entries
    int64_t *lv_tree = nullptr;    // per tree: perm base, sec base, lev base, nlev, n, data base
    // separator schedule of a shared tree (mono, k_hines_sep): on the
    // host and on the device, when the plan uses it
    std::vector<int32_t> sep;
    int32_t *sep_dev = nullptr;
    // multi-morphology trees on their own lanes (k_hines_sepm): code16 and
    // comp hold the row codes and the element map; the flat parents serve
    // Algorithm 1 on a tree that breaks down
    bool use_sepm = false;
    bps::SepMultiDev sepm;
    int32_t *flat_parent = nullptr;
    // trees the separator schedules do not take (too large for one
    // workgroup), in a plan of their own (one lane per tree, original tree
    // numbers and flat offsets) whose elements follow the separators' ones
    int64_t sep_elems = 0;
    bps_hines_plan *rest = nullptr;
};

namespace bps {

constexpr int kRing = 16;       // LDS ring slots per lane (power of two)
constexpr int kFar = 255;       // distance byte of a parent more than kRing rows up
constexpr int kLevelMaxN = 4096;        // tree size limit of the level schedule (LDS)
// auto: the level schedule up to this many compartments in the batch.
// Measured (one solve): trees of 512, 16 .. 1024 neurons: 77 .. 107 us with
// levels, 147 us with one lane per neuron; 2048: 135 vs 151; 4096: 259 vs 158.
// Trees of 256 .. 2048: 256 neurons 308 vs 513 us, 1024 neurons 584 vs 513.
// Multi-morphology batches compare with two lanes per tree (levels / two
// lanes): 256 trees of 512: 87 / 91 us, 1024 trees of 512: 99.5 / 93 us;
// 256 trees of 256 .. 2048: 281 / 301 us, 512 such trees: 314 / 294 us.
constexpr int64_t kLevelAutoUnknowns = 786432;
constexpr int64_t kLevelAutoUnknownsMulti = 393216;
constexpr int kHinesAhead = 8;  // rows of look-ahead for the streamed inputs
constexpr int kSimds = 1024;    // SIMDs of the GPU (256 CUs x 4)
constexpr int kSplitMin = 32;   // smallest tree put on two lanes
// Row codes of the two-lane kernel (see build_split), 16 bits: the row's
// own slot (bits 0-5), its parent's slot (bits 6-11), live (bit 12),
// whether the parent's voltage is that of the lane's previous live row in
// the substitution (bit 13, then it is in a register), and whether the
// parent's slot is in the column of the pair's even lane (bit 14: a branch
// root of the odd lane, whose parent is on the trunk).  Slot ids: 0..15 the
// lane's ring, 16..31 the pair's trunk ring (kept in the even lane's column,
// the lane that takes the trunk), 32 the lane's sink (the own slot of
// padding and waiting rows, the parent slot of roots and those).
constexpr int kSlotTrunk = 16, kSlotSink = 32, kSlots = 33;
constexpr uint16_t kCodeLive = 1u << 12, kCodeVreg = 1u << 13, kCodeEven = 1u << 14;
__host__ __device__ constexpr uint16_t row_code(int own, int par, bool live, bool vreg, bool even = false)
{
    return uint16_t(own | (par << 6) | (live ? kCodeLive : 0) | (vreg ? kCodeVreg : 0) |
                    (even ? kCodeEven : 0));
}

struct HinesArgs {
    int64_t batch, n, ld;            // mono geometry
    const int64_t *blk_off;          // multi geometry
    const int32_t *blk_rows, *lane_n, *lane_src;
    const int32_t *parent;
    const uint8_t *dist8;
    const uint16_t *code16;          // two-lane plans: row codes
    const int32_t *comp;             // two-lane plans: compartment of each row
    const double *u, *l, *d;
    double *rhs, *mwork, *gd, *gr;
    int32_t *info;
};

template <bool MONO, bool GEN, int D>
__global__ void __launch_bounds__(kWave) k_hines(HinesArgs A)
{
    __shared__ double ring_d[kRing][kWave];
    __shared__ double ring_r[kRing][kWave];
    const int k = threadIdx.x;
    int64_t base, ld;
    int32_t rows, my_n, src;
    if (MONO) {
        const int64_t s = int64_t(blockIdx.x) * kWave + k;
        base = s; ld = A.ld; rows = int32_t(A.n);
        my_n = s < A.batch ? rows : 0;
        src = s < A.batch ? int32_t(s) : -1;
    } else {
        const int64_t b = blockIdx.x;
        base = A.blk_off[b] + k; ld = kWave; rows = A.blk_rows[b];
        my_n = A.lane_n[b * kWave + k];
        src = A.lane_src[b * kWave + k];
    }
    const double *u = A.u + base, *l = A.l + base, *d = A.d + base;
    double *rhs = A.rhs + base, *mw = A.mwork + base;
    const int32_t *par = MONO ? A.parent : A.parent + base;
    const int64_t pst = MONO ? 1 : ld;   // parent stride
    double *gd = GEN ? A.gd + base : nullptr, *gr = GEN ? A.gr + base : nullptr;
    auto parent_of = [&](int32_t i) { return par[int64_t(i) * pst]; };

#pragma unroll
    for (int j = 0; j < kRing; ++j) { ring_d[j][k] = 0.0; ring_r[j][k] = 0.0; }

    int32_t bad = 0;
    // ---- leaves -> root elimination --------------------------------------
    // The streamed inputs of row i - D are loaded while row i is eliminated;
    // parent updates are accumulated with LDS atomic adds on the lane's own
    // column (no read on the elimination chain); only the row's own pending
    // value is read back.
    // The general variant's accumulators of far children come in with the
    // row's inputs, D (< kRing) rows ahead: a child more than kRing rows away
    // has been eliminated by then, and its update (a global atomic add that
    // returns nothing) precedes the load in this lane's order.
    double qu[D], ql[D], qd[D], qr[D], qgd[D], qgr[D];
    int32_t qp[D];
    static_assert(D < kRing, "far-child accumulators are read D rows ahead");
    auto load_b = [&](int j, int32_t r) {
        const bool live = r >= 1 && r < my_n;
        const int64_t o = int64_t(live ? r : 0) * ld;
        qu[j] = live ? u[o] : 0.0; ql[j] = live ? l[o] : 0.0;
        qd[j] = live ? d[o] : 1.0; qr[j] = live ? rhs[o] : 0.0;
        if (!MONO) qp[j] = live ? par[o] : 0;
        if (GEN) { qgd[j] = live ? gd[o] : 0.0; qgr[j] = live ? gr[o] : 0.0; }
    };
#pragma unroll
    for (int j = 0; j < D; ++j) load_b(j, rows - 1 - j);
    for (int32_t i0 = rows - 1; i0 >= 1; i0 -= D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int32_t i = i0 - j;
            if (i < 1) break;
            const double ui = qu[j], li = ql[j], di = qd[j], ri = qr[j];
            const double gdi = GEN ? qgd[j] : 0.0, gri = GEN ? qgr[j] : 0.0;
            const int32_t pi = MONO ? parent_of(i) : qp[j];
            load_b(j, i - D);
            if (i >= my_n) continue;
            const int64_t o = int64_t(i) * ld;
            const int slot = i & (kRing - 1);
            double pd = ring_d[slot][k], pr = ring_r[slot][k];
            ring_d[slot][k] = 0.0; ring_r[slot][k] = 0.0;
            if (GEN) { pd += gdi; pr += gri; }
            const double dd = di - pd;               // d'_i
            const double rr = ri - pr;               // rhs'_i
            if (!bad && bad_pivot(dd)) bad = i + 1;
            const double rcp = 1.0 / dd;
            const double fac = ui * rcp;             // factor of Algorithm 1
            rhs[o] = rr * rcp;                       // q_i
            mw[o] = li * rcp;                        // m_i
            if (!GEN || i - pi <= kRing) {
                const int ps = pi & (kRing - 1);
                unsafeAtomicAdd(&ring_d[ps][k], fac * li);
                unsafeAtomicAdd(&ring_r[ps][k], fac * rr);
            } else {
                unsafeAtomicAdd(&gd[int64_t(pi) * ld], fac * li);
                unsafeAtomicAdd(&gr[int64_t(pi) * ld], fac * rr);
            }
        }
    }
    double v0 = 0.0;
    if (my_n > 0) {
        double pd = ring_d[0][k], pr = ring_r[0][k];
        if (GEN) { pd += gd[0]; pr += gr[0]; }
        const double dd = d[0] - pd;
        if (!bad && bad_pivot(dd)) bad = 1;
        v0 = (rhs[0] - pr) / dd;
        rhs[0] = v0;
    }
    if (src >= 0 && A.info) A.info[src] = bad;
    // ---- root -> leaves substitution -------------------------------------
    // ring_d now holds the last kRing voltages (V of row j in slot j mod kRing);
    // a parent one row up comes straight from a register.
    ring_d[0][k] = v0;
    double vprev = v0;
    double fq[D], fm[D];
    int32_t fp[D];
    auto load_f = [&](int j, int32_t r) {
        const bool live = r < my_n;
        const int64_t o = int64_t(live ? r : 0) * ld;
        fq[j] = live ? rhs[o] : 0.0; fm[j] = live ? mw[o] : 0.0;
        if (!MONO) fp[j] = live ? par[o] : 0;
    };
#pragma unroll
    for (int j = 0; j < D; ++j) load_f(j, 1 + j);
    for (int32_t i0 = 1; i0 < rows; i0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int32_t i = i0 + j;
            if (i >= rows) break;
            const double qi = fq[j], mi = fm[j];
            const int32_t pi = MONO ? parent_of(i) : fp[j];
            load_f(j, i + D);
            if (i >= my_n) continue;
            double vp;
            if (i - pi == 1) vp = vprev;
            else if (!GEN || i - pi <= kRing) vp = ring_d[pi & (kRing - 1)][k];
            else vp = rhs[int64_t(pi) * ld];
            const double v = qi - mi * vp;
            rhs[int64_t(i) * ld] = v;
            ring_d[i & (kRing - 1)][k] = v;
            vprev = v;
        }
    }
}

// One tree shared by all lanes and parents within kRing rows: the parent
// index is wave-uniform, so the pending updates and the recent voltages stay
// in registers, indexed by a uniform slot (relative register addressing).
template <int D>
__global__ void __launch_bounds__(kWave) k_hines_mono_reg(HinesArgs A)
{
    const int k = threadIdx.x;
    const int64_t s = int64_t(blockIdx.x) * kWave + k;
    const bool act = s < A.batch;
    const int64_t ld = A.ld;
    const int32_t n = int32_t(A.n);
    // Lanes past the end of the batch shadow the last neuron: they compute
    // exactly what its own lane computes and store the same values, so the
    // hot loops need no branches (a branch around a load or store makes the
    // compiler drain every outstanding load at the join).
    const int64_t base = act ? s : A.batch - 1;
    const double *u = A.u + base, *l = A.l + base, *d = A.d + base;
    double *rhs = A.rhs + base, *mw = A.mwork + base;
    const int32_t *par = A.parent;
    double pend_d[kRing], pend_r[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) { pend_d[j] = 0.0; pend_r[j] = 0.0; }
    int32_t bad = 0;
    double qu[D], ql[D], qd[D], qr[D];
    int32_t qp[D];
    auto load_b = [&](int j, int32_t r) {
        int32_t rr = r >= 1 ? r : 1;
        rr = rr < n ? rr : n - 1;                // n == 1: row 0 (never used)
        const int64_t o = int64_t(rr) * ld;
        qu[j] = u[o]; ql[j] = l[o]; qd[j] = d[o]; qr[j] = rhs[o];
        qp[j] = par[rr];
    };
#pragma unroll
    for (int j = 0; j < D; ++j) load_b(j, n - 1 - j);
    auto elim = [&](int32_t i, double ui, double li, double di, double ri, int32_t pi) {
        const int ps = __builtin_amdgcn_readfirstlane(pi & (kRing - 1));
        const int slot = __builtin_amdgcn_readfirstlane(i & (kRing - 1));
        const double dd = di - pend_d[slot];     // d'_i
        const double rr = ri - pend_r[slot];     // rhs'_i
        pend_d[slot] = 0.0; pend_r[slot] = 0.0;
        if (!bad && bad_pivot(dd)) bad = i + 1;
        const double rcp = 1.0 / dd;
        const double fac = ui * rcp;
        const int64_t o = int64_t(i) * ld;
        rhs[o] = rr * rcp;
        mw[o] = li * rcp;
        pend_d[ps] += fac * li;
        pend_r[ps] += fac * rr;
    };
    // whole blocks of D rows (no exits inside: the loaded values land directly
    // in the look-ahead registers), then the last rows without look-ahead
    int32_t i0 = n - 1;
    for (; i0 - D + 1 >= 1; i0 -= D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const double ui = qu[j], li = ql[j], di = qd[j], ri = qr[j];
            const int32_t pi = qp[j];
            load_b(j, i0 - j - D);
            elim(i0 - j, ui, li, di, ri, pi);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (i0 - j >= 1) elim(i0 - j, qu[j], ql[j], qd[j], qr[j], qp[j]);
    const double dd0 = d[0] - pend_d[0];
    if (!bad && bad_pivot(dd0)) bad = 1;
    const double v0 = (rhs[0] - pend_r[0]) / dd0;
    rhs[0] = v0;
    if (act && A.info) A.info[s] = bad;
    // substitution: recent voltages by slot (pend_d reused)
    pend_d[0] = v0;
    double fq[D], fm[D];
    int32_t fp[D];
    auto load_f = [&](int j, int32_t r) {
        const int32_t rr = r < n ? r : n - 1;
        const int64_t o = int64_t(rr) * ld;
        fq[j] = rhs[o]; fm[j] = mw[o]; fp[j] = par[rr];
    };
#pragma unroll
    for (int j = 0; j < D; ++j) load_f(j, 1 + j);
    auto subst = [&](int32_t i, double qi, double mi, int32_t pi) {
        const int ps = __builtin_amdgcn_readfirstlane(pi & (kRing - 1));
        const double v = qi - mi * pend_d[ps];
        rhs[int64_t(i) * ld] = v;
        pend_d[__builtin_amdgcn_readfirstlane(i & (kRing - 1))] = v;
    };
    int32_t f0 = 1;
    for (; f0 + D - 1 < n; f0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const double qi = fq[j], mi = fm[j];
            const int32_t pi = fp[j];
            load_f(j, f0 + j + D);
            subst(f0 + j, qi, mi, pi);
        }
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (f0 + j < n) subst(f0 + j, fq[j], fm[j], fp[j]);
}

// Buffer-resource access to one block of the packed layout: a wave-uniform
// descriptor (base, size in bytes; accesses beyond the size read zero and
// write nothing), the lane's byte offset in a VGPR and the row's byte
// offset in an SGPR, so that a row costs one memory instruction and no
// address arithmetic.  Third descriptor word for gfx9 raw buffers.
constexpr int kBufWord3 = 0x00020000;
// The base and size are passed through readfirstlane: a descriptor the
// compiler cannot prove uniform would be used through a loop over the
// distinct values in the wavefront at every access.
__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ void *uniform_ptr(const void *p)
{
    return reinterpret_cast<void *>(uniform_i64(reinterpret_cast<int64_t>(p)));
}
struct BlockBuf {
    __amdgpu_buffer_rsrc_t r;
    __device__ BlockBuf(const void *base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0,
                                              int(__builtin_amdgcn_readfirstlane(bytes)), kBufWord3)) {}
    __device__ double ld(uint32_t lane_off, uint32_t row_off) const {
        return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, row_off, 0));
    }
    __device__ int32_t ldi(uint32_t lane_off, uint32_t row_off) const {
        return int32_t(__builtin_amdgcn_raw_buffer_load_b32(r, lane_off, row_off, 0));
    }
    __device__ int32_t ldb(uint32_t lane_off, uint32_t row_off) const {
        return int32_t(__builtin_amdgcn_raw_buffer_load_b8(r, lane_off, row_off, 0));
    }
    __device__ uint32_t ldh(uint32_t lane_off, uint32_t row_off) const {
        return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, lane_off, row_off, 0));
    }
    __device__ void st(double v, uint32_t lane_off, uint32_t row_off) const {
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, lane_off, row_off, 0);
    }
};

// Multi-morphology blocks, parents within kRing rows: branch-free loops.
// Every lane reads and writes only its own column of its block (rows past
// its neuron's size are padding of the packed layout); results of padding
// rows are masked with selects and padding is written back unchanged.
// The largest blocks set the kernel time (one wavefront per block, a serial
// chain per lane), so the instruction count per row matters: rows go
// through buffer descriptors (one instruction per access), the look-ahead
// alternates between two sets of registers (no copies), and the pending
// (d, rhs) updates of a row share one 16-byte LDS slot.
template <int D, bool GEN = false>
__global__ void __launch_bounds__(kWave) k_hines_multi(HinesArgs A)
{
    __shared__ double2 ring[kRing][kWave];
    const int k = threadIdx.x;
    const int64_t b = blockIdx.x;
    // block geometry is wave-uniform: kept in scalar registers, so that row
    // offsets can be the scalar offsets of buffer accesses
    const int64_t off = uniform_i64(A.blk_off[b]);
    const int32_t rows = __builtin_amdgcn_readfirstlane(A.blk_rows[b]);
    const int32_t my_n = A.lane_n[b * kWave + k];
    const int32_t src = A.lane_src[b * kWave + k];
    const uint32_t nbytes = uint32_t(rows) * kWave * 8u;
    const BlockBuf U(A.u + off, nbytes), L(A.l + off, nbytes), Dg(A.d + off, nbytes);
    const BlockBuf R(A.rhs + off, nbytes), MW(A.mwork + off, nbytes);
    // parents as one-byte distances i - p_i (the window holds them): a
    // quarter of the bytes of int32 indices in both sweeps
    const BlockBuf PD(A.dist8 + off, nbytes / 8);
    // GEN: a distance byte of kFar marks a parent more than kRing rows up;
    // its index comes from the packed parents, and its pending updates go
    // to the lane's global accumulators (atomic adds that return nothing),
    // which a row reads with its inputs, D (< kRing) rows ahead: every child
    // more than kRing rows away has added to them by then, in this lane's
    // order
    static_assert(!GEN || D < kRing, "far-child accumulators are read D rows ahead");
    const BlockBuf PI(GEN ? static_cast<const void *>(A.parent + off) : A.u, GEN ? nbytes / 2 : 8u);
    const BlockBuf GD(GEN ? static_cast<const void *>(A.gd + off) : A.u, GEN ? nbytes : 8u);
    const BlockBuf GR(GEN ? static_cast<const void *>(A.gr + off) : A.u, GEN ? nbytes : 8u);
    const uint32_t lo8 = uint32_t(k) * 8u, lo1 = uint32_t(k);   // lane byte offsets
    // row byte offsets (scalar: a buffer access takes its row offset from an SGPR)
    auto rb8 = [](int32_t r) { return __builtin_amdgcn_readfirstlane(uint32_t(r) * (kWave * 8u)); };
    auto rb1 = [](int32_t r) { return __builtin_amdgcn_readfirstlane(uint32_t(r) * uint32_t(kWave)); };
#pragma unroll
    for (int j = 0; j < kRing; ++j) ring[j][k] = make_double2(0.0, 0.0);
    int32_t bad = 0;

    // ---- leaves -> root ----
    struct BRow { double u, l, d, r, gd, gr; int32_t p, pi; };   // p: distance to the parent
    auto load_b = [&](BRow &q, int32_t r) {
        const int32_t rc = r >= 1 ? r : 1 < rows ? 1 : 0;
        q.u = U.ld(lo8, rb8(rc)); q.l = L.ld(lo8, rb8(rc)); q.d = Dg.ld(lo8, rb8(rc));
        q.r = R.ld(lo8, rb8(rc)); q.p = PD.ldb(lo1, rb1(rc));
        if (GEN) {
            q.gd = GD.ld(lo8, rb8(rc)); q.gr = GR.ld(lo8, rb8(rc));
            q.pi = PI.ldi(lo8 / 2, rb8(rc) / 2);
        }
    };
    auto elim = [&](int32_t i, const BRow &q) {
        const bool live = i < my_n;
        const int slot = i & (kRing - 1);
        double2 pp = ring[slot][k];
        ring[slot][k] = make_double2(0.0, 0.0);
        if (GEN) { pp.x += q.gd; pp.y += q.gr; }
        const double dd = q.d - pp.x;            // d'_i
        const double rr = q.r - pp.y;            // rhs'_i
        if (live && !bad && bad_pivot(dd)) bad = i + 1;
        const double rcp = 1.0 / dd;
        const double fac = live ? q.u * rcp : 0.0;  // factor of Algorithm 1
        R.st(live ? rr * rcp : q.r, lo8, rb8(i));   // q_i (padding unchanged)
        MW.st(live ? q.l * rcp : 0.0, lo8, rb8(i)); // m_i
        if (GEN && q.p == kFar) {
            const int64_t pe = off + int64_t(q.pi) * kWave + k;
            unsafeAtomicAdd(&A.gd[pe], fac * q.l);
            unsafeAtomicAdd(&A.gr[pe], fac * rr);
        } else {
            const int ps = (i - q.p) & (kRing - 1);
            unsafeAtomicAdd(&ring[ps][k].x, fac * q.l);
            unsafeAtomicAdd(&ring[ps][k].y, fac * rr);
        }
    };
    BRow qa[D], qb[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_b(qa[j], rows - 1 - j);
    int32_t i0 = rows - 1;
    // two groups per iteration: the group in one set is worked on while the
    // next one arrives in the other
    for (; i0 - 2 * D + 1 >= 1; i0 -= 2 * D) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qb[j], i0 - D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - j, qa[j]);
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qa[j], i0 - 2 * D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - D - j, qb[j]);
    }
    if (i0 - D + 1 >= 1) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qb[j], i0 - D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - j, qa[j]);
        i0 -= D;
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (i0 - j >= 1) elim(i0 - j, qb[j]);
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (i0 - j >= 1) elim(i0 - j, qa[j]);
    }
    const bool root = my_n > 0;
    double2 p0 = ring[0][k];
    if (GEN) { p0.x += GD.ld(lo8, 0); p0.y += GR.ld(lo8, 0); }
    const double dd0 = Dg.ld(lo8, 0) - p0.x;
    if (root && !bad && bad_pivot(dd0)) bad = 1;
    const double r0 = R.ld(lo8, 0);
    const double v0 = root ? (r0 - p0.y) / dd0 : 0.0;
    R.st(root ? v0 : r0, lo8, 0);
    if (src >= 0 && A.info) A.info[src] = bad;

    // ---- root -> leaves; ring (.x) holds recent voltages by slot, a
    // parent one row up comes from a register ----
    ring[0][k].x = v0;
    double vprev = v0;
    struct FRow { double q, m; int32_t p, pi; };     // p: distance to the parent
    auto load_f = [&](FRow &f, int32_t r) {
        const int32_t rc = r < rows ? r : rows - 1;
        f.q = R.ld(lo8, rb8(rc)); f.m = MW.ld(lo8, rb8(rc)); f.p = PD.ldb(lo1, rb1(rc));
        if (GEN) f.pi = PI.ldi(lo8 / 2, rb8(rc) / 2);
    };
    auto subst = [&](int32_t i, const FRow &f) {
        const bool live = i < my_n;
        double vr = ring[(i - f.p) & (kRing - 1)][k].x;
        // a far parent's voltage, written long before (its row differs by lane)
        if (GEN && f.p == kFar) vr = R.ld(lo8 + uint32_t(f.pi) * (kWave * 8u), 0);
        const double vp = (f.p == 1) ? vprev : vr;
        const double v = f.q - f.m * vp;
        R.st(live ? v : f.q, lo8, rb8(i));
        ring[i & (kRing - 1)][k].x = v;
        vprev = v;
    };
    FRow fa[D], fb[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_f(fa[j], 1 + j);
    int32_t f0 = 1;
    for (; f0 + 2 * D - 1 < rows; f0 += 2 * D) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fb[j], f0 + D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + j, fa[j]);
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fa[j], f0 + 2 * D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + D + j, fb[j]);
    }
    if (f0 + D - 1 < rows) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fb[j], f0 + D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + j, fa[j]);
        f0 += D;
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (f0 + j < rows) subst(f0 + j, fb[j]);
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (f0 + j < rows) subst(f0 + j, fa[j]);
    }
}

// Multi-morphology blocks in which some trees run on two lanes (an aligned
// pair; the plan's schedule, see build_split) and the others on one.  Each
// row's code names its own slot and its parent's (a lane ring, the pair's
// trunk ring, or the lane's sink), so the kernel keeps no counters and no
// row branches on its kind: padding and waiting rows read, clear and feed
// the sink, and what they store in rhs and work is never read.  Everything
// else follows k_hines_multi.
template <int D>
__global__ void __launch_bounds__(kWave) k_hines_split(HinesArgs A)
{
    // slot id s of lane k: ring[s][k]; the odd lane of a pair reaches the
    // trunk slots in the even lane's column (code bit 14)
    __shared__ double2 ring[kSlots][kWave];
    const int k = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t off = uniform_i64(A.blk_off[b]);
    const int32_t rows = __builtin_amdgcn_readfirstlane(A.blk_rows[b]);
    const int32_t src = A.lane_src[b * kWave + k];
    const uint32_t nbytes = uint32_t(rows) * kWave * 8u;
    const BlockBuf U(A.u + off, nbytes), L(A.l + off, nbytes), Dg(A.d + off, nbytes);
    const BlockBuf R(A.rhs + off, nbytes), MW(A.mwork + off, nbytes);
    const BlockBuf PC(A.code16 + off, nbytes / 4);
    const uint32_t lo8 = uint32_t(k) * 8u, lo2 = uint32_t(k) * 2u;
    auto rb8 = [](int32_t r) { return __builtin_amdgcn_readfirstlane(uint32_t(r) * (kWave * 8u)); };
    auto rb2 = [](int32_t r) { return __builtin_amdgcn_readfirstlane(uint32_t(r) * (kWave * 2u)); };
    const uint32_t kl = uint32_t(k);
#pragma unroll
    for (int j = 0; j < kSlots; ++j) ring[j][k] = make_double2(0.0, 0.0);
    // (slot ids are at most 32: build_split writes them, split_check rejects
    // a schedule with any other)
    auto own_slot = [&](uint32_t c) -> double2 & { return ring[c & 63u][kl]; };
    auto parent_slot = [&](uint32_t c) -> double2 & { return ring[(c >> 6) & 63u][kl & ~((c >> 14) & 1u)]; };
    int32_t bad = 0;

    // ---- leaves -> root ----
    struct BRow { double u, l, d, r; uint32_t c; };
    auto load_b = [&](BRow &q, int32_t r) {
        const int32_t rc = r >= 0 ? r : 0;
        q.u = U.ld(lo8, rb8(rc)); q.l = L.ld(lo8, rb8(rc)); q.d = Dg.ld(lo8, rb8(rc));
        q.r = R.ld(lo8, rb8(rc)); q.c = PC.ldh(lo2, rb2(rc));
    };
    auto elim = [&](int32_t i, const BRow &q) {
        const bool live = q.c & kCodeLive;
        double2 &own = own_slot(q.c);
        const double2 pp = own;
        own = make_double2(0.0, 0.0);
        const double dd = q.d - pp.x;            // d'_i
        const double rr = q.r - pp.y;            // rhs'_i
        if (live & bad_pivot(dd)) bad = max(bad, 1 + A.comp[off + int64_t(i) * kWave + k]);
        const double rcp = 1.0 / dd;
        const double fac = q.u * rcp;            // factor of Algorithm 1
        R.st(rr * rcp, lo8, rb8(i));             // q_i (padding: unspecified)
        MW.st(q.l * rcp, lo8, rb8(i));           // m_i
        double2 &par = parent_slot(q.c);
        unsafeAtomicAdd(&par.x, fac * q.l);
        unsafeAtomicAdd(&par.y, fac * rr);
    };
    BRow qa[D], qb[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_b(qa[j], rows - 1 - j);
    int32_t i0 = rows - 1;
    for (; i0 - 2 * D + 1 >= 0; i0 -= 2 * D) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qb[j], i0 - D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - j, qa[j]);
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qa[j], i0 - 2 * D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - D - j, qb[j]);
    }
    if (i0 - D + 1 >= 0) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_b(qb[j], i0 - D - j);
#pragma unroll
        for (int j = 0; j < D; ++j) elim(i0 - j, qa[j]);
        i0 -= D;
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (i0 - j >= 0) elim(i0 - j, qb[j]);
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (i0 - j >= 0) elim(i0 - j, qa[j]);
    }
    // a tree's info: 1 + the largest index of a bad pivot over its lanes
    const int32_t other_src = __builtin_amdgcn_mov_dpp(src, 0xB1, 0xF, 0xF, false);
    const int32_t other_bad = __builtin_amdgcn_mov_dpp(bad, 0xB1, 0xF, 0xF, false);
    const bool paired = src >= 0 && other_src == src;
    if (src >= 0 && A.info && (!paired || (k & 1) == 0)) A.info[src] = paired ? max(bad, other_bad) : bad;

    // ---- root -> leaves: a slot holds the voltage its row stored last.  The
    // sink starts at 0: a root (the first live row of its lanes here) reads
    // it as its parent's voltage ----
    ring[kSlotSink][k] = make_double2(0.0, 0.0);
    double vprev = 0.0;
    struct FRow { double q, m; uint32_t c; };
    auto load_f = [&](FRow &f, int32_t r) {
        const int32_t rc = r < rows ? r : rows - 1;
        f.q = R.ld(lo8, rb8(rc)); f.m = MW.ld(lo8, rb8(rc)); f.c = PC.ldh(lo2, rb2(rc));
    };
    auto subst = [&](int32_t i, const FRow &f) {
        const bool live = f.c & kCodeLive;
        const double vr = parent_slot(f.c).x;
        const double v = f.q - f.m * ((f.c & kCodeVreg) ? vprev : vr);
        R.st(v, lo8, rb8(i));
        own_slot(f.c).x = v;
        vprev = live ? v : vprev;
    };
    FRow fa[D], fb[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_f(fa[j], j);
    int32_t f0 = 0;
    for (; f0 + 2 * D - 1 < rows; f0 += 2 * D) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fb[j], f0 + D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + j, fa[j]);
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fa[j], f0 + 2 * D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + D + j, fb[j]);
    }
    if (f0 + D - 1 < rows) {
#pragma unroll
        for (int j = 0; j < D; ++j) load_f(fb[j], f0 + D + j);
#pragma unroll
        for (int j = 0; j < D; ++j) subst(f0 + j, fa[j]);
        f0 += D;
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (f0 + j < rows) subst(f0 + j, fb[j]);
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (f0 + j < rows) subst(f0 + j, fa[j]);
    }
}

// ---- level schedule -----------------------------------------------------------
//
// For batches of few neurons one lane per neuron leaves most of the chip
// idle.  Here one wavefront takes one neuron and parallelises inside its tree
// (the per-branch, per-level decomposition of section 4 of the Hines page):
// the tree is cut into sections (maximal unbranched paths: a node starts a
// section when it is the root or its parent has several children), nodes
// are renumbered so that each section is a contiguous range head -> tail,
// and a section's level is one more than the highest level of the sections
// hanging from its tail (leaf sections: 0).  The neuron's u, l, d, rhs are
// gathered into LDS in that order; the elimination runs level by level, one
// section per lane, from the tail to the head (the parent of every node but
// the head is the node before it, so the update is carried in registers);
// the head's update to its parent (the tail of a higher-level section) is an
// LDS atomic add.  Substitution runs the levels in reverse, head to tail.
// Between the sweeps the LDS copies of d and rhs hold m_i = l_i / d'_i and
// q_i = rhs'_i / d'_i, as in the one-lane-per-neuron kernels.  info = 1 + the
// largest index of a bad pivot, the first one Algorithm 1's order meets.
struct LevelArgs {
    int64_t ld, nwg;
    int mono;
    const int32_t *lane_src;     // multi: neuron at each position of the packed layout
    const int64_t *tree;
    const int32_t *perm, *sec, *spar, *lev;
    const double *u, *l, *d;
    double *rhs;
    int32_t *info;
};

__global__ void __launch_bounds__(kWave) k_hines_levels(LevelArgs A)
{
    extern __shared__ double lv_lds[];
    __shared__ int32_t bad;
    // A neuron's values share cache lines with its neighbours in the solver
    // layout (16 per 128-byte row segment mono, 64 per block row multi).
    // Workgroups are dispatched round-robin over the 8 XCDs, each with its
    // own L2: give the workgroups one XCD runs neighbouring positions, so
    // that a line is fetched once instead of once per XCD.
    const int64_t nb = A.nwg, bid = blockIdx.x, full = nb & ~int64_t(7);
    const int64_t pos = bid < full ? (bid & 7) * (full >> 3) + (bid >> 3) : bid;
    const int64_t s = A.mono ? pos : A.lane_src[pos];
    if (s < 0) return;               // an empty lane of the last block
    const int k = threadIdx.x;
    const int64_t *t = A.tree + (A.mono ? 0 : 6 * s);
    const int32_t *perm = A.perm + t[0], *sec = A.sec + t[1], *spar = A.spar + t[1];
    const int32_t *lev = A.lev + t[2];
    const int32_t nlev = int32_t(t[3]), n = int32_t(t[4]);
    const int64_t base = A.mono ? s : t[5];
    const int64_t stride = A.mono ? A.ld : kWave;
    double *dd = lv_lds, *rr = lv_lds + n, *uu = lv_lds + 2 * n, *ll = lv_lds + 3 * n;
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    if (k == 0) bad = 0;
    for (int32_t j = k; j < n; j += kWave) {
        const int64_t o = base + int64_t(perm[j]) * stride;
        dd[j] = A.d[o];
        rr[j] = A.rhs[o];
        const bool root = perm[j] == 0;   // no coupling above the root
        uu[j] = root ? 0.0 : A.u[o];
        ll[j] = root ? 0.0 : A.l[o];
    }
    wave_sync();
    int32_t mybad = 0;
    // ---- leaves -> root, level by level ----
    for (int32_t L = 0; L < nlev; ++L) {
        for (int32_t q = lev[L] + k; q < lev[L + 1]; q += kWave) {
            const int32_t s0 = sec[q], s1 = sec[q + 1];
            double cd = 0.0, cr = 0.0;
            for (int32_t j = s1 - 1; j >= s0; --j) {
                const double dj = dd[j] - cd, rj = rr[j] - cr;
                if (bad_pivot(dj)) mybad = max(mybad, perm[j] + 1);
                const double rc = 1.0 / dj;
                const double fac = uu[j] * rc;
                dd[j] = ll[j] * rc;        // m_j
                rr[j] = rj * rc;           // q_j
                cd = fac * ll[j];
                cr = fac * rj;
            }
            const int32_t ph = spar[q];
            if (ph >= 0) {
                unsafeAtomicAdd(&dd[ph], -cd);
                unsafeAtomicAdd(&rr[ph], -cr);
            }
        }
        wave_sync();
    }
    // ---- root -> leaves ----
    for (int32_t L = nlev - 1; L >= 0; --L) {
        for (int32_t q = lev[L] + k; q < lev[L + 1]; q += kWave) {
            const int32_t s0 = sec[q], s1 = sec[q + 1], ph = spar[q];
            double vp = ph >= 0 ? rr[ph] : 0.0;
            for (int32_t j = s0; j < s1; ++j) {
                const double v = rr[j] - dd[j] * vp;
                rr[j] = v;
                vp = v;
            }
        }
        wave_sync();
    }
    if (mybad) atomicMax(&bad, mybad);
    for (int32_t j = k; j < n; j += kWave) A.rhs[base + int64_t(perm[j]) * stride] = rr[j];
    wave_sync();
    if (k == 0 && A.info) A.info[s] = bad;
}

// Sections of one tree (parent[0] ignored), renumbered and ordered by level.
struct LevelTree {
    std::vector<int32_t> perm, sec, spar, lev;
};

static void build_level_tree(int32_t n, const int32_t *p, LevelTree &T)
{
    std::vector<int32_t> nch(n, 0), only(n, -1);
    for (int32_t i = 1; i < n; ++i) nch[p[i]]++;
    for (int32_t i = 1; i < n; ++i)
        if (nch[p[i]] == 1) only[p[i]] = i;
    std::vector<int32_t> heads;
    for (int32_t i = 0; i < n; ++i)
        if (i == 0 || nch[p[i]] != 1) heads.push_back(i);
    const int32_t ns = int32_t(heads.size());
    std::vector<int32_t> sec_of(n, -1), len(ns, 0), level(ns, 0);
    for (int32_t h = 0; h < ns; ++h) {
        int32_t c = heads[h];
        while (true) {
            sec_of[c] = h;
            ++len[h];
            if (nch[c] != 1) break;
            c = only[c];
        }
    }
    // a child section's head has a larger index than every node of its
    // parent section's head, so decreasing head order visits children first
    for (int32_t h = ns - 1; h >= 1; --h) {
        const int32_t ps = sec_of[p[heads[h]]];
        level[ps] = std::max(level[ps], level[h] + 1);
    }
    std::vector<int32_t> ord(ns);
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) {
        return level[x] != level[y] ? level[x] < level[y] : len[x] > len[y];
    });
    T.perm.assign(n, 0);
    T.sec.assign(ns + 1, n);
    T.spar.assign(ns + 1, -1);
    std::vector<int32_t> newidx(n, 0);
    int32_t pos = 0;
    for (int32_t q = 0; q < ns; ++q) {
        T.sec[q] = pos;
        int32_t c = heads[ord[q]];
        while (true) {
            T.perm[pos] = c;
            newidx[c] = pos++;
            if (nch[c] != 1) break;
            c = only[c];
        }
    }
    for (int32_t q = 0; q < ns; ++q) {
        const int32_t hd = heads[ord[q]];
        T.spar[q] = hd == 0 ? -1 : newidx[p[hd]];
    }
    const int32_t nlev = level[ord[ns - 1]] + 1;
    T.lev.assign(nlev + 1, 0);
    for (int32_t q = 0; q < ns; ++q) T.lev[level[ord[q]] + 1]++;
    for (int32_t L = 0; L < nlev; ++L) T.lev[L + 1] += T.lev[L];
}

__global__ void k_fill_zero(double *p, int64_t count)
{
    for (int64_t i = lane_id(); i < count; i += int64_t(gridDim.x) * blockDim.x) p[i] = 0.0;
}

// ---- layout transforms ---------------------------------------------------------

// mono: flat [batch][n]  <->  interleaved [n][ld].  Packing walks every
// element of the interleaved array, padding columns (s >= batch) included,
// and writes those as 0; unpacking reads the batch real columns only.
template <typename T, bool PACK>
__global__ void k_mono_transpose(int64_t n, int64_t batch, int64_t ld, const T *__restrict__ src,
                                 T *__restrict__ dst)
{
    const int64_t cols = PACK ? ld : batch;
    const int64_t total = n * cols;
    for (int64_t e = lane_id(); e < total; e += int64_t(gridDim.x) * blockDim.x) {
        const int64_t i = e / cols, s = e % cols;     // interleaved order: coalesced side
        if (PACK) dst[i * ld + s] = s < batch ? src[s * n + i] : T(0);
        else dst[s * n + i] = src[i * ld + s];
    }
}

// multi: flat (neuron after neuron)  <->  block-interleaved [rows_b][64]
template <typename T, bool PACK>
__global__ void k_multi_pack(const int64_t *__restrict__ blk_off, const int32_t *__restrict__ blk_rows,
                             const int32_t *__restrict__ lane_n, const int32_t *__restrict__ lane_src,
                             const int64_t *__restrict__ src_off, const T *__restrict__ src,
                             T *__restrict__ dst)
{
    const int64_t b = blockIdx.x;
    const int64_t rows = blk_rows[b], off = blk_off[b];
    for (int64_t e = threadIdx.x; e < rows * kWave; e += blockDim.x) {
        const int64_t i = e / kWave;
        const int k = int(e % kWave);
        const int32_t s = lane_src[b * kWave + k];
        const bool live = s >= 0 && i < lane_n[b * kWave + k];
        if (PACK) dst[off + e] = live ? src[src_off[s] + i] : T(0);
        else if (live) dst[src_off[s] + i] = src[off + e];
    }
}

// multi with trees on two lanes: the compartment of each packed element is
// listed (comp, -1 for padding), since a split tree's rows are in schedule
// order
template <typename T, bool PACK>
__global__ void k_multi_pack_map(const int64_t *__restrict__ blk_off, const int32_t *__restrict__ blk_rows,
                                 const int32_t *__restrict__ lane_src, const int32_t *__restrict__ comp,
                                 const int64_t *__restrict__ src_off, const T *__restrict__ src,
                                 T *__restrict__ dst)
{
    const int64_t b = blockIdx.x;
    const int64_t rows = blk_rows[b], off = blk_off[b];
    for (int64_t e = threadIdx.x; e < rows * kWave; e += blockDim.x) {
        const int k = int(e % kWave);
        const int32_t s = lane_src[b * kWave + k];
        const int32_t c = comp[off + e];
        const bool live = s >= 0 && c >= 0;
        if (PACK) dst[off + e] = live ? src[src_off[s] + c] : T(0);
        else if (live) dst[src_off[s] + c] = src[off + e];
    }
}

// ---- host side -------------------------------------------------------------------

template <typename T>
static bps_status upload(T **dptr, const std::vector<T> &h)
{
    if (h.empty()) { *dptr = nullptr; return BPS_OK; }
    hipError_t e = hipMalloc((void **)dptr, h.size() * sizeof(T));
    if (e != hipSuccess) BPS_FAIL(BPS_ENOMEM, "hipMalloc of %zu bytes failed: %s",
                                  h.size() * sizeof(T), hipGetErrorString(e));
    BPS_HIP(hipMemcpy(*dptr, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return BPS_OK;
}

static void free_plan(bps_hines_plan *p)
{
    if (!p) return;
    (void)hipFree(p->parent); (void)hipFree(p->dist8); (void)hipFree(p->blk_off);
    (void)hipFree(p->blk_rows);
    (void)hipFree(p->lane_n); (void)hipFree(p->lane_src); (void)hipFree(p->src_off);
    (void)hipFree(p->lv_perm); (void)hipFree(p->lv_sec); (void)hipFree(p->lv_spar);
    (void)hipFree(p->lv_lev); (void)hipFree(p->lv_tree);
    (void)hipFree(p->code16); (void)hipFree(p->comp); (void)hipFree(p->sep_dev);
    (void)hipFree(const_cast<int32_t *>(p->sepm.lanetab)); (void)hipFree(const_cast<int32_t *>(p->sepm.tabs));
    (void)hipFree(const_cast<int32_t *>(p->sepm.pos)); (void)hipFree(const_cast<int64_t *>(p->sepm.wgoff));
    (void)hipFree(p->flat_parent);
    free_plan(p->rest);
    delete p;
}

// Level schedules of the batch's trees (one for a shared tree), uploaded.
// data_base: per tree, where its values start in the solver layout (multi).
static bps_status build_levels(bps_hines_plan *P, int64_t ntrees, const int32_t *sizes,
                               const int32_t *parent, const std::vector<int64_t> &data_base)
{
    std::vector<int32_t> perm, sec, spar, lev;
    std::vector<int64_t> tree(6 * ntrees);
    int64_t off = 0;
    LevelTree T;
    for (int64_t s = 0; s < ntrees; ++s) {
        const int32_t n = sizes[s];
        build_level_tree(n, parent + off, T);
        int64_t *d = &tree[6 * s];
        d[0] = int64_t(perm.size()); d[1] = int64_t(sec.size()); d[2] = int64_t(lev.size());
        d[3] = int64_t(T.lev.size()) - 1; d[4] = n; d[5] = data_base.empty() ? 0 : data_base[s];
        perm.insert(perm.end(), T.perm.begin(), T.perm.end());
        sec.insert(sec.end(), T.sec.begin(), T.sec.end());
        spar.insert(spar.end(), T.spar.begin(), T.spar.end());
        lev.insert(lev.end(), T.lev.begin(), T.lev.end());
        P->lv_maxn = std::max(P->lv_maxn, n);
        off += n;
    }
    bps_status st;
    if ((st = upload(&P->lv_perm, perm)) != BPS_OK) return st;
    if ((st = upload(&P->lv_sec, sec)) != BPS_OK) return st;
    if ((st = upload(&P->lv_spar, spar)) != BPS_OK) return st;
    if ((st = upload(&P->lv_lev, lev)) != BPS_OK) return st;
    return upload(&P->lv_tree, tree);
}

// ---- two lanes per neuron (multi-morphology) ----------------------------------
//
// With one lane per neuron the largest trees of a batch set the time of the
// launch: their lanes run a serial chain of n rows while the rest of the
// GPU has finished.  Such a tree is split over two lanes of its wavefront
// (the per-branch decomposition of section 4 of the Hines page, done inside
// one wavefront): the trunk (the path from the root that always descends
// into the largest subtree) and the side branches hanging from it.  Lane 0
// eliminates the trunk from its deepest node upwards as each trunk node's
// branches are done; both lanes eliminate side branches, deepest attachment
// first, each branch in decreasing index order.  A trunk node's pending
// update lives in a ring of 16 slots shared by the pair (slot = its position
// on the trunk mod 16); a branch node's in the lane's own ring (slot = the
// lane's count of branch rows mod 16).  The schedule is lockstep (one row
// per lane and step, bubbles where a lane waits), and is checked here by
// replaying both sweeps' slot traffic; a tree that fails stays on one lane.
//
// Row code (one byte per row and lane): bit 7 live, bit 6 trunk row,
// bits 4-5 where the parent's pending update / voltage is (0 the lane's
// ring, 2 the trunk ring, 3 no parent), bits 0-3 the slot (a trunk row: its
// own slot; its parent is the trunk slot before it).
namespace {

struct SplitLane {
    std::vector<int32_t> node;   // per step (first sweep order): compartment, -1 waiting
    std::vector<uint16_t> code;  // per step: row_code
};

// Replays both sweeps of k_hines_split on the slot level for one tree on a
// lane pair: every pending update reaches its parent's slot before the
// parent reads it, and every parent voltage read finds the parent's.
bool split_check(int32_t n, const int32_t *p, const SplitLane lane[2])
{
    const int32_t rows = int32_t(lane[0].node.size());
    std::vector<int32_t> nch(n, 0);
    for (int32_t i = 1; i < n; ++i) ++nch[p[i]];
    struct Slot { int32_t tag = -1, count = 0; };
    // [lane][slot id]: a row's own slot in its lane's column, its parent's in
    // the even lane's when the code says so
    Slot sl[2][kSlots];
    auto at = [&](int j, int id) -> Slot & { return sl[j][id]; };
    int32_t seen = 0;
    for (int32_t s = 0; s < rows; ++s) {
        for (int j = 0; j < 2; ++j) {            // read and clear the own slot
            const uint16_t c = lane[j].code[s];
            const int own = c & 63, par = (c >> 6) & 63;
            if (own >= kSlots || par >= kSlots) return false;
            if (!(c & kCodeLive)) { if (own != kSlotSink || par != kSlotSink) return false; continue; }
            const int32_t x = lane[j].node[s];
            if (own == kSlotSink) return false;
            Slot &o = at(j, own);
            if (o.count != nch[x] || (nch[x] && o.tag != x)) return false;
            o = Slot{};
            ++seen;
        }
        for (int j = 0; j < 2; ++j) {            // add to the parent's slot
            const uint16_t c = lane[j].code[s];
            if (!(c & kCodeLive)) continue;
            const int32_t x = lane[j].node[s];
            const int par = (c >> 6) & 63;
            if ((par == kSlotSink) != (x == 0)) return false;
            if (x == 0) continue;
            Slot &q = at((c & kCodeEven) ? 0 : j, par);
            if (q.count && q.tag != p[x]) return false;
            q.tag = p[x];
            ++q.count;
        }
    }
    if (seen != n) return false;
    // substitution: steps in reverse; a slot holds the last voltage stored
    int32_t vs[2][kSlots], vprev[2] = {-1, -1};
    std::fill(&vs[0][0], &vs[0][0] + 2 * kSlots, -1);
    auto vat = [&](int j, int id) -> int32_t & { return vs[j][id]; };
    bool root_done = false;
    for (int32_t s = rows - 1; s >= 0; --s) {
        int32_t got[2] = {-2, -2};
        for (int j = 0; j < 2; ++j) {            // read the parent's voltage
            const uint16_t c = lane[j].code[s];
            if (!(c & kCodeLive)) continue;
            const int32_t x = lane[j].node[s];
            const int par = (c >> 6) & 63;
            if (x == 0) {                        // the root reads the zeroed sink, first
                if (root_done || s != rows - 1 || j != 0 || (c & kCodeVreg)) return false;
                root_done = true;
                continue;
            }
            got[j] = (c & kCodeVreg) ? vprev[j] : vat((c & kCodeEven) ? 0 : j, par);
            if (got[j] != p[x]) return false;
        }
        for (int j = 0; j < 2; ++j) {            // store the own voltage
            const uint16_t c = lane[j].code[s];
            if (!(c & kCodeLive)) continue;
            const int32_t x = lane[j].node[s];
            vat(j, c & 63) = x;
            vprev[j] = x;
        }
    }
    return root_done;
}

// The two-lane schedule of one tree (parents p, p_0 ignored); false when
// the greedy schedule does not close or fails the replay.
bool split_schedule(int32_t n, const int32_t *p, SplitLane lane[2])
{
    if (n < 2) return false;
    std::vector<int32_t> sz(n, 1), first(n + 1, 0), kids(n > 1 ? n - 1 : 0);
    for (int32_t i = n - 1; i >= 1; --i) sz[p[i]] += sz[i];
    for (int32_t i = 1; i < n; ++i) ++first[p[i] + 1];
    for (int32_t i = 0; i < n; ++i) first[i + 1] += first[i];
    {
        std::vector<int32_t> fill(first.begin(), first.end() - 1);
        for (int32_t i = 1; i < n; ++i) kids[fill[p[i]]++] = i;     // children in increasing index
    }
    std::vector<int32_t> trunk, tpos(n, -1);
    for (int32_t v = 0;;) {
        tpos[v] = int32_t(trunk.size());
        trunk.push_back(v);
        int32_t best = -1;
        for (int32_t e = first[v]; e < first[v + 1]; ++e)
            if (best < 0 || sz[kids[e]] > sz[best]) best = kids[e];
        if (best < 0) break;
        v = best;
    }
    const int32_t L = int32_t(trunk.size());
    // side branches, deepest attachment first, each in decreasing index order
    struct Branch { int32_t attach, begin, end; };
    std::vector<Branch> br;
    std::vector<int32_t> bn, stack, pending(L, 0);
    bn.reserve(n);
    for (int32_t k = L - 1; k >= 0; --k) {
        const int32_t t = trunk[k];
        for (int32_t e = first[t]; e < first[t + 1]; ++e) {
            const int32_t c = kids[e];
            if (tpos[c] >= 0) continue;
            const int32_t b0 = int32_t(bn.size());
            stack.assign(1, c);
            while (!stack.empty()) {
                const int32_t x = stack.back();
                stack.pop_back();
                bn.push_back(x);
                for (int32_t f = first[x]; f < first[x + 1]; ++f) stack.push_back(kids[f]);
            }
            std::sort(bn.begin() + b0, bn.end(), std::greater<int32_t>());
            br.push_back({k, b0, int32_t(bn.size())});
            ++pending[k];
        }
    }
    std::vector<int32_t> tstep(L, -1), cnt_of(n, -1), lane_of(n, -1);
    int32_t nextk = L - 1, cnt[2] = {0, 0}, cur[2] = {-1, -1}, pos[2] = {0, 0};
    size_t qi = 0;
    for (int j = 0; j < 2; ++j) { lane[j].node.clear(); lane[j].code.clear(); }
    for (int32_t step = 0; nextk >= 0; ++step) {
        if (step > 2 * n + 4 * kRing) return false;
        const bool ready = pending[nextk] == 0 && (nextk == L - 1 || tstep[nextk + 1] >= 0);
        for (int j = 0; j < 2; ++j) {
            if (j == 0 && ready) {
                lane[0].node.push_back(trunk[nextk]);
                tstep[nextk] = step;
                lane_of[trunk[nextk]] = 0;
                --nextk;
                continue;
            }
            if (cur[j] < 0 && qi < br.size()) { cur[j] = int32_t(qi++); pos[j] = br[cur[j]].begin; }
            if (cur[j] < 0) { lane[j].node.push_back(-1); continue; }
            const Branch &B = br[cur[j]];
            // a branch root's update goes to trunk slot (attach mod 16): the
            // trunk node 16 positions deeper must have taken its own first
            if (pos[j] + 1 == B.end && B.attach + kRing < L && tstep[B.attach + kRing] < 0) {
                lane[j].node.push_back(-1);
                continue;
            }
            const int32_t x = bn[pos[j]];
            lane[j].node.push_back(x);
            cnt_of[x] = cnt[j]++;
            lane_of[x] = j;
            if (++pos[j] == B.end) { --pending[B.attach]; cur[j] = -1; }
        }
    }
    if (qi != br.size() || cur[0] >= 0 || cur[1] >= 0) return false;
    // a tree whose trunk is most of it (a chain) gains too little from a
    // second lane to pay for the lane
    if (5 * int64_t(lane[0].node.size()) > 4 * int64_t(n)) return false;
    // slot ids: a branch row's is its count mod 16 in its lane, a trunk row's
    // 16 + its trunk position mod 16; the voltage register serves a parent
    // that is the lane's previous live row in the substitution
    auto slot_of = [&](int32_t x) {
        return tpos[x] >= 0 ? kSlotTrunk + (tpos[x] & (kRing - 1)) : cnt_of[x] & (kRing - 1);
    };
    for (int j = 0; j < 2; ++j) {
        const size_t m = lane[j].node.size();
        lane[j].code.assign(m, row_code(kSlotSink, kSlotSink, false, false));
        int32_t prev = -1;                       // previous live row, substitution order
        for (size_t t = m; t-- > 0;) {
            const int32_t x = lane[j].node[t];
            if (x < 0) continue;
            if (x != 0 && tpos[p[x]] < 0 && lane_of[p[x]] != j) return false;
            if (j == 1 && tpos[x] >= 0) return false;         // the trunk is lane 0's
            const int par = x == 0 ? kSlotSink : slot_of(p[x]);
            lane[j].code[t] = row_code(slot_of(x), par, true, x != 0 && p[x] == prev,
                                       j == 1 && par >= kSlotTrunk && par < kSlotSink);
            prev = x;
        }
    }
    return split_check(n, p, lane);
}

}  // namespace

// Multi-morphology plan with up to `want` trees on two lanes: the largest
// of at least kSplitMin compartments whose schedules close.  Units (a tree on one lane, or a
// split tree on an aligned pair of lanes) are sorted by their row count and
// dealt 64 lanes per block; a unit of m rows occupies rows m-1 .. 0 of its
// block (first sweep from the top), the rows above are padding.  Leaves
// P->nsplit = 0 and builds nothing when no tree splits.
static bps_status build_split(bps_hines_plan *P, int64_t batch, const int32_t *sizes,
                              const int32_t *parent, const std::vector<int64_t> &off, int64_t want)
{
    std::vector<SplitLane> lanes;          // two per split tree
    std::vector<int32_t> split_of(batch, -1), by_size(batch);
    std::iota(by_size.begin(), by_size.end(), 0);
    std::stable_sort(by_size.begin(), by_size.end(), [&](int32_t x, int32_t y) { return sizes[x] > sizes[y]; });
    // schedules of the candidates (the largest trees, a few more than wanted
    // in case some do not split), computed on all host threads; then taken
    // in size order
    int64_t ncand = 0;
    while (ncand < batch && sizes[by_size[ncand]] >= kSplitMin) ++ncand;
    ncand = std::min<int64_t>(ncand, want + want / 8 + 64);
    std::vector<SplitLane> cand(2 * ncand);
    std::vector<uint8_t> ok(ncand, 0);
    {
        const int64_t hw = std::min<int64_t>(16, std::thread::hardware_concurrency());
        const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(ncand / 64, hw));
        std::vector<std::thread> pool;
        for (int64_t t = 0; t < nt; ++t)
            pool.emplace_back([&, t] {
                for (int64_t c = t; c < ncand; c += nt) {
                    const int32_t s = by_size[c];
                    ok[c] = split_schedule(sizes[s], parent + off[s], &cand[2 * c]);
                }
            });
        for (auto &th : pool) th.join();
    }
    for (int64_t c = 0; c < ncand && int64_t(lanes.size() / 2) < want; ++c) {
        if (!ok[c]) continue;
        split_of[by_size[c]] = int32_t(lanes.size() / 2);
        lanes.push_back(std::move(cand[2 * c]));
        lanes.push_back(std::move(cand[2 * c + 1]));
    }
    P->nsplit = int64_t(lanes.size() / 2);
    if (P->nsplit == 0) return BPS_OK;
    auto rows_of = [&](int32_t s) {
        return split_of[s] >= 0 ? int32_t(lanes[2 * split_of[s]].node.size()) : sizes[s];
    };
    std::vector<int32_t> pairs, singles;
    for (int32_t s = 0; s < int32_t(batch); ++s) (split_of[s] >= 0 ? pairs : singles).push_back(s);
    auto by_rows = [&](int32_t x, int32_t y) { return rows_of(x) > rows_of(y); };
    std::stable_sort(pairs.begin(), pairs.end(), by_rows);
    std::stable_sort(singles.begin(), singles.end(), by_rows);
    // lane assignment: longest first; a pair starts at an even lane (an odd
    // lane takes the next single, or stays empty)
    std::vector<int32_t> lsrc;
    size_t ip = 0, is = 0;
    while (ip < pairs.size() || is < singles.size()) {
        const bool odd = lsrc.size() & 1;
        const bool take_pair = ip < pairs.size() &&
                               (is == singles.size() || rows_of(pairs[ip]) >= rows_of(singles[is]));
        if (take_pair && !odd) { lsrc.push_back(pairs[ip]); lsrc.push_back(pairs[ip]); ++ip; }
        else if (is < singles.size()) lsrc.push_back(singles[is++]);
        else lsrc.push_back(-1);
    }
    const int64_t nb = int64_t((lsrc.size() + kWave - 1) / kWave);
    lsrc.resize(size_t(nb * kWave), -1);
    std::vector<int64_t> boff(nb);
    std::vector<int32_t> brows(nb), ln(nb * kWave, 0);
    int64_t acc = 0;
    for (int64_t b = 0; b < nb; ++b) {
        int32_t rmax = 1;
        for (int k = 0; k < kWave; ++k)
            if (lsrc[b * kWave + k] >= 0) rmax = std::max(rmax, rows_of(lsrc[b * kWave + k]));
        boff[b] = acc;
        brows[b] = rmax;
        acc += int64_t(rmax) * kWave;
        P->max_rows = std::max(P->max_rows, rmax);
    }
    P->nblocks = nb;
    P->elems = acc;
    std::vector<uint16_t> code(acc, row_code(kSlotSink, kSlotSink, false, false));
    std::vector<int32_t> comp(acc, -1);
    for (int64_t b = 0; b < nb; ++b)
        for (int k = 0; k < kWave; ++k) {
            const int32_t s = lsrc[b * kWave + k];
            if (s < 0) continue;
            const int64_t base = boff[b] + k;
            if (split_of[s] >= 0) {
                const SplitLane &SL = lanes[2 * split_of[s] + (k & 1)];
                const int32_t m = int32_t(SL.node.size());
                int32_t live = 0;
                for (int32_t t = 0; t < m; ++t) {
                    const int64_t e = base + int64_t(m - 1 - t) * kWave;
                    code[e] = SL.code[t];
                    comp[e] = SL.node[t];
                    live += SL.node[t] >= 0;
                }
                ln[b * kWave + k] = live;
            } else {
                // one lane: row i is compartment i; its slot is its count
                // (n-1-i: the first sweep runs from row n-1 down) mod 16
                const int32_t n = sizes[s];
                const int32_t *ps = parent + off[s];
                for (int32_t i = 0; i < n; ++i) {
                    const int64_t e = base + int64_t(i) * kWave;
                    code[e] = i == 0 ? row_code((n - 1) & (kRing - 1), kSlotSink, true, false)
                                     : row_code((n - 1 - i) & (kRing - 1), (n - 1 - ps[i]) & (kRing - 1),
                                                true, ps[i] == i - 1);
                    comp[e] = i;
                }
                ln[b * kWave + k] = n;
            }
        }
    bps_status st;
    if ((st = upload(&P->code16, code)) != BPS_OK || (st = upload(&P->comp, comp)) != BPS_OK ||
        (st = upload(&P->blk_off, boff)) != BPS_OK || (st = upload(&P->blk_rows, brows)) != BPS_OK ||
        (st = upload(&P->lane_n, ln)) != BPS_OK || (st = upload(&P->lane_src, lsrc)) != BPS_OK)
        return st;
    return upload(&P->src_off, off);
}

bps_status hines_plan_build(bps_hines_plan **out, int64_t batch, const int32_t *sizes,
                            const int32_t *parent, int mono, int64_t ld, int sched);

// The trees a multi-morphology separator plan leaves out (skip): a one-lane
// plan of their own, retargeted to the original tree numbers (lane_src) and
// flat offsets (src_off), so that its kernels and layout transform address
// the caller's arrays and info directly; its elements follow P's.
static bps_status build_rest(bps_hines_plan *P, int64_t batch, const int32_t *sizes, const int32_t *parent,
                             const std::vector<int64_t> &off, const std::vector<char> &skip)
{
    std::vector<int32_t> ids, sz, par;
    for (int64_t s = 0; s < int64_t(skip.size()); ++s)
        if (skip[size_t(s)]) {
            ids.push_back(int32_t(s));
            sz.push_back(sizes[s]);
            par.insert(par.end(), parent + off[s], parent + off[s] + sizes[s]);
        }
    if (ids.empty()) return BPS_OK;
    bps_hines_plan *R = nullptr;
    bps_status st = hines_plan_build(&R, int64_t(ids.size()), sz.data(), par.data(), 0, 0, BPS_HINES_LANES);
    if (st != BPS_OK) return st;
    P->rest = R;
    std::vector<int32_t> ls(size_t(R->nblocks) * kWave);
    if (hipMemcpy(ls.data(), R->lane_src, ls.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
        BPS_FAIL(BPS_EHIP, "hines plan: reading the lanes of the trees left out");
    for (int32_t &v : ls)
        if (v >= 0) v = ids[size_t(v)];
    (void)hipFree(R->lane_src); R->lane_src = nullptr;
    (void)hipFree(R->src_off); R->src_off = nullptr;
    if ((st = upload(&R->lane_src, ls)) != BPS_OK || (st = upload(&R->src_off, off)) != BPS_OK) return st;
    P->elems = P->sep_elems + R->elems;
    (void)batch;
    return BPS_OK;
}

bps_status hines_plan_build(bps_hines_plan **out, int64_t batch, const int32_t *sizes,
                            const int32_t *parent, int mono, int64_t ld, int sched)
{
    auto *P = new bps_hines_plan();
    P->mono = mono ? 1 : 0;
    P->batch = batch;
    P->sched = sched;
    int32_t nmax = 0;
    int64_t total = 0;
    for (int64_t s = 0; s < (mono ? 1 : batch); ++s) {
        nmax = std::max(nmax, sizes[s]);
        total += sizes[s];
    }
    if (mono) total *= batch;
    const bool lv_fit = nmax <= kLevelMaxN;
    if (sched == BPS_HINES_LEVELS && !lv_fit) {
        delete P;
        BPS_FAIL(BPS_ENOTSUP, "level schedule needs trees of at most %d compartments", kLevelMaxN);
    }
    P->use_levels = sched == BPS_HINES_LEVELS ||
                    (sched == BPS_HINES_AUTO && lv_fit &&
                     total <= (mono ? kLevelAutoUnknowns : kLevelAutoUnknownsMulti));
    bps_status st = BPS_OK;
    if (mono) {
        const int64_t n = sizes[0];
        P->n = n;
        P->ld = ld;
        P->elems = n * ld;
        P->unknowns = n * batch;
        std::vector<int32_t> h(parent, parent + n);
        h[0] = 0;   // never read; keep it a valid index
        for (int64_t i = 1; i < n; ++i) P->max_dist = std::max<int32_t>(P->max_dist, int32_t(i - h[i]));
        st = upload(&P->parent, h);
        // separator schedules: when asked for, and by default for trees
        // it takes, unless small trees with parents within 16 in a batch
        // large enough to fill the GPU with one lane per neuron (measured:
        // 128 compartments, 16384 neurons 39.8 vs 47.2 us, 32768 neurons 63.4
        // vs 53.5 us; 256 and above faster at every batch, e.g. 512 x 65536
        // 346 vs 437 us and 512 x 256 29.8 us against 79.7 with levels;
        // parents further back leave the others the general variant)
        const bool sep_try = sched == BPS_HINES_SEP ||
                             (sched == BPS_HINES_AUTO && (n >= 256 || n * batch <= (int64_t(1) << 21) ||
                                                          P->max_dist > kRing));
        if (st == BPS_OK && sep_try) {
            std::string why;
            if (n > 2047 || n * ld * 8 > int64_t(0xFFFF0000u))
                why = n > 2047 ? "tree size above 2047" : "n * ld * 8 bytes above 4 GiB";
            else P->sep = sep_schedule(int32_t(n), parent, why);
            // with parents within 16 and at least 24576 neurons, not on 64
            // lanes nor on 32 lanes of 32 rows squeezed to more than 32
            // separators: one lane per neuron is faster there (51.2M
            // compartments per batch, separators / one lane: n = 1024 with 40
            // separators 0.870 / 0.736 ms, 1100 with 79 1.06 / 0.674, 64 lanes
            // for 1300 .. 2000 0.80 .. 0.85 / 0.71 .. 0.82; but 1000 with 25
            // 0.644 / 0.756, and 800 on 24 rows with 39 .. 56 0.619 / 0.662),
            // while its general variant takes 2.1 .. 3.5 ms for such trees
            // numbered depth first.  Smaller batches leave one lane per neuron
            // latency-bound: n = 1500 (64 lanes), 2048 .. 32768 neurons 0.046,
            // 0.087, 0.204, 0.416, 0.814 ms against 0.429, 0.431, 0.482, 0.526,
            // 0.665; n = 1024 (40 separators) 0.036, 0.069, 0.132, 0.316, 0.616
            // against 0.293, 0.297, 0.317, 0.356, 0.451
            if (sched == BPS_HINES_AUTO && P->max_dist <= kRing && batch >= 24576 && !P->sep.empty() &&
                (P->sep[6] == 64 || (P->sep[6] == 32 && P->sep[0] == 32 && P->sep[1] > 32)))
                P->sep.clear();
            if (P->sep.empty() && sched == BPS_HINES_SEP) {
                free_plan(P);
                BPS_FAIL(BPS_ENOTSUP, "BPS_HINES_SEP: %s", why.c_str());
            }
            if (!P->sep.empty()) {
                P->use_levels = false;
                st = upload(&P->sep_dev, P->sep);
            }
        }
        if (st == BPS_OK && P->use_levels) st = build_levels(P, 1, sizes, parent, {});
    } else {
        std::vector<int64_t> off(batch + 1, 0);
        for (int64_t s = 0; s < batch; ++s) off[s + 1] = off[s] + sizes[s];
        P->unknowns = off[batch];
        // separator schedules: when asked for, and by default unless the
        // trees average under 128 compartments, lie within 16 of their
        // parents and are enough for one lane per tree to fill every SIMD
        // (measured, us per solve, separators / the other choice: 70000
        // trees of 30..60 56 / 37 on one lane; depth-first numbered, whose
        // one-lane kernel is the general one, 56 / 106; 5000 of 1..100 24 / 37
        // with levels; 20000 of 60..190 36 / 51 on two lanes; 64 of 256..2048
        // 44 / 270 with levels; 32768 of 256..2048 0.38 / 0.61 ms two lanes)
        int32_t dfar = 0;
        for (int64_t s = 0; s < batch && dfar <= kRing; ++s)
            for (int32_t i = 1; i < sizes[s]; ++i) dfar = std::max(dfar, i - parent[off[s] + i]);
        const bool fills = (batch + kWave - 1) / kWave >= kSimds;
        const bool sep_auto = sched == BPS_HINES_AUTO && (off[batch] >= 128 * batch || dfar > kRing || !fills);
        SepMulti M;
        std::string why;
        std::vector<char> skip;
        const bool sep_ok = (sched == BPS_HINES_SEP || sep_auto) &&
                            sep_build_multi(batch, sizes, parent, off.data(), M, why, sep_auto ? &skip : nullptr);
        if (sched == BPS_HINES_SEP && !sep_ok) {
            free_plan(P);
            BPS_FAIL(BPS_ENOTSUP, "BPS_HINES_SEP: %s", why.c_str());
        }
        if (sep_ok) {
            P->use_levels = false;
            P->use_sepm = true;
            P->elems = M.elems;
            std::vector<int32_t> fp(parent, parent + off[batch]);
            int32_t *lt = nullptr, *tb = nullptr, *ps = nullptr;
            int64_t *wo = nullptr;
            if ((st = upload(&P->code16, M.code)) == BPS_OK && (st = upload(&P->comp, M.comp)) == BPS_OK &&
                (st = upload(&ps, M.pos)) == BPS_OK && (st = upload(&lt, M.lanetab)) == BPS_OK &&
                (st = upload(&tb, M.tabs)) == BPS_OK && (st = upload(&wo, M.wgoff)) == BPS_OK &&
                (st = upload(&P->src_off, off)) == BPS_OK)
                st = upload(&P->flat_parent, fp);
            P->sepm.nwg = M.nwg; P->sepm.elems = M.elems; P->sepm.lds = M.lds;
            P->sepm.code = P->code16; P->sepm.lanetab = lt; P->sepm.tabs = tb; P->sepm.pos = ps;
            P->sepm.wgoff = wo;
            P->sep_elems = M.elems;
            if (st == BPS_OK) st = build_rest(P, batch, sizes, parent, off, skip);
            if (st != BPS_OK) { free_plan(P); return st; }
            *out = P;
            return BPS_OK;
        }
        if (!P->use_levels && sched != BPS_HINES_LANES) {
            int32_t dmax = 0;
            for (int64_t s = 0; s < batch; ++s)
                for (int32_t i = 1; i < sizes[s]; ++i) dmax = std::max(dmax, i - parent[off[s] + i]);
            // how many trees go on two lanes: every one when asked for; by
            // default, when one lane per neuron leaves SIMDs without a
            // wavefront, the largest, until the lanes (nearly) fill one
            // wavefront per SIMD
            const int64_t want = sched == BPS_HINES_SPLIT ? batch
                               : (batch + kWave - 1) / kWave < kSimds ? int64_t(kSimds) * kWave - batch - 2 * kWave
                                                                     : 0;
            if (dmax <= kRing && want > 0) {
                st = build_split(P, batch, sizes, parent, off, want);
                if (st != BPS_OK) { free_plan(P); return st; }
                if (P->nsplit > 0) { P->max_dist = dmax; *out = P; return BPS_OK; }
            }
        }
        std::vector<int32_t> order(batch);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(),
                         [&](int32_t x, int32_t y) { return sizes[x] > sizes[y]; });
        const int64_t nb = (batch + kWave - 1) / kWave;
        P->nblocks = nb;
        std::vector<int64_t> boff(nb);
        std::vector<int32_t> brows(nb), ln(nb * kWave, 0), lsrc(nb * kWave, -1);
        int64_t acc = 0;
        for (int64_t b = 0; b < nb; ++b) {
            int32_t rmax = 0;
            for (int k = 0; k < kWave; ++k) {
                const int64_t j = b * kWave + k;
                if (j >= batch) break;
                const int32_t s = order[j];
                ln[j] = sizes[s];
                lsrc[j] = s;
                rmax = std::max(rmax, sizes[s]);
            }
            boff[b] = acc;
            brows[b] = rmax;
            acc += int64_t(rmax) * kWave;
            P->max_rows = std::max(P->max_rows, rmax);
        }
        P->elems = acc;
        std::vector<int32_t> pk(acc, 0);
        std::vector<uint8_t> d8(acc, 0);
        for (int64_t b = 0; b < nb; ++b)
            for (int k = 0; k < kWave; ++k) {
                const int32_t s = lsrc[b * kWave + k];
                if (s < 0) continue;
                for (int32_t i = 1; i < sizes[s]; ++i) {
                    const int32_t p = parent[off[s] + i];
                    pk[boff[b] + int64_t(i) * kWave + k] = p;
                    d8[boff[b] + int64_t(i) * kWave + k] = uint8_t(i - p <= kRing ? i - p : kFar);
                    P->max_dist = std::max<int32_t>(P->max_dist, i - p);
                }
            }
        st = upload(&P->dist8, d8);
        if (st == BPS_OK && (st = upload(&P->parent, pk)) == BPS_OK && (st = upload(&P->blk_off, boff)) == BPS_OK &&
            (st = upload(&P->blk_rows, brows)) == BPS_OK && (st = upload(&P->lane_n, ln)) == BPS_OK &&
            (st = upload(&P->lane_src, lsrc)) == BPS_OK)
            st = upload(&P->src_off, off);
        if (st == BPS_OK && P->use_levels) {
            // neuron s sits at lane k of block b: its values start at boff[b] + k
            std::vector<int64_t> dbase(batch, 0);
            for (int64_t b = 0; b < nb; ++b)
                for (int k = 0; k < kWave; ++k)
                    if (lsrc[b * kWave + k] >= 0) dbase[lsrc[b * kWave + k]] = boff[b] + k;
            st = build_levels(P, batch, sizes, parent, dbase);
        }
    }
    if (st != BPS_OK) { free_plan(P); return st; }
    *out = P;
    return BPS_OK;
}

bps_status hines_plan_free(bps_hines_plan *p)
{
    free_plan(p);
    return BPS_OK;
}

// The level schedule's dynamic LDS (four values per compartment of the
// largest tree) may exceed the default 64 KiB: allowed its largest amount on
// the current device.
hipError_t hines_prepare_device()
{
    const hipError_t e = hipFuncSetAttribute((const void *)k_hines_levels,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             int(4 * kLevelMaxN * sizeof(double)));
    return e != hipSuccess ? e : sep_prepare_device();
}

bool hines_plan_general(const bps_hines_plan *p)
{
    return !p->sep_dev && !p->use_sepm && p->max_dist > kRing;
}
bool hines_plan_levels(const bps_hines_plan *p) { return p->use_levels; }
size_t hines_plan_work_bytes(const bps_hines_plan *p)
{
    if (p->use_sepm)
        return size_t(p->sep_elems) * 8 + (p->rest ? hines_plan_work_bytes(p->rest) : 0);
    return size_t(p->elems) * 8 * (hines_plan_general(p) ? 3 : 1);
}
bool hines_plan_sep(const bps_hines_plan *p) { return p->sep_dev != nullptr || p->use_sepm; }
int64_t hines_plan_elems_of(const bps_hines_plan *p) { return p->elems; }
int64_t hines_plan_unknowns_of(const bps_hines_plan *p) { return p->unknowns; }
int64_t hines_plan_batch_of(const bps_hines_plan *p) { return p->batch; }
int64_t hines_plan_split_of(const bps_hines_plan *p) { return p->nsplit; }

int32_t hines_sep_blob(int32_t n, const int32_t *parent, int32_t *out, int32_t cap, std::string &why)
{
    const std::vector<int32_t> b = sep_schedule(n, parent, why);
    if (b.empty()) return 0;
    if (int64_t(b.size()) > cap) return -int32_t(b.size());
    std::copy(b.begin(), b.end(), out);
    return int32_t(b.size());
}

int32_t hines_split_rows(int32_t n, const int32_t *parent, int32_t *node, uint16_t *code, int32_t cap)
{
    SplitLane two[2];
    if (!split_schedule(n, parent, two)) return 0;
    const int32_t m = int32_t(two[0].node.size());
    if (m > cap) return -m;
    for (int j = 0; j < 2; ++j) {
        std::copy(two[j].node.begin(), two[j].node.end(), node + int64_t(j) * cap);
        std::copy(two[j].code.begin(), two[j].code.end(), code + int64_t(j) * cap);
    }
    return m;
}

template <typename T>
bps_status hines_transform(const bps_hines_plan *P, bool pack, const void *src, void *dst,
                           hipStream_t st)
{
    if (P->use_sepm) {
        BPS_HIP(sepm_pack(pack, sizeof(T) == 8, P->comp, P->sep_elems, src, dst, st));
        if (!P->rest) return BPS_OK;
        // the trees left out: their own transform, after the separators' elements
        return pack ? hines_transform<T>(P->rest, true, src, static_cast<T *>(dst) + P->sep_elems, st)
                    : hines_transform<T>(P->rest, false, static_cast<const T *>(src) + P->sep_elems, dst, st);
    }
    if (P->mono) {
        const int64_t total = P->n * (pack ? P->ld : P->batch);
        const unsigned grid = unsigned(std::min<int64_t>((total + 255) / 256, 65536));
        if (pack)
            hipLaunchKernelGGL((k_mono_transpose<T, true>), dim3(grid), dim3(256), 0, st, P->n,
                               P->batch, P->ld, (const T *)src, (T *)dst);
        else
            hipLaunchKernelGGL((k_mono_transpose<T, false>), dim3(grid), dim3(256), 0, st, P->n,
                               P->batch, P->ld, (const T *)src, (T *)dst);
    } else if (P->nsplit > 0) {
        if (pack)
            hipLaunchKernelGGL((k_multi_pack_map<T, true>), dim3(unsigned(P->nblocks)), dim3(256), 0, st,
                               P->blk_off, P->blk_rows, P->lane_src, P->comp, P->src_off,
                               (const T *)src, (T *)dst);
        else
            hipLaunchKernelGGL((k_multi_pack_map<T, false>), dim3(unsigned(P->nblocks)), dim3(256), 0, st,
                               P->blk_off, P->blk_rows, P->lane_src, P->comp, P->src_off,
                               (const T *)src, (T *)dst);
    } else {
        if (pack)
            hipLaunchKernelGGL((k_multi_pack<T, true>), dim3(unsigned(P->nblocks)), dim3(256), 0, st,
                               P->blk_off, P->blk_rows, P->lane_n, P->lane_src, P->src_off,
                               (const T *)src, (T *)dst);
        else
            hipLaunchKernelGGL((k_multi_pack<T, false>), dim3(unsigned(P->nblocks)), dim3(256), 0, st,
                               P->blk_off, P->blk_rows, P->lane_n, P->lane_src, P->src_off,
                               (const T *)src, (T *)dst);
    }
    BPS_LAUNCHED("hines layout transform");
    return BPS_OK;
}
template bps_status hines_transform<float>(const bps_hines_plan *, bool, const void *, void *, hipStream_t);
template bps_status hines_transform<double>(const bps_hines_plan *, bool, const void *, void *, hipStream_t);

bps_status hines_launch(const bps_hines_plan *P, const void *u, const void *l, const void *d,
                        void *rhs, void *work, int32_t *info, hipStream_t st)
{
    if (P->use_levels) {
        LevelArgs L{};
        L.ld = P->ld; L.mono = P->mono; L.tree = P->lv_tree; L.lane_src = P->lane_src;
        L.nwg = P->mono ? P->batch : P->nblocks * kWave;
        L.perm = P->lv_perm; L.sec = P->lv_sec; L.spar = P->lv_spar; L.lev = P->lv_lev;
        L.u = (const double *)u; L.l = (const double *)l; L.d = (const double *)d;
        L.rhs = (double *)rhs; L.info = info;
        const size_t lds = size_t(4) * P->lv_maxn * sizeof(double);
        hipLaunchKernelGGL(k_hines_levels, dim3(unsigned(L.nwg)), dim3(kWave), lds, st, L);
        BPS_LAUNCHED("k_hines_levels");
        return BPS_OK;
    }
    if (P->use_sepm) {
        const bps_status s0 = launch_hines_sepm(P->sepm, P->flat_parent, P->src_off, u, l, d, rhs, work, info, st);
        if (s0 != BPS_OK || !P->rest) return s0;
        // the trees left out, on their own elements and work
        const int64_t e = P->sep_elems;
        return hines_launch(P->rest, static_cast<const double *>(u) + e, static_cast<const double *>(l) + e,
                            static_cast<const double *>(d) + e, static_cast<double *>(rhs) + e,
                            static_cast<unsigned char *>(work) + size_t(e) * 8, info, st);
    }
    if (P->sep_dev)
        return launch_hines_sep(P->sep.data(), P->sep_dev, P->batch, P->ld, P->parent, u, l, d, rhs,
                                work, info, st);
    const bool gen = hines_plan_general(P);
    HinesArgs A{};
    A.batch = P->batch; A.n = P->n; A.ld = P->ld;
    A.blk_off = P->blk_off; A.blk_rows = P->blk_rows; A.lane_n = P->lane_n; A.lane_src = P->lane_src;
    A.parent = P->parent;
    A.dist8 = P->dist8;
    A.code16 = P->code16;
    A.comp = P->comp;
    A.u = (const double *)u; A.l = (const double *)l; A.d = (const double *)d;
    A.rhs = (double *)rhs;
    A.mwork = (double *)work;
    A.gd = gen ? A.mwork + P->elems : nullptr;
    A.gr = gen ? A.mwork + 2 * P->elems : nullptr;
    A.info = info;
    if (gen) {
        hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(256), 0, st, A.gd, 2 * P->elems);
        BPS_LAUNCHED("k_fill_zero");
    }
    const dim3 grid(unsigned(P->mono ? (P->batch + kWave - 1) / kWave : P->nblocks));
    constexpr int D = kHinesAhead;
    // A multi-morphology batch of at most one block per SIMD runs one wave
    // per SIMD anyway, and its largest blocks set the time: groups of 16
    // rows (256 VGPRs, one wave per SIMD) keep more rows in flight.
    if (P->mono) {
        if (gen) hipLaunchKernelGGL((k_hines<true, true, D>), grid, dim3(kWave), 0, st, A);
        else hipLaunchKernelGGL((k_hines_mono_reg<D>), grid, dim3(kWave), 0, st, A);
    } else {
        if (gen) hipLaunchKernelGGL((k_hines_multi<D, true>), grid, dim3(kWave), 0, st, A);
        else if (P->nsplit > 0 && P->nblocks <= kSimds)
            hipLaunchKernelGGL((k_hines_split<16>), grid, dim3(kWave), 0, st, A);
        else if (P->nsplit > 0) hipLaunchKernelGGL((k_hines_split<D>), grid, dim3(kWave), 0, st, A);
        else if (P->nblocks <= kSimds) hipLaunchKernelGGL((k_hines_multi<16>), grid, dim3(kWave), 0, st, A);
        else hipLaunchKernelGGL((k_hines_multi<D>), grid, dim3(kWave), 0, st, A);
    }
    BPS_LAUNCHED("k_hines");
    return BPS_OK;
}

}  // namespace bps
