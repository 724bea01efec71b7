// kernels.h -- host launchers of the HIP kernels (internal to libbps).
#pragma once

#include <string>
#include <vector>

#include "common.h"

namespace bps {

template <typename T>
// mask (device int32[batch] or NULL): only systems with mask[s] != 0.
bps_status launch_penta_factor(int64_t n, int64_t batch, int64_t ld, bool cyclic, bool shared,
                               const void *a, const void *b, const void *c, const void *d,
                               const void *e, void *fac, int32_t *info, hipStream_t st,
                               const int32_t *mask = nullptr);
template <typename T>
bps_status launch_penta_solve(int64_t n, int64_t batch, int64_t ld, bool shared,
                              const void *fac, void *x, hipStream_t st);
template <typename T>
bps_status launch_penta_cyclic_solve(int64_t n, int64_t batch, int64_t ld, int64_t nsteps,
                                     bool shared, const void *fac, void *x, hipStream_t st,
                                     const int32_t *mask = nullptr);
template <typename T>
bps_status launch_penta_fused(int64_t n, int64_t batch, int64_t ld, const void *a, const void *b,
                              const void *c, const void *d, const void *e, void *x, void *work,
                              int32_t *info, hipStream_t st);
// Chunked register-resident factor + solve (per-system); spike_rows(n,
// cyclic) is the chunk length (16 or 12), 0 when the path does not apply.
// Non-periodic: work holds 2 n ld values for the sequential fallback.
// Periodic: systems whose chunked elimination breaks down are left
// untouched and marked in mask (int32[batch], every entry written) for a
// second pass.
int spike_rows(int64_t n, bool cyclic);
template <typename T>
bps_status launch_penta_spike(int64_t n, int64_t batch, int64_t ld, bool cyclic, const void *a,
                              const void *b, const void *c, const void *d, const void *e, void *x,
                              void *work, int32_t *info, int32_t *mask, hipStream_t st);

// Builds the five shared diagonals of I + sigma*D4 on the device.
template <typename T>
bps_status launch_hyper_diagonals(int64_t n, double sigma, void *diag, hipStream_t st);

// Register-resident multi-step solve of I + sigma*D4 (fp64): set-up kernel
// plus the step kernel.  resident_chunk(n) is the chunk length, 0 when the
// resident path does not apply to n.
int resident_chunk(int64_t n);
size_t resident_coef_bytes(int64_t n);
// Right-hand side of every step of the resident kernel (mode bits): the
// state (0: implicit step), or the explicit stencil (e2, e1, e0, e1, e2) of
// the state (kResStencil: theta scheme; sigma is then theta * sigma), plus
// rr D2 (C^3 - C) with kResPhase (Cahn-Hilliard).
enum { kResStencil = 1, kResPhase = 2 };
// parts: the set-up kernel (coefficients into coef), the step kernel (reads
// them), or both in that order.
enum { kResSetup = 1, kResSteps = 2, kResBoth = 3 };
bps_status launch_hyper_resident(int64_t n, int64_t batch, int64_t ld, int64_t nsteps, double sigma,
                                 int mode, double e0, double e1, double e2, double rr, void *coef,
                                 void *C, hipStream_t st, int parts = kResBoth);
// Streaming theta / Cahn-Hilliard right-hand side: the explicit stencil
// (+ rr D2 (C^3 - C) when ch) into a separate array, and a strided copy
// between interleaved arrays.
template <typename T>
bps_status launch_hyper_explicit(int64_t n, int64_t batch, int64_t ldi, int64_t ldo, double e0,
                                 double e1, double e2, double rr, bool ch, const void *in,
                                 void *out, hipStream_t st);
template <typename T>
bps_status launch_copy_interleaved(int64_t n, int64_t batch, int64_t ldi, int64_t ldo,
                                   const void *in, void *out, hipStream_t st);

// Batched tridiagonal solve: register-resident chunks for n = M P, M = 16
// (else 12), 2 <= P <= 64 (tri_rows(n) is M, or 0); chunks spread over
// workgroups for n = 16 P, 64 < P <= 65535 (tri_part_chunks); else one lane
// per system.  Work: tri_work_bytes_es(n, ld, sizeof(T)) bytes.
int tri_rows(int64_t n);
int tri_part_chunks(int64_t n);
size_t tri_work_bytes_es(int64_t n, int64_t ld, size_t es);
template <typename T>
bps_status launch_tri_solve(int64_t n, int64_t batch, int64_t ld, const void *a, const void *b,
                            const void *c, void *y, void *work, int32_t *info, hipStream_t st);

// Hines systems of one shared tree on sixteen, thirty-two or sixty-four lanes per neuron
// (hines_sep.hip): the schedule of a tree (empty, reason in why, when the
// tree does not qualify), the kernel's dynamic LDS, and its launch.
std::vector<int32_t> sep_schedule(int32_t n, const int32_t *parent, std::string &why);
size_t sep_lds_bytes(const int32_t *blob);
hipError_t sep_prepare_device();
bps_status launch_hines_sep(const int32_t *blob_host, const int32_t *blob_dev, int64_t batch, int64_t ld,
                            const int32_t *parent_dev, const void *u, const void *l, const void *d,
                            void *rhs, void *work, int32_t *info, hipStream_t st);

// Multi-morphology trees, each its own separator schedule, in a
// schedule-ordered layout (hines_sep.hip): the host plan, its device copy,
// the layout transform and the launch.
struct SepMulti {
    int R = 0, lanes = 0;           // rows per lane, lanes per workgroup
    int64_t nwg = 0, elems = 0;
    size_t lds = 0;
    std::vector<uint16_t> code;      // [elems] row codes
    std::vector<int32_t> comp;       // [elems] flat compartment, -1 padding
    std::vector<int32_t> pos;        // [compartments] element of each flat compartment
    std::vector<int32_t> lanetab;    // [nwg * lanes][5]
    std::vector<int64_t> wgoff;      // [nwg + 1]
    std::vector<int32_t> tabs;
};
struct SepMultiDev {
    int64_t nwg = 0, elems = 0;
    size_t lds = 0;
    const uint16_t *code = nullptr;
    const int32_t *lanetab = nullptr, *tabs = nullptr, *pos = nullptr;
    const int64_t *wgoff = nullptr;
};
// With skip, trees that do not fit are marked there and left out (the
// schedule holds the others); without, such a tree fails the batch.
bool sep_build_multi(int64_t batch, const int32_t *sizes, const int32_t *parent, const int64_t *off,
                     SepMulti &M, std::string &why, std::vector<char> *skip = nullptr);
hipError_t sepm_pack(bool pack, bool f64, const int32_t *gcomp, int64_t elems, const void *src, void *dst,
                     hipStream_t st);
bps_status launch_hines_sepm(const SepMultiDev &S, const int32_t *parent_dev, const int64_t *src_off,
                             const void *u, const void *l, const void *d, void *rhs, void *work,
                             int32_t *info, hipStream_t st);

// Number of values of a factor buffer.
inline int64_t penta_factor_elems(int64_t n, int64_t ldf, bool cyclic) {
    return cyclic ? (9 * (n - 2) + 4) * ldf : 5 * n * ldf;
}

}  // namespace bps
