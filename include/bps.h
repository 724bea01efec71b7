/*
 * bps.h -- batched banded solvers for PDE time stepping on AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every array argument named "device"
 * is a pointer to GPU memory (hipMalloc / torch tensors); "host" arrays are
 * ordinary CPU memory.  `stream` is a hipStream_t passed as void* (NULL = the
 * default stream); every call only ENQUEUES work on it and returns without
 * synchronising, except hines_plan_create / hines_plan_create_sched /
 * hines_plan_destroy, which allocate / free device memory and synchronise.
 * No solve allocates memory.  Solve, pack and unpack calls enqueue kernels
 * only (no allocation, copy, memset or synchronisation), so a sequence of
 * them can be captured into a HIP graph and replayed.  The first call on a
 * device that needs them (bps_init, penta_factor_solve_batch,
 * hines_plan_create*) also sets the dynamic-LDS limits of the kernels that
 * use more than 64 KiB there: a host-side kernel attribute, with no stream
 * work, so that first call may itself be inside a capture.
 *
 * Sources (web-page titles; sections named as on the pages):
 *   [P] "cuPentBatch - A batched pentadiagonal solver for NVIDIA GPUs":
 *       section "Pentadiagonal solver" (A = L R factorisation steps, the
 *       forward steps for g, the back-substitution steps for x, six vectors
 *       and in-place reuse of the factors), the hyperdiffusion section
 *       (eq. (4) on a periodic domain, the centred fourth difference, the
 *       periodic pentadiagonal matrix and Navon's reduction eqs. (10)-(12)),
 *       and the section on the batched GPU implementation (interleaved
 *       layout, factorisation split from the solve: "Constant" factors once,
 *       "Rewrite" refactors every call).
 *   [H] "Simulating the behavior of the human brain on GPUs": section 2
 *       (cable equation discretised on a neuron tree, the parent vector,
 *       the Hines matrix, Algorithm 1 `solveHines(u, l, d, rhs, p, cellSize)`),
 *       section 3 (Full-Interleaved and Block-Interleaved layouts, one thread
 *       per system, layout transformed once up front), section 4 (batches of
 *       neurons with different morphologies, the per-branch / per-level
 *       decomposition, and tridiagonal systems: the Thomas algorithm of
 *       cuThomasBatch, section 4.1).  The cuPentBatch page's introduction
 *       also gives the Cahn-Hilliard model and its semi-implicit scheme.
 *
 * LAYOUTS
 *   Interleaved (the [P] and [H] layout): element (row i, system s) of an
 *   array is at index i*ld + s, 0 <= i < n, 0 <= s < batch, ld >= batch
 *   (elements, not bytes), n * ld <= 2^40.  Systems are the fastest-varying
 *   index, so one elimination step over consecutive systems is one
 *   coalesced HBM stream.
 *
 * PRECISION
 *   BPS_F64 (double) everywhere; BPS_F32 (float) for the pentadiagonal and
 *   hyperdiffusion entry points.  No pivoting (as on [P]): the solves are
 *   meant for diagonally dominant or symmetric positive definite matrices.
 *
 * ERRORS
 *   Argument checks run on the host before anything is enqueued and return
 *   BPS_EINVAL (bad sizes, NULL or misaligned pointers, unknown dtype/flags,
 *   a parent index not in [0, i)) or BPS_ENOTSUP (valid but not supported
 *   combination).  A failed HIP launch returns BPS_EHIP.  bps_last_error()
 *   gives a message for the calling thread's last failure.  Numerical
 *   breakdown is only known on the device: when an `info` array (device,
 *   int32[batch]) is given, info[s] = 0, or 1 + the first row whose pivot is
 *   zero or not finite (LAPACK style); the solution of that system is then
 *   meaningless, the others are unaffected.
 *
 * OWNERSHIP
 *   The caller owns every device buffer.  Inputs are never modified; only
 *   the arrays documented as outputs (x / rhs / C, factors, work, info) are
 *   written.  The library allocates device memory only inside
 *   hines_plan_create / hines_plan_create_sched and frees it in
 *   hines_plan_destroy.  Calls on different
 *   streams with different output buffers are independent.
 */
#ifndef BPS_H
#define BPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define BPS_API __attribute__((visibility("default")))
#else
#define BPS_API
#endif

typedef enum bps_status {
    BPS_OK = 0,
    BPS_EINVAL = 1,   /* invalid argument                       */
    BPS_ENOTSUP = 2,  /* valid but unsupported combination      */
    BPS_EHIP = 3,     /* a HIP runtime call or launch failed    */
    BPS_ENOMEM = 4    /* device allocation failed (plans only)  */
} bps_status;

typedef enum bps_dtype { BPS_F32 = 1, BPS_F64 = 2 } bps_dtype;

/* Matrix flags for bps_penta_desc.flags */
#define BPS_CYCLIC      0x1u  /* periodic: column indices wrap modulo n ([P], periodic matrix)  */
#define BPS_SHARED_COEF 0x2u  /* one set of diagonals (n values each) used by every system     */

/* Text for a status code (static storage). */
BPS_API const char *bps_status_str(int status);
/* Message describing the calling thread's most recent failure ("" if none). */
BPS_API const char *bps_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
BPS_API int bps_version(void);
/* Prepare the current device: sets, once per device, the dynamic-LDS limits
 * of the kernels whose launches may use more than 64 KiB (the chunked
 * pentadiagonal solves, the Hines level schedule) to their largest launch.
 * Host-side only (no allocation, no stream work); idempotent and
 * thread-safe.  The entry points that launch those kernels call it
 * themselves, so calling it is optional.  BPS_EHIP if the runtime refuses. */
BPS_API bps_status bps_init(void);

/* ======================================================================== */
/* Pentadiagonal systems  [P] "Pentadiagonal solver"                        */
/* ======================================================================== */

/* Describes a batch of pentadiagonal systems A_s x_s = f_s.
 * Diagonals (the [P] naming): a_i = A[i][i-2], b_i = A[i][i-1], c_i = A[i][i],
 * d_i = A[i][i+1], e_i = A[i][i+2].
 *  - default: each system has its own diagonals, interleaved [n][ld];
 *    the entries that fall outside the matrix (a_0, a_1, b_0, d_{n-1},
 *    e_{n-2}, e_{n-1}) are never read.  n >= 4.
 *  - BPS_CYCLIC: periodic matrix, column index (i+k) mod n, so every entry
 *    is used; solved by the reduction of [P] (the last two unknowns coupled
 *    through a 2x2 block, eqs. (10)-(12)) in an equivalent fused order.
 *    n >= 6.
 *  - BPS_SHARED_COEF: a..e are single vectors of n values shared by all
 *    systems (the "Constant" use of [P]: factor once, solve many).
 * ld: leading dimension (elements) of the interleaved x / f / per-system
 * diagonal arrays, ld >= batch. */
typedef struct bps_penta_desc {
    int32_t dtype;    /* BPS_F32 or BPS_F64 */
    uint32_t flags;   /* 0 or an OR of BPS_CYCLIC, BPS_SHARED_COEF */
    int64_t n;        /* rows per system */
    int64_t batch;    /* number of systems */
    int64_t ld;       /* leading dimension of interleaved arrays, >= batch */
} bps_penta_desc;

/* Bytes of the `factors` buffer that penta_factor_batch fills for `desc`
 * (0 if desc is invalid).  Its content is private to this library. */
BPS_API size_t bps_penta_factor_bytes(const bps_penta_desc *desc);

/* Factor every system ([P] factorisation steps 1-14; for BPS_CYCLIC also the
 * quantities of the periodic reduction that [P] says are computed once and
 * stored: the Schur 2x2 inverse and the coupling vectors).
 * a..e: device, per the desc layout.  factors: device, bps_penta_factor_bytes.
 * info: device int32[batch] (int32[1] with BPS_SHARED_COEF) or NULL.
 * Alignment: 8 bytes (F64) / 4 bytes (F32) for every array. */
BPS_API bps_status penta_factor_batch(const bps_penta_desc *desc,
                              const void *a, const void *b, const void *c,
                              const void *d, const void *e,
                              void *factors, int32_t *info, void *stream);

/* Solve with stored factors of a NON-periodic batch ([P] forward steps for g,
 * then back substitution).  x: device interleaved [n][ld]; holds f on entry
 * and the solution on return.  desc must equal the one used to factor. */
BPS_API bps_status penta_solve_batch(const bps_penta_desc *desc, const void *factors,
                             void *x, void *stream);

/* Solve with stored factors of a PERIODIC batch (desc has BPS_CYCLIC).
 * Same conventions as penta_solve_batch. */
BPS_API bps_status penta_cyclic_solve_batch(const bps_penta_desc *desc, const void *factors,
                                    void *x, void *stream);

/* Bytes of the `work` buffer penta_factor_solve_batch needs (0 if invalid):
 * 2*n*ld values, or for BPS_CYCLIC the periodic factors of every system
 * plus ld int32. */
BPS_API size_t bps_penta_work_bytes(const bps_penta_desc *desc);

/* Factor and solve in one pass over the data (the "Rewrite" use of [P]:
 * a new matrix every call), per-system diagonals only (flags 0 or
 * BPS_CYCLIC; BPS_SHARED_COEF gives BPS_ENOTSUP).  x: f on entry, solution
 * on return.  work: device, bps_penta_work_bytes(desc) bytes, overwritten
 * (scratch; contents undefined on return).  info: as above or NULL.
 * Non-periodic: 1 + the first row whose pivot of the page's sequential
 * elimination is zero or non-finite.  For n = M*P with M = 16 (else 12)
 * and 2 <= P <= 64 the systems are solved in M-row chunks (each eliminated
 * with its own pivots, joined by a 2x2-block interface system); a system
 * whose chunked elimination meets a zero or non-finite pivot is re-solved
 * in the same launch by the sequential elimination, so info and the
 * solution are those of the page's algorithm.
 * Periodic (BPS_CYCLIC, [P] hyperdiffusion section: Navon's reduction with
 * per-system coupling vectors): info as penta_factor_batch (1 + first bad
 * pivot of the leading n-2 block, n - 1 for a singular 2x2 corner system).
 * For n = M*P, M = 16 (else 12), P in {2, 4, ..., 64}, the chunked solve
 * applies with the chunks joined periodically (the wrap entries couple the
 * first and last chunks); systems whose chunked elimination breaks down,
 * and other n, are factored and solved by the page's periodic reduction in
 * a second pass. */
BPS_API bps_status penta_factor_solve_batch(const bps_penta_desc *desc,
                                    const void *a, const void *b, const void *c,
                                    const void *d, const void *e,
                                    void *x, void *work, int32_t *info, void *stream);

/* ======================================================================== */
/* Periodic hyperdiffusion  [P] hyperdiffusion section                      */
/* ======================================================================== */

/* Bytes of `work` for hyperdiffusion_step (shared factors; 0 if invalid). */
BPS_API size_t hyperdiffusion_work_bytes(int dtype, int64_t n, int64_t batch);

/* Advance `batch` periodic 1-D fields by `nsteps` implicit steps
 *     (I + sigma*D4) C^{k+1} = C^k,   sigma = dt / dx^4,
 * with D4 the centred fourth difference [1, -4, 6, -4, 1] wrapping modulo n
 * (periodic domain of length n*dx, eq. (4) with gamma = D = 1).
 * diagonals: NULL for the operator above, or a device array of 5*n values
 *   [a | b | c | d | e] (each n long) giving any periodic pentadiagonal
 *   matrix shared by all systems (the "constant" use of [P]).
 * C: device, interleaved [n][ld]; C^0 on entry, C^{nsteps} on return.
 * work: device, hyperdiffusion_work_bytes(dtype, n, batch) bytes.
 * The matrix is factored once per call and reused for all nsteps steps.
 * n >= 6, batch >= 1, ld >= batch, nsteps >= 0, dt and dx finite, dx != 0. */
BPS_API bps_status hyperdiffusion_step(int dtype, int64_t n, int64_t batch, int64_t ld,
                               double dt, double dx, const void *diagonals,
                               void *C, int64_t nsteps, void *work, void *stream);

/* The two halves of hyperdiffusion_step, for the "Constant" use of [P]
 * (the matrix factored once at the start, its factors reused by every
 * solve): hyperdiffusion_factor writes the factors of the operator (with the
 * quantities of the periodic reduction) into `work`; hyperdiffusion_solve
 * advances C by nsteps steps with them.  hyperdiffusion_step is the factor
 * call followed by the solve call with the same arguments.  The factors
 * depend on dtype, n, dt, dx and diagonals only: every solve call must be
 * given those exactly as the factor call was (they also select the solver),
 * with any batch, ld and nsteps; `work` (hyperdiffusion_work_bytes(dtype, n,
 * 1) bytes or more, device) is read, not written, by the solve, so one
 * factorisation serves any number of solves, on any stream ordered after
 * the factor call.  Checks as hyperdiffusion_step. */
BPS_API bps_status hyperdiffusion_factor(int dtype, int64_t n, double dt, double dx,
                                 const void *diagonals, void *work, void *stream);
BPS_API bps_status hyperdiffusion_solve(int dtype, int64_t n, int64_t batch, int64_t ld,
                                double dt, double dx, const void *diagonals, void *C,
                                int64_t nsteps, const void *work, void *stream);

/* Size of the per-GPU scratch array of hyperdiffusion_step_noalloc. */
#define BPS_NOALLOC_SCRATCH_BYTES (2u * 1024u * 1024u)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * hyperdiffusion_step without the `work` argument: same operation, other
 * arguments, checks and results.  Its work memory is a device array of
 * BPS_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU, which that GPU
 * holds from the library's first use on it until the process ends.  The
 * call allocates nothing (no hipMalloc / hipFree, no allocating library
 * routine).  BPS_EINVAL when hyperdiffusion_work_bytes(dtype, n, batch)
 * exceeds the array (n above 18725 in fp64, 37450 in fp32).  Every call on a
 * GPU uses that GPU's array, which keeps the last call's contents (each call
 * writes all the work memory it reads before reading it, so nothing needs
 * clearing): calls on one stream are ordered, but calls that overlap on one
 * GPU (on streams not ordered with each other, or from several threads at
 * once) race and give undefined results. */
BPS_API bps_status hyperdiffusion_step_noalloc(int dtype, int64_t n, int64_t batch, int64_t ld,
                                       double dt, double dx, const void *diagonals, void *C,
                                       int64_t nsteps, void *stream);

/* Bytes of `work` for hyperdiffusion_theta_step (0 if invalid). */
BPS_API size_t hyperdiffusion_theta_work_bytes(int dtype, int64_t n, int64_t batch);

/* Advance `batch` periodic 1-D fields by `nsteps` theta-scheme steps
 *     (I + theta*sigma*D4) C^{k+1} = (I - (1 - theta)*sigma*D4) C^k,
 * sigma = dt / dx^4, D4 as above ([P] hyperdiffusion section: the page's
 * Crank-Nicolson scheme is theta = 1/2, i.e. sigma_x = dt/(2 dx^4) on both
 * sides; theta = 1 is hyperdiffusion_step with the built-in operator, with
 * identical results).  The right-hand side is the explicit five-point
 * stencil with entries -se, 4 se, 1 - 6 se, 4 se, -se (se = (1-theta)*sigma);
 * the implicit matrix (a = e = si, b = d = -4 si, c = 1 + 6 si, si =
 * theta*sigma) is factored once per call.  The scheme is unconditionally
 * stable for theta >= 1/2 only; smaller theta is computed as asked.
 * C: device, interleaved [n][ld]; C^0 on entry, C^{nsteps} on return.
 * work: device, hyperdiffusion_theta_work_bytes(dtype, n, batch) bytes.
 * n >= 6, batch >= 1, ld >= batch, nsteps >= 0, dt and dx finite, dx != 0,
 * 0 <= theta <= 1 (else BPS_EINVAL). */
BPS_API bps_status hyperdiffusion_theta_step(int dtype, int64_t n, int64_t batch, int64_t ld,
                                     double dt, double dx, double theta, void *C,
                                     int64_t nsteps, void *work, void *stream);

/* ======================================================================== */
/* Cahn-Hilliard  [P] introduction (model equation and its time scheme)     */
/* ======================================================================== */

/* Bytes of `work` for cahn_hilliard_step (0 if invalid). */
BPS_API size_t cahn_hilliard_work_bytes(int dtype, int64_t n, int64_t batch);

/* Advance `batch` periodic 1-D concentration fields of the Cahn-Hilliard
 * equation dC/dt = D d_xx (C^3 - C - gamma d_xx C) by `nsteps` steps of the
 * semi-implicit scheme: the phase-separation term at the old time level,
 * the fourth-order term with the theta family,
 *     (I + theta*sigma*D4) C^{k+1} = (I - (1 - theta)*sigma*D4) C^k
 *                                    + r * D2 ((C^k)^3 - C^k),
 * r = mobility*dt/(dx*dx), sigma = gamma*r/(dx*dx), D2 = [1, -2, 1] and D4 =
 * [1, -4, 6, -4, 1] wrapping modulo n.  theta = 1 is the semi-implicit scheme
 * (fourth-order term fully implicit); theta = 1/2 treats it like the page's
 * Crank-Nicolson hyperdiffusion step.  The implicit matrix is factored once
 * per call; the explicit side is the stencil of hyperdiffusion_theta_step
 * plus the phase-separation term.  Stability of the explicit term is the
 * caller's concern (steps are computed as asked).
 * C: device, interleaved [n][ld]; C^0 on entry, C^{nsteps} on return.
 * work: device, cahn_hilliard_work_bytes(dtype, n, batch) bytes.
 * n >= 6, batch >= 1, ld >= batch, nsteps >= 0, dt and dx finite, dx != 0,
 * gamma and mobility finite and >= 0, 0 <= theta <= 1 (else BPS_EINVAL). */
BPS_API bps_status cahn_hilliard_step(int dtype, int64_t n, int64_t batch, int64_t ld,
                              double dt, double dx, double gamma, double mobility,
                              double theta, void *C, int64_t nsteps, void *work,
                              void *stream);

/* ======================================================================== */
/* Tridiagonal systems  [H] section 4.1 (Thomas algorithm, cuThomasBatch)   */
/* ======================================================================== */

/* Bytes of `work` for tri_solve_batch with this n and ld (n*ld values, a
 * little more for n = 16*P with P > 64; 0 if invalid). */
BPS_API size_t tri_work_bytes(int dtype, int64_t n, int64_t ld);

/* Solve `batch` independent tridiagonal systems A u = y, row i of system s
 * holding a_i (column i-1), b_i (diagonal) and c_i (column i+1); a_0 and
 * c_{n-1} lie outside the matrix and are ignored.
 * a, b, c, y: device, interleaved [n][ld] (element (i, s) at i*ld + s);
 * a, b, c are not modified; y holds the right-hand sides on entry and the
 * solutions on return.  work: device, tri_work_bytes(dtype, n, ld) bytes,
 * scratch (contents undefined on return).  info: device int32[batch] or
 * NULL: 0, or 1 + the first row whose pivot of the page's Thomas
 * elimination (no pivoting) is zero or non-finite.
 * For n = M*P with M = 16 (else 12) and 2 <= P <= 64 the systems are solved
 * in M-row chunks (each eliminated with its own pivots, joined by a scalar
 * tridiagonal interface system); a system whose chunked elimination meets a
 * zero or non-finite pivot is re-solved in the same launch by the
 * sequential Thomas algorithm, so info and the solution are those of the
 * page's method.
 * For n = 16*P with 64 < P <= 65535 the chunks of a system are spread
 * over many workgroups (per-chunk elimination, the interface system solved
 * by this same routine, then each chunk's substitution), with the same
 * sequential rescue.  Other n: one lane per system (cuThomasBatch).
 * n >= 1, 1 <= batch <= 2^31 - 64, ld >= batch (else BPS_EINVAL). */
BPS_API bps_status tri_solve_batch(int dtype, int64_t n, int64_t batch, int64_t ld,
                           const void *a, const void *b, const void *c, void *y,
                           void *work, int32_t *info, void *stream);

/* ======================================================================== */
/* Hines tree-tridiagonal systems  [H] sections 2-4                         */
/* ======================================================================== */

/* Matrix of one neuron with n compartments ([H] section 2):
 *   A[i][i] = d_i,  A[p_i][i] = u_i ("upper"),  A[i][p_i] = l_i ("lower"),
 * parent p_i in [0, i) for i >= 1 (each parent numbered before its child);
 * p_0 and u_0, l_0 are not read.  Solved by Algorithm 1 of [H] (leaves-to-
 * root elimination, then root-to-leaves substitution). */
typedef struct bps_hines_plan bps_hines_plan;

/* Build a plan (host work + device upload; synchronises).
 * mono != 0 (one morphology for all neurons, [H] section 3):
 *   sizes: host int32[1] = {n}; parent: host int32[n];
 *   solver layout: Full-Interleaved [n][ld], ld >= batch (ld = 0 means batch).
 * mono == 0 (one morphology per neuron, [H] section 4):
 *   sizes: host int32[batch] compartments per neuron (>= 1);
 *   parent: host int32[sum(sizes)], each neuron's parents (local indices)
 *   one neuron after another.  The plan sorts neurons by size and packs
 *   them 64 per block (one wavefront), each block interleaved with its own
 *   row count (the Block-Interleaved layout of [H] with BS = 64); ld is
 *   ignored.  Use hines_pack / hines_unpack to convert data.
 * Fails with BPS_EINVAL if any p_i is outside [0, i). */
BPS_API bps_status hines_plan_create(bps_hines_plan **plan, int64_t batch, const int32_t *sizes,
                             const int32_t *parent, int mono, int64_t ld);
BPS_API bps_status hines_plan_destroy(bps_hines_plan *plan);

/* Schedules of hines_solve_batch ([H] sections 3 and 4):
 *   BPS_HINES_LANES   one lane per neuron over the whole tree (the page's
 *                     Full-/Block-Interleaved kernels);
 *   BPS_HINES_SPLIT   as LANES, but in a multi-morphology batch whose parents
 *                     all lie within 16 compartments every tree of 32 or more
 *                     compartments runs on two lanes of its wavefront (the
 *                     per-branch decomposition of section 4 inside a
 *                     wavefront: the side branches hanging from the trunk,
 *                     the path from the root into the largest subtrees, are
 *                     eliminated on both lanes, the trunk on the first as
 *                     its branches finish); a tree whose two-lane schedule
 *                     does not shorten it stays on one lane.  Mono plans:
 *                     as LANES;
 *   BPS_HINES_SEP     single compartments (separators) cut each tree into
 *                     components with at most one separator below each;
 *                     lanes eliminate whole components (Algorithm 1 inside
 *                     each, holding their rows' factors in registers), the
 *                     components' Schur complements on the separators form a
 *                     smaller tree system solved by Algorithm 1, then the
 *                     lanes substitute their rows: the per-branch
 *                     decomposition of section 4 with the pages' solve of
 *                     the reduced system, each compartment's values read and
 *                     written once.  Mono plans (trees of at most 2047
 *                     compartments whose components fit 16, 32 or 64
 *                     lanes of 32 rows): sixteen, thirty-two or sixty-four
 *                     lanes per neuron in the Full-Interleaved layout.  Multi-morphology plans (trees
 *                     of at most 8191 compartments): every tree on as many
 *                     lanes as it needs, trees packed into workgroups of 128
 *                     lanes, the plan's layout in schedule order (element
 *                     (w, t, k) = workgroup w, step t, lane k; the
 *                     separators' own rows among the lanes' rows; see
 *                     hines_sep_multi_layout).  The elimination order differs
 *                     from Algorithm 1's on the separators and on the paths
 *                     from them up to their components' roots, so results
 *                     differ by rounding; a neuron any of whose pivots in
 *                     this order is zero or not finite is solved again by
 *                     Algorithm 1 in the same call (its info is Algorithm
 *                     1's).  A lane keeps its pending updates and
 *                     voltages in eight slots, given per lane from the
 *                     tree's own order (parents may lie anywhere before
 *                     their children): components are made small enough
 *                     that no lane holds more than eight at once.
 *                     BPS_ENOTSUP for larger trees or when no partition
 *                     fits the lanes (32 rows each);
 *   BPS_HINES_LEVELS  one wavefront per neuron: the tree cut into its
 *                     unbranched sections, grouped by level (the page's
 *                     per-branch / per-level decomposition of section 4),
 *                     one section per lane and level, with the neuron held
 *                     in LDS; for batches too small to fill the GPU with one
 *                     lane per neuron.  Trees of at most 4096 compartments;
 *   BPS_HINES_AUTO    SEP for trees it takes: mono plans whose tree has a
 *                     parent more than 16 compartments back, or has at
 *                     least 256 compartments or a batch of at most 2^21
 *                     compartments in all, unless (parents within 16, at
 *                     least 24576 neurons) its schedule takes 64 lanes, or
 *                     32 lanes of 32 rows with more than 32 separators;
 *                     multi-morphology plans
 *                     unless the trees average under 128 compartments, have all
 *                     their parents within 16 and fill the GPU with one
 *                     lane each (at least 1024 blocks of 64); trees too
 *                     large for one workgroup of SEP's layout, if any, are
 *                     solved one lane each, their elements after the
 *                     others' (asked for explicitly, SEP takes every tree
 *                     or gives BPS_ENOTSUP).  Otherwise:
 *                     LEVELS for batches whose trees fit and that hold at
 *                     most 786432 compartments in all (mono) or 393216
 *                     (multi-morphology), else LANES; when one lane per
 *                     neuron would leave SIMDs of the GPU without a
 *                     wavefront (fewer than 1024 blocks of 64 neurons), the
 *                     largest trees go on two lanes as in SPLIT until the
 *                     blocks nearly fill them (what hines_plan_create
 *                     chooses).
 * Every schedule takes the same arguments; the solver layout is the plan's
 * (elements per array: hines_plan_elems; convert with hines_pack and
 * hines_unpack): a tree on two lanes has its compartments in the order its
 * schedule visits them. */
enum { BPS_HINES_AUTO = 0, BPS_HINES_LANES = 1, BPS_HINES_LEVELS = 2, BPS_HINES_SPLIT = 3,
       BPS_HINES_SEP = 4 };

/* hines_plan_create with an explicit schedule.  BPS_ENOTSUP for
 * BPS_HINES_LEVELS with a tree above 4096 compartments; BPS_EINVAL for an
 * unknown schedule. */
BPS_API bps_status hines_plan_create_sched(bps_hines_plan **plan, int64_t batch,
                                   const int32_t *sizes, const int32_t *parent, int mono,
                                   int64_t ld, int schedule);

/* 1 if the plan solves with the level schedule, else 0. */
BPS_API int hines_plan_uses_levels(const bps_hines_plan *plan);
/* Number of trees the plan solves on two lanes (0 for a NULL plan). */
BPS_API int64_t hines_plan_split(const bps_hines_plan *plan);
/* 1 if the plan solves with BPS_HINES_SEP (separator schedules), else 0. */
BPS_API int hines_plan_uses_sep(const bps_hines_plan *plan);

/* The schedule BPS_HINES_SEP would give one tree (host only, no device
 * needed; for inspection and host-side tests), as int32 words:
 *   [0] R rows per lane, [1] ns separators, [2] nc components, [3] npc
 *   components with a separator below, [4] nh compartments on those
 *   components' paths, [5] n, [6] lanes per neuron (16, 32 or 64), [7]
 *   neurons per workgroup (16, 8 with 32 lanes, 8 or 4 with 64);
 *   then codes [lanes][R]: lane k's step t of the first sweep (the second
 *   takes the steps in reverse): bits 0-10 the compartment, 11-13 its slot
 *   in the lane's ring of pending updates and voltages, 14-16 its parent's
 *   slot, 17 live (else padding), 18 on a path, 19 first row of a path, 20
 *   root of its component;
 *   then [lanes][3] per lane the numbers of its first component, first path
 *   row and first component with a path (each numbered in the order the
 *   lanes visit them, lane by lane);
 *   then ns x 5 words per separator (in descending compartment order): the
 *   compartment, its parent in the separator tree (-1 none), the component
 *   it hangs below (-1 when its parent is a separator or it is the root),
 *   and the range [b, e) of its components in the list below;
 *   then nc x 3 words per component: its parent separator (-1 for the
 *   root's component), the separator below it (-1 none), its path index
 *   (-1 none); then nc words: components listed by parent separator.
 *   parent: host int32[n], p_i in [0, i) (parent[0] ignored).
 * Returns the number of words written to out (at most cap), 0 if the tree
 * does not qualify (reason in bps_last_error), -1 on invalid arguments or
 * cap below the words needed. */
BPS_API int32_t hines_sep_schedule(int32_t n, const int32_t *parent, int32_t *out, int32_t cap);

/* The two-lane schedule BPS_HINES_SPLIT would give one tree (host only, no
 * device needed; for inspection and host-side tests).
 *   parent: host int32[n], p_i in [0, i) (parent[0] ignored).
 *   node, code: host arrays of 2*cap entries; lane j's step t (first sweep
 *   order, t < rows; the substitution takes the steps in reverse) is
 *   node[j*cap + t], the compartment it eliminates (-1 while the lane
 *   waits), and code[j*cap + t]: bits 0-5 the row's slot, bits 6-11 its
 *   parent's slot (slot ids 0..15 the lane's ring of pending updates and
 *   voltages, 16..31 the pair's trunk ring, 32 none), bit 12 live, bit 13
 *   the parent is the lane's previous live row of the substitution.
 * Returns the number of rows (steps), 0 if the tree stays on one lane, -1
 * on invalid arguments or cap below the rows (message in bps_last_error). */
BPS_API int32_t hines_split_schedule(int32_t n, const int32_t *parent, int32_t *node,
                                     uint16_t *code, int32_t cap);

/* The schedule BPS_HINES_SEP gives a multi-morphology batch (host only, no
 * device needed; for inspection and host-side tests).  sizes, parent as
 * for hines_plan_create with mono == 0.  dims: host int64[6], set to the
 * number of workgroups, the elements per value array of the
 * schedule-ordered layout (element (w, t, k) = workgroup w, step t < R,
 * lane k < K at ((w R + t) K + k)), R, the kernel's LDS bytes per
 * workgroup, the words of the workgroups' tables, and K, the lanes per
 * workgroup.  When every other pointer is non-NULL they receive (sized
 * from a first call with NULL arrays): code[elems] the row codes (bits 0-2
 * the row's ring slot, 3-5 its parent's, 6 live, 7 on a path, 8 first row
 * of a path, 9 root of its component, 10 a separator's own row),
 * comp[elems] the flat compartment of each element (-1 padding),
 * pos[sum(sizes)] the element of each flat compartment,
 * lanetab[workgroups * K][5] per lane its tree's slot in the workgroup (-1
 * unused) and its first component, path row, path component and separator
 * numbers, wgoff[workgroups + 1] and tabs: per workgroup 8 header words
 * (trees, separators, components, path components, path rows, 16-bit
 * table entries), 5 words per tree (separator range, lane range, tree
 * number) and 16-bit tables (per separator: its parent separator, the
 * component it hangs below, its range of components below; per component:
 * parent separator, lower separator, path index; the component list), all
 * numbered within the workgroup.
 * Returns 1, 0 if the batch does not qualify (reason in bps_last_error),
 * -1 on invalid arguments. */
BPS_API int32_t hines_sep_multi_layout(int64_t batch, const int32_t *sizes, const int32_t *parent,
                                       int64_t *dims, uint16_t *code, int32_t *comp, int32_t *pos,
                                       int32_t *lanetab, int64_t *wgoff, int32_t *tabs);

/* Elements of one value array (u, l, d or rhs) in the plan's solver layout. */
BPS_API int64_t hines_plan_elems(const bps_hines_plan *plan);
/* Real compartments (sum of sizes, or n*batch for mono). */
BPS_API int64_t hines_plan_unknowns(const bps_hines_plan *plan);

/* Layout transforms ([H] section 3: done once, off the time-stepping loop).
 * flat: device, the neurons' values one neuron after another (sum(sizes)
 * values; n*batch for mono, neuron-major).  packed: device,
 * hines_plan_elems values in the solver layout.  Padding entries of the
 * packed layout are written as 0 by hines_pack; no result depends on them,
 * and a solve may leave any value in those of rhs. */
BPS_API bps_status hines_pack(const bps_hines_plan *plan, int dtype, const void *flat,
                      void *packed, void *stream);
BPS_API bps_status hines_unpack(const bps_hines_plan *plan, int dtype, const void *packed,
                        void *flat, void *stream);

/* Bytes of `work` hines_solve_batch needs for this plan. */
BPS_API size_t hines_work_bytes(const bps_hines_plan *plan, int dtype);

/* Solve every neuron ([H] Algorithm 1) with the plan's schedule (one lane
 * per neuron, two lanes for split trees, separator schedules (sixteen,
 * thirty-two or sixty-four lanes per neuron, or every tree on its own
 * lanes), or one
 * wavefront per neuron).
 * u, l, d: device, solver layout, not modified.  rhs: device, solver layout,
 * right-hand side on entry, voltages V on return (as in [H]).  work: device,
 * hines_work_bytes bytes.  info: device int32[batch] indexed by the ORIGINAL
 * neuron number, or NULL; a nonzero value is 1 + the first compartment, in
 * Algorithm 1's elimination order (n-1 down to 1, then the root 0), whose
 * pivot is zero or not finite, whatever order the schedule eliminates in.
 * dtype must be BPS_F64. */
BPS_API bps_status hines_solve_batch(const bps_hines_plan *plan, int dtype,
                             const void *u, const void *l, const void *d,
                             void *rhs, void *work, int32_t *info, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BPS_H */
