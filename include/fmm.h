/*
 * fmm.h -- C-ABI of the MI355X (gfx950) fast-multipole gravity library
 * (libmbg_fmm.so).
 *
 * What it computes (jz-fmm project page):
 *   phi_i = -G sum_{j != i} m_j / |x_i - x_j|        ("From particle pairs to
 *   a_i   = -grad phi_i                                node pairs", direct-sum
 *                                                      equation; self term omitted)
 * approximated by the fast multipole method: Cartesian multipole moments of
 * every octree cell ("Describing the source and the receiving region", moment
 * equations), multipole-to-local translations of accepted cell pairs into local
 * Taylor coefficients ("Calculating a node-node interaction", the two closed
 * forms), the opening criterion theta = |l_A + l_B| / |c_A - c_B| with the pair
 * opened iff theta >= theta_max (same section), and the upward / interaction /
 * downward passes with a direct near field ("Combining near and far
 * interactions").  G = 1 (scale the outputs by G), no softening.
 *
 * Conventions shared by every call:
 *   - Order p: multipoles and locals keep total degree <= p and the
 *     translation keeps |n| + |m| <= p.  0 <= p <= FMM_MAX_ORDER.
 *   - The octree root is the cube anchored at the per-axis minimum of the
 *     positions with the smallest power-of-two side >= the largest extent;
 *     keys have 21 bits per axis (x the most significant bit of each triple);
 *     a cell is a leaf iff it holds <= leaf_size particles or is at level 21;
 *     expansion centres are geometric cell centres; cells are numbered
 *     breadth first (level, then key).  The criterion is evaluated exactly in
 *     integer cell units: accept iff 3 (h_A + h_B)^2 < fl(theta^2) |c_A - c_B|^2.
 *   - The walk splits the coarser non-leaf of a rejected pair (both when the
 *     levels are equal); accepted pairs are translated (M2L), rejected leaf
 *     pairs are summed directly (P2P).  Lists are directed, per target, with
 *     sources ascending.
 *   - Positions are row-major [N][3], masses [N], phi [N], acc [N][3], all in
 *     the plan's dtype and all DEVICE pointers owned by the caller; outputs are
 *     in the caller's particle order.
 *   - Every call returns an fmm_status code and never aborts.  Work is ordered
 *     on the HIP stream passed in (NULL = the default stream).  A plan is not
 *     thread-safe; distinct plans may run concurrently on distinct streams.
 *   - The same inputs and plan give bitwise-identical results on the same GPU:
 *     every accumulation has a fixed owner and a fixed order (no floating-point
 *     atomics).  (jz-fmm page, "Why reversibility matters": the force must be
 *     reproducible.)
 */
#ifndef MBG_FMM_H
#define MBG_FMM_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMM_MAX_ORDER 10
/* Largest octree a build accepts: node ids are 32-bit.  (Clustered inputs with
 * a small leaf size can need more cells than particles, so N < 2^31 alone does
 * not bound it.) */
#define FMM_MAX_NODES 2147483647LL

typedef struct fmm_plan_s* fmm_plan_t; /* opaque, owned by the library */

enum fmm_dtype { FMM_F32 = 0, FMM_F64 = 1 };

enum fmm_status {
  FMM_OK = 0,
  FMM_ERR_ARG = -1,       /* argument out of range / NULL pointer */
  FMM_ERR_STATE = -2,     /* eval or copy before a successful build */
  FMM_ERR_OOM = -3,       /* device allocation failed */
  FMM_ERR_HIP = -4,       /* a HIP runtime call failed, or a bounded wait of a kernel
                           * (the sort's look-back over its tiles) was given up */
  FMM_ERR_NONFINITE = -5, /* NaN or Inf in positions or masses */
  FMM_ERR_NODEVICE = -6   /* no HIP device visible */
};

/* Stage indices of fmm_stats_t.stage_ms (filled when timing is enabled). */
enum fmm_stage {
  FMM_STAGE_KEYS = 0,  /* bounding box + Morton keys            */
  FMM_STAGE_SORT = 1,  /* radix sort + gather into sorted order */
  FMM_STAGE_TREE = 2,  /* octree build                          */
  FMM_STAGE_WALK = 3,  /* dual-tree walk, M2L and P2P lists     */
  FMM_STAGE_UP = 4,    /* P2M + M2M + M2L source records (build, second stream) */
  FMM_STAGE_M2L = 5,   /* M2L of the own entries, sibling kernel (build, second stream) */
  FMM_STAGE_DOWN = 6,  /* L2L (build; L2P is timed as a kernel)  */
  FMM_STAGE_P2P = 7,   /* the single P2P (+ combine) launch     */
  FMM_STAGE_TAIL = 8,  /* M2L of the transposed tails (build)   */
  FMM_STAGE_VJP = 9,   /* the whole fmm_vjp call                */
  FMM_N_STAGES = 10
};

/* Kernel indices of fmm_stats_t.kernel_ms: single launches inside the M2L
 * and P2P stages (filled when timing is enabled; 0 for a kernel that did not
 * run). */
enum fmm_kernel {
  FMM_KERNEL_M2L_SIB = 0,     /* M2L over the sibling unions (own entries) */
  FMM_KERNEL_M2L_TAIL = 1,    /* M2L over the transposed tails            */
  FMM_KERNEL_P2P = 2,         /* near-field pair sums                     */
  FMM_KERNEL_P2P_COMBINE = 3, /* ordered sum of split leaves' partials    */
  FMM_KERNEL_VJP_M2L_SIB = 4, /* fmm_vjp: sibling M2L of the sensitivity moments */
  FMM_KERNEL_VJP_P2P = 5,     /* fmm_vjp: near-field pair sums            */
  FMM_KERNEL_P2M = 6,         /* leaf moments (build, second stream)      */
  FMM_KERNEL_L2P = 7,         /* far field at the particles (eval)        */
  FMM_N_KERNELS = 8
};

typedef struct {
  int64_t n, n_nodes, n_leaves, n_m2l, n_p2p;
  int32_t depth, order, leaf_size, dtype;
  double theta;
  double lo[3], side;    /* root cube */
  float stage_ms[FMM_N_STAGES]; /* mean over the timed steps, see fmm_set_timing */
  int32_t walk_retries;  /* workspace regrowths during the last walk */
  float kernel_ms[FMM_N_KERNELS]; /* mean over the timed builds (sibling M2L, P2M), evals or VJPs */
  int32_t timed_builds;  /* builds, evals and VJPs the means are taken over */
  int32_t timed_evals;
  int32_t timed_vjps;
  int32_t walk_one_block; /* 1: the last walk sorted its transposed keys (and formed the
                           * near-field list offsets) in the one-block path, taken when the
                           * plan's previous walk had few of them; 0: multi-block path */
} fmm_stats_t;

/* Create a plan for N particles.  N in [1, 2^31), order in [0, FMM_MAX_ORDER],
 * theta in (0, 1), leaf_size >= 1, dtype FMM_F32 or FMM_F64.  Allocates the
 * N-sized device workspace on the current device; data-dependent buffers grow
 * on demand during builds (grow-only, freed by fmm_destroy). */
int fmm_plan(fmm_plan_t* out, int64_t n, int order, double theta, int leaf_size, int dtype);

/* Sort the particles, build the octree and the interaction lists, form the
 * multipoles (P2M, M2M), translate them along every M2L entry and pass the
 * locals down to the leaves (L2L): the whole far field up to the leaves'
 * local expansions.  pos [N][3] and
 * mass [N] are device arrays in the plan's dtype; they are copied into the
 * plan's sorted layout, so the caller may reuse them once `stream` has passed
 * this call.  The multipoles need the tree only and the own-entry M2L the
 * walk's unions only: both run on a second stream owned by the plan, which
 * starts after the tree and overlaps the walk; the next fmm_eval or fmm_build
 * on any stream waits for it.  Synchronizes `stream` twice (tree size, list
 * sizes), once more per walk repeat when the list pools have to grow (see
 * fmm_set_walk_pool_hint).  Returns FMM_ERR_NONFINITE (and leaves the plan un-built)
 * if any input is NaN/Inf, FMM_ERR_OOM if the octree of these positions would
 * need more than FMM_MAX_NODES cells.
 *
 * Builds, evals and VJPs of one plan run in the order they are called, on
 * whatever streams: a call on a stream other than the previous call's waits
 * (on the device) for the end of that call before its first launch. */
int fmm_build(fmm_plan_t plan, const void* pos, const void* mass, void* stream);

/* Evaluate potential and acceleration of every particle: the leaves' local
 * expansions at the particles (L2P) plus the near field (P2P), written in the
 * caller's order.  phi [N] and acc [N][3] are device arrays in the plan's
 * dtype.  Asynchronous on `stream`; may be repeated after one build (the
 * build's results are only read). */
int fmm_eval(fmm_plan_t plan, void* phi, void* acc, void* stream);

/* Vector-Jacobian product of the evaluation (jz-fmm page, "Following
 * sensitivities backwards"): given the sensitivities phi_bar = dS/dphi [N] and
 * acc_bar = dS/da [N][3] of a scalar S, writes
 *   pos_bar [N][3] = dS/dpos = -phi_bar_i a_i - (Hess phi)(x_i) acc_bar_i
 *                              + m_i grad Psi(x_i),
 *   mass_bar [N]   = dS/dmass = Psi(x_i),
 * Psi being the potential of monopoles phi_bar and point dipoles acc_bar at the
 * particles (self term omitted).  The page's two contributions: the next
 * higher derivative (the Hessian) of the original evaluation, and an FMM whose
 * sources are the sensitivities acting as dipole moments.  Both use the plan's
 * tree, lists and order: the Hessian comes from the leaf locals of order p (one
 * degree below the acceleration), so build the plan one order higher than the
 * forward evaluation to keep the accuracy of that evaluation.  All arrays are
 * device arrays in the plan's dtype, in the caller's order.  Requires a built
 * plan (FMM_ERR_STATE otherwise); runs the forward's leaf locals itself if no
 * fmm_eval followed the build.  Asynchronous on `stream`; repeatable; ordered
 * after the plan's previous call like fmm_build.  Its own workspace (sensitivity records and
 * expansions, about 2 N + 3 n_nodes K values of the dtype) is allocated by the
 * first call after a build that needs more, grow-only like the plan's. */
int fmm_vjp(fmm_plan_t plan, const void* phi_bar, const void* acc_bar, void* pos_bar,
            void* mass_bar, void* stream);

/* Reversible integer-lattice kick-drift-kick steps (jz-fmm page, "Why
 * reversibility matters": positions and velocities on an integer lattice, the
 * force in floating point, an update undone by subtracting the same integer
 * increment).  State: q [N][3] and u [N][3], device int64 arrays, updated in
 * place; x = q dx, v = u dv.  Each step, with s = direction (+1 forward, -1
 * backward) and a the acceleration of the plan at the current x:
 *   u += s rint(a (dt/2)/dv);  q += s rint(u dt dv/dx);  u += s rint(a' (dt/2)/dv)
 * where a' is the acceleration at the new positions; every increment is one
 * fp64 product rounded half to even.  Because the evaluation is bitwise
 * reproducible, n steps backward undo n steps forward exactly.  mass [N] is a
 * device array in the plan's dtype.  Each call evaluates the force n_steps + 1
 * times (fmm_build + fmm_eval on the plan, whose previous build it replaces)
 * and synchronizes `stream` at the end.  FMM_ERR_ARG for a null pointer,
 * n_steps < 0, direction not +-1, dx or dv not positive or a non-finite
 * dt; FMM_ERR_NONFINITE if positions or masses are not finite, or an increment
 * is not finite or exceeds 2^62 in magnitude (the state is then unspecified). */
int fmm_lattice_steps(fmm_plan_t plan, int64_t* q, int64_t* u, const void* mass, double dx,
                      double dv, double dt, int n_steps, int direction, void* stream);

/* Free the plan and its workspace (synchronizes the device). */
int fmm_destroy(fmm_plan_t plan);

/* Static string for a status code. */
const char* fmm_strerror(int code);

/* Bits with which the walk packs a node id into its transposed
 * (kind, target, source) keys, for a tree of n_nodes cells: the smallest
 * b >= 1 with 2^b > n_nodes.  A key takes 2 b + 1 bits, at most 63 for
 * n_nodes <= FMM_MAX_NODES.
 * FMM_ERR_ARG for a null pointer or n_nodes outside [1, FMM_MAX_NODES].
 * Host only; touches no device. */
int fmm_node_id_bits(int64_t n_nodes, int* bits);

/* Near field of sibling leaves summed mutually (1) or directed (0, the
 * default).  The leaf children of one parent touch, so all their particle
 * pairs (a leaf with itself included) are near-field pairs in both
 * directions; with 1, one kernel sums each such unordered pair once and adds
 * it to both particles (for groups of at most 256 particles), and the directed
 * near field skips those list entries (the jaccpot issue's mutual
 * interactions, restricted to pairs whose two sides one workgroup holds).
 * Results agree with the directed form to rounding and stay bitwise
 * reproducible.  Takes effect at the next fmm_build; the VJP is unaffected. */
int fmm_set_mutual_near_field(fmm_plan_t plan, int enable);

/* Size of the walk's work pools at the start of each build, in entries per
 * tree node (-1, the default: 128 per node, grown from build to build as
 * needed).  A pool that runs out during a build is regrown from the measured
 * use and the walk repeated (fmm_stats_t.walk_retries counts the repeats;
 * FMM_ERR_OOM after 12); small values trade memory for repeats.  Lists and
 * results do not depend on it.  FMM_ERR_ARG for values below -1. */
int fmm_set_walk_pool_hint(fmm_plan_t plan, int64_t entries_per_node);

/* HIP-event timing: 1 = the stages and the main kernels, 2 = the main
 * kernels and the fmm_vjp stage only (the other stage_ms stay 0), 3 = the
 * near-field kernels (P2P and its combine) and the fmm_vjp stage only,
 * 0 = off.  Events
 * are recorded between launches on the stream that runs them (the caller's;
 * the plan's second stream for the upward stage); their times are collected
 * at the next synchronization the library makes anyway (the first one of the
 * next build) or by fmm_stats, so timing adds no synchronization.  Each event
 * is a marker in the stream, though, and the stage events (about thirty per
 * build and eval) make a step measurably slower (17 % at 4096 particles, 4 %
 * at 10^6), the twelve kernel events 5 % and 1.5 %.  Enabling resets the
 * means; FMM_ERR_ARG for other values. */
int fmm_set_timing(fmm_plan_t plan, int enable);

/* Sizes of the last build and, with timing on, the mean stage and kernel times
 * since timing was enabled (synchronizes the device). */
int fmm_stats(fmm_plan_t plan, fmm_stats_t* out);

/* ---- introspection (host copies for parity checks; each synchronizes) ---- */

/* sorted_keys [N] and perm [N] (perm[k] = caller index of sorted particle k). */
int fmm_copy_keys(fmm_plan_t plan, uint64_t* sorted_keys, int32_t* perm);

/* Node arrays [n_nodes], breadth-first order; NULL skips an array.
 * first_child is -1 for leaves. */
int fmm_copy_tree(fmm_plan_t plan, uint8_t* level, uint64_t* prefix, int32_t* begin,
                  int32_t* count, int32_t* parent, int32_t* first_child, uint8_t* n_child);

/* Interaction lists in CSR by target node: m2l_off [n_nodes+1], m2l_src
 * [n_m2l], p2p_off [n_nodes+1], p2p_src [n_p2p]; NULL skips an array. */
int fmm_copy_lists(fmm_plan_t plan, int64_t* m2l_off, int32_t* m2l_src, int64_t* p2p_off,
                   int32_t* p2p_src);

/* Multipoles and locals of the last build, [n_nodes][C(p+3,3)] fp64, for
 * multi-indices (a,b,c) ordered by degree, then a descending, then b
 * descending.  mpole = raw moments sum_j m_j s^(a,b,c) about the cell centre;
 * local = derivatives d^(a,b,c) phi at the cell centre (with every ancestor's
 * contribution translated in).  NULL skips one. */
int fmm_copy_expansions(fmm_plan_t plan, double* mpole, double* local);

/* ---- reference ---- */

/* Direct summation at chosen targets (jz-fmm page, "From particle pairs to node
 * pairs": the direct sum with the self term omitted), for accuracy
 * measurements: for t < n_targets, phi[t] and acc[3t..3t+2] of particle
 * targets[t] (caller indices in [0, n)) from all n particles.  pos [n][3],
 * mass [n], phi [n_targets] and acc [n_targets][3] are device arrays in the
 * dtype; targets [n_targets] is a device int64 array.  Sums run in fp64 in a
 * fixed order (bitwise reproducible).  Independent of any plan; allocates a
 * temporary workspace of 2 KiB per target and synchronizes `stream`.  Returns
 * FMM_ERR_ARG for null pointers, n < 1, n_targets < 0 or a bad dtype; a
 * target index outside [0, n) gets NaN results. */
int fmm_direct(const void* pos, const void* mass, int64_t n, const int64_t* targets,
               int64_t n_targets, int dtype, void* phi, void* acc, void* stream);

/* fmm_direct for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same results bit for bit, with the workspace in a
 * static device array of the library (8 MiB per device, held until the
 * process ends) instead of a temporary allocation.  Calls no hipMalloc,
 * hipFree or other allocating routine, and does not synchronize: the results
 * are ready when `stream` passes the call.  Every call on one device shares
 * that array: calls that overlap on one device (on different streams, or from
 * different threads) race and give undefined results.  FMM_ERR_ARG as
 * fmm_direct, and for n_targets > FMM_DIRECT_NOALLOC_MAX_TARGETS. */
#define FMM_DIRECT_NOALLOC_MAX_TARGETS 4096
int fmm_direct_noalloc(const void* pos, const void* mass, int64_t n, const int64_t* targets,
                       int64_t n_targets, int dtype, void* phi, void* acc, void* stream);

/* ---- measurement ---- */

/* Measured vector multiply-add rates of the current device, in TFLOP/s (two
 * flops per multiply-add): a kernel of independent fma chains filling every
 * compute unit, best of three timed runs after one warm-up, for fp64 and for
 * fp32 as this library compiles it (no packed two-wide fp32 operations).  The
 * benchmark reports the fraction of these next to the published peaks.
 * Allocates a small output buffer and synchronizes `stream`. */
int fmm_measure_peaks(double* fp64_tflops, double* fp32_tflops, void* stream);

#ifdef __cplusplus
}
#endif
#endif
