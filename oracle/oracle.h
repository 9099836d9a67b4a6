/*
 * oracle.h -- plain CPU reference of the fast-multipole gravity evaluation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this; only the test-suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source, header or table with the GPU
 * library.
 *
 * Everything is fp64 (fp32 inputs are widened exactly by the caller), G = 1,
 * no softening.  Source: the jz-fmm project page (sections "From particle pairs
 * to node pairs", "Describing the source and the receiving region",
 * "Calculating a node-node interaction", "Combining near and far
 * interactions").  The readings taken where the page is silent are listed in
 * oracle.c next to the code that implements them.
 *
 * Coefficient layout used by the copy-out functions (shared *convention*
 * with the GPU library's introspection call, not shared code): multi-indices
 * (a,b,c) with a+b+c <= p, ordered by total degree d = 0..p, then a
 * descending, then b descending.  Multipoles are the raw power sums
 * M_(a,b,c) = sum_j m_j sx^a sy^b sz^c about the cell centre; locals are the
 * derivatives L_(a,b,c) = d^a_x d^b_y d^c_z Phi at the cell centre.
 */
#ifndef MBG_ORACLE_H
#define MBG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARG = -1,
  ORACLE_ERR_OOM = -3,
  ORACLE_ERR_NONFINITE = -5
};

typedef struct oracle_result oracle_result;

/* Number of coefficients of an expansion of total degree p: C(p+3,3). */
int oracle_ncoef(int order);

/* Thread count for the OpenMP loops (0 = leave the runtime default). */
void oracle_set_threads(int n);

/* O(N^2) direct sum, self term omitted by index.  Targets are indices into
 * pos; phi[t], acc[3t..3t+2] receive target t's results. */
int oracle_direct(int64_t n, const double* pos, const double* mass,
                  int64_t n_targets, const int64_t* targets,
                  double* phi, double* acc);

/* Full FMM evaluation.  If n_sample > 0, only the leaves holding the listed
 * particles (and their ancestors) are treated as targets: the tree, keys and
 * all multipoles are complete, the interaction lists are exact for the marked
 * targets and empty for the others, and phi/acc are valid for every particle
 * of a marked leaf (NaN elsewhere).  stage_mask bit 0 = run the numeric
 * passes (clear it to stop after the walk).  stage_mask bit 1 = digest mode:
 * the walk stores no lists but a digest of every target's two lists (see
 * oracle_copy_digests), walking the pairs below level 4 in parallel; no
 * numeric pass runs.  It serves sizes whose lists would not fit host memory. */
int oracle_fmm(int64_t n, const double* pos, const double* mass, int order,
               double theta, int leaf_size, int64_t n_sample,
               const int64_t* sample, int stage_mask, oracle_result** out);
void oracle_free(oracle_result* r);

/* sizes[0..6] = n_nodes, n_leaves, depth, n_m2l, n_p2p, n_marked_nodes, K */
void oracle_sizes(const oracle_result* r, int64_t* sizes);
/* root cube: lo[3] anchor, *side = power-of-two cube side */
void oracle_root(const oracle_result* r, double* lo, double* side);
/* stage wall times in seconds: [keys+sort, tree, walk, p2m+m2m, m2l, l2l+l2p, p2p, total] */
void oracle_times(const oracle_result* r, double* t8);
void oracle_copy_keys(const oracle_result* r, uint64_t* sorted_keys, int32_t* perm);
void oracle_copy_tree(const oracle_result* r, uint8_t* level, uint64_t* prefix,
                      int32_t* begin, int32_t* count, int32_t* parent,
                      int32_t* first_child, uint8_t* n_child);
void oracle_copy_lists(const oracle_result* r, int64_t* m2l_off, int32_t* m2l_src,
                       int64_t* p2p_off, int32_t* p2p_src);
void oracle_copy_mark(const oracle_result* r, uint8_t* node_mark);
/* Per target node [n_nodes]: the number of entries of its M2L and P2P lists
 * and the order-independent hash sum_s h(s) mod 2^64 of their sources, h(s) =
 * the (s+1)-th output of SplitMix64 seeded with 0.  From the walk in digest
 * mode, else from the stored lists. */
int oracle_copy_digests(const oracle_result* r, uint64_t* m2l_cnt, uint64_t* m2l_hash,
                        uint64_t* p2p_cnt, uint64_t* p2p_hash);
/* node_count x K arrays in the layout above; NULL skips one */
void oracle_copy_expansions(const oracle_result* r, double* mpole, double* local);
/* results in the caller's particle order */
void oracle_copy_result(const oracle_result* r, double* phi, double* acc);

/* Single-operator entry points, for pinning each step on its own. */
int oracle_p2m(int order, int64_t n, const double* pos, const double* mass,
               const double* centre, double* mpole);
int oracle_m2m(int order, const double* mpole_child, const double* d,
               double* mpole_parent_accum);
int oracle_dtensor(int order, const double* r, double* dtens);
int oracle_m2l(int order, const double* mpole, const double* r, double* local_accum);
int oracle_l2l(int order, const double* local_parent, const double* d,
               double* local_child_accum);
int oracle_l2p(int order, const double* local, const double* delta,
               double* phi, double* acc);
int oracle_morton(int64_t n, const double* pos, double* lo, double* side,
                  uint64_t* keys);

/* Vector-Jacobian products for S = sum_i pb_i phi_i + ab_i . a_i (pb [n],
 * ab [n][3], caller's order): xbar [n][3] = dS/dpos, mbar [n] = dS/dmass.
 * oracle_direct_vjp is the exact gradient of the direct sum (O(N^2));
 * oracle_fmm_vjp is the fast multipole form of the jz-fmm page on the tree and
 * lists of oracle_fmm with the same order, theta and leaf size (and the same
 * sampled mode: n_sample > 0 restricts the targets, NaN elsewhere). */
int oracle_direct_vjp(int64_t n, const double* pos, const double* mass,
                      const double* pb, const double* ab, double* xbar, double* mbar);
int oracle_fmm_vjp(int64_t n, const double* pos, const double* mass, int order,
                   double theta, int leaf_size, int64_t n_sample, const int64_t* sample,
                   const double* pb, const double* ab, double* xbar, double* mbar);
/* Moments of monopoles q [n] and point dipoles dip [n][3] about centre. */
int oracle_p2m_dipole(int order, int64_t n, const double* pos, const double* q,
                      const double* dip, const double* centre, double* mpole);
/* n_steps kick-drift-kick steps on the integer lattice x = q dx, v = u dv,
 * forward (direction +1) or backward (-1), updating q [n][3] and u [n][3] in
 * place; forces from oracle_fmm with the given order, theta and leaf size.
 * *min_margin: the closest any kick came to a rounding boundary (relative). */
int oracle_lattice_steps(int64_t n, int64_t* q, int64_t* u, const double* mass, double dx,
                         double dv, double dt, int n_steps, int direction, int order,
                         double theta, int leaf_size, double* min_margin);
/* Hessian of the local polynomial at offset delta: H6 = xx, yy, zz, xy, xz, yz. */
int oracle_l2p_hessian(int order, const double* local, const double* delta, double* H6);

#ifdef __cplusplus
}
#endif
#endif
