// fmm_internal.h -- plan object and kernel-launcher declarations shared by the
// HIP sources of libmbg_fmm.so.  Not installed; the public interface is
// include/fmm.h.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/fmm.h"

namespace mbg {

constexpr int KEY_BITS = 21;
constexpr int MAX_LEVELS = KEY_BITS + 1;  // levels 0..21

// Number of Cartesian coefficients of total degree <= p: C(p+3, 3).
constexpr int ncoef(int p) { return (p + 1) * (p + 2) * (p + 3) / 6; }
// Source record of a node for the M2L: its KR folded (traceless-form)
// moments (element size wb), then its centre as three fp64 words at the next
// 8-byte boundary, padded to a multiple of 16 bytes so that records can be
// moved in 16-byte pieces.
constexpr int mrec_centre_byte(int K, int wb) { return (K * wb + 7) / 8 * 8; }
constexpr int mrec_bytes(int K, int wb) { return (mrec_centre_byte(K, wb) + 24 + 15) / 16 * 16; }
constexpr int mrec_stride(int K, int wb) { return mrec_bytes(K, wb) / wb; }  // in elements

// Root cube and key scale, computed on the device.
struct RootInfo {
  double lo[3];
  double side;   // power of two
  double scale;  // 2^21 / side (exact)
};

// Work octaves in the launch orders (descending: octave 63 - floor(log2 w)).
constexpr int ORDER_OCT = 64;

// Device scalars written by kernels and read back at the build syncs.
constexpr int POOL_SHARDS = 512;
enum { POOL_CU = 0, POOL_U = 1, POOL_PU = 2, N_POOLS = 3 };
struct Control;
struct OsBufs;
// The walk's bookkeeping runs without a host check in between: after a pool
// or list overflow every kernel that indexes the walk's results does nothing,
// and the host repeats the walk with larger buffers.
__host__ __device__ inline bool walk_aborted(const Control* c);
struct Control {
  RootInfo root;  // the root cell, for the host
  int32_t nonfinite;
  int32_t pad0;
  int64_t n_nodes;
  int64_t n_leaves;
  int64_t level_off[MAX_LEVELS + 1];
  int64_t leaves_at_level[MAX_LEVELS];
  int64_t n_m2l;
  int64_t n_p2p;
  int64_t own_m2l_total, own_p2p_total;  // walk: entries found at the target's own level
  // (summed on the host from per-shard counts, so that the groups' additions
  // spread over many addresses)
  int64_t n_trm, n_trp;                   // walk: transposed M2L and P2P entries
  int64_t n_p2p_tasks, n_p2p_part;        // near-field tasks and partial-sum slots
  int64_t n_tail_tasks;                   // transposed-tail M2L tasks
  int32_t pool_overflow;                  // a sharded pool ran out of room
  int32_t list_overflow;                  // the transposed keys or the P2P lists ran out of room
  int64_t n_tr;                           // walk: n_trm + n_trp (the transposed keys)
  int64_t pool_used[N_POOLS][POOL_SHARDS];  // per pool and shard: entries handed out
  int64_t own_used[2][POOL_SHARDS];          // per shard: own M2L / P2P entries found
  // launch orders (work octaves, heaviest first) of the near-field tasks and
  // of the sibling M2L groups: per-octave counts and placement cursors
  int32_t task_oct[ORDER_OCT], task_cur[ORDER_OCT];
  int32_t group_oct[ORDER_OCT], group_cur[ORDER_OCT];
  int32_t n_split;  // leaves whose near field is split over several tasks
  int32_t tr_small_over;  // the one-block transposed-key path had too many keys
  int32_t sort_err;       // a single-pass sort gave up a wait (its order is wrong)
  int32_t pad1;
};
__host__ __device__ inline bool walk_aborted(const Control* c) {
  return (c->pool_overflow | c->list_overflow) != 0;
}
// Grow-only device buffer.
struct DBuf {
  void* p = nullptr;
  size_t cap = 0;
};

struct fmm_plan_impl;

}  // namespace mbg

struct fmm_plan_s {
  int64_t n;
  int order, K, leaf, dtype;
  double theta, t2;
  int device;
  int n_cu = 0;  // compute units of the device
  double clock_hz = 2.4e9;  // their peak clock (from the device when it reports one)
  bool built = false, evaluated = false, timing = false;
  bool timing_stages = false;   // timing: the stage events
  bool timing_kernels = false;  // timing: every main kernel's (else the near field's only)
  bool l2l_pulled = false;  // last eval used the one-launch downward pass

  // N-sized
  mbg::DBuf keys, keys_alt, idx, idx_alt, pts, far, perm_inv;
  mbg::DBuf lcp, wlev, wtmp, leaf_level, leaf_of;
  mbg::DBuf radix_hist, scan_tmp;
  mbg::DBuf os_state, os_dword;  // single-pass sorts: counters and histograms, tile status words
  mbg::DBuf root, ctrl, bbox_part;
  // node-sized
  mbg::DBuf nlevel, nprefix, nbegin, ncount, nparent, nfirst, nnchild, ncentre, nq, ngeo;
  mbg::DBuf leaves, lvl_blkcnt;
  mbg::DBuf mpole, mred, local, lfin;
  // VJP: sensitivity records (N), far parts (N), and the sensitivity
  // expansions (node-sized), apart from the forward's so that evals and VJPs
  // of one build can alternate
  mbg::DBuf vrec, vfar, vmpole, vmred, vlocal, vlfin;
  // lattice integrator: positions, potential and acceleration of the current
  // lattice state, and the overflow flag
  mbg::DBuf lat_pos, lat_phi, lat_acc, lat_flag;
  // walk: sharded pools (carry unions, M2L unions, P2P unions, transposed
  // M2L and P2P keys) and per-node slices / counts
  mbg::DBuf pool[mbg::N_POOLS];
  mbg::DBuf cu_off, cu_cnt, u_off, u_cnt, pu_off, pu_cnt, own_m2l, own_p2p;
  mbg::DBuf trm_cnt, trp_cnt, trm_base, trp_base;  // per parent index: transposed entries
  mbg::DBuf rootgen;
  mbg::DBuf tr_cnt_m2l, tr_start_m2l;  // [kind][node] run lengths / starts in the sorted keys
  mbg::DBuf tr_keys, tr_keys_alt, tr_vals, tr_vals_alt;
  const uint64_t* tr_sorted = nullptr;  // sorted transposed keys (one of tr_keys / tr_keys_alt)
  int64_t n_tr = 0;
  int key_shift = 0;
  mbg::DBuf m2l_off, m2l_src, p2p_off, p2p_src;
  bool m2l_lists_ready = false;  // per-target M2L lists materialized (on request only)
  // near-field tasks (target leaf x bounded slice of its list)
  mbg::DBuf p2p_task, p2p_part, p2p_toff, p2p_poff, tot_m2l, tot_p2p;
  mbg::DBuf split_leaves;  // positions (in the leaf list) of the split leaves, any order
  // mutual near field of sibling groups (optional): per-node flags
  mbg::DBuf mut_flag;
  bool mutual = false;      // the plan's setting
  bool mut_built = false;   // the flags of the current build exist
  int64_t n_split = 0;
  // non-leaf nodes in id order; the parents of level l are parents[pbeg[l] .. pbeg[l+1])
  mbg::DBuf parents, m2l_order;
  int64_t n_parents = 0, n_union = 0;
  int64_t pbeg[mbg::MAX_LEVELS + 2] = {0};
  // transposed-tail M2L tasks: per-leaf task offsets, tasks, partial locals
  mbg::DBuf tail_toff, tail_task, tail_part;
  int64_t n_tail_tasks = 0;
  int64_t n_p2p_tasks = 0, n_p2p_part = 0;

  // host copies of the last build's sizes
  int64_t n_nodes = 0, n_leaves = 0, n_m2l = 0, n_p2p = 0;
  int depth = 0;
  int64_t level_off[mbg::MAX_LEVELS + 1] = {0};
  int64_t leaves_at_level[mbg::MAX_LEVELS + 1] = {0};
  int walk_retries = 0;
  mbg::RootInfo root_host{};

  int64_t shard_cap[mbg::N_POOLS] = {0, 0, 0};  // entries per shard, per pool
  int64_t cap_tr = 0, cap_p2p = 0;  // room for transposed keys / near-field list entries
  int64_t cap_nodes = 0;  // room for nodes of the tree's second phase (0: none yet)
  int64_t last_own_m2l = 0;         // own M2L entries of the last build (sibling M2L issue)
  bool tr_small_ok = false;  // the last walk's transposed keys fit the one-block path
  bool walk_one_block = false;  // the last walk attempt took it
  int64_t pool_hint = -1;  // walk pool entries per node at each build; -1: automatic

  mbg::Control* ctrl_host = nullptr;  // pinned
  // The upward pass (P2M, M2M, M2L source records) depends only on the tree, so
  // a build issues it on a second stream of its own, where it overlaps the
  // walk; the eval's stream, and the next build's, wait for ev_up.
  // The sibling M2L (own entries) needs the unions and their launch order
  // only: the build issues it on the same stream after the upward pass, once
  // the walk has ordered the groups (ev_order), so it overlaps the rest of the
  // walk.  It writes `local`; the eval leaves `local` as it is and writes the
  // leaves' complete locals into `lfin`, so evals can repeat.
  hipStream_t up_stream = nullptr;
  hipEvent_t ev_tree = nullptr, ev_order = nullptr, ev_up = nullptr;
  hipEvent_t ev_rec = nullptr;  // the M2L source records are written (second stream)
  bool up_issued = false;
  // Every build, eval and VJP records ev_done on its stream at its end, and
  // the next call on another stream waits for it: calls on one plan run in the
  // order they are issued, whatever streams they are given (they rewrite or
  // read the same workspace).
  hipEvent_t ev_done = nullptr;
  hipEvent_t ev_ctrl = nullptr;  // the tree's control block copied to the host
  hipStream_t last_stream = nullptr;
  bool done_issued = false;
  hipEvent_t ev[2 * FMM_N_STAGES] = {};
  hipEvent_t kev[2 * FMM_N_KERNELS] = {};  // begin/end of single kernel launches
  bool kran[FMM_N_KERNELS] = {};          // the kernel ran in the last eval
  bool pend_build = false, pend_eval = false, pend_vjp = false;  // events not yet collected
  double stage_sum[FMM_N_STAGES] = {0}, kernel_sum[FMM_N_KERNELS] = {0};
  int32_t n_timed_builds = 0, n_timed_evals = 0, n_timed_vjps = 0;
};

namespace mbg {

// ---- launchers (each enqueues on `st`; return hipError_t) ----
hipError_t launch_bbox(const void* pos, const void* mass, int64_t n, int dtype, double* part,
                       int nblk, RootInfo* root, Control* ctrl, hipStream_t st);
hipError_t launch_keys(const void* pos, int64_t n, int dtype, const RootInfo* root,
                       uint64_t* keys, int32_t* idx, hipStream_t st);
hipError_t launch_radix_sort(uint64_t* keys, int32_t* idx, uint64_t* keys_alt, int32_t* idx_alt,
                             int64_t n, int32_t* hist, int32_t* scan_tmp, bool* in_alt,
                             hipStream_t st, const OsBufs* os = nullptr);
hipError_t launch_gather(const void* pos, const void* mass, const int32_t* perm, int64_t n,
                         int dtype, void* pts, hipStream_t st);
// Box, keys, stable sort and gather of a set of at most FRONT_MID_MAX particles
// in one launch: the same root, sorted keys, permutation and records as
// launch_bbox + launch_keys + launch_radix_sort + launch_gather (two instances:
// up to FRONT_MAX particles, and up to FRONT_MID_MAX).
constexpr int FRONT_MAX = 8000;
constexpr int FRONT_MID_MAX = 11264;
hipError_t launch_front_small(const void* pos, const void* mass, int64_t n, int dtype,
                              uint64_t* keys_sorted, int32_t* perm, void* pts, RootInfo* root,
                              Control* ctrl, hipStream_t st);
size_t radix_hist_ints(int64_t n);
size_t scan_tmp_bytes(int64_t n);

// Exclusive scan of int64 (in may alias out).  If total != nullptr the grand
// total is written there.
// r (1 to 3) int64 arrays of length n scanned together: exclusive scan of
// in[i] into out[i] (in place allowed), the total at out[i][n] and, if dst and
// dst[i] are given, at dst[i]; tmp: scan_tmp_bytes(n) * r bytes
hipError_t scan_exclusive_multi_i64(int r, const int64_t* const* in, int64_t* const* out,
                                    int64_t* const* dst, int64_t n, void* tmp, hipStream_t st);
hipError_t scan_exclusive_i64(const int64_t* in, int64_t* out, int64_t n, int64_t* total,
                              void* tmp, hipStream_t st);
hipError_t scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n, int32_t* total,
                              void* tmp, hipStream_t st);

struct TreeArrays {
  uint8_t* level;
  uint64_t* prefix;
  int32_t *begin, *count, *parent, *first_child;
  uint8_t* n_child;
  double* centre;  // [n_nodes][3]
  uint64_t* q;     // packed integer cell coords qx<<42 | qy<<21 | qz
  int4* geo;       // centre and half-width in units of 1/2^22 of the root side; leaf flag bit 30
};

hipError_t launch_tree_phase1(const uint64_t* keys, int64_t n, int leaf, int8_t* lcp, int8_t* wlev,
                              int8_t* wtmp, int8_t* leaf_level, int64_t* blkcnt, void* scan_tmp,
                              Control* ctrl, hipStream_t st);
size_t tree_blkcnt_len(int64_t n);
// The nodes from the first phase's counts in `ctrl`, into arrays of `cap`
// nodes (leaf_flag and leaf_scan: cap + 1 entries each).  It needs no host
// value of the node count, so it can be queued before that count is read
// back; with more nodes than `cap` it writes no node and the caller repeats it
// with room.
hipError_t launch_tree_phase2(const uint64_t* keys, int64_t n, int leaf, const int8_t* lcp,
                              const int8_t* leaf_level, const int64_t* blkcnt_scanned,
                              int64_t cap, const RootInfo* root, const TreeArrays& t,
                              int32_t* leaf_flag, int32_t* leaf_scan, int32_t* leaves,
                              int32_t* leaf_of, int32_t* parents, void* scan_tmp,
                              const Control* ctrl, hipStream_t st);

// ---- walk ----
// Sharded bump allocator: shard sh owns [sh * shard_cap, (sh+1) * shard_cap).
template <typename T>
struct Pool {
  T* data;
  int64_t shard_cap;
  int64_t* used;  // [POOL_SHARDS]
};
struct WalkArgs {
  const int4* geo;
  const int32_t* first_child;
  const uint8_t* n_child;
  const int32_t* parent;
  double t2;
  const int32_t* parents;  // non-leaf nodes, id order
  int64_t pbeg, pcnt;      // the parents of this step: parents[pbeg .. pbeg + pcnt)
  // pools of packed entries (node << 8) | child mask
  Pool<uint64_t> cu, u, pu;
  // per parent node: slices of its carry union, M2L union, P2P union
  int64_t *cu_off, *u_off, *pu_off;
  int32_t *cu_cnt, *u_cnt, *pu_cnt;
  int32_t *own_m2l, *own_p2p;  // per node: entries found at its own level
  int64_t *trm_cnt, *trp_cnt;  // per parent index: transposed entries it emits
  const int64_t *trm_base, *trp_base;  // their exclusive scans (emission pass)
  uint64_t* tr_keys;           // transposed keys, M2L then P2P (emission pass)
  int64_t tr_cap;              // room in tr_keys (more keys: list_overflow)
  const int64_t* n_trm;        // device total of the M2L ones
  const uint64_t* rootgen;     // the root's generator: one entry, the root itself
  int key_shift;
  Control* ctrl;
};
// one step: the children of the parents of one level, counted and written
hipError_t launch_walk(const WalkArgs& a, hipStream_t st);
// after the walk, every parent at once: the transposed keys (a.pbeg = 0,
// a.pcnt = all); also clears run_cnt[0 .. run_n) for the run step
hipError_t launch_tr_emit(const WalkArgs& a, int32_t* run_cnt, int64_t run_n, hipStream_t st);
hipError_t launch_walk_reset(Control* ctrl, uint64_t* rootgen, int root_leaf, int32_t* own_m2l,
                             int32_t* own_p2p, hipStream_t st);
hipError_t launch_walk_root_leaf(const int64_t* p2p_off, int32_t* p2p_src, hipStream_t st);

// n: room in keys; the keys present are min(*n_dev, n) (nothing after a walk abort)
hipError_t launch_tr_runs(const uint64_t* keys, int64_t n, const int64_t* n_dev,
                          const Control* ctrl, int key_shift, int kind_bit, int64_t n_nodes,
                          int64_t* start, int32_t* cnt, hipStream_t st);
hipError_t launch_walk_offsets(int64_t n_nodes, const int32_t* own, const int32_t* tr_cnt,
                               int64_t* tot, hipStream_t st);
// At most TRS_MAX transposed keys and TRS_MAX_NODES nodes (key_shift <= 17):
// the transposed sort, runs, run lengths, near-field list sizes and offsets
// (launch_radix_sort_bits + launch_tr_runs + launch_walk_offsets + the
// offsets scan) in one launch; keys_out gets the sorted keys.  More keys:
// list_overflow and tr_small_over are set.
constexpr int TRS_MAX = 8192;
constexpr int64_t TRS_MAX_NODES = 65536;
hipError_t launch_tr_small(const uint64_t* keys_in, int64_t cap, Control* ctrl, int key_shift,
                           int64_t n_nodes, uint64_t* keys_out, int64_t* start, int32_t* cnt,
                           const int32_t* own, int64_t* tot, int64_t* p2p_off, hipStream_t st);
// sorted transposed keys of one kind -> after each target's own entries
// (keys as launch_tr_runs; src has room for cap entries, more: list_overflow)
hipError_t launch_tr_scatter(const uint64_t* keys, int64_t n, const int64_t* n_dev,
                             Control* ctrl, int key_shift, int kind_bit, int kind,
                             int64_t n_nodes, const int64_t* off, const int32_t* own,
                             const int64_t* start, int32_t* src, int64_t cap, hipStream_t st);
// per-target own entries from the unions of their parents (root-leaf case included)
// (ctrl: null, or stop after a walk abort; src has room for cap entries)
hipError_t launch_union_scatter(const int32_t* parents, int64_t n_parents,
                                const int32_t* first_child, const uint8_t* n_child,
                                const uint64_t* pool, const int64_t* uoff, const int32_t* ucnt,
                                const int64_t* off, int32_t* src, int64_t cap, Control* ctrl,
                                hipStream_t st);


// LSD radix sort over the low `bits` bits; returns in *in_alt whether the
// result ended in (keys_alt, idx_alt).
// stable LSD sort of keys by bits [lo_bit, lo_bit + bits) (idx/idx_alt may be
// null for keys only); *in_alt tells which buffer holds the result
// Single-pass placement of each digit (decoupled look-back over the tiles):
// the passes' digit counts and tile counters, and the tiles' status words.
constexpr int OS_MAX_PASSES = 8;
struct OsState {
  uint32_t tile_ctr[OS_MAX_PASSES];
  int32_t hist[OS_MAX_PASSES][512];
};
struct OsBufs {
  OsState* state;   // cleared by the sort itself
  uint64_t* dword;  // os_dword_words(n) words, all zero when first allocated
  int32_t* err;     // set to 1 when a wait of the look-back was given up
};
size_t os_dword_words(int64_t n);
hipError_t launch_radix_sort_bits(uint64_t* keys, int32_t* idx, uint64_t* keys_alt,
                                  int32_t* idx_alt, int64_t n, int lo_bit, int bits,
                                  int32_t* hist, int32_t* scan_tmp, bool* in_alt,
                                  hipStream_t st, const int64_t* n_dev = nullptr,
                                  const Control* stop = nullptr, const OsBufs* os = nullptr);
// (n_dev: sort min(*n_dev, n) keys, n being the room in the buffers; stop:
// sort nothing after a walk abort; os: one launch per digit instead of three)

// ---- numeric passes ----
hipError_t launch_p2m(int dtype, int order, const void* pts, const int32_t* leaves,
                      int64_t n_leaves, const int32_t* begin, const int32_t* count,
                      const double* centre, void* mpole, hipStream_t st);
// M2M over every level of the tree, deepest parents first (level_off: the
// node ranges of levels 0 .. depth; parents at levels depth - 1 .. 0)
hipError_t launch_m2m_levels(int dtype, int order, const int64_t* level_off, int depth,
                             const int32_t* first_child, const uint8_t* n_child,
                             const double* centre, void* mpole, hipStream_t st);
// M2L: the root's local is cleared, the sibling blocks write every child's own
// entries (from its parent's M2L union), and the leaves' transposed tails (runs
// of the sorted transposed keys) are evaluated as tasks of at most TAIL_E
// entries and subtracted per leaf.
constexpr int TAIL_E = 64;
struct TailTask {
  int64_t e0;  // first entry in the sorted transposed keys
  int32_t n;   // entries (1..TAIL_E)
  int32_t li;  // index into the leaf list
};
struct M2LArgs {
  int64_t n_nodes;
  const int32_t* parents;
  int64_t n_parents;
  const int32_t* first_child;
  const uint8_t* n_child;
  const uint64_t* upool;  // packed (source << 8) | child mask
  const int64_t* u_off;   // per parent node
  const int32_t* u_cnt;
  const int32_t* leaves;
  int64_t n_leaves;
  const TailTask* tasks;
  int64_t n_tasks;
  const int64_t* toff;    // per leaf: first task (n_leaves + 1)
  const uint64_t* keys;   // sorted transposed keys; source = key & src_mask
  uint64_t src_mask;
  const double* centre;
  const void* mrec;       // source records (folded moments + centre)
  void* part;             // task partials (n_tasks x K)
  void* local;
  const Control* stop;    // null, or: the sibling kernel does nothing after a pool overflow
  hipEvent_t* ev;         // null, or begin/end events of the sibling and tail kernels
  bool* ran;              // with ev: set when the kernel was launched
  int64_t max_blocks;     // > 0: grid cap of the sibling kernel (its waves loop over parents)
};
// own entries: clears the root's local, then the sibling kernel writes the
// local of every other node (a.local)
hipError_t launch_m2l_sib(int dtype, int order, const M2LArgs& a, hipStream_t st);
// transposed tails: task partials into a.part; with combine, also subtracts
// each leaf's partials, in task order, from a.local
hipError_t launch_m2l_tails(int dtype, int order, const M2LArgs& a, bool combine,
                            hipStream_t st);
// launch order of the sibling M2L groups (parents with longer unions first),
// written to order[0 .. np) (counts in ctrl->group_oct, cursors group_cur,
// both zero at the start)
hipError_t launch_m2l_order(const int32_t* parents, int64_t np, const int32_t* u_cnt,
                            Control* ctrl, int32_t* order, hipStream_t st);

hipError_t launch_tail_fill(const int32_t* leaves, int64_t n_leaves, const int64_t* tr_start,
                            const int32_t* tr_cnt, const int64_t* toff, TailTask* tasks,
                            hipStream_t st);
// downward pass in one launch (orders with register kernels; false: not
// available, use the per-level L2L): out[leaf] = local[leaf] - its tail
// partials (toff / part, may be null) + every ancestor's local shifted to it
bool launch_l2l_pull(int dtype, int order, const int32_t* leaves, int64_t n_leaves,
                     const int32_t* parent, const double* centre, const void* local,
                     const int64_t* toff, const void* part, void* out, hipStream_t st);
// dst row r = src row r for the n listed rows of row_bytes bytes each
hipError_t launch_copy_rows(const int32_t* rows, int64_t n, int64_t row_bytes, const void* src,
                            void* dst, hipStream_t st);
// one level of the level-by-level L2L (skip_leaves: the n_child array, to leave
// leaves untouched; register kernels only)
hipError_t launch_l2l(int dtype, int order, int64_t lvl_begin, int64_t lvl_count,
                      const int32_t* parent, const double* centre, void* local,
                      const uint8_t* skip_leaves, hipStream_t st);
hipError_t launch_l2p(int dtype, int order, int64_t n, const void* pts, const int32_t* leaf_of,
                      const double* centre, const void* local, void* far, hipStream_t st);
size_t p2p_task_bytes();
// per leaf: near-field tasks, their partial-sum slots (0 for one task) and
// transposed-tail M2L tasks (tr_cnt: the leaves' transposed M2L run lengths)
hipError_t launch_leaf_task_counts(const int32_t* leaves, int64_t n_leaves, const int64_t* off,
                                   const int32_t* count, const int32_t* tr_cnt, int64_t* ntask,
                                   int64_t* npart, int64_t* ntail, int32_t* split, Control* ctrl,
                                   hipStream_t st);
// the tasks in launch order (heavier octaves of work first; ctrl->task_oct
// counted by launch_leaf_task_counts, task_cur zero at the start)
hipError_t launch_p2p_task_fill(const int32_t* leaves, int64_t n_leaves, int64_t n_tasks,
                                const int64_t* task_off, const int64_t* part_off,
                                const int64_t* off, const int32_t* count, Control* ctrl,
                                void* tasks, hipStream_t st);
// mutual near field of sibling groups: mut[leaf] = 1 where the group (the
// leaf children of one parent) holds 1..256 particles, 0 elsewhere
hipError_t launch_mutual_flags(const int32_t* parents, int64_t np, const int32_t* first_child,
                               const uint8_t* n_child, const int32_t* count, uint8_t* mut,
                               int64_t n_nodes, hipStream_t st);
// far[k] += the flagged groups' own pair sums (both sides of every pair once)
hipError_t launch_p2p_mutual(int dtype, int64_t np, const int32_t* parents,
                             const int32_t* first_child, const uint8_t* n_child,
                             const int32_t* begin, const int32_t* count, const void* pts,
                             void* far, hipStream_t st);
// mut / parent: null, or the flags above (entries of flagged groups' siblings
// and of the leaf itself are skipped)
hipError_t launch_p2p(int dtype, const void* tasks, int64_t n_tasks, const int32_t* leaves,
                      int64_t n_leaves, const int64_t* task_off, const int64_t* part_off,
                      const int32_t* begin, const int32_t* count, const uint8_t* mut,
                      const int32_t* parent, const int32_t* src,
                      const void* pts, const void* far, const int32_t* perm, void* phi, void* acc,
                      void* part, const int32_t* split, int64_t n_split, hipEvent_t* ev, bool* ran,
                      hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// ---- integer-lattice kick-drift-kick ----
// pos [N][3] = q dx in the dtype
hipError_t launch_lat_pos(int dtype, int64_t n, const int64_t* q, double dx, void* pos,
                          hipStream_t st);
// u += s rint(acc c); q += s rint(u c); *flag |= 1 on an increment that does
// not fit (or is not finite)
hipError_t launch_lat_kick(int dtype, int64_t n, int64_t* u, const void* acc, double c, int s,
                           int* flag, hipStream_t st);
hipError_t launch_lat_drift(int64_t n, int64_t* q, const int64_t* u, double c, int s, int* flag,
                            hipStream_t st);

// ---- vector-Jacobian product ----
// rec[k] = P8 (sorted particle k, pb and ab of caller index perm[k])
hipError_t launch_vjp_gather(int dtype, int64_t n, const void* pts, const int32_t* perm,
                             const void* pb, const void* ab, void* rec, hipStream_t st);
// leaf moments of the monopoles pb and dipoles ab held in the records
hipError_t launch_p2m_dip(int dtype, int order, const void* rec, const int32_t* leaves,
                          int64_t n_leaves, const int32_t* begin, const int32_t* count,
                          const double* centre, void* mpole, hipStream_t st);
// far-field parts per sorted particle: (Psi, -pb a - (Hess phi) ab + m grad Psi),
// from the forward's leaf locals and the sensitivity leaf locals
hipError_t launch_l2p_vjp(int dtype, int order, int64_t n, const void* rec, const int32_t* leaf_of,
                          const double* centre, const void* local, const void* blocal, void* out,
                          hipStream_t st);
// near field of the VJP on the forward's tasks; writes mbar [N] and xbar [N][3]
// in the caller's order (far parts from `far`)
hipError_t launch_p2p_vjp(int dtype, const void* tasks, int64_t n_tasks, const int32_t* leaves,
                          int64_t n_leaves, const int64_t* task_off, const int64_t* part_off,
                          const int32_t* begin, const int32_t* count, const int32_t* src,
                          const void* recs, const void* far, const int32_t* perm, void* mbar,
                          void* xbar, void* part, const int32_t* split, int64_t n_split,
                          hipEvent_t* ev, bool* ran, hipStream_t st);
// expansions in the plan's dtype/convention -> fp64 raw moments / derivatives
// traceless source records for the M2L: folded moments + centre, per node
hipError_t launch_m2l_records(int dtype, int order, int64_t n_nodes, const double* centre,
                              const void* mpole, void* mred, hipStream_t st);
hipError_t launch_export_expansions(int dtype, int order, int64_t n_nodes, const void* mpole,
                                    const void* local, double* mp_out, double* lc_out,
                                    hipStream_t st);

}  // namespace mbg
