// fmm_api.hip -- host side of the C-ABI in include/fmm.h: plan and workspace
// management, stage sequencing, the two build synchronizations, timing and
// introspection copies.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "fmm_internal.h"

using namespace mbg;


namespace {

int status_of(hipError_t e) {
  if (e == hipSuccess) return FMM_OK;
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return FMM_ERR_OOM;
  return FMM_ERR_HIP;
}

#define TRY_HIP(x)                     \
  do {                                 \
    hipError_t _e = (x);               \
    if (_e != hipSuccess) return status_of(_e); \
  } while (0)
#define TRY(x)                    \
  do {                            \
    int _r = (x);                 \
    if (_r != FMM_OK) return _r;  \
  } while (0)

// Grow-only allocation (with 1/8 slack so that small fluctuations between
// builds do not reallocate).
int grow(DBuf& b, size_t bytes) {
  if (bytes == 0) bytes = 16;
  if (bytes <= b.cap) return FMM_OK;
  if (b.p) {
    hipError_t e = hipFree(b.p);
    if (e != hipSuccess) return status_of(e);
  }
  b.p = nullptr;
  b.cap = 0;
  size_t want = bytes + bytes / 8;
  want = (want + 255) & ~(size_t)255;
  if (hipMalloc(&b.p, want) != hipSuccess) {
    b.p = nullptr;
    return FMM_ERR_OOM;
  }
  b.cap = want;
  return FMM_OK;
}

// grow(), and a new allocation cleared to zero (in stream order)
int grow_cleared(DBuf& b, size_t bytes, hipStream_t st) {
  const void* before = b.p;
  const size_t cap0 = b.cap;
  TRY(grow(b, bytes));
  // a new allocation, even at the old address
  if (b.p != before || b.cap != cap0) TRY_HIP(hipMemsetAsync(b.p, 0, b.cap, st));
  return FMM_OK;
}


void release(DBuf& b) {
  if (b.p) (void)hipFree(b.p);
  b.p = nullptr;
  b.cap = 0;
}

template <typename T>
T* P(DBuf& b) {
  return static_cast<T*>(b.p);
}

// The particle sort places each digit in one launch (look-back over the
// tiles) for up to OS_SORT_MAX keys, where that measured faster than per-tile
// histograms, their scan and a scatter; above, with all of a pass's tiles
// resident at once, the chains of the look-back made it slower (10^6 keys:
// 0.246 -> 0.320 ms; 4*10^7: 5.94 -> 6.60 ms), and so they did for the walk's
// transposed-key sort at every size measured.
constexpr int64_t OS_SORT_MAX = (int64_t)1 << 17;
// The sort's buffers for up to n keys (grown, new status words cleared).
static int os_bufs(fmm_plan_t p, int64_t n, hipStream_t st, OsBufs* out, const OsBufs** use) {
  *use = nullptr;
  if (n > OS_SORT_MAX) return FMM_OK;
  TRY(grow(p->os_state, sizeof(OsState)));
  TRY(grow_cleared(p->os_dword, 8 * os_dword_words(n), st));
  *out = OsBufs{P<OsState>(p->os_state), P<uint64_t>(p->os_dword),
                &P<Control>(p->ctrl)->sort_err};
  *use = out;
  return FMM_OK;
}

size_t wbytes(int dtype) { return dtype == FMM_F64 ? 8 : 4; }

void rec(fmm_plan_t p, int stage, int end, hipStream_t st) {
  // the whole fmm_vjp call is timed in either mode
  if (p->timing && (p->timing_stages || stage == FMM_STAGE_VJP))
    (void)hipEventRecord(p->ev[2 * stage + end], st);
}

int bbox_blocks(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (int)std::min<int64_t>(std::max<int64_t>(b, 1), 1024);
}

// Timing: events are read only after a synchronization that follows them.
// The first three build stages are collected at the end of their build (after
// its last synchronization); the walk and upward stages (the latter on the
// second stream, which the next build's stream waits for before its first
// synchronization) and the eval's stages and kernels at the first
// synchronization of the next build, or by fmm_stats.
double elapsed(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) {
    (void)hipGetLastError();
    ms = 0.f;
  }
  return (double)ms;
}
void collect_early_build(fmm_plan_t p) {
  if (!p->timing) return;
  if (p->timing_stages)
    for (int s = FMM_STAGE_KEYS; s <= FMM_STAGE_TREE; s++)
      p->stage_sum[s] += elapsed(p->ev[2 * s], p->ev[2 * s + 1]);
  p->pend_build = true;  // the walk stage is still pending
}
void collect_pending(fmm_plan_t p) {
  if (p->pend_build) {
    if (p->timing_stages)
      for (int s : {FMM_STAGE_WALK, FMM_STAGE_UP, FMM_STAGE_M2L, FMM_STAGE_TAIL, FMM_STAGE_DOWN})
        p->stage_sum[s] += elapsed(p->ev[2 * s], p->ev[2 * s + 1]);
    for (int k : {FMM_KERNEL_M2L_SIB, FMM_KERNEL_P2M, FMM_KERNEL_M2L_TAIL})
      if (p->kran[k]) p->kernel_sum[k] += elapsed(p->kev[2 * k], p->kev[2 * k + 1]);
    p->n_timed_builds++;
    p->pend_build = false;
  }
  if (p->pend_eval) {
    if (p->timing_stages)
      p->stage_sum[FMM_STAGE_P2P] +=
          elapsed(p->ev[2 * FMM_STAGE_P2P], p->ev[2 * FMM_STAGE_P2P + 1]);
    for (int k : {FMM_KERNEL_P2P, FMM_KERNEL_P2P_COMBINE, FMM_KERNEL_L2P})
      if (p->kran[k]) p->kernel_sum[k] += elapsed(p->kev[2 * k], p->kev[2 * k + 1]);
    p->n_timed_evals++;
    p->pend_eval = false;
  }
  if (p->pend_vjp) {
    p->stage_sum[FMM_STAGE_VJP] +=
        elapsed(p->ev[2 * FMM_STAGE_VJP], p->ev[2 * FMM_STAGE_VJP + 1]);
    for (int k : {FMM_KERNEL_VJP_M2L_SIB, FMM_KERNEL_VJP_P2P})
      if (p->kran[k]) p->kernel_sum[k] += elapsed(p->kev[2 * k], p->kev[2 * k + 1]);
    p->n_timed_vjps++;
    p->pend_vjp = false;
  }
}

// Calls on one plan run in the order they are issued: a build, eval or VJP
// on a stream other than the previous call's first waits for the end of that
// call (they rewrite or read the same workspace: sorted particles, lists,
// task tables, partial sums), and records its own end for the next one.
int order_after_previous(fmm_plan_t p, hipStream_t st) {
  if (p->done_issued && st != p->last_stream) TRY_HIP(hipStreamWaitEvent(st, p->ev_done, 0));
  return FMM_OK;
}
int mark_done(fmm_plan_t p, hipStream_t st) {
  TRY_HIP(hipEventRecord(p->ev_done, st));
  p->last_stream = st;
  p->done_issued = true;
  return FMM_OK;
}

int sync_ctrl(fmm_plan_t p, hipStream_t st) {
  TRY_HIP(hipMemcpyAsync(p->ctrl_host, p->ctrl.p, sizeof(Control), hipMemcpyDeviceToHost, st));
  TRY_HIP(hipStreamSynchronize(st));
  return FMM_OK;
}


// ---------------- walk ----------------
int bits_for(int64_t v) {  // bits to hold 0..v (v < 2^62)
  int b = 1;
  while (b < 62 && ((int64_t)1 << b) <= v) b++;
  return b;
}

// Arguments of the M2L kernels for the current build.
M2LArgs m2l_args(fmm_plan_t p) {
  M2LArgs ma{};
  ma.n_nodes = p->n_nodes;
  ma.parents = P<int32_t>(p->m2l_order);
  ma.n_parents = p->n_parents;
  ma.first_child = P<int32_t>(p->nfirst);
  ma.n_child = P<uint8_t>(p->nnchild);
  ma.upool = P<uint64_t>(p->pool[POOL_U]);
  ma.u_off = P<int64_t>(p->u_off);
  ma.u_cnt = P<int32_t>(p->u_cnt);
  ma.leaves = P<int32_t>(p->leaves);
  ma.n_leaves = p->n_leaves;
  ma.tasks = P<TailTask>(p->tail_task);
  ma.n_tasks = p->n_tail_tasks;
  ma.toff = P<int64_t>(p->tail_toff);
  ma.keys = p->tr_sorted;
  ma.src_mask = (1ull << p->key_shift) - 1ull;
  ma.centre = P<double>(p->ncentre);
  ma.mrec = p->mred.p;
  ma.part = p->tail_part.p;
  ma.local = p->local.p;
  return ma;
}

// P2M, M2M (deepest level first) and the M2L source records on the second
// stream (ordered after the tree by ev_tree).
int issue_upward(fmm_plan_t p) {
  hipStream_t us = p->up_stream;
  const int dt = p->dtype, ord = p->order;
  const double* centre = P<double>(p->ncentre);
  rec(p, FMM_STAGE_UP, 0, us);
  if (p->timing_kernels) TRY_HIP(hipEventRecord(p->kev[2 * FMM_KERNEL_P2M], us));
  TRY_HIP(launch_p2m(dt, ord, p->pts.p, P<int32_t>(p->leaves), p->n_leaves,
                     P<int32_t>(p->nbegin), P<int32_t>(p->ncount), centre, p->mpole.p, us));
  if (p->timing_kernels) {
    TRY_HIP(hipEventRecord(p->kev[2 * FMM_KERNEL_P2M + 1], us));
    p->kran[FMM_KERNEL_P2M] = true;
  }
  TRY_HIP(launch_m2m_levels(dt, ord, p->level_off, p->depth, P<int32_t>(p->nfirst),
                            P<uint8_t>(p->nnchild), centre, p->mpole.p, us));
  TRY_HIP(launch_m2l_records(dt, ord, p->n_nodes, centre, p->mpole.p, p->mred.p, us));
  TRY_HIP(hipEventRecord(p->ev_rec, us));  // the M2L source records are written
  rec(p, FMM_STAGE_UP, 1, us);
  return FMM_OK;
}

// The sibling M2L on the second stream: after the upward pass (same stream)
// and the launch order (ev_order on the walk's stream).  ev_up marks its end.
// `capped`: two blocks (one wave per SIMD each) per compute unit, so that its
// waves never take all of a SIMD's registers and the walk's short kernels
// beside it (which raise their issue priority) find room on every unit.
int issue_sibling_m2l(fmm_plan_t p, hipStream_t st, bool capped) {
  hipStream_t us = p->up_stream;
  TRY_HIP(hipEventRecord(p->ev_order, st));
  TRY_HIP(hipStreamWaitEvent(us, p->ev_order, 0));
  M2LArgs ma = m2l_args(p);
  ma.ev = p->timing_kernels ? p->kev + 2 * FMM_KERNEL_M2L_SIB : nullptr;
  ma.ran = p->kran + FMM_KERNEL_M2L_SIB;
  ma.max_blocks = capped ? 2 * (int64_t)std::max(p->n_cu, 1) : 0;
  ma.stop = P<Control>(p->ctrl);  // the walk may still be repeated
  rec(p, FMM_STAGE_M2L, 0, us);
  TRY_HIP(launch_m2l_sib(p->dtype, p->order, ma, us));
  rec(p, FMM_STAGE_M2L, 1, us);
  TRY_HIP(hipEventRecord(p->ev_up, us));
  return FMM_OK;
}

// Expected duration of the sibling M2L over `own` own entries: about
// 444 ((p + 1) / 5)^4 flops per entry, at the fraction of the device's vector
// rate (compute units x 128 fp64 or unpacked fp32 flops per clock x clock)
// that the kernel reaches: about 0.46 in fp64 and 0.76 in fp32.
static double sibling_seconds(const fmm_plan_t p, int64_t own) {
  const double q = (p->order + 1) / 5.0;
  const double flops = 444.0 * q * q * q * q * (double)own;
  const double rate = 128.0 * (double)std::max(p->n_cu, 1) * p->clock_hz;
  return flops / ((p->dtype == FMM_F64 ? 0.46 : 0.76) * rate);
}

int run_walk(fmm_plan_t p, hipStream_t st) {
  const int depth = p->depth;
  const int64_t nn = p->n_nodes;
  const int64_t nl = p->n_leaves;
  const int64_t np = nn - nl;
  for (DBuf* b : {&p->cu_off, &p->u_off, &p->pu_off}) TRY(grow(*b, (size_t)nn * 8));
  for (DBuf* b : {&p->trm_cnt, &p->trp_cnt}) TRY(grow(*b, (size_t)std::max<int64_t>(np, 1) * 8));
  for (DBuf* b : {&p->trm_base, &p->trp_base})
    TRY(grow(*b, (size_t)(std::max<int64_t>(np, 1) + 1) * 8));
  for (DBuf* b : {&p->cu_cnt, &p->u_cnt, &p->pu_cnt, &p->own_m2l, &p->own_p2p})
    TRY(grow(*b, (size_t)nn * 4));
  TRY(grow(p->rootgen, 8));
  TRY(grow(p->tr_cnt_m2l, (size_t)2 * nn * 4));  // [kind][node]
  TRY(grow(p->tr_start_m2l, (size_t)2 * nn * 8));
  TRY(grow(p->tot_p2p, (size_t)(nn + 1) * 8));
  TRY(grow(p->p2p_off, (size_t)(nn + 1) * 8));
  TRY(grow(p->p2p_toff, (size_t)(nl + 1) * 8));
  TRY(grow(p->p2p_poff, (size_t)(nl + 1) * 8));
  TRY(grow(p->tail_toff, (size_t)(nl + 1) * 8));
  TRY(grow(p->scan_tmp, 3 * scan_tmp_bytes(std::max(nn, nl) + 1)));
  // the parents of level l (non-leaf nodes, id order) are parents[pbeg[l] .. pbeg[l + 1])
  p->n_parents = np;
  p->pbeg[0] = 0;
  for (int l = 0; l <= MAX_LEVELS; l++) {
    const int64_t cnt = l < MAX_LEVELS ? (p->level_off[l + 1] - p->level_off[l]) : 0;
    const int64_t lv = l < MAX_LEVELS ? p->leaves_at_level[l] : 0;
    p->pbeg[l + 1] = p->pbeg[l] + (cnt - lv);
  }
  if (p->pbeg[MAX_LEVELS + 1] != np) return FMM_ERR_HIP;
  // first guesses for the pools (regrown from the measured use on overflow)
  // (a group reserves its candidate count in each of the three unions): 128
  // entries per node and at least 2048 per shard, kept from build to build;
  // with a caller's hint, exactly hint entries per node at every build
  if (p->pool_hint >= 0) {
    const int64_t cap = std::max<int64_t>((p->pool_hint * nn + 4096) / POOL_SHARDS, 1);
    for (int k = 0; k < N_POOLS; k++) p->shard_cap[k] = cap;
  } else {
    const int64_t guess = 128 * nn + 4096;
    for (int k = 0; k < N_POOLS; k++)
      p->shard_cap[k] =
          std::max<int64_t>(p->shard_cap[k], std::max<int64_t>(guess / POOL_SHARDS, 2048));
  }

  WalkArgs a{};
  a.geo = P<int4>(p->ngeo);
  a.first_child = P<int32_t>(p->nfirst);
  a.n_child = P<uint8_t>(p->nnchild);
  a.parent = P<int32_t>(p->nparent);
  a.t2 = p->t2;
  a.parents = P<int32_t>(p->parents);
  a.cu_off = P<int64_t>(p->cu_off);
  a.u_off = P<int64_t>(p->u_off);
  a.pu_off = P<int64_t>(p->pu_off);
  a.trm_cnt = P<int64_t>(p->trm_cnt);
  a.trp_cnt = P<int64_t>(p->trp_cnt);
  a.trm_base = P<int64_t>(p->trm_base);
  a.trp_base = P<int64_t>(p->trp_base);
  a.cu_cnt = P<int32_t>(p->cu_cnt);
  a.u_cnt = P<int32_t>(p->u_cnt);
  a.pu_cnt = P<int32_t>(p->pu_cnt);
  a.own_m2l = P<int32_t>(p->own_m2l);
  a.own_p2p = P<int32_t>(p->own_p2p);
  a.rootgen = P<uint64_t>(p->rootgen);
  a.key_shift = bits_for(nn);
  p->key_shift = a.key_shift;
  const int kind_bit = 2 * a.key_shift;
  a.ctrl = P<Control>(p->ctrl);
  Control* dctrl = P<Control>(p->ctrl);
  const int root_leaf = (depth == 0) ? 1 : 0;
  int32_t* leaves = P<int32_t>(p->leaves);
  int64_t* toff = P<int64_t>(p->p2p_toff);
  int64_t* poff = P<int64_t>(p->p2p_poff);

  // Room for the transposed keys and the near-field lists.  The transposed
  // keys' sort, run search and scatter are launched over their room, so it
  // follows the previous walk's exact count with 1/16 slack (a first guess
  // per node before any walk; 48 per node was 5x the use on the 4*10^7
  // sphere); a walk that finds more repeats with the exact count.  The lists'
  // room only takes memory and is kept from build to build.
  p->cap_tr = p->n_tr > 0 ? p->n_tr + p->n_tr / 16 + 4096 : 48 * nn + 4096;
  p->cap_p2p = std::max<int64_t>(p->cap_p2p, 128 * nn + 4096);

  // The whole walk, its lists and its task counts are issued without a host
  // check: a pool or list that runs out of room sets a flag, every later
  // kernel that indexes the walk's results then does nothing, and the one
  // synchronization at the end finds the flag, regrows from the counts and
  // repeats.
  p->walk_retries = 0;
  for (;;) {
    for (int k = 0; k < N_POOLS; k++)
      TRY(grow(p->pool[k], (size_t)p->shard_cap[k] * POOL_SHARDS * 8));
    TRY(grow(p->tr_keys, (size_t)p->cap_tr * 8));
    TRY(grow(p->tr_keys_alt, (size_t)p->cap_tr * 8));
    TRY(grow(p->radix_hist, 4 * radix_hist_ints(p->cap_tr)));
    TRY(grow(p->scan_tmp, scan_tmp_bytes((int64_t)radix_hist_ints(p->cap_tr))));
    TRY(grow(p->p2p_src, (size_t)p->cap_p2p * 4));
    Pool<uint64_t>* pools[N_POOLS] = {&a.cu, &a.u, &a.pu};
    for (int k = 0; k < N_POOLS; k++)
      *pools[k] = Pool<uint64_t>{P<uint64_t>(p->pool[k]), p->shard_cap[k], dctrl->pool_used[k]};
    TRY_HIP(launch_walk_reset(dctrl, P<uint64_t>(p->rootgen), root_leaf, a.own_m2l, a.own_p2p,
                              st));
    for (int l = 0; l < depth; l++) {
      a.pbeg = p->pbeg[l];
      a.pcnt = p->pbeg[l + 1] - p->pbeg[l];
      TRY_HIP(launch_walk(a, st));
    }
    {  // offsets of every group's transposed keys, in group order; totals to the control block
      const int64_t* in[2] = {a.trm_cnt, a.trp_cnt};
      int64_t* out[2] = {P<int64_t>(p->trm_base), P<int64_t>(p->trp_base)};
      int64_t* dst[2] = {&dctrl->n_trm, &dctrl->n_trp};
      TRY_HIP(scan_exclusive_multi_i64(2, in, out, dst, np, p->scan_tmp.p, st));
    }
    // the upward pass, once the first attempt's walk launches are all queued
    // (its host launch time then overlaps the walk instead of delaying it)
    if (p->walk_retries == 0) TRY(issue_upward(p));

    // launch order of the M2L sibling blocks; then the sibling M2L itself on
    // the second stream, where it overlaps the rest of the walk.  A short one
    // (under a millisecond, estimated from the last build's own entries)
    // starts now on a capped grid, so that it runs beside the transposed sort
    // and the rest of the walk (2 % off the 10^6 step); a long one waits for
    // the transposed sort and takes the whole GPU (capped, it ran 12 % slower
    // on the 4*10^7 sphere).
    TRY(grow(p->m2l_order, (size_t)std::max<int64_t>(np, 1) * 4));
    TRY_HIP(launch_m2l_order(a.parents, np, a.u_cnt, dctrl, P<int32_t>(p->m2l_order), st));
    const bool sib_early = sibling_seconds(p, p->last_own_m2l) < 1e-3;
    if (sib_early) TRY(issue_sibling_m2l(p, st, true));

    // transposed entries: emitted in group order (ascending source for each
    // target), then stably sorted on (kind, target); run lengths per target
    int32_t* tr_cnt = P<int32_t>(p->tr_cnt_m2l);
    int64_t* tr_start = P<int64_t>(p->tr_start_m2l);
    a.tr_keys = P<uint64_t>(p->tr_keys);
    a.tr_cap = p->cap_tr;
    a.n_trm = &dctrl->n_trm;
    a.pbeg = 0;
    a.pcnt = np;
    TRY_HIP(launch_tr_emit(a, tr_cnt, 2 * nn, st));  // also clears tr_cnt
    int64_t* p2p_off = P<int64_t>(p->p2p_off);
    const uint64_t* sorted = nullptr;
    // few transposed keys (as many as the last walk had, when that fitted
    // comfortably): sort, runs and the near-field offsets in one launch
    const bool tr_small = p->tr_small_ok && a.key_shift <= 17 && nn <= TRS_MAX_NODES;
    p->walk_one_block = tr_small;
    if (tr_small) {
      TRY_HIP(launch_tr_small(P<uint64_t>(p->tr_keys), p->cap_tr, dctrl, a.key_shift, nn,
                              P<uint64_t>(p->tr_keys_alt), tr_start, tr_cnt, a.own_p2p,
                              P<int64_t>(p->tot_p2p), p2p_off, st));
      sorted = P<uint64_t>(p->tr_keys_alt);
    } else {
      bool in_alt = false;
      TRY_HIP(launch_radix_sort_bits(P<uint64_t>(p->tr_keys), nullptr,
                                     P<uint64_t>(p->tr_keys_alt), nullptr, p->cap_tr,
                                     a.key_shift, a.key_shift + 1, P<int32_t>(p->radix_hist),
                                     P<int32_t>(p->scan_tmp), &in_alt, st, &dctrl->n_tr, dctrl));
      sorted = in_alt ? P<uint64_t>(p->tr_keys_alt) : P<uint64_t>(p->tr_keys);
      TRY_HIP(launch_tr_runs(sorted, p->cap_tr, &dctrl->n_tr, dctrl, a.key_shift, kind_bit, nn,
                             tr_start, tr_cnt, st));
    }
    p->tr_sorted = sorted;
    // a long sibling M2L beside the rest of the walk, after the transposed sort
    // (beside that sort, on a full grid, the sort's kernels were starved)
    if (!sib_early) TRY(issue_sibling_m2l(p, st, false));

    // P2P lists: own entries (from the parents' P2P unions) then transposed ones
    if (!tr_small) {
      TRY_HIP(launch_walk_offsets(nn, a.own_p2p, tr_cnt + nn, P<int64_t>(p->tot_p2p), st));
      const int64_t* in[1] = {P<int64_t>(p->tot_p2p)};
      int64_t* out[1] = {p2p_off};
      int64_t* dst[1] = {&dctrl->n_p2p};
      TRY_HIP(scan_exclusive_multi_i64(1, in, out, dst, nn, p->scan_tmp.p, st));
    }
    int32_t* p2p_src = P<int32_t>(p->p2p_src);
    TRY_HIP(launch_union_scatter(a.parents, np, a.first_child, a.n_child, a.pu.data, a.pu_off,
                                 a.pu_cnt, p2p_off, p2p_src, p->cap_p2p, dctrl, st));
    if (root_leaf) TRY_HIP(launch_walk_root_leaf(p2p_off, p2p_src, st));
    TRY_HIP(launch_tr_scatter(sorted, p->cap_tr, &dctrl->n_tr, dctrl, a.key_shift, kind_bit, 1,
                              nn, p2p_off, a.own_p2p, tr_start + nn, p2p_src, p->cap_p2p, st));

    // near-field tasks, their partial slots and the transposed-tail M2L tasks,
    // per leaf; offsets and totals (to the control block) in one scan
    int64_t* ttoff = P<int64_t>(p->tail_toff);
    TRY(grow(p->split_leaves, (size_t)std::max<int64_t>(nl, 1) * 4));
    TRY_HIP(launch_leaf_task_counts(leaves, nl, p2p_off, P<int32_t>(p->ncount), tr_cnt, toff,
                                    poff, ttoff, P<int32_t>(p->split_leaves), dctrl, st));
    {
      const int64_t* in[3] = {toff, poff, ttoff};
      int64_t* out[3] = {toff, poff, ttoff};
      int64_t* dst[3] = {&dctrl->n_p2p_tasks, &dctrl->n_p2p_part, &dctrl->n_tail_tasks};
      TRY_HIP(scan_exclusive_multi_i64(3, in, out, dst, nl, p->scan_tmp.p, st));
    }
    TRY(sync_ctrl(p, st));
    const Control& c = *p->ctrl_host;
    if (!c.pool_overflow && !c.list_overflow) break;
    // repeat with more room: the second stream's kernels of this attempt
    // (the sibling M2L reads the pools) end first
    if (++p->walk_retries > 12) return FMM_ERR_OOM;
    TRY_HIP(hipStreamSynchronize(p->up_stream));
    if (c.tr_small_over) p->tr_small_ok = false;  // the multi-block path from here on
    if (c.pool_overflow) {  // the levels after the first overflow did not run: grow at least twofold
      for (int k = 0; k < N_POOLS; k++) {
        int64_t mx = 0;
        for (int sh = 0; sh < POOL_SHARDS; sh++) mx = std::max(mx, c.pool_used[k][sh]);
        if (mx > p->shard_cap[k]) p->shard_cap[k] = std::max(mx + mx / 2, 2 * p->shard_cap[k]);
      }
    } else {  // the walk is complete: the exact sizes are known
      int64_t own_p = c.own_p2p_total;
      for (int sh = 0; sh < POOL_SHARDS; sh++) own_p += c.own_used[1][sh];
      const int64_t ntr = c.n_trm + c.n_trp, np2p = own_p + c.n_trp;
      if (ntr > p->cap_tr) p->cap_tr = ntr + ntr / 8;
      if (np2p > p->cap_p2p) p->cap_p2p = np2p + np2p / 8;
    }
  }
  const Control& c = *p->ctrl_host;
  int64_t nu = 0, own_m = 0, own_p = c.own_p2p_total;  // the root's, when it is a leaf
  for (int sh = 0; sh < POOL_SHARDS; sh++) {
    nu += c.pool_used[POOL_U][sh];
    own_m += c.own_used[0][sh];
    own_p += c.own_used[1][sh];
  }
  const int64_t ntm = c.n_trm, ntp = c.n_trp;
  p->n_union = nu;  // room reserved for the M2L unions (an upper bound)
  p->n_m2l = own_m + ntm;
  p->n_p2p = own_p + ntp;
  p->n_tr = ntm + ntp;
  p->tr_small_ok = p->n_tr <= 3 * TRS_MAX / 4;  // for the next build
  p->last_own_m2l = own_m;
  p->m2l_lists_ready = false;
  if (c.n_p2p != p->n_p2p || c.n_tr != p->n_tr) return FMM_ERR_HIP;
  p->n_p2p_tasks = c.n_p2p_tasks;
  p->n_p2p_part = c.n_p2p_part;
  p->n_split = c.n_split;
  p->n_tail_tasks = c.n_tail_tasks;
  TRY(grow(p->p2p_task, (size_t)std::max<int64_t>(p->n_p2p_tasks, 1) * p2p_task_bytes()));
  TRY(grow(p->p2p_part, (size_t)std::max<int64_t>(p->n_p2p_part, 1) * 4 * wbytes(p->dtype)));
  TRY_HIP(launch_p2p_task_fill(leaves, nl, p->n_p2p_tasks, toff, poff, P<int64_t>(p->p2p_off),
                               P<int32_t>(p->ncount), dctrl, p->p2p_task.p, st));
  TRY(grow(p->tail_task, (size_t)std::max<int64_t>(p->n_tail_tasks, 1) * sizeof(TailTask)));
  TRY(grow(p->tail_part,
           (size_t)std::max<int64_t>(p->n_tail_tasks, 1) * p->K * wbytes(p->dtype)));
  TRY_HIP(launch_tail_fill(leaves, nl, P<int64_t>(p->tr_start_m2l), P<int32_t>(p->tr_cnt_m2l),
                           P<int64_t>(p->tail_toff), P<TailTask>(p->tail_task), st));
  p->mut_built = false;
  if (p->mutual) {
    TRY(grow(p->mut_flag, (size_t)nn));
    TRY_HIP(launch_mutual_flags(a.parents, np, a.first_child, a.n_child, P<int32_t>(p->ncount),
                                P<uint8_t>(p->mut_flag), nn, st));
    p->mut_built = true;
  }
  return FMM_OK;
}

// Per-target M2L lists (own entries from the parents' M2L unions, then the
// transposed tail), built only when they are asked for.
int materialize_m2l_lists(fmm_plan_t p, hipStream_t st) {
  if (p->m2l_lists_ready) return FMM_OK;
  const int64_t nn = p->n_nodes;
  TRY(grow(p->tot_m2l, (size_t)(nn + 1) * 8));
  TRY(grow(p->m2l_off, (size_t)(nn + 1) * 8));
  TRY(grow(p->m2l_src, (size_t)std::max<int64_t>(p->n_m2l, 1) * 4));
  int64_t* off = P<int64_t>(p->m2l_off);
  const int32_t* own = P<int32_t>(p->own_m2l);
  TRY_HIP(launch_walk_offsets(nn, own, P<int32_t>(p->tr_cnt_m2l), P<int64_t>(p->tot_m2l), st));
  TRY_HIP(scan_exclusive_i64(P<int64_t>(p->tot_m2l), off, nn, off + nn, p->scan_tmp.p, st));
  TRY_HIP(launch_union_scatter(P<int32_t>(p->parents), p->n_parents, P<int32_t>(p->nfirst),
                               P<uint8_t>(p->nnchild), P<uint64_t>(p->pool[POOL_U]),
                               P<int64_t>(p->u_off), P<int32_t>(p->u_cnt), off,
                               P<int32_t>(p->m2l_src), p->n_m2l, nullptr, st));
  if (p->n_tr > 0)
    TRY_HIP(launch_tr_scatter(p->tr_sorted, p->n_tr, nullptr, nullptr, p->key_shift,
                              2 * p->key_shift, 0, nn, off, own, P<int64_t>(p->tr_start_m2l),
                              P<int32_t>(p->m2l_src), p->n_m2l, st));
  TRY_HIP(hipStreamSynchronize(st));
  p->m2l_lists_ready = true;
  return FMM_OK;
}

// The leaves' complete forward locals in lfin: the M2L of the transposed
// tails, then the downward pass (one launch at orders <= 6, else level by
// level on a copy of `local`).  Records the tail stage and the start of the
// downward stage.  With the one-launch pass the tails only write their
// partials and need only the source records, so they start before the
// own-entry M2L on the second stream has finished (in its shadow); the pass
// itself waits for that M2L.
int leaf_locals(fmm_plan_t p, hipStream_t st) {
  const int dt = p->dtype, ord = p->order;
  const double* centre = P<double>(p->ncentre);
  int32_t* leaves = P<int32_t>(p->leaves);
  const int64_t nn = p->n_nodes;
  const size_t lbytes = (size_t)nn * p->K * wbytes(dt);
  const bool pull = ord <= 6;  // the one-launch downward pass

  TRY_HIP(hipStreamWaitEvent(st, pull ? p->ev_rec : p->ev_up, 0));
  rec(p, FMM_STAGE_TAIL, 0, st);
  M2LArgs ma = m2l_args(p);
  ma.ev = p->timing_kernels ? p->kev + 2 * FMM_KERNEL_M2L_TAIL : nullptr;
  ma.ran = p->kran + FMM_KERNEL_M2L_TAIL;
  if (!pull) {  // the level-by-level pass works on a copy
    TRY_HIP(hipMemcpyAsync(p->lfin.p, p->local.p, lbytes, hipMemcpyDeviceToDevice, st));
    ma.local = p->lfin.p;
  }
  TRY_HIP(launch_m2l_tails(dt, ord, ma, !pull, st));
  rec(p, FMM_STAGE_TAIL, 1, st);
  if (pull) TRY_HIP(hipStreamWaitEvent(st, p->ev_up, 0));  // the own-entry locals

  rec(p, FMM_STAGE_DOWN, 0, st);
  p->l2l_pulled = pull && launch_l2l_pull(dt, ord, leaves, p->n_leaves, P<int32_t>(p->nparent),
                                          centre, p->local.p,
                                          p->n_tail_tasks > 0 ? P<int64_t>(p->tail_toff) : nullptr,
                                          p->tail_part.p, p->lfin.p, st);
  if (pull && !p->l2l_pulled) return FMM_ERR_HIP;
  if (p->l2l_pulled) {
    TRY_HIP(hipGetLastError());
  } else {
    for (int l = 1; l <= p->depth; l++)
      TRY_HIP(launch_l2l(dt, ord, p->level_off[l], p->level_off[l + 1] - p->level_off[l],
                         P<int32_t>(p->nparent), centre, p->lfin.p, nullptr, st));
  }
  return FMM_OK;
}

}  // namespace

extern "C" {

const char* fmm_strerror(int code) {
  switch (code) {
    case FMM_OK: return "ok";
    case FMM_ERR_ARG: return "invalid argument";
    case FMM_ERR_STATE: return "plan not built";
    case FMM_ERR_OOM: return "device out of memory";
    case FMM_ERR_HIP: return "HIP runtime error";
    case FMM_ERR_NONFINITE: return "non-finite position or mass";
    case FMM_ERR_NODEVICE: return "no HIP device";
    default: return "unknown status";
  }
}

int fmm_plan(fmm_plan_t* out, int64_t n, int order, double theta, int leaf_size, int dtype) {
  if (!out) return FMM_ERR_ARG;
  *out = nullptr;
  if (n < 1 || n >= ((int64_t)1 << 31) || order < 0 || order > FMM_MAX_ORDER || !(theta > 0.0) ||
      !(theta < 1.0) || leaf_size < 1 || (dtype != FMM_F32 && dtype != FMM_F64))
    return FMM_ERR_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return FMM_ERR_NODEVICE;
  fmm_plan_t p = new (std::nothrow) fmm_plan_s();
  if (!p) return FMM_ERR_OOM;
  p->n = n;
  p->order = order;
  p->K = ncoef(order);
  p->leaf = leaf_size;
  p->dtype = dtype;
  p->theta = theta;
  p->t2 = theta * theta;  // one rounding, as the criterion specifies
  int rc = FMM_OK;
  auto fail = [&](int r) {
    fmm_destroy(p);
    return r;
  };
  if (hipGetDevice(&p->device) != hipSuccess ||
      hipDeviceGetAttribute(&p->n_cu, hipDeviceAttributeMultiprocessorCount, p->device) !=
          hipSuccess)
    return fail(FMM_ERR_HIP);
  {
    int khz = 0;  // peak engine clock; only the scheduling estimate above uses it
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, p->device) == hipSuccess &&
        khz > 0)
      p->clock_hz = 1e3 * (double)khz;
  }
  const size_t w = wbytes(dtype);
  if ((rc = grow(p->keys, 8 * n)) || (rc = grow(p->keys_alt, 8 * n)) || (rc = grow(p->idx, 4 * n)) ||
      (rc = grow(p->idx_alt, 4 * n)) || (rc = grow(p->pts, 4 * w * n)) ||
      (rc = grow(p->far, 4 * w * n)) || (rc = grow(p->lcp, n)) || (rc = grow(p->leaf_level, n)) ||
      (rc = grow(p->leaf_of, 4 * n)) || (rc = grow(p->radix_hist, 4 * radix_hist_ints(n))) ||
      (rc = grow(p->scan_tmp, scan_tmp_bytes(std::max<int64_t>(n, 1 << 20)))) ||
      (rc = grow(p->root, sizeof(RootInfo))) || (rc = grow(p->ctrl, sizeof(Control))) ||
      (rc = grow(p->bbox_part, 6 * 8 * 1024)) || (rc = grow(p->lvl_blkcnt, 8 * tree_blkcnt_len(n))))
    return fail(rc);
  if ((int64_t)leaf_size < n) {
    if ((rc = grow(p->wlev, (size_t)(n + leaf_size))) || (rc = grow(p->wtmp, (size_t)(n + leaf_size))))
      return fail(rc);
  }
  if (hipHostMalloc((void**)&p->ctrl_host, sizeof(Control), hipHostMallocDefault) != hipSuccess)
    return fail(FMM_ERR_OOM);
  for (int i = 0; i < 2 * FMM_N_STAGES; i++)
    if (hipEventCreate(&p->ev[i]) != hipSuccess) return fail(FMM_ERR_HIP);
  for (int i = 0; i < 2 * FMM_N_KERNELS; i++)
    if (hipEventCreate(&p->kev[i]) != hipSuccess) return fail(FMM_ERR_HIP);
  // default priority, like every stream of the library
  if (hipStreamCreateWithFlags(&p->up_stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_tree, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_order, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_up, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_rec, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_done, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&p->ev_ctrl, hipEventDisableTiming) != hipSuccess)
    return fail(FMM_ERR_HIP);
  *out = p;
  return FMM_OK;
}

int fmm_destroy(fmm_plan_t p) {
  if (!p) return FMM_ERR_ARG;
  (void)hipDeviceSynchronize();
  DBuf* bufs[] = {&p->keys,       &p->keys_alt,    &p->idx,         &p->idx_alt,
                  &p->pts,        &p->far,         &p->perm_inv,    &p->lcp,
                  &p->wlev,       &p->wtmp,        &p->leaf_level,  &p->leaf_of,
                  &p->radix_hist, &p->scan_tmp,    &p->os_state,    &p->os_dword,
                  &p->root,       &p->ctrl,
                  &p->bbox_part,  &p->nlevel,      &p->nprefix,     &p->nbegin,
                  &p->ncount,     &p->nparent,     &p->nfirst,      &p->nnchild,
                  &p->ncentre,    &p->nq,          &p->ngeo,        &p->leaves,
                  &p->lvl_blkcnt, &p->mpole,       &p->mred,        &p->local,       &p->lfin,
                  &p->vrec,       &p->vfar,        &p->vmpole,      &p->vmred,
                  &p->vlocal,     &p->vlfin,
                  &p->lat_pos,    &p->lat_phi,     &p->lat_acc,     &p->lat_flag,
                  &p->pool[0],
                  &p->pool[1],    &p->pool[2],
                  &p->cu_off,     &p->cu_cnt,      &p->u_off,       &p->u_cnt,
                  &p->pu_off,     &p->pu_cnt,      &p->trm_cnt,     &p->trp_cnt,
                  &p->trm_base,   &p->trp_base,
                  &p->own_m2l,    &p->own_p2p,     &p->rootgen,     &p->tr_cnt_m2l,
                  &p->tr_start_m2l, &p->tr_keys,   &p->tr_keys_alt, &p->tr_vals,
                  &p->tr_vals_alt, &p->m2l_off,    &p->m2l_src,     &p->p2p_off,
                  &p->p2p_src,    &p->p2p_task,    &p->p2p_part,    &p->p2p_toff,
                  &p->split_leaves, &p->mut_flag,
                  &p->p2p_poff,   &p->tot_m2l,     &p->tot_p2p,     &p->parents,
                  &p->m2l_order,
                  &p->tail_toff,  &p->tail_task,   &p->tail_part};
  for (DBuf* b : bufs) release(*b);
  if (p->ctrl_host) (void)hipHostFree(p->ctrl_host);
  for (int i = 0; i < 2 * FMM_N_STAGES; i++)
    if (p->ev[i]) (void)hipEventDestroy(p->ev[i]);
  for (int i = 0; i < 2 * FMM_N_KERNELS; i++)
    if (p->kev[i]) (void)hipEventDestroy(p->kev[i]);
  if (p->ev_tree) (void)hipEventDestroy(p->ev_tree);
  if (p->ev_order) (void)hipEventDestroy(p->ev_order);
  if (p->ev_up) (void)hipEventDestroy(p->ev_up);
  if (p->ev_rec) (void)hipEventDestroy(p->ev_rec);
  if (p->ev_done) (void)hipEventDestroy(p->ev_done);
  if (p->ev_ctrl) (void)hipEventDestroy(p->ev_ctrl);
  if (p->up_stream) (void)hipStreamDestroy(p->up_stream);
  delete p;
  return FMM_OK;
}

int fmm_node_id_bits(int64_t n_nodes, int* bits) {
  if (!bits || n_nodes < 1 || n_nodes > FMM_MAX_NODES) return FMM_ERR_ARG;
  *bits = bits_for(n_nodes);
  return FMM_OK;
}

int fmm_set_mutual_near_field(fmm_plan_t p, int enable) {
  if (!p || (enable != 0 && enable != 1)) return FMM_ERR_ARG;
  p->mutual = enable == 1;
  return FMM_OK;
}

int fmm_set_walk_pool_hint(fmm_plan_t p, int64_t entries_per_node) {
  if (!p || entries_per_node < -1) return FMM_ERR_ARG;
  p->pool_hint = entries_per_node;
  return FMM_OK;
}

int fmm_set_timing(fmm_plan_t p, int enable) {
  if (!p || enable < 0 || enable > 3) return FMM_ERR_ARG;
  p->timing = enable != 0;
  p->timing_stages = enable == 1;
  p->timing_kernels = enable == 1 || enable == 2;
  if (p->timing) {
    TRY_HIP(hipSetDevice(p->device));
    TRY_HIP(hipDeviceSynchronize());
    p->pend_build = p->pend_eval = p->pend_vjp = false;
    for (double& x : p->stage_sum) x = 0.0;
    for (double& x : p->kernel_sum) x = 0.0;
    p->n_timed_builds = p->n_timed_evals = p->n_timed_vjps = 0;
  }
  return FMM_OK;
}

namespace {
int build_impl(fmm_plan_t p, const void* pos, const void* mass, hipStream_t st);
int eval_impl(fmm_plan_t p, void* phi, void* acc, hipStream_t st);
int vjp_impl(fmm_plan_t p, const void* phi_bar, const void* acc_bar, void* pos_bar,
             void* mass_bar, hipStream_t st);
}  // namespace

int fmm_build(fmm_plan_t p, const void* pos, const void* mass, void* stream) {
  if (!p || !pos || !mass) return FMM_ERR_ARG;
  hipStream_t st = (hipStream_t)stream;
  TRY_HIP(hipSetDevice(p->device));
  p->built = false;
  TRY(order_after_previous(p, st));
  const int rc = build_impl(p, pos, mass, st);
  const int rd = mark_done(p, st);
  return rc != FMM_OK ? rc : rd;
}

int fmm_eval(fmm_plan_t p, void* phi, void* acc, void* stream) {
  if (!p || !phi || !acc) return FMM_ERR_ARG;
  if (!p->built) return FMM_ERR_STATE;
  hipStream_t st = (hipStream_t)stream;
  TRY_HIP(hipSetDevice(p->device));
  TRY(order_after_previous(p, st));
  const int rc = eval_impl(p, phi, acc, st);
  const int rd = mark_done(p, st);
  return rc != FMM_OK ? rc : rd;
}

int fmm_vjp(fmm_plan_t p, const void* phi_bar, const void* acc_bar, void* pos_bar,
            void* mass_bar, void* stream) {
  if (!p || !phi_bar || !acc_bar || !pos_bar || !mass_bar) return FMM_ERR_ARG;
  if (!p->built) return FMM_ERR_STATE;
  hipStream_t st = (hipStream_t)stream;
  TRY_HIP(hipSetDevice(p->device));
  TRY(order_after_previous(p, st));
  const int rc = vjp_impl(p, phi_bar, acc_bar, pos_bar, mass_bar, st);
  const int rd = mark_done(p, st);
  return rc != FMM_OK ? rc : rd;
}

}  // extern "C"

namespace {

int build_impl(fmm_plan_t p, const void* pos, const void* mass, hipStream_t st) {
  p->evaluated = false;
  const int64_t n = p->n;
  Control* ctrl = P<Control>(p->ctrl);
  RootInfo* root = P<RootInfo>(p->root);
  // the previous build's second stream reads the sorted particles, the tree
  // and the walk's unions
  if (p->up_issued) TRY_HIP(hipStreamWaitEvent(st, p->ev_up, 0));

  rec(p, FMM_STAGE_KEYS, 0, st);
  TRY_HIP(launch_fill_zero(ctrl, sizeof(Control), st));
  if (n <= FRONT_MID_MAX) {
    // small sets: box, keys, sort and gather in one launch (timed as the keys stage)
    TRY_HIP(launch_front_small(pos, mass, n, p->dtype, P<uint64_t>(p->keys), P<int32_t>(p->idx),
                               p->pts.p, root, ctrl, st));
    rec(p, FMM_STAGE_KEYS, 1, st);
    rec(p, FMM_STAGE_SORT, 0, st);
    rec(p, FMM_STAGE_SORT, 1, st);
  } else {
    const int nbb = bbox_blocks(n);
    TRY_HIP(launch_bbox(pos, mass, n, p->dtype, P<double>(p->bbox_part), nbb, root, ctrl, st));
    TRY_HIP(launch_keys(pos, n, p->dtype, root, P<uint64_t>(p->keys), P<int32_t>(p->idx), st));
    rec(p, FMM_STAGE_KEYS, 1, st);

    rec(p, FMM_STAGE_SORT, 0, st);
    bool sorted_alt = false;
    OsBufs osb;
    const OsBufs* os = nullptr;
    TRY(os_bufs(p, n, st, &osb, &os));
    TRY_HIP(launch_radix_sort(P<uint64_t>(p->keys), P<int32_t>(p->idx),
                              P<uint64_t>(p->keys_alt), P<int32_t>(p->idx_alt), n,
                              P<int32_t>(p->radix_hist), P<int32_t>(p->scan_tmp), &sorted_alt,
                              st, os));
    if (sorted_alt) {  // the sorted keys and permutation are the plan's from here on
      std::swap(p->keys, p->keys_alt);
      std::swap(p->idx, p->idx_alt);
    }
    TRY_HIP(launch_gather(pos, mass, P<int32_t>(p->idx), n, p->dtype, p->pts.p, st));
    rec(p, FMM_STAGE_SORT, 1, st);
  }

  rec(p, FMM_STAGE_TREE, 0, st);
  TRY_HIP(launch_tree_phase1(P<uint64_t>(p->keys), n, p->leaf, P<int8_t>(p->lcp),
                             P<int8_t>(p->wlev), P<int8_t>(p->wtmp), P<int8_t>(p->leaf_level),
                             P<int64_t>(p->lvl_blkcnt), p->scan_tmp.p, ctrl, st));
  // The second phase needs no host value of the node count: with room from
  // the previous build it is queued before the count is read back and runs
  // while the host waits for the copy; the phase is repeated with room when
  // the tree has more nodes than that.
  const size_t w = wbytes(p->dtype);
  auto grow_nodes = [&](int64_t m) -> int {
    TRY(grow(p->nlevel, m));
    TRY(grow(p->nprefix, 8 * m));
    TRY(grow(p->nbegin, 4 * m));
    TRY(grow(p->ncount, 4 * m));
    TRY(grow(p->nparent, 4 * m));
    TRY(grow(p->nfirst, 4 * m));
    TRY(grow(p->nnchild, m));
    TRY(grow(p->ncentre, 24 * m));
    TRY(grow(p->nq, 8 * m));
    TRY(grow(p->ngeo, 16 * m));
    TRY(grow(p->leaves, 4 * (3 * m + 2)));
    TRY(grow(p->parents, 4 * m));
    TRY(grow(p->scan_tmp, scan_tmp_bytes(m + 1)));
    return FMM_OK;
  };
  auto phase2 = [&](int64_t cap) -> int {
    TreeArrays t{P<uint8_t>(p->nlevel),  P<uint64_t>(p->nprefix), P<int32_t>(p->nbegin),
                 P<int32_t>(p->ncount),  P<int32_t>(p->nparent),  P<int32_t>(p->nfirst),
                 P<uint8_t>(p->nnchild), P<double>(p->ncentre),   P<uint64_t>(p->nq),
                 P<int4>(p->ngeo)};
    int32_t* lv = P<int32_t>(p->leaves);
    TRY_HIP(launch_tree_phase2(P<uint64_t>(p->keys), n, p->leaf, P<int8_t>(p->lcp),
                               P<int8_t>(p->leaf_level), P<int64_t>(p->lvl_blkcnt), cap, root, t,
                               lv + cap, lv + 2 * cap + 1, lv, P<int32_t>(p->leaf_of),
                               P<int32_t>(p->parents), p->scan_tmp.p, ctrl, st));
    return FMM_OK;
  };
  const int64_t cap = p->cap_nodes;
  if (cap > 0) {
    TRY(grow_nodes(cap));
    TRY_HIP(hipMemcpyAsync(p->ctrl_host, p->ctrl.p, sizeof(Control), hipMemcpyDeviceToHost, st));
    TRY_HIP(hipEventRecord(p->ev_ctrl, st));
    TRY(phase2(cap));
    TRY_HIP(hipEventSynchronize(p->ev_ctrl));
  } else {
    TRY(sync_ctrl(p, st));
  }
  p->root_host = p->ctrl_host->root;
  if (p->ctrl_host->nonfinite) return FMM_ERR_NONFINITE;
  if (p->ctrl_host->sort_err) return FMM_ERR_HIP;  // a sort gave up a wait: its order is wrong
  const Control& c = *p->ctrl_host;
  const int64_t nn = c.level_off[MAX_LEVELS];
  // node ids are 32-bit, and the walk packs (kind, target, source) node ids
  // into 64-bit keys of 2 * fmm_node_id_bits(nn) + 1 bits
  if (nn > FMM_MAX_NODES) return FMM_ERR_OOM;
  p->n_nodes = nn;
  p->depth = 0;
  p->n_leaves = 0;
  for (int l = 0; l <= MAX_LEVELS; l++) p->level_off[l] = c.level_off[l];
  for (int l = 0; l < MAX_LEVELS; l++) {
    p->leaves_at_level[l] = c.leaves_at_level[l];
    p->n_leaves += c.leaves_at_level[l];
    if (c.level_off[l + 1] > c.level_off[l]) p->depth = l;
  }
  if (nn > cap) {  // no room queued (first build), or too little: the phase with room
    if (cap > 0) TRY_HIP(hipStreamSynchronize(st));  // the queued phase ends before any regrowth
    TRY(grow_nodes(nn));
    TRY(phase2(nn));
  }
  p->cap_nodes = nn + nn / 8 + 1024;  // the next build's room
  TRY(grow(p->mpole, w * p->K * nn));
  TRY(grow(p->mred, (size_t)mrec_bytes((p->order + 1) * (p->order + 1), (int)w) * nn));
  TRY(grow(p->local, w * p->K * nn));
  TRY(grow(p->lfin, w * p->K * nn));
  rec(p, FMM_STAGE_TREE, 1, st);
  // the previous step's events completed before the synchronization above;
  // they are read while the tree's second phase runs, before this build
  // records the walk's, the upward pass's and the kernels' events again
  collect_pending(p);
  for (int k = 0; k < FMM_N_KERNELS; k++) p->kran[k] = false;

  // the upward pass goes on the second stream after the tree; it is issued
  // by the walk once its level launches are queued (host launch time then
  // overlaps the walk's execution instead of delaying it)
  hipStream_t us = p->up_stream;
  TRY_HIP(hipEventRecord(p->ev_tree, st));
  TRY_HIP(hipStreamWaitEvent(us, p->ev_tree, 0));
  p->up_issued = true;  // ev_up is recorded by the walk, after the sibling M2L

  rec(p, FMM_STAGE_WALK, 0, st);
  const int wrc = run_walk(p, st);
  if (wrc != FMM_OK) {
    (void)hipEventRecord(p->ev_up, us);  // the next call still waits for this stream
    return wrc;
  }
  rec(p, FMM_STAGE_WALK, 1, st);
  // the leaves' complete locals (transposed-tail M2L, downward pass) need
  // nothing the eval brings: queued here, they run while the host returns
  // and issues the eval
  TRY(leaf_locals(p, st));
  rec(p, FMM_STAGE_DOWN, 1, st);
  collect_early_build(p);  // keys, sort and tree ended before the walk's last sync
  p->built = true;
  p->evaluated = true;  // the locals are complete
  return FMM_OK;
}

int eval_impl(fmm_plan_t p, void* phi, void* acc, hipStream_t st) {
  // the leaves' complete locals (lfin) come from the build
  if (p->timing_kernels) TRY_HIP(hipEventRecord(p->kev[2 * FMM_KERNEL_L2P], st));
  TRY_HIP(launch_l2p(p->dtype, p->order, p->n, p->pts.p, P<int32_t>(p->leaf_of),
                     P<double>(p->ncentre), p->lfin.p, p->far.p, st));
  if (p->timing_kernels) {
    TRY_HIP(hipEventRecord(p->kev[2 * FMM_KERNEL_L2P + 1], st));
    p->kran[FMM_KERNEL_L2P] = true;
  }

  rec(p, FMM_STAGE_P2P, 0, st);
  int32_t* leaves = P<int32_t>(p->leaves);
  const uint8_t* mut = nullptr;
  if (p->mut_built) {  // the sibling groups' pairs, both sides at once, into `far`
    TRY_HIP(launch_p2p_mutual(p->dtype, p->n_parents, P<int32_t>(p->parents),
                              P<int32_t>(p->nfirst), P<uint8_t>(p->nnchild),
                              P<int32_t>(p->nbegin), P<int32_t>(p->ncount), p->pts.p, p->far.p,
                              st));
    mut = P<uint8_t>(p->mut_flag);
  }
  TRY_HIP(launch_p2p(p->dtype, p->p2p_task.p, p->n_p2p_tasks, leaves, p->n_leaves,
                     P<int64_t>(p->p2p_toff), P<int64_t>(p->p2p_poff), P<int32_t>(p->nbegin),
                     P<int32_t>(p->ncount), mut, P<int32_t>(p->nparent),
                     P<int32_t>(p->p2p_src), p->pts.p, p->far.p,
                     P<int32_t>(p->idx), phi, acc, p->p2p_part.p,
                     P<int32_t>(p->split_leaves), p->n_split,
                     p->timing ? p->kev + 2 * FMM_KERNEL_P2P : nullptr,
                     p->kran + FMM_KERNEL_P2P, st));
  rec(p, FMM_STAGE_P2P, 1, st);
  p->pend_eval = p->timing;
  return FMM_OK;
}

int vjp_impl(fmm_plan_t p, const void* phi_bar, const void* acc_bar, void* pos_bar,
             void* mass_bar, hipStream_t st) {
  const int dt = p->dtype, ord = p->order;
  const int64_t n = p->n, nn = p->n_nodes;
  const size_t w = wbytes(dt);
  TRY(grow(p->vrec, 8 * w * n));
  TRY(grow(p->vfar, 4 * w * n));
  TRY(grow(p->vmpole, w * p->K * nn));
  TRY(grow(p->vmred, (size_t)mrec_bytes((ord + 1) * (ord + 1), (int)w) * nn));
  TRY(grow(p->vlocal, w * p->K * nn));
  TRY(grow(p->vlfin, w * p->K * nn));
  TRY_HIP(hipStreamWaitEvent(st, p->ev_up, 0));
  // the forward's leaf locals (lfin, from the build) give the Hessian term
  rec(p, FMM_STAGE_VJP, 0, st);
  const double* centre = P<double>(p->ncentre);
  int32_t* leaves = P<int32_t>(p->leaves);
  // sensitivity sources: monopoles pb and dipoles ab at the particles, on the
  // forward's tree and lists
  TRY_HIP(launch_vjp_gather(dt, n, p->pts.p, P<int32_t>(p->idx), phi_bar, acc_bar, p->vrec.p, st));
  TRY_HIP(launch_p2m_dip(dt, ord, p->vrec.p, leaves, p->n_leaves, P<int32_t>(p->nbegin),
                         P<int32_t>(p->ncount), centre, p->vmpole.p, st));
  TRY_HIP(launch_m2m_levels(dt, ord, p->level_off, p->depth, P<int32_t>(p->nfirst),
                            P<uint8_t>(p->nnchild), centre, p->vmpole.p, st));
  TRY_HIP(launch_m2l_records(dt, ord, nn, centre, p->vmpole.p, p->vmred.p, st));
  M2LArgs ma = m2l_args(p);
  ma.mrec = p->vmred.p;
  ma.local = p->vlocal.p;
  ma.ev = p->timing_kernels ? p->kev + 2 * FMM_KERNEL_VJP_M2L_SIB : nullptr;
  ma.ran = p->kran + FMM_KERNEL_VJP_M2L_SIB;
  TRY_HIP(launch_m2l_sib(dt, ord, ma, st));
  ma.ev = nullptr;
  ma.ran = nullptr;
  const bool pull = ord <= 6;
  if (!pull) {
    TRY_HIP(hipMemcpyAsync(p->vlfin.p, p->vlocal.p, (size_t)nn * p->K * w,
                           hipMemcpyDeviceToDevice, st));
    ma.local = p->vlfin.p;
  }
  TRY_HIP(launch_m2l_tails(dt, ord, ma, !pull, st));
  if (pull) {
    if (!launch_l2l_pull(dt, ord, leaves, p->n_leaves, P<int32_t>(p->nparent), centre,
                         p->vlocal.p, p->n_tail_tasks > 0 ? P<int64_t>(p->tail_toff) : nullptr,
                         p->tail_part.p, p->vlfin.p, st))
      return FMM_ERR_HIP;
    TRY_HIP(hipGetLastError());
  } else {
    for (int l = 1; l <= p->depth; l++)
      TRY_HIP(launch_l2l(dt, ord, p->level_off[l], p->level_off[l + 1] - p->level_off[l],
                         P<int32_t>(p->nparent), centre, p->vlfin.p, nullptr, st));
  }
  TRY_HIP(launch_l2p_vjp(dt, ord, n, p->vrec.p, P<int32_t>(p->leaf_of), centre, p->lfin.p,
                         p->vlfin.p, p->vfar.p, st));
  TRY_HIP(launch_p2p_vjp(dt, p->p2p_task.p, p->n_p2p_tasks, leaves, p->n_leaves,
                         P<int64_t>(p->p2p_toff), P<int64_t>(p->p2p_poff), P<int32_t>(p->nbegin),
                         P<int32_t>(p->ncount), P<int32_t>(p->p2p_src), p->vrec.p, p->vfar.p,
                         P<int32_t>(p->idx), mass_bar, pos_bar, p->p2p_part.p,
                         P<int32_t>(p->split_leaves), p->n_split,
                         p->timing ? p->kev + 2 * FMM_KERNEL_VJP_P2P : nullptr,
                         p->kran + FMM_KERNEL_VJP_P2P, st));
  rec(p, FMM_STAGE_VJP, 1, st);
  p->pend_vjp = p->timing;
  return FMM_OK;
}

}  // namespace

extern "C" {

int fmm_lattice_steps(fmm_plan_t p, int64_t* q, int64_t* u, const void* mass, double dx,
                      double dv, double dt, int n_steps, int direction, void* stream) {
  if (!p || !q || !u || !mass || n_steps < 0 || (direction != 1 && direction != -1) ||
      !(dx > 0.0) || !(dv > 0.0) || !std::isfinite(dx) || !std::isfinite(dv) ||
      !std::isfinite(dt))
    return FMM_ERR_ARG;
  if (n_steps == 0) return FMM_OK;
  hipStream_t st = (hipStream_t)stream;
  TRY_HIP(hipSetDevice(p->device));
  TRY(order_after_previous(p, st));  // the lattice buffers feed the builds below
  const int dt_ = p->dtype;
  const int64_t n = p->n;
  const size_t w = wbytes(dt_);
  TRY(grow(p->lat_pos, 3 * w * n));
  TRY(grow(p->lat_phi, w * n));
  TRY(grow(p->lat_acc, 3 * w * n));
  TRY(grow(p->lat_flag, sizeof(int)));
  int* flag = P<int>(p->lat_flag);
  TRY_HIP(launch_fill_zero(flag, sizeof(int), st));
  const double ck = 0.5 * dt / dv, cd = dt * dv / dx;
  auto force = [&]() -> int {  // acceleration of the current lattice positions
    TRY_HIP(launch_lat_pos(dt_, n, q, dx, p->lat_pos.p, st));
    TRY(fmm_build(p, p->lat_pos.p, mass, stream));
    return fmm_eval(p, p->lat_phi.p, p->lat_acc.p, stream);
  };
  TRY(force());
  for (int s = 0; s < n_steps; s++) {
    TRY_HIP(launch_lat_kick(dt_, n, u, p->lat_acc.p, ck, direction, flag, st));
    TRY_HIP(launch_lat_drift(n, q, u, cd, direction, flag, st));
    TRY(force());
    TRY_HIP(launch_lat_kick(dt_, n, u, p->lat_acc.p, ck, direction, flag, st));
  }
  int h = 0;
  TRY_HIP(hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, st));
  TRY_HIP(hipStreamSynchronize(st));
  return h ? FMM_ERR_NONFINITE : FMM_OK;
}

int fmm_stats(fmm_plan_t p, fmm_stats_t* out) {
  if (!p || !out) return FMM_ERR_ARG;
  std::memset(out, 0, sizeof(*out));
  out->n = p->n;
  out->order = p->order;
  out->leaf_size = p->leaf;
  out->dtype = p->dtype;
  out->theta = p->theta;
  out->walk_retries = p->walk_retries;
  out->walk_one_block = p->walk_one_block ? 1 : 0;
  if (p->built) {
    out->n_nodes = p->n_nodes;
    out->n_leaves = p->n_leaves;
    out->n_m2l = p->n_m2l;
    out->n_p2p = p->n_p2p;
    out->depth = p->depth;
    for (int a = 0; a < 3; a++) out->lo[a] = p->root_host.lo[a];
    out->side = p->root_host.side;
  }
  if (p->timing) {
    TRY_HIP(hipSetDevice(p->device));
    TRY_HIP(hipDeviceSynchronize());
    collect_pending(p);
    const double nb = std::max(1, p->n_timed_builds), ne = std::max(1, p->n_timed_evals),
                 nv = std::max(1, p->n_timed_vjps);
    for (int s = 0; s < FMM_N_STAGES; s++)
      out->stage_ms[s] = (float)(p->stage_sum[s] / (s == FMM_STAGE_P2P   ? ne
                                                     : s == FMM_STAGE_VJP ? nv
                                                                          : nb));
    for (int k = 0; k < FMM_N_KERNELS; k++)
      out->kernel_ms[k] =
          (float)(p->kernel_sum[k] / (k == FMM_KERNEL_M2L_SIB || k == FMM_KERNEL_P2M ||
                                              k == FMM_KERNEL_M2L_TAIL
                                          ? nb
                                      : k == FMM_KERNEL_VJP_M2L_SIB || k == FMM_KERNEL_VJP_P2P
                                          ? nv
                                          : ne));
    out->timed_builds = p->n_timed_builds;
    out->timed_evals = p->n_timed_evals;
    out->timed_vjps = p->n_timed_vjps;
  }
  return FMM_OK;
}

int fmm_copy_keys(fmm_plan_t p, uint64_t* keys, int32_t* perm) {
  if (!p) return FMM_ERR_ARG;
  if (!p->built) return FMM_ERR_STATE;
  TRY_HIP(hipDeviceSynchronize());
  if (keys) TRY_HIP(hipMemcpy(keys, p->keys.p, 8 * p->n, hipMemcpyDeviceToHost));
  if (perm) TRY_HIP(hipMemcpy(perm, p->idx.p, 4 * p->n, hipMemcpyDeviceToHost));
  return FMM_OK;
}

int fmm_copy_tree(fmm_plan_t p, uint8_t* level, uint64_t* prefix, int32_t* begin, int32_t* count,
                  int32_t* parent, int32_t* first_child, uint8_t* n_child) {
  if (!p) return FMM_ERR_ARG;
  if (!p->built) return FMM_ERR_STATE;
  TRY_HIP(hipDeviceSynchronize());
  const size_t m = (size_t)p->n_nodes;
  if (level) TRY_HIP(hipMemcpy(level, p->nlevel.p, m, hipMemcpyDeviceToHost));
  if (prefix) TRY_HIP(hipMemcpy(prefix, p->nprefix.p, 8 * m, hipMemcpyDeviceToHost));
  if (begin) TRY_HIP(hipMemcpy(begin, p->nbegin.p, 4 * m, hipMemcpyDeviceToHost));
  if (count) TRY_HIP(hipMemcpy(count, p->ncount.p, 4 * m, hipMemcpyDeviceToHost));
  if (parent) TRY_HIP(hipMemcpy(parent, p->nparent.p, 4 * m, hipMemcpyDeviceToHost));
  if (first_child) TRY_HIP(hipMemcpy(first_child, p->nfirst.p, 4 * m, hipMemcpyDeviceToHost));
  if (n_child) TRY_HIP(hipMemcpy(n_child, p->nnchild.p, m, hipMemcpyDeviceToHost));
  return FMM_OK;
}

int fmm_copy_lists(fmm_plan_t p, int64_t* m2l_off, int32_t* m2l_src, int64_t* p2p_off,
                   int32_t* p2p_src) {
  if (!p) return FMM_ERR_ARG;
  if (!p->built) return FMM_ERR_STATE;
  TRY_HIP(hipSetDevice(p->device));
  TRY_HIP(hipDeviceSynchronize());
  if (m2l_off || m2l_src) TRY(materialize_m2l_lists(p, nullptr));
  const size_t m = (size_t)p->n_nodes + 1;
  if (m2l_off) TRY_HIP(hipMemcpy(m2l_off, p->m2l_off.p, 8 * m, hipMemcpyDeviceToHost));
  if (p2p_off) TRY_HIP(hipMemcpy(p2p_off, p->p2p_off.p, 8 * m, hipMemcpyDeviceToHost));
  if (m2l_src && p->n_m2l)
    TRY_HIP(hipMemcpy(m2l_src, p->m2l_src.p, 4 * (size_t)p->n_m2l, hipMemcpyDeviceToHost));
  if (p2p_src && p->n_p2p)
    TRY_HIP(hipMemcpy(p2p_src, p->p2p_src.p, 4 * (size_t)p->n_p2p, hipMemcpyDeviceToHost));
  return FMM_OK;
}

int fmm_copy_expansions(fmm_plan_t p, double* mpole, double* local) {
  if (!p) return FMM_ERR_ARG;
  if (!p->evaluated) return FMM_ERR_STATE;
  TRY_HIP(hipDeviceSynchronize());
  const size_t m = (size_t)p->n_nodes * p->K;
  double *dm = nullptr, *dl = nullptr;
  if (hipMalloc(&dm, 8 * m) != hipSuccess) return FMM_ERR_OOM;
  if (hipMalloc(&dl, 8 * m) != hipSuccess) {
    (void)hipFree(dm);
    return FMM_ERR_OOM;
  }
  // The eval's complete locals are in lfin: every node's with the
  // level-by-level pass, the leaves' only with the one-launch pass.  There
  // the internal nodes' full locals (own M2L part in `local`, parent's shifted
  // in, level by level) are rebuilt on a copy, and the leaves' rows taken from
  // lfin.
  void* lsrc = p->lfin.p;
  void* tmp = nullptr;
  const size_t lbytes = m * wbytes(p->dtype);
  int rc = FMM_OK;
  if (p->l2l_pulled) {
    if (hipMalloc(&tmp, lbytes) != hipSuccess) rc = FMM_ERR_OOM;
    if (rc == FMM_OK)
      rc = status_of(hipMemcpy(tmp, p->local.p, lbytes, hipMemcpyDeviceToDevice));
    for (int l = 1; rc == FMM_OK && l <= p->depth; l++)
      rc = status_of(launch_l2l(p->dtype, p->order, p->level_off[l],
                                p->level_off[l + 1] - p->level_off[l], P<int32_t>(p->nparent),
                                P<double>(p->ncentre), tmp, P<uint8_t>(p->nnchild), nullptr));
    if (rc == FMM_OK)
      rc = status_of(launch_copy_rows(P<int32_t>(p->leaves), p->n_leaves,
                                      (int64_t)p->K * (int64_t)wbytes(p->dtype), p->lfin.p, tmp,
                                      nullptr));
    lsrc = tmp;
  }
  if (rc == FMM_OK)
    rc = status_of(launch_export_expansions(p->dtype, p->order, p->n_nodes, p->mpole.p, lsrc, dm,
                                            dl, nullptr));
  if (rc == FMM_OK) rc = status_of(hipDeviceSynchronize());
  if (rc == FMM_OK && mpole) rc = status_of(hipMemcpy(mpole, dm, 8 * m, hipMemcpyDeviceToHost));
  if (rc == FMM_OK && local) rc = status_of(hipMemcpy(local, dl, 8 * m, hipMemcpyDeviceToHost));
  (void)hipFree(dm);
  (void)hipFree(dl);
  if (tmp) (void)hipFree(tmp);
  return rc;
}

}  // extern "C"
