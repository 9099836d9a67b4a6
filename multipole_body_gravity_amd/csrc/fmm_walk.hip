// fmm_walk.hip -- the dual-tree walk that emits the M2L and P2P lists.
//
// jz-fmm project page, "Calculating a node-node interaction" (opening criterion)
// and "Combining near and far interactions" (accept well-separated pairs for
// multipole-to-local translations, refine the rest, sum the remaining nearby
// pairs directly).  The pair walk from (root, root) -- accept -> M2L, two
// leaves -> P2P, otherwise split the coarser non-leaf (both when the levels are
// equal) -- is evaluated here target by target, one tree level per step:
//
//   * at step s every node t of level s receives as candidates the "carry" of
//     its parent (the parent's rejected partners), each carried leaf kept as
//     it is and each carried non-leaf replaced by its children;
//   * a leaf t additionally keeps receiving, at steps s+1, s+2, ..., the
//     children of the non-leaf partners it rejected at the previous step
//     (the pair walk splits only the non-leaf side there);
//   * each candidate c is accepted (M2L t<-c) or rejected; a rejected c goes
//     to t's carry if t is a non-leaf, to t's P2P list if both are leaves,
//     and to t's pending carry otherwise.
//
// Candidates are enumerated in ascending node order, so each step appends a
// sorted run of sources, and runs of later steps hold deeper (larger) ids:
// every target's lists come out sorted by source without a sort.  Pass 1
// counts list lengths and materializes the carries; after a scan of the
// per-target totals, pass 2 re-classifies and writes the lists in place.
// Carry slices are allocated with an integer atomic counter: their placement
// varies between runs, their contents and the final lists do not.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int WK_THREADS = 256;
constexpr int WK_WAVES = WK_THREADS / WAVE;
constexpr uint32_t QMASK = 0x1fffffu;

// Opening criterion in units of half the finer cell's side: centres and
// half-widths become integers, |c_A - c_B|^2 and 3 (h_A + h_B)^2 are exact in
// fp64 (< 2^46), and the only rounding is the product with fl(theta^2).
__device__ __forceinline__ bool accept_pair(int la, uint64_t qa, int lb, uint64_t qb, double t2) {
  const int lm = max(la, lb);
  const int ha = 1 << (lm - la), hb = 1 << (lm - lb);
  const int ax = ha * (2 * (int)((qa >> 42) & QMASK) + 1), bx = hb * (2 * (int)((qb >> 42) & QMASK) + 1);
  const int ay = ha * (2 * (int)((qa >> 21) & QMASK) + 1), by = hb * (2 * (int)((qb >> 21) & QMASK) + 1);
  const int az = ha * (2 * (int)(qa & QMASK) + 1), bz = hb * (2 * (int)(qb & QMASK) + 1);
  const double dx = (double)(ax - bx), dy = (double)(ay - by), dz = (double)(az - bz);
  const double r2 = dx * dx + dy * dy + dz * dz;  // exact
  const double s = (double)(ha + hb);
  const double lhs = 3.0 * (s * s);  // exact
  return lhs < t2 * r2;
}

enum { CAND_NONE = 0, CAND_M2L = 1, CAND_P2P = 2, CAND_CARRY = 3 };

struct Target {
  int32_t t;
  int lt;
  uint64_t qt;
  bool leaf;
};

__device__ __forceinline__ int classify(const WalkArgs& a, const Target& T, int32_t c) {
  const int lc = a.level[c];
  const uint64_t qc = a.q[c];
  if (accept_pair(T.lt, T.qt, lc, qc, a.t2)) return CAND_M2L;
  if (!T.leaf) return CAND_CARRY;
  return (a.n_child[c] == 0) ? CAND_P2P : CAND_CARRY;
}

// Visit the candidates of a generator slice in ascending node order, 64 at a
// time: first the carried leaves (levels < s, kept as they are), then the
// children of the carried non-leaves (level s).  Each phase follows the sorted
// generator order, and every id of the first phase is smaller than every id
// of the second.  f(active, cand) is called by the whole wave (it may use
// ballots).
template <typename F>
__device__ __forceinline__ void for_each_candidate(const WalkArgs& a, int64_t g0, int gc, F&& f) {
  const int lane = __lane_id();
  for (int phase = 0; phase < 2; phase++) {
    for (int c0 = 0; c0 < gc; c0 += WAVE) {
      const int j = c0 + lane;
      int nc = 0, fc = 0;
      if (j < gc) {
        const int32_t g = a.carry[g0 + j];
        const int k = a.n_child[g];
        if (phase == 0 && k == 0) {
          nc = 1;
          fc = g;
        } else if (phase == 1 && k != 0) {
          nc = k;
          fc = a.first_child[g];
        }
      }
      const int incl = wave_incl_scan(nc);
      const int excl = incl - nc;
      const int tot = __shfl(incl, WAVE - 1, WAVE);
      for (int b = 0; b < tot; b += WAVE) {
        const int qi = b + lane;
        const bool active = qi < tot;
        // smallest lane h with incl[h] > qi
        int h = 0;
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1) {
          const int probe = h + step - 1;
          const int v = __shfl(incl, probe, WAVE);
          if (v <= qi) h += step;
        }
        h = min(h, WAVE - 1);
        const int fch = __shfl(fc, h, WAVE);
        const int exh = __shfl(excl, h, WAVE);
        f(active, (int32_t)(fch + (qi - exh)));
      }
    }
  }
}

// Item record of step s, index i in [0, amax) (type A) or [amax, amax+lvl_count)
// (type B: the level-s node lvl_begin + i - amax).
__device__ __forceinline__ void item_source(const WalkArgs& a, int64_t i, int32_t& t, int64_t& g0,
                                            int& gc, bool pass1) {
  const int64_t gi = a.base + i;
  if (i < a.amax) {
    t = a.it.tgt[gi];
    g0 = a.it.gen_off[gi];
    gc = a.it.gen_cnt[gi];
    return;
  }
  t = (int32_t)(a.lvl_begin + (i - a.amax));
  if (pass1) {
    const int64_t pitem = a.prev_base + a.prev_amax + (a.parent[t] - a.prev_lvl_begin);
    g0 = a.it.carry_off[pitem];
    gc = a.it.carry_cnt[pitem];
    a.it.tgt[gi] = t;
    a.it.gen_off[gi] = g0;
    a.it.gen_cnt[gi] = gc;
  } else {
    g0 = a.it.gen_off[gi];
    gc = a.it.gen_cnt[gi];
  }
}

__global__ void __launch_bounds__(WK_THREADS) k_walk_pass1(WalkArgs a) {
  if (a.ctrl->carry_overflow) return;
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  const int64_t nA = a.ctrl->nA[a.step];
  const int64_t n_items = nA + a.lvl_count;
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < n_items;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int64_t i = (j < nA) ? j : a.amax + (j - nA);
    int32_t t;
    int64_t g0;
    int gc;
    item_source(a, i, t, g0, gc, true);
    Target T{t, a.level[t], a.q[t], a.n_child[t] == 0};
    int n_m2l = 0, n_p2p = 0, n_carry = 0;
    for_each_candidate(a, g0, gc, [&](bool act, int32_t c) {
      const int ty = act ? classify(a, T, c) : CAND_NONE;
      n_m2l += __popcll(__ballot(ty == CAND_M2L));
      n_p2p += __popcll(__ballot(ty == CAND_P2P));
      n_carry += __popcll(__ballot(ty == CAND_CARRY));
    });
    int64_t off = 0;
    if (n_carry > 0) {
      if (lane == 0) off = (int64_t)atomicAdd((unsigned long long*)&a.ctrl->carry_used,
                                              (unsigned long long)n_carry);
      off = __shfl(off, 0, WAVE);
      if (off + n_carry > a.carry_cap) {
        if (lane == 0) atomicOr(&a.ctrl->carry_overflow, 1);
        return;  // results are discarded; the host regrows the pool and retries
      }
      int64_t cur = off;
      for_each_candidate(a, g0, gc, [&](bool act, int32_t c) {
        const int ty = act ? classify(a, T, c) : CAND_NONE;
        const uint64_t m = __ballot(ty == CAND_CARRY);
        if (ty == CAND_CARRY) a.carry[cur + __popcll(m & lt)] = c;
        cur += __popcll(m);
      });
    }
    if (lane == 0) {
      const int64_t gi = a.base + i;
      a.it.carry_off[gi] = off;
      a.it.carry_cnt[gi] = n_carry;
      a.tot_m2l[t] += n_m2l;
      a.tot_p2p[t] += n_p2p;
      if (T.leaf && n_carry > 0) {  // the leaf keeps refining its partners next step
        const int slot = atomicAdd(&a.ctrl->nA[a.step + 1], 1);
        const int64_t ni = a.next_base + slot;
        a.it.tgt[ni] = t;
        a.it.gen_off[ni] = off;
        a.it.gen_cnt[ni] = n_carry;
      }
    }
  }
}

__global__ void __launch_bounds__(WK_THREADS) k_walk_pass2(WalkArgs a) {
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  const int64_t nA = a.ctrl->nA[a.step];
  const int64_t n_items = nA + a.lvl_count;
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < n_items;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int64_t i = (j < nA) ? j : a.amax + (j - nA);
    int32_t t;
    int64_t g0;
    int gc;
    item_source(a, i, t, g0, gc, false);
    Target T{t, a.level[t], a.q[t], a.n_child[t] == 0};
    const int64_t m0 = a.m2l_off[t] + a.cur_m2l[t];
    const int64_t p0 = a.p2p_off[t] + a.cur_p2p[t];
    int64_t cm = 0, cp = 0;
    for_each_candidate(a, g0, gc, [&](bool act, int32_t c) {
      const int ty = act ? classify(a, T, c) : CAND_NONE;
      const uint64_t mm = __ballot(ty == CAND_M2L);
      const uint64_t mp = __ballot(ty == CAND_P2P);
      if (ty == CAND_M2L) a.m2l_src[m0 + cm + __popcll(mm & lt)] = c;
      if (ty == CAND_P2P) a.p2p_src[p0 + cp + __popcll(mp & lt)] = c;
      cm += __popcll(mm);
      cp += __popcll(mp);
    });
    if (lane == 0) {
      a.cur_m2l[t] += cm;
      a.cur_p2p[t] += cp;
    }
  }
}

// Step 0: the root paired with itself.  A leaf root gives the single list entry
// P2P(root <- root); otherwise the root's carry is {root} for its children.
__global__ void k_walk_root(int pass, int root_leaf, WalkArgs a) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (pass == 1) {
    if (root_leaf) {
      a.tot_p2p[0] = 1;
    } else {
      a.carry[0] = 0;
      a.ctrl->carry_used = 1;
      const int64_t gi = a.base;
      a.it.tgt[gi] = 0;
      a.it.gen_off[gi] = 0;
      a.it.gen_cnt[gi] = 0;
      a.it.carry_off[gi] = 0;
      a.it.carry_cnt[gi] = 1;
    }
  } else if (root_leaf) {
    a.p2p_src[a.p2p_off[0]] = 0;
  }
}

__global__ void k_walk_reset(Control* c) {
  const int i = threadIdx.x;
  if (i <= MAX_LEVELS) c->nA[i] = 0;
  if (i == 0) {
    c->carry_overflow = 0;
    c->carry_used = 0;
  }
}

__global__ void k_walk_totals(const int64_t* m2l_total, const int64_t* p2p_total, Control* c) {
  if (threadIdx.x == 0) {
    c->n_m2l = *m2l_total;
    c->n_p2p = *p2p_total;
  }
}

hipError_t launch_walk_root(int pass, int root_leaf, const WalkArgs& a, hipStream_t st) {
  k_walk_root<<<1, 64, 0, st>>>(pass, root_leaf, a);
  return hipGetLastError();
}
hipError_t launch_walk_reset(Control* ctrl, hipStream_t st) {
  k_walk_reset<<<1, 64, 0, st>>>(ctrl);
  return hipGetLastError();
}
hipError_t launch_walk_totals(const int64_t* m2l_total, const int64_t* p2p_total, Control* ctrl,
                              hipStream_t st) {
  k_walk_totals<<<1, 64, 0, st>>>(m2l_total, p2p_total, ctrl);
  return hipGetLastError();
}

static unsigned walk_grid(const WalkArgs& a) {
  int64_t ub = a.amax + a.lvl_count;
  int64_t blocks = (ub + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

hipError_t launch_walk_pass1(const WalkArgs& a, hipStream_t st) {
  k_walk_pass1<<<walk_grid(a), WK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}
hipError_t launch_walk_pass2(const WalkArgs& a, hipStream_t st) {
  k_walk_pass2<<<walk_grid(a), WK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mbg
