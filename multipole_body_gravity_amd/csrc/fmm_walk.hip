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
//     its parent (the parent's rejected partners): each carried leaf is kept
//     as it is, each carried non-leaf is replaced by its children;
//   * each candidate c is accepted (M2L t <- c) or rejected; a rejected c goes
//     to t's carry if t is a non-leaf, and to t's P2P list if t and c are both
//     leaves.
//
// The pair walk also refines the partners of a leaf t past t's own level
// (only the non-leaf side can split).  Those pairs are exactly the pairs in
// which a deeper target sees t as a carried leaf, and the acceptance test is
// symmetric, so they are emitted from that side: when a target of level s
// accepts a carried leaf c of a coarser level, the entry (c <- target) is
// added to c's list as well, and likewise for leaf-leaf rejections.  Such
// transposed entries are appended in any order and put in place by a radix
// sort of (target, source) keys; a target's own entries (sources at its level
// or coarser) come first, its transposed ones (deeper sources) after, so every
// list ends sorted by source, as the pair walk's canonical order requires.
//
// Pass 1 counts each target's own entries and writes its carry and its
// transposed entries; the transposed entries are then sorted, counted per
// target, and after a scan of the per-target totals pass 2 re-classifies and
// writes the own entries in place.  Carry slices and transposed entries are
// placed by sharded bump allocators (integer atomics spread over 512 counters
// by target): their placement varies between runs, the final lists do not.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int WK_THREADS = 256;
constexpr int WK_WAVES = WK_THREADS / WAVE;
constexpr uint32_t QMASK = 0x1fffffu;

// Opening criterion, theta = |l_A + l_B| / |c_A - c_B| with l = (h, h, h):
// accept iff 3 (h_A + h_B)^2 < fl(theta^2) |c_A - c_B|^2.  Centres and
// half-widths are integers in units of 1/2^22 of the root side, so both squares
// are exact in fp64 (< 2^47) and the only rounding is the product with
// fl(theta^2); a change of unit by a power of two scales both sides exactly,
// so the decision equals the one taken in units of the finer cell.
constexpr int GEO_LEAF = 1 << 30;
__device__ __forceinline__ bool accept_pair(const int4& A, const int4& B, double t2) {
  const double dx = (double)(A.x - B.x), dy = (double)(A.y - B.y), dz = (double)(A.z - B.z);
  const double r2 = dx * dx + dy * dy + dz * dz;  // exact
  const double s = (double)((A.w & (GEO_LEAF - 1)) + (B.w & (GEO_LEAF - 1)));
  const double lhs = 3.0 * (s * s);  // exact
  return lhs < t2 * r2;
}

enum { CAND_NONE = 0, CAND_M2L = 1, CAND_P2P = 2, CAND_CARRY = 3 };

struct Target {
  int32_t t;
  int4 g;
  bool leaf;
};

__device__ __forceinline__ int classify(const WalkArgs& a, const Target& T, int32_t c) {
  const int4 g = a.geo[c];
  if (accept_pair(T.g, g, a.t2)) return CAND_M2L;
  if (!T.leaf) return CAND_CARRY;
  return (g.w & GEO_LEAF) ? CAND_P2P : CAND_CARRY;
}

// Visit the candidates of a generator slice in ascending node order, 64 at a
// time: first the carried leaves (levels < s, kept as they are: phase 0), then
// the children of the carried non-leaves (level s: phase 1).  Each phase
// follows the sorted generator order, and every id of phase 0 is smaller than
// every id of phase 1.  f(active, cand, phase) is called by the whole wave.
template <typename F>
__device__ __forceinline__ void for_each_candidate(const WalkArgs& a, int64_t g0, int gc, F&& f) {
  const int lane = __lane_id();
  for (int phase = 0; phase < 2; phase++) {
    for (int c0 = 0; c0 < gc; c0 += WAVE) {
      const int j = c0 + lane;
      int nc = 0, fc = 0;
      if (j < gc) {
        const int32_t g = a.carry.data[g0 + j];
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
        f(active, (int32_t)(fch + (qi - exh)), phase);
      }
    }
  }
}

__device__ __forceinline__ int shard_of(int32_t t) {
  return (int)(((uint32_t)t * 2654435761u) >> 23) & (POOL_SHARDS - 1);
}

// Wave-wide allocation of n entries from shard sh (lane 0 bumps the counter).
// Returns the global offset, or -1 when the shard is full (overflow flagged).
template <typename T>
__device__ __forceinline__ int64_t pool_alloc(const Pool<T>& p, int sh, int n, Control* ctrl) {
  int64_t off = 0;
  if (__lane_id() == 0)
    off = (int64_t)atomicAdd((unsigned long long*)&p.used[sh], (unsigned long long)n);
  off = __shfl(off, 0, WAVE);
  if (off + n > p.shard_cap) {
    if (__lane_id() == 0) atomicOr(&ctrl->pool_overflow, 1);
    return -1;
  }
  return (int64_t)sh * p.shard_cap + off;
}

__global__ void __launch_bounds__(WK_THREADS) k_walk_pass1(WalkArgs a) {
  // after an overflow the parents' carries may be missing: do nothing, the
  // host regrows the pools and repeats pass 1
  if (a.ctrl->pool_overflow) return;
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < a.lvl_count;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int32_t t = (int32_t)(a.lvl_begin + j);
    const int32_t par = a.parent[t];
    const int64_t g0 = a.carry_off[par];
    const int gc = a.carry_cnt[par];
    Target T{t, a.geo[t], (a.geo[t].w & GEO_LEAF) != 0};
    int n_m2l = 0, n_p2p = 0, n_carry = 0, n_trm = 0, n_trp = 0;
    for_each_candidate(a, g0, gc, [&](bool act, int32_t c, int phase) {
      const int ty = act ? classify(a, T, c) : CAND_NONE;
      const bool m = ty == CAND_M2L, p = ty == CAND_P2P, k = ty == CAND_CARRY && !T.leaf;
      const int cm = __popcll(__ballot(m)), cp = __popcll(__ballot(p));
      n_m2l += cm;
      n_p2p += cp;
      n_carry += __popcll(__ballot(k));
      if (phase == 0) {  // carried leaves of coarser levels: transposed entries
        n_trm += cm;
        n_trp += cp;
      }
    });
    const int sh = shard_of(t);
    int64_t off = 0;
    bool ok = true;
    if (n_carry > 0) {
      off = pool_alloc(a.carry, sh, n_carry, a.ctrl);
      ok = off >= 0;
    }
    int64_t om = 0, op = 0;
    if (ok && n_trm > 0) {
      om = pool_alloc(a.trm, sh, n_trm, a.ctrl);
      ok = om >= 0;
    }
    if (ok && n_trp > 0) {
      op = pool_alloc(a.trp, sh, n_trp, a.ctrl);
      ok = op >= 0;
    }
    if (!ok) continue;  // results are discarded; the host regrows the pools and retries
    if (n_carry + n_trm + n_trp > 0) {
      int64_t ck = off, cm = om, cp = op;
      for_each_candidate(a, g0, gc, [&](bool act, int32_t c, int phase) {
        const int ty = act ? classify(a, T, c) : CAND_NONE;
        const uint64_t bk = __ballot(ty == CAND_CARRY && !T.leaf);
        if (ty == CAND_CARRY && !T.leaf) a.carry.data[ck + __popcll(bk & lt)] = c;
        ck += __popcll(bk);
        if (phase == 0) {
          const uint64_t key = ((uint64_t)(uint32_t)c << a.key_shift) | (uint32_t)t;
          const uint64_t bm = __ballot(ty == CAND_M2L), bp = __ballot(ty == CAND_P2P);
          if (ty == CAND_M2L) a.trm.data[cm + __popcll(bm & lt)] = key;
          if (ty == CAND_P2P) a.trp.data[cp + __popcll(bp & lt)] = key;
          cm += __popcll(bm);
          cp += __popcll(bp);
        }
      });
    }
    if (lane == 0) {
      a.carry_off[t] = off;
      a.carry_cnt[t] = n_carry;
      a.own_m2l[t] = n_m2l;
      a.own_p2p[t] = n_p2p;
    }
  }
}

__global__ void __launch_bounds__(WK_THREADS) k_walk_pass2(WalkArgs a) {
  const uint64_t lt = lanemask_lt();
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < a.lvl_count;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int32_t t = (int32_t)(a.lvl_begin + j);
    const int32_t par = a.parent[t];
    const int64_t g0 = a.carry_off[par];
    const int gc = a.carry_cnt[par];
    Target T{t, a.geo[t], (a.geo[t].w & GEO_LEAF) != 0};
    const int64_t m0 = a.m2l_off[t], p0 = a.p2p_off[t];
    int64_t cm = 0, cp = 0;
    for_each_candidate(a, g0, gc, [&](bool act, int32_t c, int) {
      const int ty = act ? classify(a, T, c) : CAND_NONE;
      const uint64_t mm = __ballot(ty == CAND_M2L);
      const uint64_t mp = __ballot(ty == CAND_P2P);
      if (ty == CAND_M2L) a.m2l_src[m0 + cm + __popcll(mm & lt)] = c;
      if (ty == CAND_P2P) a.p2p_src[p0 + cp + __popcll(mp & lt)] = c;
      cm += __popcll(mm);
      cp += __popcll(mp);
    });
  }
}

// Step 0: the root paired with itself.  A leaf root gives the single list entry
// P2P(root <- root); otherwise the root's carry is {root} for its children.
__global__ void k_walk_root(int pass, int root_leaf, WalkArgs a) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (pass == 1) {
    a.own_m2l[0] = 0;
    a.carry_off[0] = 0;
    if (root_leaf) {
      a.own_p2p[0] = 1;
      a.carry_cnt[0] = 0;
    } else {
      a.own_p2p[0] = 0;
      const int sh = shard_of(0);
      const int64_t off = (int64_t)sh * a.carry.shard_cap + a.carry.used[sh];
      a.carry.data[off] = 0;
      a.carry.used[sh] += 1;
      a.carry_off[0] = off;
      a.carry_cnt[0] = 1;
    }
  } else if (root_leaf) {
    a.p2p_src[a.p2p_off[0]] = 0;
  }
}

__global__ void k_walk_reset(Control* c) {
  for (int i = threadIdx.x; i < 3 * POOL_SHARDS; i += blockDim.x) (&c->pool_used[0][0])[i] = 0;
  if (threadIdx.x == 0) {
    c->pool_overflow = 0;
    c->own_m2l_total = 0;
    c->own_p2p_total = 0;
  }
}

// Sum of the own counts (list sizes are known before the transposed sort);
// block partial sums are added with integer atomics (order-independent).
__global__ void k_walk_own_totals(int64_t n, const int32_t* om, const int32_t* op, Control* c) {
  __shared__ int64_t sm[WK_THREADS], sp[WK_THREADS];
  int64_t a = 0, b = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    a += om[i];
    b += op[i];
  }
  sm[threadIdx.x] = a;
  sp[threadIdx.x] = b;
  __syncthreads();
  for (int s = WK_THREADS / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sm[threadIdx.x] += sm[threadIdx.x + s];
      sp[threadIdx.x] += sp[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    atomicAdd((unsigned long long*)&c->own_m2l_total, (unsigned long long)sm[0]);
    atomicAdd((unsigned long long*)&c->own_p2p_total, (unsigned long long)sp[0]);
  }
}

// One block per shard: copy the shard's used entries to the dense array
// (transposed M2L pool first, then the P2P pool with the kind bit set).
__global__ void k_tr_compact(Pool<uint64_t> trm, Pool<uint64_t> trp, int kind_bit, uint64_t* dst) {
  const int sh = blockIdx.x % POOL_SHARDS;
  const int kind = blockIdx.x / POOL_SHARDS;
  const Pool<uint64_t>& p = kind ? trp : trm;
  __shared__ int64_t base;
  if (threadIdx.x == 0) {
    int64_t b = 0;
    if (kind)
      for (int i = 0; i < POOL_SHARDS; i++) b += trm.used[i];
    for (int i = 0; i < sh; i++) b += p.used[i];
    base = b;
  }
  __syncthreads();
  const int64_t n = p.used[sh];
  const uint64_t kb = (uint64_t)kind << kind_bit;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
    dst[base + i] = p.data[(int64_t)sh * p.shard_cap + i] | kb;
}

// Runs of equal (kind, target) in the sorted keys: first index and end index.
__global__ void k_tr_runs(const uint64_t* keys, int64_t n, int sh, int kind_bit, int64_t n_nodes,
                          int64_t* start, int32_t* cnt) {
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const uint64_t g = keys[k] >> sh;  // kind and target
  const int kind = (int)(keys[k] >> kind_bit);
  const int64_t c = (int64_t)(g & ((1ull << (kind_bit - sh)) - 1ull));
  const int64_t slot = (int64_t)kind * n_nodes + c;
  if (k == 0 || (keys[k - 1] >> sh) != g) start[slot] = k;
  if (k == n - 1 || (keys[k + 1] >> sh) != g) cnt[slot] = (int32_t)(k + 1);  // end, for now
}

// run ends -> run lengths
__global__ void k_tr_lengths(int64_t m, const int64_t* start, int32_t* cnt) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < m && cnt[i] > 0) cnt[i] = (int32_t)(cnt[i] - start[i]);
}

__global__ void k_walk_offsets(int64_t n, const int32_t* om, const int32_t* op, const int32_t* cm,
                               const int32_t* cp, int64_t* totm, int64_t* totp) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  totm[i] = (int64_t)om[i] + cm[i];
  totp[i] = (int64_t)op[i] + cp[i];
}

__global__ void k_walk_copy_totals(const int64_t* m2l_total, const int64_t* p2p_total,
                                   const int64_t* task_total, const int64_t* part_total,
                                   const int64_t* union_total, const int64_t* tail_total,
                                   Control* c) {
  if (threadIdx.x == 0) {
    c->n_m2l = *m2l_total;
    c->n_p2p = *p2p_total;
    c->n_p2p_tasks = *task_total;
    c->n_p2p_part = *part_total;
    c->n_union = *union_total;
    c->n_tail_tasks = *tail_total;
  }
}

// The children of a non-leaf P all receive the same candidates (P's carry,
// expanded), so their own M2L sources are the candidates accepted by at least
// one child.  One wave per parent enumerates them once, in ascending order,
// and keeps each accepted candidate with a mask of the accepting children.
__global__ void __launch_bounds__(WK_THREADS)
    k_union(int pass, WalkArgs a, const int32_t* parents, int64_t n_parents, int64_t* cnt_off,
            int32_t* usrc, uint8_t* umask) {
  const uint64_t lt = lanemask_lt();
  const int lane = __lane_id();
  for (int64_t pi = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; pi < n_parents;
       pi += (int64_t)gridDim.x * WK_WAVES) {
    const int32_t P = parents[pi];
    const int nc = a.n_child[P];
    const int32_t fc = a.first_child[P];
    int4 mine = make_int4(0, 0, 0, 0);
    if (lane < nc) mine = a.geo[fc + lane];
    int4 cg[8];
#pragma unroll
    for (int t = 0; t < 8; t++) {
      cg[t].x = __shfl(mine.x, t, WAVE);
      cg[t].y = __shfl(mine.y, t, WAVE);
      cg[t].z = __shfl(mine.z, t, WAVE);
      cg[t].w = __shfl(mine.w, t, WAVE);
    }
    const int64_t g0 = a.carry_off[P];
    const int gc = a.carry_cnt[P];
    int64_t base = pass == 2 ? cnt_off[pi] : 0;
    int64_t n = 0;
    for_each_candidate(a, g0, gc, [&](bool act, int32_t c, int) {
      uint32_t m = 0;
      if (act) {
        const int4 g = a.geo[c];
#pragma unroll
        for (int t = 0; t < 8; t++)
          if (t < nc && accept_pair(cg[t], g, a.t2)) m |= 1u << t;
      }
      const uint64_t b = __ballot(m != 0);
      if (pass == 2 && m != 0) {
        const int64_t o = base + n + __popcll(b & lt);
        usrc[o] = c;
        umask[o] = (uint8_t)m;
      }
      n += __popcll(b);
    });
    if (pass == 1 && lane == 0) cnt_off[pi] = n;
  }
}

hipError_t launch_union(int pass, const WalkArgs& a, const int32_t* parents, int64_t n_parents,
                        int64_t* ucount_or_off, int32_t* usrc, uint8_t* umask, hipStream_t st) {
  if (n_parents <= 0) return hipSuccess;
  int64_t blocks = (n_parents + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 16384) blocks = 16384;
  k_union<<<(unsigned)blocks, WK_THREADS, 0, st>>>(pass, a, parents, n_parents, ucount_or_off,
                                                  usrc, umask);
  return hipGetLastError();
}

// Sorted transposed keys -> after each target's own entries.
__global__ void k_tr_scatter(const uint64_t* keys, int64_t n, int sh, int kind_bit,
                             int64_t n_nodes, const int64_t* m2l_off, const int32_t* own_m2l,
                             const int64_t* start_m2l, int32_t* m2l_src, const int64_t* p2p_off,
                             const int32_t* own_p2p, const int64_t* start_p2p, int32_t* p2p_src) {
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const uint64_t key = keys[k];
  const int kind = (int)(key >> kind_bit);
  const int64_t c = (int64_t)((key >> sh) & ((1ull << (kind_bit - sh)) - 1ull));
  const int32_t src = (int32_t)(key & ((1ull << sh) - 1ull));
  if (kind == 0)
    m2l_src[m2l_off[c] + own_m2l[c] + (k - start_m2l[c])] = src;
  else
    p2p_src[p2p_off[c] + own_p2p[c] + (k - start_p2p[c])] = src;
}

hipError_t launch_walk_root(int pass, int root_leaf, const WalkArgs& a, hipStream_t st) {
  k_walk_root<<<1, 64, 0, st>>>(pass, root_leaf, a);
  return hipGetLastError();
}
hipError_t launch_walk_reset(Control* ctrl, hipStream_t st) {
  k_walk_reset<<<1, 256, 0, st>>>(ctrl);
  return hipGetLastError();
}
hipError_t launch_walk_own_totals(int64_t n_nodes, const int32_t* own_m2l, const int32_t* own_p2p,
                                  Control* ctrl, hipStream_t st) {
  int64_t blocks = (n_nodes + WK_THREADS - 1) / WK_THREADS;
  if (blocks > 1024) blocks = 1024;
  k_walk_own_totals<<<(unsigned)blocks, WK_THREADS, 0, st>>>(n_nodes, own_m2l, own_p2p, ctrl);
  return hipGetLastError();
}
hipError_t launch_tr_compact(const WalkArgs& a, int kind_bit, uint64_t* dst, hipStream_t st) {
  k_tr_compact<<<2 * POOL_SHARDS, 256, 0, st>>>(a.trm, a.trp, kind_bit, dst);
  return hipGetLastError();
}
hipError_t launch_tr_runs(const uint64_t* keys, int64_t n, int key_shift, int kind_bit,
                          int64_t n_nodes, int64_t* start, int32_t* cnt, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_tr_runs<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(keys, n, key_shift, kind_bit, n_nodes,
                                                         start, cnt);
  k_tr_lengths<<<(unsigned)((2 * n_nodes + 255) / 256), 256, 0, st>>>(2 * n_nodes, start, cnt);
  return hipGetLastError();
}
hipError_t launch_walk_offsets(int64_t n_nodes, const int32_t* own_m2l, const int32_t* own_p2p,
                               const int32_t* cnt_m2l, const int32_t* cnt_p2p, int64_t* tot_m2l,
                               int64_t* tot_p2p, hipStream_t st) {
  k_walk_offsets<<<(unsigned)((n_nodes + 255) / 256), 256, 0, st>>>(n_nodes, own_m2l, own_p2p,
                                                                    cnt_m2l, cnt_p2p, tot_m2l,
                                                                    tot_p2p);
  return hipGetLastError();
}
hipError_t launch_walk_copy_totals(const int64_t* m2l_total, const int64_t* p2p_total,
                                   const int64_t* task_total, const int64_t* part_total,
                                   const int64_t* union_total, const int64_t* tail_total,
                                   Control* ctrl, hipStream_t st) {
  k_walk_copy_totals<<<1, 64, 0, st>>>(m2l_total, p2p_total, task_total, part_total, union_total,
                                       tail_total, ctrl);
  return hipGetLastError();
}
hipError_t launch_tr_scatter(const uint64_t* keys, int64_t n, int key_shift, int kind_bit,
                             int64_t n_nodes, const int64_t* m2l_off, const int32_t* own_m2l,
                             const int64_t* start_m2l, int32_t* m2l_src, const int64_t* p2p_off,
                             const int32_t* own_p2p, const int64_t* start_p2p, int32_t* p2p_src,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_tr_scatter<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
      keys, n, key_shift, kind_bit, n_nodes, m2l_off, own_m2l, start_m2l, m2l_src, p2p_off,
      own_p2p, start_p2p, p2p_src);
  return hipGetLastError();
}

static unsigned walk_grid(const WalkArgs& a) {
  int64_t blocks = (a.lvl_count + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 16384) blocks = 16384;
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
