// fmm_walk.hip -- the dual-tree walk that emits the M2L and P2P lists.
//
// jz-fmm project page, "Calculating a node-node interaction" (opening criterion)
// and "Combining near and far interactions" (accept well-separated pairs for
// multipole-to-local translations, refine the rest, sum the remaining nearby
// pairs directly).  The pair walk from (root, root) -- accept -> M2L, two
// leaves -> P2P, otherwise split the coarser non-leaf (both when the levels are
// equal) -- is evaluated here one tree level per step, per sibling group:
//
//   * the children of a node X all receive the same candidates: X's "carry"
//     (X's rejected partners) with each carried leaf kept as it is and each
//     carried non-leaf replaced by its children;
//   * each candidate c is tested against every child t: accepted -> M2L
//     (t <- c); rejected with t and c both leaves -> P2P (t <- c); rejected
//     with t a non-leaf -> c goes to t's carry.
//
// One wave per X enumerates the candidates once per pass and keeps, for the
// group, three unions of (candidate, 8-bit mask of children): the M2L union,
// the P2P union and the carry union.  A child's own list (or carry) is the
// union's entries with its bit set, in enumeration order.
//
// The pair walk also refines the partners of a leaf t past t's own level
// (only the non-leaf side can split).  Those pairs are exactly the pairs in
// which a deeper target sees t as a carried leaf, and the acceptance test is
// symmetric, so they are emitted from that side: when a target accepts a
// carried leaf c of a coarser level, the entry (c <- target) is added to c's
// list as well, and likewise for leaf-leaf rejections.  Such transposed
// entries are appended in any order and put in place by a radix sort of
// (target, source) keys; a target's own entries (sources at its level or
// coarser) come first, its transposed ones (deeper sources) after, so every
// list ends sorted by source, as the pair walk's canonical order requires.
//
// A step enumerates each group's candidates once: their number, known from the
// carry alone, reserves room for the three unions (sharded bump allocators,
// integer atomics spread over 512 counters by node: placement varies between
// runs, the lists do not), and the transposed entries are only counted.  After
// the last step one launch over every group re-tests the carried leaves only
// and writes the transposed keys at offsets from a scan over the groups in id
// order: for a fixed target the keys come out with ascending sources, so a
// stable sort on (kind, target) alone puts every transposed list in order.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int WK_THREADS = 256;
constexpr int WK_WAVES = WK_THREADS / WAVE;
constexpr int WALK_TAB = 8 * WAVE;  // candidates of 64 carried entries (<= 8 children each)
// Generators of at most GEN_T entries are read once, by the counting pass,
// which also keeps each entry's child count and first candidate in the wave's
// LDS for both enumeration passes (each pass over memory is a chain of
// dependent loads per 64 entries).
constexpr int GEN_T = 4 * WAVE;

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

// Visit the candidates of the group of X in ascending node order, 64 at a time:
// first the carried leaves (levels < s, kept as they are: phase 0), then the
// children of the carried non-leaves (level s: phase 1).  X's carry is the
// entries of its parent's carry union with X's bit set (for the root: the
// root).  f(active, cand, geo of cand, phase) is called by the whole wave; the
// geometry of the next 64 candidates is loaded before f runs on the current
// ones, so its latency overlaps their classification.  tab: the wave's LDS
// table of WALK_TAB candidates.  gk, gf (null: read the generator): per entry
// its node's child count (-1 without X's bit) and its first candidate (the
// node itself when it is a leaf, else its first child), from the counting pass.
template <typename F>
__device__ __forceinline__ void for_each_candidate(const WalkArgs& a, int32_t X, int32_t* tab,
                                                   const int* gk, const int32_t* gf, F&& f) {
  const int lane = __lane_id();
  const uint64_t* gen;
  int gc, slot;
  if (X == 0) {
    gen = a.rootgen;
    gc = 1;
    slot = 0;
  } else {
    const int32_t Y = uniform(a.parent[X]);
    gen = a.cu.data + uniform(a.cu_off[Y]);
    gc = uniform(a.cu_cnt[Y]);
    slot = X - uniform(a.first_child[Y]);
  }
  for (int phase = 0; phase < 2; phase++) {
    for (int c0 = 0; c0 < gc; c0 += WAVE) {
      const int j = c0 + lane;
      int nc = 0, fc = 0;
      if (j < gc) {
        if (gk) {
          const int k = gk[j];
          if ((phase == 0 && k == 0) || (phase == 1 && k > 0)) {
            nc = k == 0 ? 1 : k;
            fc = gf[j];
          }
        } else {
          const uint64_t e = gen[j];
          if ((e >> slot) & 1u) {
            const int32_t g = (int32_t)(e >> 8);
            const int k = a.n_child[g];
            if (phase == 0 && k == 0) {
              nc = 1;
              fc = g;
            } else if (phase == 1 && k != 0) {
              nc = k;
              fc = a.first_child[g];
            }
          }
        }
      }
      // the (at most 8 x 64) candidates of these entries, in order, in the
      // wave's LDS table
      const int incl = wave_incl_scan(nc);
      const int excl = incl - nc;
      const int tot = read_lane(incl, WAVE - 1);
      for (int k = 0; k < nc; k++) tab[excl + k] = fc + k;
      __builtin_amdgcn_wave_barrier();
      int32_t cn = 0;
      int4 gn = make_int4(0, 0, 0, 0);
      if (lane < tot) {
        cn = tab[lane];
        gn = a.geo[cn];
      }
      for (int b = 0; b < tot; b += WAVE) {
        const bool active = b + lane < tot;
        const int32_t c = cn;
        const int4 g = gn;
        if (b + WAVE + lane < tot) {
          cn = tab[b + WAVE + lane];
          gn = a.geo[cn];
        }
        f(active, c, g, phase);
      }
      __builtin_amdgcn_wave_barrier();  // the table is read before it is refilled
    }
  }
}

__device__ __forceinline__ int shard_of(int32_t t) {
  return (int)(((uint32_t)t * 2654435761u) >> 23) & (POOL_SHARDS - 1);
}

// The children of X: geometry of child t in cg[t]; masks of the leaf children
// and of all children.
struct Group {
  int4 cg[8];
  uint32_t leafmask, allmask;
  int nc;
  int32_t fc;
};

__device__ __forceinline__ Group load_group(const WalkArgs& a, int32_t X) {
  Group G;
  const int lane = __lane_id();
  G.nc = uniform((int)a.n_child[X]);
  G.fc = uniform(a.first_child[X]);
  int4 mine = make_int4(0, 0, 0, 0);
  if (lane < G.nc) mine = a.geo[G.fc + lane];
#pragma unroll
  for (int t = 0; t < 8; t++) {
    G.cg[t].x = __shfl(mine.x, t, WAVE);
    G.cg[t].y = __shfl(mine.y, t, WAVE);
    G.cg[t].z = __shfl(mine.z, t, WAVE);
    G.cg[t].w = __shfl(mine.w, t, WAVE);
  }
  G.allmask = (1u << G.nc) - 1u;
  G.leafmask = (uint32_t)__ballot(lane < G.nc && (mine.w & GEO_LEAF) != 0) & G.allmask;
  return G;
}

// Classify a candidate of geometry g for every child: masks of M2L, P2P and carry.
__device__ __forceinline__ void classify(const WalkArgs& a, const Group& G, const int4& g,
                                         uint32_t& mM, uint32_t& mP, uint32_t& mC) {
  uint32_t acc = 0;
#pragma unroll
  for (int t = 0; t < 8; t++)
    if (accept_pair(G.cg[t], g, a.t2)) acc |= 1u << t;
  acc &= G.allmask;
  const uint32_t rej = G.allmask & ~acc;
  mM = acc;
  mP = (g.w & GEO_LEAF) ? (rej & G.leafmask) : 0u;
  mC = rej & ~G.leafmask;
}

// 8 counters of up to 2^32 - 1 in four 64-bit words: bit t of m adds one to counter t
__device__ __forceinline__ void add_bits(uint64_t (&c)[4], uint32_t m) {
#pragma unroll
  for (int k = 0; k < 4; k++)
    c[k] += (uint64_t)((m >> (2 * k)) & 1u) | ((uint64_t)((m >> (2 * k + 1)) & 1u) << 32);
}

// The generator of X (its carry): the entries of its parent's carry union with
// X's bit set; for the root, the root.
struct Gen {
  const uint64_t* e;
  int n, slot;
};
__device__ __forceinline__ Gen generator(const WalkArgs& a, int32_t X) {
  if (X == 0) return Gen{a.rootgen, 1, 0};
  const int32_t Y = uniform(a.parent[X]);
  return Gen{a.cu.data + uniform(a.cu_off[Y]), uniform(a.cu_cnt[Y]),
             X - uniform(a.first_child[Y])};
}

__global__ void __launch_bounds__(WK_THREADS) k_walk(WalkArgs a) {
  // after an overflow the carry unions may be incomplete: do nothing, the host
  // regrows the pools and repeats the walk
  if (a.ctrl->pool_overflow) return;
  __shared__ int32_t tab_all[WK_WAVES][WALK_TAB];
  __shared__ int gk_all[WK_WAVES][GEN_T];
  __shared__ int32_t gf_all[WK_WAVES][GEN_T];
  int32_t* tab = tab_all[threadIdx.x / WAVE];
  int* gk = gk_all[threadIdx.x / WAVE];
  int32_t* gf = gf_all[threadIdx.x / WAVE];
  const int lane = __lane_id();
  const uint64_t lt = lanemask_lt();
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < a.pcnt;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int64_t pi = a.pbeg + j;
    const int32_t X = uniform(a.parents[pi]);
    const Group G = load_group(a, X);
    // number of candidates: carried leaves count 1, carried non-leaves their children
    const Gen gen = generator(a, X);
    const bool inlds = gen.n <= GEN_T;
    int nc_lane = 0;
    if (inlds) {  // all loads of a step issued before the first is used
      constexpr int R = GEN_T / WAVE;
      uint64_t e[R];
      int k[R];
#pragma unroll
      for (int r = 0; r < R; r++) e[r] = r * WAVE + lane < gen.n ? gen.e[r * WAVE + lane] : 0ull;
#pragma unroll
      for (int r = 0; r < R; r++)
        k[r] = r * WAVE + lane < gen.n && ((e[r] >> gen.slot) & 1u)
                   ? (int)a.n_child[(int32_t)(e[r] >> 8)]
                   : -1;
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int32_t g = (int32_t)(e[r] >> 8);
        gk[r * WAVE + lane] = k[r];
        gf[r * WAVE + lane] = k[r] > 0 ? a.first_child[g] : g;
        nc_lane += k[r] < 0 ? 0 : (k[r] == 0 ? 1 : k[r]);
      }
    } else {
      for (int c0 = lane; c0 < gen.n; c0 += WAVE) {
        const uint64_t e = gen.e[c0];
        if ((e >> gen.slot) & 1u) {
          const int k = a.n_child[(int32_t)(e >> 8)];
          nc_lane += k == 0 ? 1 : k;
        }
      }
    }
    const int64_t ncand = wave_sum((int64_t)nc_lane);
    // room for up to ncand entries in each union; one atomic per pool, issued together
    const int sh = shard_of(X);
    int64_t o[3] = {0, 0, 0};
    if (lane == 0 && ncand > 0) {
      o[0] = (int64_t)atomicAdd((unsigned long long*)&a.cu.used[sh], (unsigned long long)ncand);
      o[1] = (int64_t)atomicAdd((unsigned long long*)&a.u.used[sh], (unsigned long long)ncand);
      o[2] = (int64_t)atomicAdd((unsigned long long*)&a.pu.used[sh], (unsigned long long)ncand);
    }
    bool ok = true;
#pragma unroll
    for (int k = 0; k < 3; k++) {
      o[k] = __shfl(o[k], 0, WAVE);
      const Pool<uint64_t>& P = k == 0 ? a.cu : (k == 1 ? a.u : a.pu);
      ok = ok && o[k] + ncand <= P.shard_cap;
      o[k] += (int64_t)sh * P.shard_cap;
    }
    if (!ok) {  // results are discarded; the host regrows the pools and retries
      if (lane == 0) atomicOr(&a.ctrl->pool_overflow, 1);
      continue;
    }
    int64_t kU = 0, kPU = 0, kCU = 0;
    uint32_t ntm = 0, ntp = 0;  // per lane
    uint64_t cm[4] = {0, 0, 0, 0}, cp[4] = {0, 0, 0, 0};
    const int* gkp = inlds ? gk : nullptr;
    for_each_candidate(a, X, tab, gkp, gf, [&](bool act, int32_t c, const int4& g, int phase) {
      uint32_t mM = 0, mP = 0, mC = 0;
      if (act) classify(a, G, g, mM, mP, mC);
      const uint64_t packed = (uint64_t)(uint32_t)c << 8;
      const uint64_t bU = __ballot(mM != 0), bP = __ballot(mP != 0), bC = __ballot(mC != 0);
      if (mM) a.u.data[o[1] + kU + __popcll(bU & lt)] = packed | mM;
      if (mP) a.pu.data[o[2] + kPU + __popcll(bP & lt)] = packed | mP;
      if (mC) a.cu.data[o[0] + kCU + __popcll(bC & lt)] = packed | mC;
      kU += __popcll(bU);
      kPU += __popcll(bP);
      kCU += __popcll(bC);
      add_bits(cm, mM);
      add_bits(cp, mP);
      if (phase == 0) {  // carried leaves of coarser levels: transposed entries
        ntm += __popc(mM);
        ntp += __popc(mP);
      }
    });
#pragma unroll
    for (int k = 0; k < 4; k++) {
      cm[k] = wave_sum(cm[k]);
      cp[k] = wave_sum(cp[k]);
    }
    const int64_t tm = wave_sum((int64_t)ntm), tp = wave_sum((int64_t)ntp);
    int64_t om = 0, op = 0;  // the group's own entries, for the list totals
#pragma unroll
    for (int k = 0; k < 4; k++) {
      om += (int64_t)(cm[k] & 0xffffffffu) + (int64_t)(cm[k] >> 32);
      op += (int64_t)(cp[k] & 0xffffffffu) + (int64_t)(cp[k] >> 32);
    }
    if (lane == 0) {
      if (om) atomicAdd((unsigned long long*)&a.ctrl->own_used[0][sh], (unsigned long long)om);
      if (op) atomicAdd((unsigned long long*)&a.ctrl->own_used[1][sh], (unsigned long long)op);
      a.cu_off[X] = o[0];
      a.cu_cnt[X] = (int32_t)kCU;
      a.u_off[X] = o[1];
      a.u_cnt[X] = (int32_t)kU;
      a.pu_off[X] = o[2];
      a.pu_cnt[X] = (int32_t)kPU;
      a.trm_cnt[pi] = tm;
      a.trp_cnt[pi] = tp;
    }
    if (lane < G.nc) {
      const int k = lane >> 1, hi = lane & 1;
      uint64_t vm = 0, vp = 0;
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (q == k) {
          vm = cm[q];
          vp = cp[q];
        }
      a.own_m2l[G.fc + lane] = (int32_t)(hi ? (vm >> 32) : (vm & 0xffffffffu));
      a.own_p2p[G.fc + lane] = (int32_t)(hi ? (vp >> 32) : (vp & 0xffffffffu));
    }
  }
}

// Transposed keys, every group at once: the carried leaves of X's generator are
// tested again against X's children; (c <- child) keys go to the group's slot of
// the M2L part (accepted) or the P2P part (leaf-leaf rejected), candidate by
// candidate, children in order.
constexpr int TRE_U = 4;  // chunks of generator entries per round of k_tr_emit
__global__ void __launch_bounds__(WK_THREADS) k_tr_emit(WalkArgs a, int32_t* run_cnt,
                                                         int64_t run_n) {
  bookkeeping_priority();
  // the run lengths of the next step start at zero (targets without a run)
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < run_n;
       i += (int64_t)gridDim.x * blockDim.x)
    run_cnt[i] = 0;
  if (a.ctrl->pool_overflow) return;  // the unions are incomplete
  const uint64_t lt = lanemask_lt();
  const int lane = __lane_id();
  const int64_t ntm_all = *a.n_trm;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int64_t ntr = ntm_all + a.ctrl->n_trp;
    a.ctrl->n_tr = ntr;
    if (ntr > a.tr_cap) a.ctrl->list_overflow = 1;
  }
  if (ntm_all + a.ctrl->n_trp > a.tr_cap) return;  // no room: repeated with more
  for (int64_t pi = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; pi < a.pcnt;
       pi += (int64_t)gridDim.x * WK_WAVES) {
    if (uniform(a.trm_cnt[pi]) + uniform(a.trp_cnt[pi]) == 0) continue;
    const int32_t X = uniform(a.parents[pi]);
    const Group G = load_group(a, X);
    const Gen gen = generator(a, X);
    int64_t om = a.trm_base[pi], op = ntm_all + a.trp_base[pi];
    const uint64_t hiK = 1ull << (2 * a.key_shift);
    // TRE_U chunks of 64 entries per round: their entries, child counts and
    // geometry are loaded together, so that a long generator (a sparse leaf
    // next to a dense cluster has ~10^5 carried candidates) costs one chain of
    // dependent loads per TRE_U chunks; the keys are then written chunk by
    // chunk, in entry order, as with one chunk per round
    for (int c0 = 0; c0 < gen.n; c0 += TRE_U * WAVE) {
      uint64_t e[TRE_U];
#pragma unroll
      for (int u = 0; u < TRE_U; u++) {
        const int j = c0 + u * WAVE + lane;
        e[u] = j < gen.n ? gen.e[j] : 0ull;  // 0: no slot bit, inactive
      }
      int kc[TRE_U];
      int4 gc[TRE_U];
#pragma unroll
      for (int u = 0; u < TRE_U; u++) {
        kc[u] = 1;
        gc[u] = make_int4(0, 0, 0, 0);
        if ((e[u] >> gen.slot) & 1u) {
          const int32_t c = (int32_t)(e[u] >> 8);
          kc[u] = a.n_child[c];
          gc[u] = a.geo[c];
        }
      }
#pragma unroll
      for (int u = 0; u < TRE_U; u++) {
        uint32_t mM = 0, mP = 0, mC = 0;
        if (kc[u] == 0) classify(a, G, gc[u], mM, mP, mC);
        const int nm = __popc(mM), np = __popc(mP);
        const int im = wave_incl_scan(nm), ip = wave_incl_scan(np);
        int64_t wm = om + (im - nm), wp = op + (ip - np);
        const uint64_t hiC = (uint64_t)(uint32_t)(e[u] >> 8) << a.key_shift;
        for (uint32_t m = mM; m; m &= m - 1) a.tr_keys[wm++] = hiC | (uint32_t)(G.fc + __ffs(m) - 1);
        for (uint32_t m = mP; m; m &= m - 1)
          a.tr_keys[wp++] = hiK | hiC | (uint32_t)(G.fc + __ffs(m) - 1);
        om += __shfl(im, WAVE - 1, WAVE);
        op += __shfl(ip, WAVE - 1, WAVE);
      }
    }
    (void)lt;
  }
}


// Walk set-up: pools empty, no overflow, the root's generator; the own-entry
// totals start with the root's (itself as its only P2P entry when it is a leaf).
__global__ void k_walk_reset(Control* c, uint64_t* rootgen, int root_leaf, int32_t* own_m2l,
                             int32_t* own_p2p) {
  if (threadIdx.x == 0) {  // (also when the walk is repeated within one build)
    c->list_overflow = 0;
    c->n_tr = 0;
    c->n_split = 0;
    c->tr_small_over = 0;
  }
  for (int i = threadIdx.x; i < N_POOLS * POOL_SHARDS; i += blockDim.x)
    (&c->pool_used[0][0])[i] = 0;
  for (int i = threadIdx.x; i < 2 * POOL_SHARDS; i += blockDim.x) (&c->own_used[0][0])[i] = 0;
  for (int i = threadIdx.x; i < ORDER_OCT; i += blockDim.x) {
    c->task_oct[i] = c->task_cur[i] = 0;
    c->group_oct[i] = c->group_cur[i] = 0;
  }
  if (threadIdx.x == 0) {
    own_m2l[0] = 0;  // the root is nobody's child: its own counts are set here
    own_p2p[0] = root_leaf;
    c->pool_overflow = 0;
    c->own_m2l_total = 0;
    c->own_p2p_total = root_leaf;
    rootgen[0] = (0ull << 8) | 1ull;  // node 0, slot 0
  }
}

// Sum of the own counts (list sizes are known before the transposed sort);
// block partial sums are added with integer atomics (order-independent).

// Runs of equal (kind, target) in the sorted keys: first index and end index.
__global__ void k_tr_runs(const uint64_t* keys, int64_t cap, const int64_t* n_dev,
                          const Control* ctrl, int sh, int kind_bit, int64_t n_nodes,
                          int64_t* start, int32_t* cnt) {
  bookkeeping_priority();
  if (walk_aborted(ctrl)) return;
  const int64_t n = min(*n_dev, cap);
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
  bookkeeping_priority();
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < m && cnt[i] > 0) cnt[i] = (int32_t)(cnt[i] - start[i]);
}

__global__ void k_walk_offsets(int64_t n, const int32_t* own, const int32_t* tr_cnt,
                               int64_t* tot) {
  bookkeeping_priority();
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  tot[i] = (int64_t)own[i] + tr_cnt[i];
}


// Few transposed keys (at most TRS_MAX, nodes at most TRS_MAX_NODES): one
// block of 1024 threads does what the multi-block path does in twelve
// dependent launches.  The keys are stably sorted on their (kind, target)
// bits in LDS (two 9-bit passes; wave w owns the w-th sixteenth of the current
// order, counts its digits, the counts are scanned over waves and digits and
// each wave places its elements in order, so equal digits keep their order),
// written to keys_out, and their runs give start[slot] and cnt[slot] (slot =
// kind * n_nodes + target; cnt was cleared by the emission).  Then tot[i] =
// own[i] + cnt[n_nodes + i] and p2p_off = its exclusive scan, with the total
// at p2p_off[n_nodes] and in ctrl->n_p2p.  More keys than TRS_MAX: the lists
// are marked as overflowing (the walk is repeated, on the multi-block path).
constexpr int TRS_THREADS = 1024;
constexpr int TRS_WAVES = TRS_THREADS / WAVE;
constexpr int TRS_BATCH = TRS_MAX / TRS_THREADS;  // 64-element batches per wave and pass

__global__ void __launch_bounds__(TRS_THREADS)
    k_tr_small(const uint64_t* __restrict__ keys_in, int64_t cap, Control* ctrl, int sh,
               int64_t n_nodes, uint64_t* __restrict__ keys_out, int64_t* __restrict__ start,
               int32_t* __restrict__ cnt, const int32_t* __restrict__ own,
               int64_t* __restrict__ tot, int64_t* __restrict__ p2p_off) {
  bookkeeping_priority();
  __shared__ uint64_t skey[TRS_MAX];
  __shared__ int16_t ping[2][TRS_MAX];
  __shared__ int wc[TRS_WAVES][512];
  __shared__ int64_t wsum64[TRS_WAVES];
  __shared__ int wsum[TRS_WAVES];
  if (walk_aborted(ctrl)) return;
  const int64_t nd = min(ctrl->n_tr, cap);
  if (nd > TRS_MAX) {
    if (threadIdx.x == 0) {
      ctrl->list_overflow = 1;
      ctrl->tr_small_over = 1;
    }
    return;
  }
  const int n = (int)nd;
  const int tid = threadIdx.x, w = tid / WAVE, lane = __lane_id();
  for (int i = tid; i < n; i += TRS_THREADS) {
    skey[i] = keys_in[i];
    ping[0][i] = (int16_t)i;
  }
  __syncthreads();
  const int per = TRS_BATCH * WAVE;  // the wave's part of the order
  const int c0 = min(n, w * per), c1 = min(n, c0 + per);
  const uint64_t lt = lanemask_lt();
  const int bits = sh + 1;  // kind and target
  const int passes = (bits + 8) / 9;
  for (int pass = 0; pass < passes; pass++) {
    const int16_t* src = ping[pass & 1];
    int16_t* dst = ping[(pass & 1) ^ 1];
    const int shift = sh + 9 * pass;
    const uint32_t dmask = (1u << min(9, sh + bits - shift)) - 1u;
    for (int d = lane; d < 512; d += WAVE) wc[w][d] = 0;
    __builtin_amdgcn_wave_barrier();
    int16_t sv[TRS_BATCH];
    int dg[TRS_BATCH];
#pragma unroll
    for (int b = 0; b < TRS_BATCH; b++) {
      const int i = c0 + b * WAVE + lane;
      sv[b] = i < c1 ? src[i] : (int16_t)0;
      dg[b] = i < c1 ? (int)((skey[sv[b]] >> shift) & dmask) : -1;
    }
#pragma unroll
    for (int b = 0; b < TRS_BATCH; b++)
      if (dg[b] >= 0) atomicAdd(&wc[w][dg[b]], 1);
    __syncthreads();
    int incl = 0, acc = 0;
    if (tid < 512) {  // digit tid: start of each wave's part within the digit
      for (int q = 0; q < TRS_WAVES; q++) {
        const int c = wc[q][tid];
        wc[q][tid] = acc;
        acc += c;
      }
      incl = wave_incl_scan(acc);
      if (lane == WAVE - 1) wsum[w] = incl;
    }
    __syncthreads();
    if (tid < 512) {
      int dstart = incl - acc;
      for (int q = 0; q < w; q++) dstart += wsum[q];
      for (int q = 0; q < TRS_WAVES; q++) wc[q][tid] += dstart;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < TRS_BATCH; b++) {
      if (c0 + b * WAVE >= c1) break;  // wave-uniform
      const int d = dg[b];
      uint64_t mask = __ballot(d >= 0);
#pragma unroll
      for (int k = 0; k < 9; k++) {
        const uint64_t bb = __ballot((d >> k) & 1);
        mask &= ((d >> k) & 1) ? bb : ~bb;
      }
      const int before = d >= 0 ? wc[w][d] : 0;
      __builtin_amdgcn_wave_barrier();
      if (d >= 0) {
        dst[before + __popcll(mask & lt)] = sv[b];
        if ((mask & lt) == 0) wc[w][d] = before + __popcll(mask);
      }
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }
  const int16_t* ord = ping[passes & 1];
  const uint64_t gmask = (1ull << (sh + 1)) - 1ull;  // kind and target, above the source
  // sorted keys and the run starts
  for (int k = tid; k < n; k += TRS_THREADS) {
    const uint64_t key = skey[ord[k]];
    keys_out[k] = key;
    const uint64_t g = (key >> sh) & gmask;
    if (k == 0 || ((skey[ord[k - 1]] >> sh) & gmask) != g) {
      const int64_t slot = (int64_t)(g >> sh) * n_nodes + (int64_t)(g & ((1ull << sh) - 1ull));
      start[slot] = k;
    }
  }
  __syncthreads();  // the starts are visible to the whole block
  for (int k = tid; k < n; k += TRS_THREADS) {
    const uint64_t g = (skey[ord[k]] >> sh) & gmask;
    if (k == n - 1 || ((skey[ord[k + 1]] >> sh) & gmask) != g) {
      const int64_t slot = (int64_t)(g >> sh) * n_nodes + (int64_t)(g & ((1ull << sh) - 1ull));
      cnt[slot] = (int32_t)(k + 1 - start[slot]);
    }
  }
  __syncthreads();  // the run lengths are visible to the whole block
  // near-field list sizes and their exclusive scan: thread t takes a
  // contiguous range of nodes
  const int64_t chunk = (n_nodes + TRS_THREADS - 1) / TRS_THREADS;
  const int64_t i0 = min(n_nodes, (int64_t)tid * chunk), i1 = min(n_nodes, i0 + chunk);
  int64_t part = 0;
  for (int64_t i = i0; i < i1; i++) {
    const int64_t t = (int64_t)own[i] + cnt[n_nodes + i];
    tot[i] = t;
    part += t;
  }
  const int64_t winc = wave_incl_scan(part);
  if (lane == WAVE - 1) wsum64[w] = winc;
  __syncthreads();
  int64_t off = winc - part, total = 0;
  for (int q = 0; q < TRS_WAVES; q++) {
    if (q < w) off += wsum64[q];
    total += wsum64[q];
  }
  for (int64_t i = i0; i < i1; i++) {
    p2p_off[i] = off;
    off += tot[i];
  }
  if (tid == 0) {
    p2p_off[n_nodes] = total;
    ctrl->n_p2p = total;
  }
}

hipError_t launch_tr_small(const uint64_t* keys_in, int64_t cap, Control* ctrl, int key_shift,
                           int64_t n_nodes, uint64_t* keys_out, int64_t* start, int32_t* cnt,
                           const int32_t* own, int64_t* tot, int64_t* p2p_off, hipStream_t st) {
  if (key_shift > 17 || n_nodes > TRS_MAX_NODES) return hipErrorInvalidValue;
  k_tr_small<<<1, TRS_THREADS, 0, st>>>(keys_in, cap, ctrl, key_shift, n_nodes, keys_out, start,
                                        cnt, own, tot, p2p_off);
  return hipGetLastError();
}

// Sorted transposed keys of one kind -> after each target's own entries.
__global__ void k_tr_scatter(const uint64_t* keys, int64_t kcap, const int64_t* n_dev,
                             Control* ctrl, int sh, int kind_bit, int kind, int64_t n_nodes,
                             const int64_t* off, const int32_t* own, const int64_t* start,
                             int32_t* src, int64_t cap) {
  bookkeeping_priority();
  if (ctrl && walk_aborted(ctrl)) return;
  const int64_t n = n_dev ? min(*n_dev, kcap) : kcap;
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const uint64_t key = keys[k];
  if ((int)(key >> kind_bit) != kind) return;
  const int64_t c = (int64_t)((key >> sh) & ((1ull << (kind_bit - sh)) - 1ull));
  const int64_t o = off[c] + own[c] + (k - start[c]);
  if (o < cap)
    src[o] = (int32_t)(key & ((1ull << sh) - 1ull));
  else if (ctrl)
    ctrl->list_overflow = 1;
}

// One wave per parent X: child t's own entries are the entries of X's union
// with bit t set, in union order; they go to src[off[child] ...].
__global__ void __launch_bounds__(WK_THREADS)
    k_union_scatter(const int32_t* parents, int64_t n_parents, const int32_t* first_child,
                    const uint8_t* n_child, const uint64_t* pool, const int64_t* uoff,
                    const int32_t* ucnt, const int64_t* off, int32_t* src, int64_t cap,
                    Control* ctrl) {
  bookkeeping_priority();
  if (ctrl && walk_aborted(ctrl)) return;
  const uint64_t lt = lanemask_lt();
  const int lane = __lane_id();
  for (int64_t j = (int64_t)blockIdx.x * WK_WAVES + threadIdx.x / WAVE; j < n_parents;
       j += (int64_t)gridDim.x * WK_WAVES) {
    const int32_t X = uniform(parents[j]);
    const int nc = uniform((int)n_child[X]);
    const int32_t fc = uniform(first_child[X]);
    const int64_t u0 = uniform(uoff[X]);
    const int un = uniform(ucnt[X]);
    int64_t base[8];
#pragma unroll
    for (int t = 0; t < 8; t++) base[t] = t < nc ? off[fc + t] : 0;
    for (int e0 = 0; e0 < un; e0 += WAVE) {
      uint64_t v = 0;
      if (e0 + lane < un) v = pool[u0 + e0 + lane];
      const int32_t id = (int32_t)(v >> 8);
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const bool has = (v >> t) & 1u;
        const uint64_t b = __ballot(has);
        if (has) {
          const int64_t o = base[t] + __popcll(b & lt);
          if (o < cap)
            src[o] = id;
          else if (ctrl)
            ctrl->list_overflow = 1;
        }
        base[t] += __popcll(b);
      }
    }
  }
}

// The root is nobody's child: its own counts are set here.  A leaf root has the
// single list entry P2P(root <- root).
// A root that is a leaf: its only P2P entry is itself.
__global__ void k_walk_root_leaf(const int64_t* p2p_off, int32_t* p2p_src) {
  bookkeeping_priority();
  if (threadIdx.x == 0) p2p_src[p2p_off[0]] = 0;
}
hipError_t launch_walk_root_leaf(const int64_t* p2p_off, int32_t* p2p_src, hipStream_t st) {
  k_walk_root_leaf<<<1, 64, 0, st>>>(p2p_off, p2p_src);
  return hipGetLastError();
}

hipError_t launch_walk_reset(Control* ctrl, uint64_t* rootgen, int root_leaf, int32_t* own_m2l,
                             int32_t* own_p2p, hipStream_t st) {
  k_walk_reset<<<1, 256, 0, st>>>(ctrl, rootgen, root_leaf, own_m2l, own_p2p);
  return hipGetLastError();
}
hipError_t launch_tr_runs(const uint64_t* keys, int64_t n, const int64_t* n_dev,
                          const Control* ctrl, int key_shift, int kind_bit, int64_t n_nodes,
                          int64_t* start, int32_t* cnt, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_tr_runs<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(keys, n, n_dev, ctrl, key_shift,
                                                         kind_bit, n_nodes, start, cnt);
  k_tr_lengths<<<(unsigned)((2 * n_nodes + 255) / 256), 256, 0, st>>>(2 * n_nodes, start, cnt);
  return hipGetLastError();
}
hipError_t launch_walk_offsets(int64_t n_nodes, const int32_t* own, const int32_t* tr_cnt,
                               int64_t* tot, hipStream_t st) {
  if (n_nodes <= 0) return hipSuccess;
  k_walk_offsets<<<(unsigned)((n_nodes + 255) / 256), 256, 0, st>>>(n_nodes, own, tr_cnt, tot);
  return hipGetLastError();
}
hipError_t launch_tr_scatter(const uint64_t* keys, int64_t n, const int64_t* n_dev,
                             Control* ctrl, int key_shift, int kind_bit, int kind,
                             int64_t n_nodes, const int64_t* off, const int32_t* own,
                             const int64_t* start, int32_t* src, int64_t cap, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_tr_scatter<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(keys, n, n_dev, ctrl, key_shift,
                                                            kind_bit, kind, n_nodes, off, own,
                                                            start, src, cap);
  return hipGetLastError();
}
hipError_t launch_union_scatter(const int32_t* parents, int64_t n_parents,
                                const int32_t* first_child, const uint8_t* n_child,
                                const uint64_t* pool, const int64_t* uoff, const int32_t* ucnt,
                                const int64_t* off, int32_t* src, int64_t cap, Control* ctrl,
                                hipStream_t st) {
  if (n_parents <= 0) return hipSuccess;
  int64_t blocks = (n_parents + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 16384) blocks = 16384;
  k_union_scatter<<<(unsigned)blocks, WK_THREADS, 0, st>>>(
      parents, n_parents, first_child, n_child, pool, uoff, ucnt, off, src, cap, ctrl);
  return hipGetLastError();
}
hipError_t launch_walk(const WalkArgs& a, hipStream_t st) {
  if (a.pcnt <= 0) return hipSuccess;
  int64_t blocks = (a.pcnt + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 16384) blocks = 16384;
  k_walk<<<(unsigned)blocks, WK_THREADS, 0, st>>>(a);
  return hipGetLastError();
}
hipError_t launch_tr_emit(const WalkArgs& a, int32_t* run_cnt, int64_t run_n, hipStream_t st) {
  int64_t blocks = (std::max<int64_t>(a.pcnt, 1) + WK_WAVES - 1) / WK_WAVES;
  if (blocks > 16384) blocks = 16384;
  k_tr_emit<<<(unsigned)blocks, WK_THREADS, 0, st>>>(a, run_cnt, run_n);
  return hipGetLastError();
}

}  // namespace mbg
