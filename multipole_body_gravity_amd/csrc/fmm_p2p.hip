// fmm_p2p.hip -- near field between leaf cells, plus the final combine.
//
// jz-fmm project page: the direct sum Phi(x_i) = -G sum_{j != i} m_j/|x_i - x_j|
// with the self term omitted ("From particle pairs to node pairs"), applied to
// the leaf pairs the walk did not accept ("Combining near and far
// interactions": at the leaves, add the remaining nearby interactions
// directly).  The far field computed by L2P is added here and the result is
// written in the caller's particle order.
//
// Work split.  A task is one target leaf and a slice of at most TASK_E source
// leaves of its list (a sparse leaf next to dense clusters can have ~10^5
// source leaves; slicing keeps every wave's work bounded).  One wave per task:
// the source particles of a group of list entries are enumerated in list order
// (an LDS table maps each particle to its entry) and staged 128 at a time
// through LDS; each lane holds two targets, so one LDS read serves two pairs,
// the target pairs x source slices fill the 64 lanes, and the slices of one
// target are summed in a fixed order.  A leaf with one task writes its final
// result directly; a leaf with several tasks writes per-task partial sums that
// a second kernel adds in task order.  Every sum has a fixed order.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int P2P_THREADS = 256;
constexpr int P2P_WAVES = P2P_THREADS / WAVE;
constexpr int TASK_E = 256;  // source leaves per task

struct P2PTask {
  int64_t e0, e1;  // slice of the target leaf's list
  int64_t part;    // first partial slot, or -1 when the task is the leaf's only one
  int32_t leaf;    // target leaf node
  int32_t pad;
};

__device__ __forceinline__ double p2p_rsqrt(double x) {
  // hardware estimate (relative error ~2^-24) + one Newton step
  // y <- y + (y/2)(1 - x y^2): relative error ~(3/2) e^2 < 1e-14, far below the
  // rounding noise of the pair sums at the tolerances the results are held to
  const double y = __builtin_amdgcn_rsq(x);
  const double e = fma(-x * y, y, 1.0);
  return fma(0.5 * y, e, y);
}
// Twice the same Newton-refined value, y (3 - x y^2), in three operations
// instead of four: the forward near field sums with it and scales its sums
// once per target by exact powers of two.
__device__ __forceinline__ double p2p_rsqrt_x2(double x) {
  const double y = __builtin_amdgcn_rsq(x);
  return y * fma(-x * y, y, 3.0);
}
__device__ __forceinline__ float p2p_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

// ---- task construction (build time) ----
__global__ void k_leaf_task_counts(const int32_t* leaves, int64_t n_leaves, const int64_t* off,
                                   const int32_t* count, const int32_t* tr_cnt, int64_t* ntask,
                                   int64_t* npart, int64_t* ntail, int32_t* split, Control* ctrl) {
  bookkeeping_priority();
  __shared__ int oct[ORDER_OCT];
  for (int b = threadIdx.x; b < ORDER_OCT; b += blockDim.x) oct[b] = 0;
  __syncthreads();
  int64_t li = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (li < n_leaves) {
    const int32_t a = leaves[li];
    const int64_t len = off[a + 1] - off[a];
    const int64_t nt = len <= TASK_E ? 1 : (len + TASK_E - 1) / TASK_E;
    ntask[li] = nt;
    npart[li] = nt > 1 ? nt * (int64_t)count[a] : 0;
    ntail[li] = ((int64_t)tr_cnt[a] + TAIL_E - 1) / TAIL_E;
    if (nt > 1) split[atomicAdd(&ctrl->n_split, 1)] = (int32_t)li;  // for the combine
    // launch-order octaves of the leaf's tasks: nt - 1 full ones and the last
    const uint64_t c = (uint64_t)count[a];
    if (nt > 1) atomicAdd(&oct[work_octave(c * TASK_E)], (int)(nt - 1));
    atomicAdd(&oct[work_octave(c * (uint64_t)(len - (nt - 1) * TASK_E))], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < ORDER_OCT; b += blockDim.x)
    if (oct[b]) atomicAdd(&ctrl->task_oct[b], oct[b]);
}

// One thread per task: find its leaf by binary search over the task offsets.
// Task k (leaf order) is built and placed in launch order: heavier octaves of
// work (targets x source leaves) first, so the longest waves do not start
// last; a block's tasks of one octave stay together, so that tasks running
// together mostly share their sources in L2.  Every task's sums (and its
// partial slots) are independent of where and when it runs.
__global__ void __launch_bounds__(256)
    k_p2p_task_fill(const int32_t* leaves, int64_t n_leaves, int64_t n_tasks,
                    const int64_t* task_off, const int64_t* part_off, const int64_t* off,
                    const int32_t* count, Control* ctrl, P2PTask* tasks) {
  bookkeeping_priority();
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  P2PTask t{};
  int o = -1;
  if (k < n_tasks) {
    int64_t lo = 0, hi = n_leaves;  // last li with task_off[li] <= k
    while (hi - lo > 1) {
      int64_t mid = (lo + hi) >> 1;
      if (task_off[mid] <= k)
        lo = mid;
      else
        hi = mid;
    }
    const int64_t li = lo;
    const int32_t a = leaves[li];
    const int64_t nt = task_off[li + 1] - task_off[li];
    const int64_t kk = k - task_off[li];
    t.e0 = off[a] + kk * TASK_E;
    t.e1 = min(off[a + 1], t.e0 + TASK_E);
    t.part = nt > 1 ? part_off[li] + kk * (int64_t)count[a] : -1;
    t.leaf = a;
    t.pad = 0;
    o = work_octave((uint64_t)count[a] * (uint64_t)(t.e1 - t.e0));
  }
  const int64_t slot = octave_slot<ORDER_OCT>(o, ctrl->task_oct, ctrl->task_cur);
  if (k < n_tasks && slot >= 0 && slot < n_tasks) tasks[slot] = t;
}


// ---- near-field sums ----
constexpr int TILE = 2 * WAVE;       // source particles staged per round

typedef __attribute__((address_space(1))) void p2p_gvoid_t;
typedef __attribute__((address_space(3))) void p2p_lvoid_t;
// one 16-byte piece of a source record in LDS
struct alignas(16) Piece16 {
  uint64_t a, b;
};

// Pair interactions.  Each adds one source's contribution to the four
// per-target sums that the task writes.
//
// Forward: potential and acceleration of target i from source j.
// In fp64 the pair uses z = 2/|r| (p2p_rsqrt_x2), so the sums are 2 phi and
// 8 a; the task scales them by S_PHI = 1/2 and S_ACC = 1/8 (exact) once per
// target.  17 vector operations per pair, one of them the quarter-rate
// inverse square root estimate.
template <typename T>
struct ForcePair {
  using Rec = P4<T>;  // x, y, z, m
  static constexpr int MAXQ = 2048;  // source particles per owner table
  static constexpr T S_PHI = sizeof(T) == 8 ? (T)0.5 : (T)1;
  static constexpr T S_ACC = sizeof(T) == 8 ? (T)0.125 : (T)1;
  static __device__ __forceinline__ void add(const Rec& pi, const Rec& pj, T& fp, T& fx, T& fy,
                                             T& fz) {
    const T dx = pi.x - pj.x, dy = pi.y - pj.y, dz = pi.z - pj.z;
    const T r2 = dx * dx + dy * dy + dz * dz;
    T rinv;
    if constexpr (sizeof(T) == 8)
      rinv = p2p_rsqrt_x2(r2);
    else
      rinv = p2p_rsqrt(r2);
    const T mr = pj.m * rinv;
    const T mr3 = mr * rinv * rinv;
    fp -= mr;
    fx -= mr3 * dx;
    fy -= mr3 * dy;
    fz -= mr3 * dz;
  }
};

// VJP: the record of a particle is its position and mass, then the
// sensitivities pb = dS/dphi and ab = dS/da of its outputs.  With r = x_i - x_j
// the pair contributes to
//   Psi(x_i)  = sum_j -pb_j/|r| + ab_j . r/|r|^3                 (dS/dm_i)
//   xbar_i    = sum_j [ s r + w - 3 (r . w) r/|r|^2 ] / |r|^3,
//   s = pb_i m_j + m_i pb_j,   w = m_i ab_j - m_j ab_i,
// which is -pb_i a_i - (Hess Phi) ab_i + m_i grad Psi restricted to the pair:
// the near-field part of the VJP's position gradient.
template <typename T>
struct VjpPair {
  using Rec = P8<T>;
  static constexpr T S_PHI = (T)1, S_ACC = (T)1;
  // a smaller owner table keeps a block of four waves under 40 KB of LDS,
  // so that four blocks fit a compute unit
  static constexpr int MAXQ = 1024;
  static __device__ __forceinline__ void add(const Rec& ti, const Rec& sj, T& ps, T& gx, T& gy,
                                             T& gz) {
    const T dx = ti.p.x - sj.p.x, dy = ti.p.y - sj.p.y, dz = ti.p.z - sj.p.z;
    const T r2 = dx * dx + dy * dy + dz * dz;
    const T rinv = p2p_rsqrt(r2);
    const T rinv2 = rinv * rinv;
    const T rinv3 = rinv * rinv2;
    const T s = ti.c.x * sj.p.m + ti.p.m * sj.c.x;
    const T wx = ti.p.m * sj.c.y - sj.p.m * ti.c.y;
    const T wy = ti.p.m * sj.c.z - sj.p.m * ti.c.z;
    const T wz = ti.p.m * sj.c.m - sj.p.m * ti.c.m;
    const T rw = dx * wx + dy * wy + dz * wz;
    const T coef = s - (T)3 * rw * rinv2;
    gx += rinv3 * (coef * dx + wx);
    gy += rinv3 * (coef * dy + wy);
    gz += rinv3 * (coef * dz + wz);
    const T ad = sj.c.y * dx + sj.c.z * dy + sj.c.m * dz;
    ps += rinv3 * ad - sj.c.x * rinv;
  }
};

// Lane layout for a chunk of tc <= 128 targets: each lane holds two targets
// (2g, 2g + 1), so one source read from LDS serves two pairs.  With
// G = ceil(tc / 2) target pairs and ns = floor(64 / G) source slices, lane
// l < G ns serves pair g = l % G and slice sl = l / G, taking sources sl,
// sl + ns, ...; the few remaining lanes repeat slice 0 of their pair and their
// sums are dropped.  Sources are staged TT = ns floor(128 / ns) at a time, so
// in every full stage each lane takes exactly TT / ns sources.
// The staged source records are kept as NH planes of 16-byte pieces (plane
// h holds bytes 16h .. 16h + 15 of every record): global-to-LDS copies fill
// a plane 64 records at a time, and the lanes reading consecutive records of
// one plane touch consecutive 16-byte slots.
template <typename T, typename Rec, int MAXQ>
struct P2PShared {
  static constexpr int NH = (int)(sizeof(Rec) / 16);
  union {
    Piece16 tile[NH][TILE];
    T red[8][WAVE];
  };
  union {
    uint8_t owner[MAXQ];  // list entry (within the group of 64) of each source particle
    T fin[WAVE];  // after the staging: the targets' sums, one per lane (rounds of <= 16 targets)
  };
  int32_t sbase[WAVE];  // per entry: first particle minus its first source index
};

// The tasks of one wave.  Per target, out1[perm] = far.x + sum0 and
// out3[3 perm + a] = far.(y, z, m)[a] + sum(a + 1); a split leaf writes its
// four sums per task into `part` instead.
// mut (null: none): per leaf, 1 when its sibling group's near field (its own
// leaf and its sibling leaves) is summed by the mutual kernel; those entries
// are then skipped here (parent: the node parents, to recognise siblings).
template <typename T, class Pair>
__device__ __forceinline__ void p2p_tasks(const P2PTask* __restrict__ tasks, int64_t n_tasks,
                                          const int32_t* __restrict__ begin,
                                          const int32_t* __restrict__ count,
                                          const uint8_t* __restrict__ mut,
                                          const int32_t* __restrict__ parent,
                                          const int32_t* __restrict__ src,
                                          const typename Pair::Rec* __restrict__ pts,
                                          const P4<T>* __restrict__ far,
                                          const int32_t* __restrict__ perm, T* __restrict__ out1,
                                          T* __restrict__ out3, T* __restrict__ part,
                                          P2PShared<T, typename Pair::Rec, Pair::MAXQ>& sh) {
  using Rec = typename Pair::Rec;
  constexpr int MAXQ = Pair::MAXQ;
  constexpr int NH = P2PShared<T, Rec, MAXQ>::NH;
  static_assert(sizeof(Rec) == 16 * NH, "records are whole 16-byte pieces");
  auto staged = [&](int s) -> Rec {  // record s of the current stage
    union {
      Rec r;
      Piece16 q[NH];
    } u;
#pragma unroll
    for (int h = 0; h < NH; h++) u.q[h] = sh.tile[h][s];
    return u.r;
  };
  const int lane = __lane_id();
  // fp64: the wave index in a scalar register (fewer vector registers and
  // instructions); the fp32 kernel ran slower with it on the 256^3 lattice
  const int w = sizeof(T) == 8 ? uniform((int)(threadIdx.x / WAVE)) : (int)(threadIdx.x / WAVE);
  for (int64_t ti = (int64_t)blockIdx.x * P2P_WAVES + w; ti < n_tasks;
       ti += (int64_t)gridDim.x * P2P_WAVES) {
    const P2PTask task = tasks[ti];
    const int32_t a = task.leaf;
    const int32_t tb = begin[a], tn = count[a];
    // sibling entries (the leaf itself included) summed by the mutual kernel
    const int32_t skip_par = (mut && mut[a]) ? uniform(parent[a]) : -2;
    for (int32_t t0 = 0; t0 < tn; t0 += 2 * WAVE) {
      const int tc = min(2 * WAVE, tn - t0);
      const int G = (tc + 1) >> 1;
      // small quotients through the hardware reciprocal: each true quotient is
      // at least 0.5 / 64 away from an integer, far above the estimate's error
      const float rg = __builtin_amdgcn_rcpf((float)G);
      const int ns = uniform((int)(((float)WAVE + 0.5f) * rg));  // floor(64 / G)
      const int sl0 = (int)(((float)lane + 0.5f) * rg);          // floor(lane / G)
      const int g = lane - sl0 * G;
      const int sl = sl0 < ns ? sl0 : 0;
      const int per = uniform((int)(((float)TILE + 0.5f) * __builtin_amdgcn_rcpf((float)ns)));
      const int TT = ns * per;
      const int32_t i0 = tb + t0 + 2 * g;
      const bool two = 2 * g + 1 < tc;
      const Rec p0 = pts[i0];
      const Rec p1 = pts[two ? i0 + 1 : i0];
      T a0 = 0, a1 = 0, a2 = 0, a3 = 0, b0 = 0, b1 = 0, b2 = 0, b3 = 0;
      bool self = false;
      for (int64_t eg = task.e0; eg < task.e1;) {
        int32_t sb = 0, sc = 0;
        if (eg + lane < task.e1) {
          const int32_t b = src[eg + lane];
          if (skip_par >= 0 && parent[b] == skip_par) {
            // a sibling leaf or the leaf itself: in the mutual kernel's sums
          } else if (b == a) {
            self = true;  // the target leaf itself: summed below with the self test
          } else {
            sb = begin[b];
            sc = count[b];
          }
        }
        int incl = wave_incl_scan(sc);
        // take the longest prefix of entries whose particles fit the owner table
        // (at least one entry; a single larger one needs no table)
        const int H = max(1, (int)__popcll(__ballot(incl <= MAXQ)));
        const int inclH = __shfl(incl, H - 1, WAVE);
        if (lane >= H) {
          sc = 0;
          incl = inclH;
        }
        const int excl = incl - sc;
        const int tot = __shfl(incl, WAVE - 1, WAVE);
        const bool one = tot > MAXQ;  // one entry, particles sb[0] + q
        sh.sbase[lane] = sb - excl;
        if (!one)
          for (int k = 0; k < sc; k++) sh.owner[excl + k] = (uint8_t)lane;
        __builtin_amdgcn_wave_barrier();
        for (int q0 = 0; q0 < tot; q0 += TT) {
#pragma unroll
          for (int r = 0; r < TILE / WAVE; r++) {
            const int k = r * WAVE + lane;
            const int q = q0 + k;
            if (k < TT && q < tot) {
              // record k of the stage straight into LDS, piece h into plane h
              // (fp64: the record index in 32 bits, particle indices fit an int;
              // the fp32 kernel ran slower on the 256^3 lattice with it)
              const int32_t sbq = sh.sbase[one ? 0 : sh.owner[q]];
              const unsigned char* g = (const unsigned char*)(sizeof(T) == 8 ? pts + (sbq + q)
                                                                             : pts + sbq + q);
#pragma unroll
              for (int h = 0; h < NH; h++)
                __builtin_amdgcn_global_load_lds((p2p_gvoid_t*)(g + 16 * h),
                                                 (p2p_lvoid_t*)&sh.tile[h][r * WAVE], 16, 0, 0);
            }
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the stage has landed in LDS
          __builtin_amdgcn_wave_barrier();
          const int nv = min(TT, tot - q0);
          if (nv == TT) {
            // a full stage: the same number of sources on every lane
            // the trip count is uniform: the counter is kept in a scalar
            // register, so the loop control costs no vector instructions
            const int per_s = __builtin_amdgcn_readfirstlane(per);
            for (int k = 0; k < per_s; k = __builtin_amdgcn_readfirstlane(k + 1)) {
              const Rec pj = staged(sl + k * ns);
              Pair::add(p0, pj, a0, a1, a2, a3);
              Pair::add(p1, pj, b0, b1, b2, b3);
            }
          } else {
            for (int s = sl; s < nv; s += ns) {
              const Rec pj = staged(s);
              Pair::add(p0, pj, a0, a1, a2, a3);
              Pair::add(p1, pj, b0, b1, b2, b3);
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
        eg += H;
      }
      if (__ballot(self) != 0ull) {
        for (int32_t s = sl; s < tn; s += ns) {
          const Rec pj = pts[tb + s];
          if (tb + s != i0) Pair::add(p0, pj, a0, a1, a2, a3);  // self term omitted
          if (tb + s != i0 + 1) Pair::add(p1, pj, b0, b1, b2, b3);
        }
      }
      sh.red[0][lane] = a0;
      sh.red[1][lane] = a1;
      sh.red[2][lane] = a2;
      sh.red[3][lane] = a3;
      sh.red[4][lane] = b0;
      sh.red[5][lane] = b1;
      sh.red[6][lane] = b2;
      sh.red[7][lane] = b3;
      __builtin_amdgcn_wave_barrier();
      // Each target's four sums add its ns slices in slice order; lane pair g
      // holds targets 2g, 2g + 1 (member 4 (l & 1) of red).  Up to 16 targets
      // in the round, the 4 tc sums (target l = v / 4, component c = v % 4)
      // are formed one per lane, so most lanes work, and staged in fin; then
      // one lane per target writes all four.
      const bool spread = tc <= WAVE / 4;
      if (spread) {
        if (lane < 4 * tc) {
          const int l = lane >> 2, c = lane & 3;
          const int gg = l >> 1, m = 4 * (l & 1) + c;
          T sv = 0;
          for (int q = 0; q < ns; q++) sv += sh.red[m][q * G + gg];
          sh.fin[lane] = sv;
        }
        __builtin_amdgcn_wave_barrier();
      }
      for (int l = lane; l < tc; l += WAVE) {
        T s0, s1, s2, s3;
        if (spread) {
          s0 = sh.fin[4 * l];
          s1 = sh.fin[4 * l + 1];
          s2 = sh.fin[4 * l + 2];
          s3 = sh.fin[4 * l + 3];
        } else {
          const int gg = l >> 1, m = 4 * (l & 1);
          s0 = 0, s1 = 0, s2 = 0, s3 = 0;
          for (int q = 0; q < ns; q++) {
            s0 += sh.red[m][q * G + gg];
            s1 += sh.red[m + 1][q * G + gg];
            s2 += sh.red[m + 2][q * G + gg];
            s3 += sh.red[m + 3][q * G + gg];
          }
        }
        s0 *= Pair::S_PHI;  // exact powers of two
        s1 *= Pair::S_ACC;
        s2 *= Pair::S_ACC;
        s3 *= Pair::S_ACC;
        const int32_t i = tb + t0 + l;
        if (task.part < 0) {
          const P4<T> f = far[i];
          const int64_t o = perm[i];
          out1[o] = f.x + s0;
          out3[3 * o] = f.y + s1;
          out3[3 * o + 1] = f.z + s2;
          out3[3 * o + 2] = f.m + s3;
        } else {
          T* pp = part + 4 * (task.part + t0 + l);
          pp[0] = s0;
          pp[1] = s1;
          pp[2] = s2;
          pp[3] = s3;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(P2P_THREADS) __attribute__((amdgpu_waves_per_eu(6, 8)))
    k_p2p(const P2PTask* __restrict__ tasks, int64_t n_tasks, const int32_t* __restrict__ begin,
          const int32_t* __restrict__ count, const uint8_t* __restrict__ mut,
          const int32_t* __restrict__ parent, const int32_t* __restrict__ src,
          const P4<T>* __restrict__ pts, const P4<T>* __restrict__ far,
          const int32_t* __restrict__ perm, T* __restrict__ phi, T* __restrict__ acc,
          T* __restrict__ part) {
  __shared__ P2PShared<T, P4<T>, ForcePair<T>::MAXQ> sh_all[P2P_WAVES];
  const int w = sizeof(T) == 8 ? uniform((int)(threadIdx.x / WAVE)) : (int)(threadIdx.x / WAVE);
  p2p_tasks<T, ForcePair<T>>(tasks, n_tasks, begin, count, mut, parent, src, pts, far, perm, phi,
                             acc, part, sh_all[w]);
}

// VJP near field: out1 = dS/dm, out3 = dS/dx, with `far` holding the far-field
// parts of both (Psi and the position gradient) in sorted order.
template <typename T>
__global__ void __launch_bounds__(P2P_THREADS) __attribute__((amdgpu_waves_per_eu(4, 8)))
    k_p2p_vjp(const P2PTask* __restrict__ tasks, int64_t n_tasks, const int32_t* __restrict__ begin,
              const int32_t* __restrict__ count, const int32_t* __restrict__ src,
              const P8<T>* __restrict__ recs, const P4<T>* __restrict__ far,
              const int32_t* __restrict__ perm, T* __restrict__ mbar, T* __restrict__ xbar,
              T* __restrict__ part) {
  __shared__ P2PShared<T, P8<T>, VjpPair<T>::MAXQ> sh_all[P2P_WAVES];
  const int w = sizeof(T) == 8 ? uniform((int)(threadIdx.x / WAVE)) : (int)(threadIdx.x / WAVE);
  p2p_tasks<T, VjpPair<T>>(tasks, n_tasks, begin, count, nullptr, nullptr, src, recs, far, perm,
                           mbar, xbar, part, sh_all[w]);
}

// ---- mutual near field of sibling groups ----
// The leaf children of one parent are adjacent cells, so every pair of them
// (and every leaf with itself) is a near-field pair in both directions: the
// group's particles U interact all with all.  One wave per parent sums each
// unordered particle pair of U once and adds it to both particles (the pair's
// terms are equal and opposite in the acceleration, equal in the potential),
// in a fixed order, into the far-field records (which L2P has written); the
// directed kernel then skips these entries.  The group's records are staged in
// LDS.  Rows i come in tiles of 16 (lane & 15), four columns j at a time
// (lane >> 4), j > i only: the i-side terms stay in registers and are summed
// over the four lanes of a row at the end of the tile, the j-side terms of one
// column are summed over its 16 lanes by DPP moves inside the row; both go
// into per-particle sums in LDS.  Groups of more than MUT_MAX particles are
// left to the directed kernel.
constexpr int MUT_MAX = 256;

// sum over the 16 lanes of a row; every lane of the row gets it
template <typename T>
__device__ __forceinline__ T sum16(T x) {
  x += dpp_move<DPP_QUAD_XOR1>(x);
  x += dpp_move<DPP_QUAD_XOR2>(x);
  x += dpp_move<DPP_ROW_HALF_MIRROR>(x);
  x += dpp_move<DPP_ROW_MIRROR>(x);
  return x;
}

// Build time: mut[c] = 1 for the leaf children c of parents whose leaf children
// hold 1 .. MUT_MAX particles (a root leaf keeps the 0 it was cleared to).
__global__ void k_mutual_flags(const int32_t* parents, int64_t np, const int32_t* first_child,
                               const uint8_t* n_child, const int32_t* count, uint8_t* mut) {
  bookkeeping_priority();
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= np) return;
  const int32_t X = parents[i], fc = first_child[X];
  const int nc = n_child[X];
  int u = 0;
  for (int c = 0; c < nc; c++)
    if (n_child[fc + c] == 0) u += count[fc + c];
  const uint8_t on = (u > 0 && u <= MUT_MAX) ? 1 : 0;
  for (int c = 0; c < nc; c++)
    if (n_child[fc + c] == 0) mut[fc + c] = on;
}

template <typename T>
__global__ void __launch_bounds__(P2P_THREADS)
    k_p2p_mutual(int64_t np, const int32_t* __restrict__ parents,
                 const int32_t* __restrict__ first_child, const uint8_t* __restrict__ n_child,
                 const int32_t* __restrict__ begin, const int32_t* __restrict__ count,
                 const P4<T>* __restrict__ pts, P4<T>* __restrict__ far) {
  __shared__ P4<T> urec_all[P2P_WAVES][MUT_MAX];
  __shared__ int32_t uidx_all[P2P_WAVES][MUT_MAX];
  __shared__ T acc_all[P2P_WAVES][4][MUT_MAX];
  __shared__ T red_all[P2P_WAVES][4][WAVE];
  const int lane = __lane_id();
  const int w = uniform((int)(threadIdx.x / WAVE));
  P4<T>* urec = urec_all[w];
  int32_t* uidx = uidx_all[w];
  T(*acc)[MUT_MAX] = acc_all[w];
  T(*red)[WAVE] = red_all[w];
  for (int64_t pi = (int64_t)blockIdx.x * P2P_WAVES + w; pi < np;
       pi += (int64_t)gridDim.x * P2P_WAVES) {
    const int32_t X = uniform(parents[pi]);
    const int nc = uniform((int)n_child[X]);
    const int32_t fc = uniform(first_child[X]);
    int lc = 0, lb = 0;
    if (lane < nc && n_child[fc + lane] == 0) {
      lc = count[fc + lane];
      lb = begin[fc + lane];
    }
    const int incl = wave_incl_scan(lc);
    const int u = uniform(read_lane(incl, WAVE - 1));
    if (u == 0 || u > MUT_MAX) continue;
    const int excl = incl - lc;
    // U: the leaf children's particles in child order
    for (int t = 0; t < nc; t++) {
      const int s0 = uniform(read_lane(excl, t)), c0 = uniform(read_lane(lc, t)),
                b0 = uniform(read_lane(lb, t));
      for (int q = lane; q < c0; q += WAVE) {
        urec[s0 + q] = pts[b0 + q];
        uidx[s0 + q] = b0 + q;
      }
    }
    for (int q = lane; q < u; q += WAVE) acc[0][q] = acc[1][q] = acc[2][q] = acc[3][q] = (T)0;
    __builtin_amdgcn_wave_barrier();
    const int ri = lane & 15, g = lane >> 4;
    for (int r0 = 0; r0 < u; r0 += 16) {
      const int i = r0 + ri;
      const P4<T> pi_ = urec[i < u ? i : 0];
      T s0 = 0, s1 = 0, s2 = 0, s3 = 0;  // i side
      for (int j0 = r0; j0 < u; j0 += 4) {
        const int j = j0 + g;
        T v0 = 0, v1 = 0, v2 = 0, v3 = 0;  // j side
        if (i < u && j < u && j > i) {
          const P4<T> pj = urec[j];
          const T dx = pi_.x - pj.x, dy = pi_.y - pj.y, dz = pi_.z - pj.z;
          const T r2 = dx * dx + dy * dy + dz * dz;
          const T rinv = p2p_rsqrt(r2);
          const T rinv2 = rinv * rinv;
          const T mjr = pj.m * rinv, mir = pi_.m * rinv;
          const T mjr3 = mjr * rinv2, mir3 = mir * rinv2;
          s0 -= mjr;
          s1 -= mjr3 * dx;
          s2 -= mjr3 * dy;
          s3 -= mjr3 * dz;
          v0 = -mir;
          v1 = mir3 * dx;
          v2 = mir3 * dy;
          v3 = mir3 * dz;
        }
        v0 = sum16(v0);
        v1 = sum16(v1);
        v2 = sum16(v2);
        v3 = sum16(v3);
        if (ri == 0 && j < u) {
          acc[0][j] += v0;
          acc[1][j] += v1;
          acc[2][j] += v2;
          acc[3][j] += v3;
        }
      }
      red[0][lane] = s0;
      red[1][lane] = s1;
      red[2][lane] = s2;
      red[3][lane] = s3;
      __builtin_amdgcn_wave_barrier();
      if (lane < 16 && i < u) {
#pragma unroll
        for (int c = 0; c < 4; c++)
          acc[c][i] += ((red[c][lane] + red[c][lane + 16]) + red[c][lane + 32]) + red[c][lane + 48];
      }
      __builtin_amdgcn_wave_barrier();
    }
    for (int q = lane; q < u; q += WAVE) {
      P4<T> f = far[uidx[q]];
      f.x += acc[0][q];
      f.y += acc[1][q];
      f.z += acc[2][q];
      f.m += acc[3][q];
      far[uidx[q]] = f;
    }
    __builtin_amdgcn_wave_barrier();  // the stage and sums are read before the next group
  }
}

// Leaves split over several tasks, one block per leaf: thread (t, s) adds the
// partials of tasks s, s + nsl, ... of target t in order, then the nsl slices
// of each target are added in slice order.
constexpr int CB_THREADS = 256;

template <typename T>
__global__ void __launch_bounds__(CB_THREADS)
    k_p2p_combine(const int32_t* leaves, const int32_t* split, int64_t n_split,
                  const int64_t* task_off,
                  const int64_t* part_off, const int32_t* begin, const int32_t* count,
                  const T* part, const P4<T>* far, const int32_t* perm, T* phi, T* acc) {
  __shared__ T red[4][CB_THREADS];
  for (int64_t j = blockIdx.x; j < n_split; j += gridDim.x) {  // the split leaves only
    const int64_t li = split[j];
    const int64_t nt = task_off[li + 1] - task_off[li];
    const int32_t a = leaves[li];
    const int32_t tn = count[a], tb = begin[a];
    for (int32_t t0 = 0; t0 < tn; t0 += CB_THREADS) {
      const int tc = min(CB_THREADS, tn - t0);
      const int nsl = CB_THREADS / tc;
      const int t = threadIdx.x % tc, sl = threadIdx.x / tc;
      T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
      if (sl < nsl) {
        for (int64_t k = sl; k < nt; k += nsl) {
          const T* pp = part + 4 * (part_off[li] + k * tn + t0 + t);
          s0 += pp[0];
          s1 += pp[1];
          s2 += pp[2];
          s3 += pp[3];
        }
      }
      red[0][threadIdx.x] = s0;
      red[1][threadIdx.x] = s1;
      red[2][threadIdx.x] = s2;
      red[3][threadIdx.x] = s3;
      __syncthreads();
      if ((int)threadIdx.x < tc) {
        T r0 = 0, r1 = 0, r2 = 0, r3 = 0;
        for (int s = 0; s < nsl; s++) {
          r0 += red[0][s * tc + threadIdx.x];
          r1 += red[1][s * tc + threadIdx.x];
          r2 += red[2][s * tc + threadIdx.x];
          r3 += red[3][s * tc + threadIdx.x];
        }
        const int32_t i = tb + t0 + threadIdx.x;
        const P4<T> f = far[i];
        const int64_t o = perm[i];
        phi[o] = f.x + r0;
        acc[3 * o] = f.y + r1;
        acc[3 * o + 1] = f.z + r2;
        acc[3 * o + 2] = f.m + r3;
      }
      __syncthreads();
    }
  }
}

size_t p2p_task_bytes() { return sizeof(P2PTask); }

hipError_t launch_leaf_task_counts(const int32_t* leaves, int64_t n_leaves, const int64_t* off,
                                   const int32_t* count, const int32_t* tr_cnt, int64_t* ntask,
                                   int64_t* npart, int64_t* ntail, int32_t* split, Control* ctrl,
                                   hipStream_t st) {
  if (n_leaves == 0) return hipSuccess;
  k_leaf_task_counts<<<(unsigned)((n_leaves + 255) / 256), 256, 0, st>>>(
      leaves, n_leaves, off, count, tr_cnt, ntask, npart, ntail, split, ctrl);
  return hipGetLastError();
}

hipError_t launch_p2p_task_fill(const int32_t* leaves, int64_t n_leaves, int64_t n_tasks,
                                const int64_t* task_off, const int64_t* part_off,
                                const int64_t* off, const int32_t* count, Control* ctrl,
                                void* tasks, hipStream_t st) {
  if (n_tasks == 0) return hipSuccess;
  const unsigned g = (unsigned)((n_tasks + 255) / 256);
  k_p2p_task_fill<<<g, 256, 0, st>>>(leaves, n_leaves, n_tasks, task_off, part_off, off, count,
                                     ctrl, (P2PTask*)tasks);
  return hipGetLastError();
}

hipError_t launch_mutual_flags(const int32_t* parents, int64_t np, const int32_t* first_child,
                               const uint8_t* n_child, const int32_t* count, uint8_t* mut,
                               int64_t n_nodes, hipStream_t st) {
  hipError_t e = launch_fill_zero(mut, (size_t)n_nodes, st);
  if (e != hipSuccess || np <= 0) return e;
  k_mutual_flags<<<(unsigned)((np + 255) / 256), 256, 0, st>>>(parents, np, first_child, n_child,
                                                               count, mut);
  return hipGetLastError();
}

hipError_t launch_p2p_mutual(int dtype, int64_t np, const int32_t* parents,
                             const int32_t* first_child, const uint8_t* n_child,
                             const int32_t* begin, const int32_t* count, const void* pts,
                             void* far, hipStream_t st) {
  if (np <= 0) return hipSuccess;
  int64_t blocks = (np + P2P_WAVES - 1) / P2P_WAVES;
  if (blocks > 65535) blocks = 65535;
  if (dtype == FMM_F64)
    k_p2p_mutual<double><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        np, parents, first_child, n_child, begin, count, (const P4<double>*)pts, (P4<double>*)far);
  else
    k_p2p_mutual<float><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        np, parents, first_child, n_child, begin, count, (const P4<float>*)pts, (P4<float>*)far);
  return hipGetLastError();
}

hipError_t launch_p2p(int dtype, const void* tasks, int64_t n_tasks, const int32_t* leaves,
                      int64_t n_leaves, const int64_t* task_off, const int64_t* part_off,
                      const int32_t* begin, const int32_t* count, const uint8_t* mut,
                      const int32_t* parent, const int32_t* src,
                      const void* pts, const void* far, const int32_t* perm, void* phi, void* acc,
                      void* part, const int32_t* split, int64_t n_split, hipEvent_t* ev, bool* ran,
                      hipStream_t st) {
  // ev (optional): begin/end of the pair kernel, then of the combine
  if (n_tasks == 0) return hipSuccess;
  int64_t blocks = (n_tasks + P2P_WAVES - 1) / P2P_WAVES;
  if (blocks > 65535) blocks = 65535;
  const int64_t cblocks = n_split < 65535 ? n_split : 65535;
  if (ev) (void)hipEventRecord(ev[0], st);
  if (dtype == FMM_F64)
    k_p2p<double><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        (const P2PTask*)tasks, n_tasks, begin, count, mut, parent, src, (const P4<double>*)pts,
        (const P4<double>*)far, perm, (double*)phi, (double*)acc, (double*)part);
  else
    k_p2p<float><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        (const P2PTask*)tasks, n_tasks, begin, count, mut, parent, src, (const P4<float>*)pts,
        (const P4<float>*)far, perm, (float*)phi, (float*)acc, (float*)part);
  if (ev) {
    (void)hipEventRecord(ev[1], st);
    ran[0] = true;
  }
  if (n_split > 0) {
    if (ev) (void)hipEventRecord(ev[2], st);
    if (dtype == FMM_F64)
      k_p2p_combine<double><<<(unsigned)cblocks, CB_THREADS, 0, st>>>(
          leaves, split, n_split, task_off, part_off, begin, count, (const double*)part,
          (const P4<double>*)far, perm, (double*)phi, (double*)acc);
    else
      k_p2p_combine<float><<<(unsigned)cblocks, CB_THREADS, 0, st>>>(
          leaves, split, n_split, task_off, part_off, begin, count, (const float*)part,
          (const P4<float>*)far, perm, (float*)phi, (float*)acc);
    if (ev) {
      (void)hipEventRecord(ev[3], st);
      ran[1] = true;
    }
  }
  return hipGetLastError();
}

hipError_t launch_p2p_vjp(int dtype, const void* tasks, int64_t n_tasks, const int32_t* leaves,
                          int64_t n_leaves, const int64_t* task_off, const int64_t* part_off,
                          const int32_t* begin, const int32_t* count, const int32_t* src,
                          const void* recs, const void* far, const int32_t* perm, void* mbar,
                          void* xbar, void* part, const int32_t* split, int64_t n_split,
                          hipEvent_t* ev, bool* ran, hipStream_t st) {
  // ev (optional): begin/end of the pair kernel
  if (n_tasks == 0) return hipSuccess;
  int64_t blocks = (n_tasks + P2P_WAVES - 1) / P2P_WAVES;
  if (blocks > 65535) blocks = 65535;
  const int64_t cblocks = n_split < 65535 ? n_split : 65535;
  if (ev) (void)hipEventRecord(ev[0], st);
  if (dtype == FMM_F64)
    k_p2p_vjp<double><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        (const P2PTask*)tasks, n_tasks, begin, count, src, (const P8<double>*)recs,
        (const P4<double>*)far, perm, (double*)mbar, (double*)xbar, (double*)part);
  else
    k_p2p_vjp<float><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        (const P2PTask*)tasks, n_tasks, begin, count, src, (const P8<float>*)recs,
        (const P4<float>*)far, perm, (float*)mbar, (float*)xbar, (float*)part);
  if (ev) {
    (void)hipEventRecord(ev[1], st);
    ran[0] = true;
  }
  if (n_split > 0) {
    // the split leaves' partials: the same ordered combine as the forward
    if (dtype == FMM_F64)
      k_p2p_combine<double><<<(unsigned)cblocks, CB_THREADS, 0, st>>>(
          leaves, split, n_split, task_off, part_off, begin, count, (const double*)part,
          (const P4<double>*)far, perm, (double*)mbar, (double*)xbar);
    else
      k_p2p_combine<float><<<(unsigned)cblocks, CB_THREADS, 0, st>>>(
          leaves, split, n_split, task_off, part_off, begin, count, (const float*)part,
          (const P4<float>*)far, perm, (float*)mbar, (float*)xbar);
  }
  return hipGetLastError();
}

}  // namespace mbg
