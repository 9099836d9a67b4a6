// fmm_m2l.hip -- batched Cartesian multipole-to-local translation.
//
// jz-fmm project page, "Calculating a node-node interaction": with R = c_A - c_B
// the translation needs only the source moments and R (the page prints the
// monopole and dipole terms of Phi_B(c_A) and grad Phi_B(c_A)).  Taylor-
// expanding -m_j / |R + dx - s_j| in dx and s_j gives, for total degree p,
//     L_n(A) += - sum_{|m| <= p - |n|} Mt_m(B) D^(n+m)(R),
//     Mt_m = (-1)^|m| M_m / m!,   D^k = d^k (1/|R|).
// The derivative tensor D is built on chip for every pair from R alone (no
// operator is streamed from memory), by the recurrence for derivatives of
// f(|r|^2/2): with F_j = d^j f/du^j,
//     R^(j)_(k+e_x) = x R^(j+1)_k + k_x R^(j+1)_(k-e_x)   (same for y, z),
//     R^(j)_0 = F_j = (-1)^j (2j-1)!! / |r|^(2j+1),   D^k = R^(0)_k.
//
// The translation runs in its traceless form: since D is harmonic
// (D_(k+2x) + D_(k+2y) + D_(k+2z) = 0), the moment components with m_z >= 2
// are folded once per node onto m_z <= 1 (same degree, so the truncation is
// unchanged), the pair loop forms L_n for n_z <= 1 only, and the L_n with
// n_z >= 2 follow from L_n = -L_(n-2z+2x) - L_(n-2z+2y).  At order 4 that is
// 155 terms per pair instead of 210 (1365 instead of 3003 at order 8); the
// result equals the full sum up to rounding.
//
// Every summation runs in a fixed order (fixed butterflies, no atomics), so
// results do not depend on scheduling.
#include <algorithm>

#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int M2L_THREADS = 256;

// 1/sqrt(x) in fp64: hardware estimate refined by one step of the cubically
// convergent iteration y <- y (1 + e/2 + 3e^2/8), e = 1 - x y^2 (the series of
// (1 - e)^(-1/2)); the estimate's relative error ~2^-22 becomes < 2^-60.
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  double e = fma(-x * y, y, 1.0);
  return fma(y * e, fma(e, 0.375, 0.5), y);
}
__device__ __forceinline__ float rsqrt_any(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ double rsqrt_any(double x) { return rsqrt_f64(x); }

// Sum over the 8 lanes 8t .. 8t + 7 by DPP moves inside the row: pairs, then
// quads, then the two quads (half mirror); all 8 lanes get the same value.
template <typename T>
__device__ __forceinline__ T sum8(T x) {
  x += dpp_move<DPP_QUAD_XOR1>(x);
  x += dpp_move<DPP_QUAD_XOR2>(x);
  x += dpp_move<DPP_ROW_HALF_MIRROR>(x);
  return x;
}

// ---------------- source records ----------------
// Thread per node: fold the moments (components with m_z >= 2 onto m_z - 2,
// largest z first) and store the (P+1)^2 remaining ones with the centre.
template <typename T, int P>
__global__ void k_m2l_records(int64_t n_nodes, const double* __restrict__ centre,
                              const T* __restrict__ mpole, unsigned char* __restrict__ mred) {
  constexpr int K = Tabs<P>::K, KR = HTabs<P>::KR;
  constexpr int RB = mrec_bytes(KR, sizeof(T)), CB = mrec_centre_byte(KR, sizeof(T));
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n_nodes) return;
  T M[K];
#pragma unroll
  for (int k = 0; k < K; k++) M[k] = mpole[i * K + k];
  static_for<0, HTabs<P>::NF>([&](auto fc) {
    constexpr int f = decltype(fc)::value;
    M[htabs<P>.fd[f]] -= M[htabs<P>.fs[f]];
  });
  T* out = (T*)(mred + i * RB);
  static_for<0, KR>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    out[r] = M[htabs<P>.rfull[r]];
  });
  double* c = (double*)(mred + i * RB + CB);
  c[0] = centre[3 * i];
  c[1] = centre[3 * i + 1];
  c[2] = centre[3 * i + 2];
}

// reduced accumulators (n_z <= 1) -> all K coefficients, by the harmonic relation
template <typename T, int P>
__device__ __forceinline__ void unfold_locals(const T (&acc)[HTabs<P>::KR], T (&L)[Tabs<P>::K]) {
  static_for<0, HTabs<P>::KR>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    L[htabs<P>.rfull[r]] = acc[r];
  });
  static_for<0, HTabs<P>::NRC>([&](auto ec) {
    constexpr int e = decltype(ec)::value;
    L[htabs<P>.rd[e]] = -L[htabs<P>.r1[e]] - L[htabs<P>.r2[e]];
  });
}

// ---------------- sibling blocks ----------------
// The children of one parent receive the same candidates, so their own sources
// are the union U of the candidates any child accepts (built with the walk,
// each entry carrying an 8-bit mask of the accepting children).  One wave per
// parent: lane l = 8 t + j pairs child slot t with source slot j of a chunk of
// 8 union entries.  The chunk's source records (moments + centre) are copied
// from HBM straight into LDS by 16-byte global-to-LDS loads, NS chunks ahead in
// a ring, so no registers hold data in flight and each record is read once for
// up to 8 children.  Each lane keeps the partial local expansion of child t
// over its source slot; the 8 slots are summed by a fixed butterfly at the end
// and the children's locals are written (not added).
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

template <typename T, int P>
struct SibCfg {
  // waves per SIMD the register budget is cut for: two at order 6 (256
  // registers, a few spilled, instead of 284 and one wave)
  static constexpr int WPE = P == 6 && sizeof(T) == 8 ? 2 : 1;
  static constexpr int KR = HTabs<P>::KR;
  static constexpr int RB = mrec_bytes(KR, sizeof(T));       // record bytes
  static constexpr int CB = mrec_centre_byte(KR, sizeof(T)); // centre offset in a record
  static constexpr int PC = RB / 16;                        // 16-byte pieces per record
  static constexpr int NI = (8 * PC + WAVE - 1) / WAVE;     // copy instructions per chunk
  static constexpr int SB = NI * WAVE * 16;                 // ring stage bytes
  static constexpr int NS = NI <= 3 ? 3 : 2;                // ring depth (chunks)
  static constexpr int WIN = 256;                           // union entries per id window
  static constexpr int WAIT = (NS - 1) * NI;                // copies allowed in flight
};

// Derivatives D_k of 1/|r| up to total degree P (graded layout) and the
// traceless contraction acc[n] += Mt[m] D[n+m] together: the recurrence levels
// j = P .. 1 first, then every final derivative (level 0) is formed and used at
// once by the terms that read it, so the D table is never live as a whole.
// Every index is a compile-time constant: all of it stays in registers, and
// derivatives no term reads (k_z > 2) are never formed.
template <typename T, int P>
__device__ __forceinline__ void dtensor_contract(T x, T y, T z, const T* Ms,
                                                 T (&acc)[HTabs<P>::KR]) {
  constexpr int NR = Tabs<P>::NR;
  constexpr int R0 = tabs<P>.roff[0];  // level 0: the final derivatives
  const T r2 = x * x + y * y + z * z;
  const T rinv = rsqrt_any(r2);
  const T rinv2 = rinv * rinv;
  T g[P + 1];
  g[0] = rinv;
#pragma unroll
  for (int j = 0; j < P; j++) g[j + 1] = (T)(-(2 * j + 1)) * g[j] * rinv2;
  T R[NR];
  static_for<0, NR>([&](auto ec) {
    constexpr int e = decltype(ec)::value;
    constexpr int ax = tabs<P>.raxis[e];
    T v;
    if constexpr (ax < 0) {
      v = g[tabs<P>.rlev[e]];
    } else {
      const T u = ax == 0 ? x : (ax == 1 ? y : z);
      constexpr int s1 = tabs<P>.rs1[e];
      constexpr int s2 = tabs<P>.rs2[e];
      if constexpr (s2 >= 0)
        v = u * R[s1] + (T)tabs<P>.rc2[e] * R[s2];
      else
        v = u * R[s1];
    }
    R[e] = v;
    if constexpr (e >= R0) {  // a final derivative: its terms now
      constexpr int k = e - R0;
      static_for<htabs<P>.ko[k], htabs<P>.ko[k + 1]>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        acc[htabs<P>.kn[q]] += Ms[htabs<P>.km[q]] * v;
      });
    }
  });
}

template <typename T, int P>
__global__ void __launch_bounds__(M2L_THREADS) __attribute__((amdgpu_waves_per_eu(SibCfg<T, P>::WPE, 8)))
    k_m2l_sib(int64_t n_parents, const int32_t* __restrict__ parents,
              const int32_t* __restrict__ first_child, const uint8_t* __restrict__ n_child,
              const uint64_t* __restrict__ upool, const int64_t* __restrict__ u_off,
              const int32_t* __restrict__ u_cnt, const double* __restrict__ centre,
              const unsigned char* __restrict__ mrec, T* __restrict__ local,
              const Control* __restrict__ stop) {
  // after a pool overflow the unions are incomplete: the walk is repeated
  if (stop && stop->pool_overflow) return;
  using C = SibCfg<T, P>;
  constexpr int K = Tabs<P>::K, KR = C::KR;
  constexpr int WPB = M2L_THREADS / WAVE;
  __shared__ __attribute__((aligned(16))) unsigned char ring[WPB][C::NS][C::SB];
  __shared__ int32_t wid[WPB][C::WIN];
  __shared__ uint8_t wmk[WPB][C::WIN];
  // the wave index in a scalar register (fewer vector registers and
  // instructions), except at orders 7 and 8, where it raised the spills
  const int lane = __lane_id(),
            w = P <= 6 ? uniform((int)(threadIdx.x / WAVE)) : (int)(threadIdx.x / WAVE);
  const int t = lane >> 3, j = lane & 7;
  // this lane's piece of each copy instruction: record slot ps (8 = padding) and piece pq
  int ps[C::NI], pq[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; i++) {
    const int f = WAVE * i + lane;
    ps[i] = f < 8 * C::PC ? f / C::PC : 8;
    pq[i] = f < 8 * C::PC ? f - (f / C::PC) * C::PC : 0;
  }
  for (int64_t pi = (int64_t)blockIdx.x * WPB + w; pi < n_parents;
       pi += (int64_t)gridDim.x * WPB) {
    // wave-uniform values are moved to scalar registers so that the loop
    // conditions below are uniform branches
    const int32_t par = uniform(parents[pi]);
    const int nc = uniform((int)n_child[par]);
    const int64_t ch = (int64_t)uniform(first_child[par]) + t;
    double cx = 0.0, cy = 0.0, cz = 0.0;
    if (t < nc) {
      cx = centre[3 * ch];
      cy = centre[3 * ch + 1];
      cz = centre[3 * ch + 2];
    }
    const int64_t u0 = uniform(u_off[par]), u1 = u0 + uniform(u_cnt[par]);
    T acc[KR];
#pragma unroll
    for (int k = 0; k < KR; k++) acc[k] = (T)0;
    for (int64_t w0 = u0; w0 < u1; w0 += C::WIN) {
      const int n = (int)min((int64_t)C::WIN, u1 - w0);
      const int nch = (n + 7) >> 3;
      // id window, padded to whole chunks with (node 0, empty mask)
      for (int e = lane; e < 8 * nch; e += WAVE) {
        int32_t id = 0;
        uint8_t mk = 0;
        if (e < n) {
          const uint64_t v = upool[w0 + e];
          id = (int32_t)(v >> 8);
          mk = (uint8_t)(v & 0xff);
        }
        wid[w][e] = id;
        wmk[w][e] = mk;
      }
      __builtin_amdgcn_wave_barrier();
      // copy chunk c into ring stage c % NS; chunks past the end copy node 0's
      // record into the free stage, so every step issues the same NI copies
      auto issue = [&](int c) {
        unsigned char* stage = ring[w][c % C::NS];
        const int cc = min(c, nch - 1);
#pragma unroll
        for (int i = 0; i < C::NI; i++) {
          int64_t node = 0;
          if (c < nch && ps[i] < 8) node = wid[w][8 * cc + ps[i]];
          const unsigned char* g = mrec + node * C::RB + 16 * pq[i];
          __builtin_amdgcn_global_load_lds((gvoid_t*)g, (lvoid_t*)(stage + i * WAVE * 16), 16, 0,
                                           0);
        }
      };
#pragma unroll
      for (int c = 0; c < C::NS - 1; c++) issue(c);
      for (int c = 0; c < nch; c++) {
        issue(c + C::NS - 1);
        // copies complete in issue order: at most WAIT newer ones may remain
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::WAIT) : "memory");
        const unsigned char* rec = ring[w][c % C::NS] + j * C::RB;
        const uint32_t m = wmk[w][8 * c + j];
        if ((m >> t) & 1u) {
          const double* cs = (const double*)(rec + C::CB);
          const T rx = (T)(cx - cs[0]), ry = (T)(cy - cs[1]), rz = (T)(cz - cs[2]);
          dtensor_contract<T, P>(rx, ry, rz, (const T*)rec, acc);
        }
        asm volatile("" ::: "memory");  // this stage is read before it is refilled
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // padding copies land before reuse
    }
#pragma unroll
    for (int r = 0; r < KR; r++) {
      T x = acc[r];
      x = sum8(x);
      acc[r] = -x;  // G = 1: L = -sum
    }
    T L[K];
    unfold_locals<T, P>(acc, L);
    T* Lc = local + ch * K;
    static_for<0, K>([&](auto nc_) {
      constexpr int n = decltype(nc_)::value;
      if (t < nc && (n & 7) == j) Lc[n] = L[n];
    });
  }
}

// ---------------- transposed tails ----------------
// A leaf's transposed entries (a run of the sorted transposed keys) come from
// deeper targets that accepted it; their lengths vary widely (0 to thousands),
// so they are cut into tasks of at most TAIL_E entries.  A wave takes 8
// consecutive tasks: lane l = 8 t + j walks entries j, j + 8, ... of task t, the
// 8 lanes of a task are summed by a fixed butterfly and the task's partial
// local is stored; a second kernel subtracts each leaf's task partials, in task
// order, from its local.
template <typename T, int P>
__global__ void __launch_bounds__(M2L_THREADS)
    k_m2l_tail(int64_t n_tasks, const TailTask* __restrict__ tasks,
               const int32_t* __restrict__ leaves, const uint64_t* __restrict__ keys,
               uint64_t src_mask, const double* __restrict__ centre,
               const unsigned char* __restrict__ mrec, T* __restrict__ part) {
  constexpr int K = Tabs<P>::K, KR = HTabs<P>::KR;
  constexpr int RB = mrec_bytes(KR, sizeof(T));
  constexpr int CB = mrec_centre_byte(KR, sizeof(T));
  const int lane = __lane_id();
  const int t = lane >> 3, j = lane & 7;
  const int64_t wid = (int64_t)blockIdx.x * (M2L_THREADS / WAVE) + threadIdx.x / WAVE;
  const int64_t nw = (int64_t)gridDim.x * (M2L_THREADS / WAVE);
  for (int64_t g = wid; 8 * g < n_tasks; g += nw) {
    const int64_t ti = 8 * g + t;
    int n = 0;
    int64_t e0 = 0, a = 0;
    if (ti < n_tasks) {
      const TailTask tk = tasks[ti];
      n = tk.n;
      e0 = tk.e0;
      a = leaves[tk.li];
    }
    const double ax = ti < n_tasks ? centre[3 * a] : 0.0;
    const double ay = ti < n_tasks ? centre[3 * a + 1] : 0.0;
    const double az = ti < n_tasks ? centre[3 * a + 2] : 0.0;
    T acc[KR];
#pragma unroll
    for (int k = 0; k < KR; k++) acc[k] = (T)0;
    // software pipeline (when the registers allow: low orders): the next
    // entry's record is loaded while the current one is used, and the key
    // after it one step earlier still
    constexpr bool PIPE = KR * sizeof(T) <= 200;
    T Mn[KR];
    double cn[3];
    auto load_rec = [&](uint64_t key) {
      const unsigned char* rb = mrec + (int64_t)(key & src_mask) * RB;
      const T* Mb = (const T*)rb;
#pragma unroll
      for (int k = 0; k < KR; k++) Mn[k] = Mb[k];
      const double* cb = (const double*)(rb + CB);
      cn[0] = cb[0];
      cn[1] = cb[1];
      cn[2] = cb[2];
    };
    if constexpr (PIPE) {
      uint64_t knext = j + 8 < n ? keys[e0 + j + 8] : 0ull;
      if (j < n) load_rec(keys[e0 + j]);
      for (int e = j; e < n; e += 8) {
        T M[KR];
#pragma unroll
        for (int k = 0; k < KR; k++) M[k] = Mn[k];
        const T rx = (T)(ax - cn[0]), ry = (T)(ay - cn[1]), rz = (T)(az - cn[2]);
        if (e + 8 < n) load_rec(knext);
        if (e + 16 < n) knext = keys[e0 + e + 16];
        dtensor_contract<T, P>(rx, ry, rz, M, acc);
      }
    } else {
      for (int e = j; e < n; e += 8) {
        load_rec(keys[e0 + e]);
        const T rx = (T)(ax - cn[0]), ry = (T)(ay - cn[1]), rz = (T)(az - cn[2]);
        dtensor_contract<T, P>(rx, ry, rz, Mn, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < KR; r++) {
      T x = acc[r];
      x = sum8(x);
      acc[r] = x;
    }
    T S[K];
    unfold_locals<T, P>(acc, S);  // the relation is linear: it holds for partial sums too
    T* Pt = part + ti * K;
    static_for<0, K>([&](auto nc) {
      constexpr int q = decltype(nc)::value;
      if (ti < n_tasks && (q & 7) == j) Pt[q] = S[q];
    });
  }
}

// thread per (leaf, coefficient): L -= sum of the leaf's task partials, in order
template <typename T>
__global__ void k_m2l_tail_combine(int64_t n_leaves, int K, const int32_t* __restrict__ leaves,
                                   const int64_t* __restrict__ toff, const T* __restrict__ part,
                                   T* __restrict__ local) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= n_leaves * K) return;
  const int64_t li = g / K;
  const int n = (int)(g - li * K);
  const int64_t t0 = toff[li], t1 = toff[li + 1];
  if (t0 == t1) return;
  T s = (T)0;
  for (int64_t q = t0; q < t1; q++) s += part[q * K + n];
  local[(int64_t)leaves[li] * K + n] -= s;
}


__global__ void k_tail_fill(const int32_t* leaves, int64_t n_leaves, const int64_t* tr_start,
                            const int32_t* tr_cnt, const int64_t* toff, TailTask* tasks) {
  bookkeeping_priority();
  const int64_t li = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (li >= n_leaves) return;
  const int64_t a = leaves[li];
  if (tr_cnt[a] == 0) return;
  const int64_t e0 = tr_start[a], e1 = e0 + tr_cnt[a];
  int64_t q = toff[li];
  for (int64_t e = e0; e < e1; e += TAIL_E, q++)
    tasks[q] = TailTask{e, (int32_t)min((int64_t)TAIL_E, e1 - e), (int32_t)li};
}


hipError_t launch_tail_fill(const int32_t* leaves, int64_t n_leaves, const int64_t* tr_start,
                            const int32_t* tr_cnt, const int64_t* toff, TailTask* tasks,
                            hipStream_t st) {
  if (n_leaves <= 0) return hipSuccess;
  k_tail_fill<<<(unsigned)((n_leaves + 255) / 256), 256, 0, st>>>(leaves, n_leaves, tr_start,
                                                                   tr_cnt, toff, tasks);
  return hipGetLastError();
}

// Launch order of the sibling blocks: longer unions (by octave) first, so that
// the longest waves do not start last; a stable sort keeps id order inside an
// octave, so that blocks running together mostly share source records in L2.
// Each parent's result does not depend on when it runs.
// Launch order of the sibling M2L groups: longer unions first (octaves of the
// union length), each block's groups of one octave together.
__global__ void __launch_bounds__(256) k_group_octaves(const int32_t* parents, int64_t np,
                                                       const int32_t* u_cnt, Control* ctrl) {
  __shared__ int oct[ORDER_OCT];
  for (int b = threadIdx.x; b < ORDER_OCT; b += blockDim.x) oct[b] = 0;
  __syncthreads();
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < np) atomicAdd(&oct[work_octave((uint64_t)(uint32_t)u_cnt[parents[i]])], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < ORDER_OCT; b += blockDim.x)
    if (oct[b]) atomicAdd(&ctrl->group_oct[b], oct[b]);
}
__global__ void __launch_bounds__(256) k_group_place(const int32_t* parents, int64_t np,
                                                     const int32_t* u_cnt, Control* ctrl,
                                                     int32_t* order) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int o = i < np ? work_octave((uint64_t)(uint32_t)u_cnt[parents[i]]) : -1;
  const int64_t slot = octave_slot<ORDER_OCT>(o, ctrl->group_oct, ctrl->group_cur);
  if (i < np && slot >= 0 && slot < np) order[slot] = parents[i];
}

hipError_t launch_m2l_order(const int32_t* parents, int64_t np, const int32_t* u_cnt,
                            Control* ctrl, int32_t* order, hipStream_t st) {
  if (np <= 0) return hipSuccess;
  const unsigned g = (unsigned)((np + 255) / 256);
  k_group_octaves<<<g, 256, 0, st>>>(parents, np, u_cnt, ctrl);
  k_group_place<<<g, 256, 0, st>>>(parents, np, u_cnt, ctrl, order);
  return hipGetLastError();
}

template <typename T>
static void records_dispatch(int order, unsigned g, hipStream_t st, int64_t n, const double* c,
                             const T* m, unsigned char* r) {
  switch (order) {
#define REC_CASE(P) \
  case P:           \
    k_m2l_records<T, P><<<g, 256, 0, st>>>(n, c, m, r); \
    break;
    REC_CASE(0) REC_CASE(1) REC_CASE(2) REC_CASE(3) REC_CASE(4)
    REC_CASE(5) REC_CASE(6) REC_CASE(7) REC_CASE(8) REC_CASE(9) REC_CASE(10)
#undef REC_CASE
    default:
      break;
  }
}

hipError_t launch_m2l_records(int dtype, int order, int64_t n_nodes, const double* centre,
                              const void* mpole, void* mred, hipStream_t st) {
  if (n_nodes <= 0) return hipSuccess;
  const unsigned g = (unsigned)((n_nodes + 255) / 256);
  if (dtype == FMM_F64)
    records_dispatch<double>(order, g, st, n_nodes, centre, (const double*)mpole,
                             (unsigned char*)mred);
  else
    records_dispatch<float>(order, g, st, n_nodes, centre, (const float*)mpole,
                            (unsigned char*)mred);
  return hipGetLastError();
}

static unsigned m2l_grid(int64_t waves) {
  int64_t blocks = (waves + (M2L_THREADS / WAVE) - 1) / (M2L_THREADS / WAVE);
  if (blocks > 65535) blocks = 65535;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

template <typename T>
static void m2l_sib_dispatch(int order, hipStream_t st, const M2LArgs& a) {
  unsigned gs = m2l_grid(a.n_parents);
  if (a.max_blocks > 0 && (int64_t)gs > a.max_blocks) gs = (unsigned)a.max_blocks;
  const unsigned char* rec = (const unsigned char*)a.mrec;
  if (a.n_parents <= 0) return;
  // a.ev (optional): begin/end events of the sibling kernel
  if (a.ev) (void)hipEventRecord(a.ev[0], st);
  switch (order) {
#define M2L_SIB(P)                                                                           \
  case P:                                                                                    \
    k_m2l_sib<T, P><<<gs, M2L_THREADS, 0, st>>>(a.n_parents, a.parents, a.first_child,        \
                                                a.n_child, a.upool, a.u_off, a.u_cnt,        \
                                                a.centre, rec, (T*)a.local, a.stop);         \
    break;
    M2L_SIB(0) M2L_SIB(1) M2L_SIB(2) M2L_SIB(3) M2L_SIB(4)
    M2L_SIB(5) M2L_SIB(6) M2L_SIB(7) M2L_SIB(8) M2L_SIB(9) M2L_SIB(10)
#undef M2L_SIB
    default:
      break;
  }
  if (a.ev) {
    (void)hipEventRecord(a.ev[1], st);
    a.ran[0] = true;
  }
}

template <typename T>
static void m2l_tail_dispatch(int order, hipStream_t st, const M2LArgs& a, bool combine) {
  if (a.n_tasks <= 0) return;
  const unsigned gt = m2l_grid((a.n_tasks + 7) / 8);
  const unsigned char* rec = (const unsigned char*)a.mrec;
  // a.ev (optional): begin/end events of the tail kernel
  if (a.ev) (void)hipEventRecord(a.ev[0], st);
  switch (order) {
#define M2L_TAIL(P)                                                                          \
  case P:                                                                                    \
    k_m2l_tail<T, P><<<gt, M2L_THREADS, 0, st>>>(a.n_tasks, a.tasks, a.leaves, a.keys,        \
                                                 a.src_mask, a.centre, rec, (T*)a.part);     \
    break;
    M2L_TAIL(0) M2L_TAIL(1) M2L_TAIL(2) M2L_TAIL(3) M2L_TAIL(4)
    M2L_TAIL(5) M2L_TAIL(6) M2L_TAIL(7) M2L_TAIL(8) M2L_TAIL(9) M2L_TAIL(10)
#undef M2L_TAIL
    default:
      break;
  }
  if (a.ev) {
    (void)hipEventRecord(a.ev[1], st);
    a.ran[0] = true;
  }
  if (combine) {
    const int K = ncoef(order);
    const unsigned g = (unsigned)((a.n_leaves * K + 255) / 256);
    k_m2l_tail_combine<T><<<g, 256, 0, st>>>(a.n_leaves, K, a.leaves, a.toff,
                                             (const T*)a.part, (T*)a.local);
  }
}

hipError_t launch_m2l_sib(int dtype, int order, const M2LArgs& a, hipStream_t st) {
  if (a.n_nodes <= 0) return hipSuccess;
  // the root is nobody's child: its local (no far-field terms) is cleared
  const size_t kb = (size_t)ncoef(order) * (dtype == FMM_F64 ? 8 : 4);
  hipError_t e = launch_fill_zero(a.local, kb, st);
  if (e != hipSuccess) return e;
  if (dtype == FMM_F64)
    m2l_sib_dispatch<double>(order, st, a);
  else
    m2l_sib_dispatch<float>(order, st, a);
  return hipGetLastError();
}

hipError_t launch_m2l_tails(int dtype, int order, const M2LArgs& a, bool combine,
                            hipStream_t st) {
  if (dtype == FMM_F64)
    m2l_tail_dispatch<double>(order, st, a, combine);
  else
    m2l_tail_dispatch<float>(order, st, a, combine);
  return hipGetLastError();
}

}  // namespace mbg
