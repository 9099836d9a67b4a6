// fmm_expand.hip -- upward and downward passes: P2M, M2M, L2L, L2P.
//
// jz-fmm project page:
//   * "Describing the source and the receiving region": Cartesian mass moments
//     about the cell centre (M = sum m, M1 = sum m s, M2 = sum m s s, higher
//     moments alike) and the local Taylor polynomial about the receiving
//     centre, whose gradient gives a = -grad Phi;
//   * "Combining near and far interactions": leaf moments, children's moments
//     translated to the parent centre, parents' locals translated to the
//     children, then evaluated at the particles.
//
// Storage convention (this library's choice): the moment array holds the
// scaled moments Mt_m = (-1)^|m| M_m / m! -- with it the translation of a child
// to its parent is Mt_m(P) = sum_{k<=m} Mt_k(child) (-d)^(m-k)/(m-k)!, d =
// c_child - c_P, and the multipole-to-local step becomes a plain contraction.
// The local array holds the derivatives L_n = d^n Phi at the cell centre.
#include <algorithm>
#include <type_traits>

#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int MAXK = ncoef(FMM_MAX_ORDER);

struct MiTable {
  int8_t a[MAXK], b[MAXK], c[MAXK];
};
__constant__ MiTable c_mi;

static constexpr MiTable make_table() {
  MiTable t{};
  int k = 0;
  for (int d = 0; d <= FMM_MAX_ORDER; d++)
    for (int a = d; a >= 0; a--)
      for (int b = d - a; b >= 0; b--) {
        t.a[k] = (int8_t)a;
        t.b[k] = (int8_t)b;
        t.c[k] = (int8_t)(d - a - b);
        k++;
      }
  return t;
}

static hipError_t ensure_table() {
  static bool done = false;
  if (done) return hipSuccess;
  static const MiTable t = make_table();
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(c_mi), &t, sizeof(t));
  if (e == hipSuccess) done = true;
  return e;
}

__constant__ double c_inv_int[FMM_MAX_ORDER + 2] = {0.0,        1.0,       0.5,       1.0 / 3.0,
                                                     0.25,       0.2,       1.0 / 6.0, 1.0 / 7.0,
                                                     0.125,      1.0 / 9.0, 0.1,       1.0 / 11.0};

// x^n / n!
__device__ __forceinline__ double pow_over_fact(double x, int n) {
  double r = 1.0;
  for (int i = 1; i <= n; i++) r = r * x * c_inv_int[i];
  return r;
}

constexpr int EX_THREADS = 256;
constexpr int EX_WAVES = EX_THREADS / WAVE;
constexpr int PP = FMM_MAX_ORDER + 1;  // entries of a 1-d power table
constexpr int MAXCH = 8;
constexpr int KSLOTS = (MAXK + WAVE - 1) / WAVE;  // coefficients per lane in the wave-per-leaf kernels

// ---------------- register-resident variants ----------------
// Used wherever they beat the wave-per-node kernels further down: P2M, M2M
// and L2L up to order 8 in fp64 (at order 8 M2M and L2L spill some registers
// and are still 3.4x and 2.2x faster, measured on the 256^3 lattice), up to 6
// in fp32 (the fp32 instances spill from 7 on), the one-launch downward pass
// and the dipole P2M up to 6.
// P2M, one thread per leaf: the leaf's particles are read in order and every
// scaled moment is accumulated in registers.
template <typename T, int P>
__global__ void __launch_bounds__(256)
    k_p2m_reg(const P4<T>* pts, const int32_t* leaves, int64_t n_leaves, const int32_t* begin,
              const int32_t* count, const double* centre, T* mpole) {
  constexpr int K = Tabs<P>::K;
  constexpr int RS = K;  // moments stored densely
  const int64_t li = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (li >= n_leaves) return;
  const int32_t node = leaves[li];
  const double cx = centre[3 * node], cy = centre[3 * node + 1], cz = centre[3 * node + 2];
  double acc[K];
#pragma unroll
  for (int k = 0; k < K; k++) acc[k] = 0.0;
  const int32_t j0 = begin[node], j1 = j0 + count[node];
  for (int32_t j = j0; j < j1; j++) {
    const P4<T> p = pts[j];
    const double sx = cx - (double)p.x, sy = cy - (double)p.y, sz = cz - (double)p.z;  // -s
    double px[P + 1], py[P + 1], pz[P + 1];
    px[0] = (double)p.m;  // the mass rides on the x table
    py[0] = pz[0] = 1.0;
#pragma unroll
    for (int q = 1; q <= P; q++) {
      px[q] = px[q - 1] * sx * (1.0 / q);
      py[q] = py[q - 1] * sy * (1.0 / q);
      pz[q] = pz[q - 1] * sz * (1.0 / q);
    }
    static_for<0, K>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      acc[k] += px[tabs<P>.a[k]] * py[tabs<P>.b[k]] * pz[tabs<P>.c[k]];
    });
  }
  T* out = mpole + (int64_t)node * RS;
#pragma unroll
  for (int k = 0; k < K; k++) out[k] = (T)acc[k];
}

// M2M, eight lanes per parent: lane c translates child c to the parent centre
// (Mt_m += Mt_k(child) (-d)^(m-k)/(m-k)!, all in registers), then the eight
// lanes are added by a fixed butterfly and lane c writes coefficients c, c+8, ...
template <int P>
struct M2MTab {
  static constexpr int NT = binom_c(P + 6, 6);
  int m[NT], k[NT], ea[NT], eb[NT], ec[NT];
  int nt;
  constexpr M2MTab() : m(), k(), ea(), eb(), ec(), nt(0) {
    constexpr int K = (P + 1) * (P + 2) * (P + 3) / 6;
    int t = 0;
    for (int mi = 0; mi < K; mi++)
      for (int ki = 0; ki < K; ki++) {
        int ma = tabs<P>.a[mi], mb = tabs<P>.b[mi], mc = tabs<P>.c[mi];
        int ka = tabs<P>.a[ki], kb = tabs<P>.b[ki], kc = tabs<P>.c[ki];
        if (ka <= ma && kb <= mb && kc <= mc) {
          m[t] = mi;
          k[t] = ki;
          ea[t] = ma - ka;
          eb[t] = mb - kb;
          ec[t] = mc - kc;
          t++;
        }
      }
    nt = t;
  }
};
template <int P>
inline constexpr M2MTab<P> m2m_tab{};

// Parent pi of a level (nodes lvl_begin .. lvl_begin + lvl_count - 1) on a
// group of 8 lanes, lane c shifting child c; the children's terms are summed
// by shuffles inside the group, so all 8 lanes take part.
template <typename T, int P>
__device__ __forceinline__ void m2m_group(int64_t pi, int c, int64_t lvl_begin, int64_t lvl_count,
                                          const int32_t* first_child, const uint8_t* n_child,
                                          const double* centre, T* mpole) {
  constexpr int K = Tabs<P>::K;
  constexpr int RS = K;  // moments stored densely
  constexpr int NTM = m2m_tab<P>.nt;
  const bool valid_p = pi < lvl_count;
  const int64_t Pn = lvl_begin + (valid_p ? pi : 0);
  const int nc = valid_p ? n_child[Pn] : 0;
  double acc[K];
#pragma unroll
  for (int k = 0; k < K; k++) acc[k] = 0.0;
  if (c < nc) {
    const int64_t ch = first_child[Pn] + c;
    const double nx = centre[3 * Pn] - centre[3 * ch], ny = centre[3 * Pn + 1] - centre[3 * ch + 1],
                 nz = centre[3 * Pn + 2] - centre[3 * ch + 2];  // -d
    double px[P + 1], py[P + 1], pz[P + 1];
    px[0] = py[0] = pz[0] = 1.0;
#pragma unroll
    for (int q = 1; q <= P; q++) {
      px[q] = px[q - 1] * nx * (1.0 / q);
      py[q] = py[q - 1] * ny * (1.0 / q);
      pz[q] = pz[q - 1] * nz * (1.0 / q);
    }
    const T* Mc = mpole + ch * RS;
    double M[K];
#pragma unroll
    for (int k = 0; k < K; k++) M[k] = (double)Mc[k];
    static_for<0, NTM>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      acc[m2m_tab<P>.m[t]] += M[m2m_tab<P>.k[t]] * (px[m2m_tab<P>.ea[t]] * py[m2m_tab<P>.eb[t]] *
                                                    pz[m2m_tab<P>.ec[t]]);
    });
  }
#pragma unroll
  for (int k = 0; k < K; k++) {
    double v = acc[k];
    v += __shfl_xor(v, 1, WAVE);
    v += __shfl_xor(v, 2, WAVE);
    v += __shfl_xor(v, 4, WAVE);
    acc[k] = v;
  }
  if (valid_p && nc > 0) {
    T* out = mpole + Pn * RS;
    static_for<0, K>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if ((k & 7) == c) out[k] = (T)acc[k];
    });
  }
}

template <typename T, int P>
__global__ void __launch_bounds__(256)
    k_m2m_reg(int64_t lvl_begin, int64_t lvl_count, const int32_t* first_child,
              const uint8_t* n_child, const double* centre, T* mpole) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  m2m_group<T, P>(g >> 3, (int)(g & 7), lvl_begin, lvl_count, first_child, n_child, centre,
                  mpole);
}

// The top of the tree, where each level has few parents, in one block: level
// by level up to the root, a block barrier between levels (a level's moments
// are read by the next one up).  One launch instead of one per level, whose
// fixed cost exceeds these levels' work.
constexpr int64_t M2M_TOP_MAX = 64;  // parents per level taken by the one-block pass
template <int P>
constexpr int m2m_top_threads() { return P <= 4 ? 512 : 256; }  // as the registers allow
struct M2MLevels {
  int64_t off[MAX_LEVELS + 1];
};
template <typename T, int P>
__global__ void __launch_bounds__(m2m_top_threads<P>())
    k_m2m_top(M2MLevels lv, int l_top, const int32_t* first_child, const uint8_t* n_child,
              const double* centre, T* mpole) {
  constexpr int G = m2m_top_threads<P>() / 8;  // parents per round
  for (int l = l_top; l >= 0; l--) {
    const int64_t b = lv.off[l], cnt = lv.off[l + 1] - b;
    for (int64_t p0 = 0; p0 < cnt; p0 += G)
      m2m_group<T, P>(p0 + threadIdx.x / 8, (int)(threadIdx.x & 7), b, cnt, first_child, n_child,
                      centre, mpole);
    __syncthreads();
  }
}

// L2L, one thread per child: L_n(child) += sum_{|n|+|k|<=p} L_(n+k)(parent) d^k/k!.
template <int P>
struct L2LTab {
  static constexpr int NT = binom_c(P + 6, 6);
  int n[NT], src[NT], ka[NT], kb[NT], kc[NT];
  constexpr L2LTab() : n(), src(), ka(), kb(), kc() {
    constexpr int K = (P + 1) * (P + 2) * (P + 3) / 6;
    int t = 0;
    for (int ni = 0; ni < K; ni++)
      for (int ki = 0; ki < K; ki++)
        if (tabs<P>.d[ni] + tabs<P>.d[ki] <= P) {
          n[t] = ni;
          src[t] = mi_index(tabs<P>.a[ni] + tabs<P>.a[ki], tabs<P>.b[ni] + tabs<P>.b[ki],
                            tabs<P>.c[ni] + tabs<P>.c[ki]);
          ka[t] = tabs<P>.a[ki];
          kb[t] = tabs<P>.b[ki];
          kc[t] = tabs<P>.c[ki];
          t++;
        }
  }
};
template <int P>
inline constexpr L2LTab<P> l2l_tab{};

template <typename T, int P>
__global__ void __launch_bounds__(256)
    k_l2l_reg(int64_t lvl_begin, int64_t lvl_count, const int32_t* parent, const double* centre,
              T* local, const uint8_t* skip_leaves) {
  constexpr int K = Tabs<P>::K;
  constexpr int NTL = L2LTab<P>::NT;
  const int64_t ci = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (ci >= lvl_count) return;
  const int64_t a = lvl_begin + ci;
  if (skip_leaves && skip_leaves[a] == 0) return;  // (n_child given: leaves are complete)
  const int64_t Pn = parent[a];
  const double dx = centre[3 * a] - centre[3 * Pn], dy = centre[3 * a + 1] - centre[3 * Pn + 1],
               dz = centre[3 * a + 2] - centre[3 * Pn + 2];
  double px[P + 1], py[P + 1], pz[P + 1];
  px[0] = py[0] = pz[0] = 1.0;
#pragma unroll
  for (int q = 1; q <= P; q++) {
    px[q] = px[q - 1] * dx * (1.0 / q);
    py[q] = py[q - 1] * dy * (1.0 / q);
    pz[q] = pz[q - 1] * dz * (1.0 / q);
  }
  const T* Lp = local + Pn * K;
  T* Lc = local + a * K;
  double L[K], acc[K];
#pragma unroll
  for (int k = 0; k < K; k++) {
    L[k] = (double)Lp[k];
    acc[k] = (double)Lc[k];
  }
  static_for<0, NTL>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    acc[l2l_tab<P>.n[t]] += L[l2l_tab<P>.src[t]] *
                            (px[l2l_tab<P>.ka[t]] * py[l2l_tab<P>.kb[t]] * pz[l2l_tab<P>.kc[t]]);
  });
#pragma unroll
  for (int k = 0; k < K; k++) Lc[k] = (T)acc[k];
}

// Downward pass for orders <= 6, one thread per leaf: Taylor shifts of a
// degree-p polynomial are exact and compose, so the leaf's local is the sum of
// its own M2L local (own entries, minus the sum of its transposed-tail task
// partials in task order) and of every ancestor's M2L local shifted straight
// to the leaf centre (leaf first, then up to the root; the same sums as the
// level-by-level pass in another association).  `local` is only read; the
// result goes to out[leaf], so one launch replaces one launch per level.
template <typename T, int P>
__global__ void __launch_bounds__(256)
    k_l2l_pull(const int32_t* leaves, int64_t n_leaves, const int32_t* parent,
               const double* centre, const T* local, const int64_t* toff, const T* part,
               T* out) {
  constexpr int K = Tabs<P>::K;
  constexpr int NTL = L2LTab<P>::NT;
  const int64_t li = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (li >= n_leaves) return;
  const int64_t a = leaves[li];
  const T* La = local + a * K;
  double acc[K];
  if (toff && toff[li + 1] > toff[li]) {
    T s[K];
#pragma unroll
    for (int k = 0; k < K; k++) s[k] = (T)0;
    for (int64_t q = toff[li]; q < toff[li + 1]; q++) {
#pragma unroll
      for (int k = 0; k < K; k++) s[k] += part[q * K + k];
    }
#pragma unroll
    for (int k = 0; k < K; k++) acc[k] = (double)(La[k] - s[k]);
  } else {
#pragma unroll
    for (int k = 0; k < K; k++) acc[k] = (double)La[k];
  }
  const double cx = centre[3 * a], cy = centre[3 * a + 1], cz = centre[3 * a + 2];
  // ancestor q's M2L local, its centre and its parent
  auto fetch = [&](int64_t q, double (&L)[K], double (&c)[3], int64_t& up) {
    const T* Lq = local + q * K;
#pragma unroll
    for (int k = 0; k < K; k++) L[k] = (double)Lq[k];
    c[0] = centre[3 * q];
    c[1] = centre[3 * q + 1];
    c[2] = centre[3 * q + 2];
    up = parent[q];
  };
  // add L shifted from the centre c to the leaf centre
  auto shift_add = [&](const double (&L)[K], const double (&c)[3]) {
    const double dx = cx - c[0], dy = cy - c[1], dz = cz - c[2];
    double px[P + 1], py[P + 1], pz[P + 1];
    px[0] = py[0] = pz[0] = 1.0;
#pragma unroll
    for (int r = 1; r <= P; r++) {
      px[r] = px[r - 1] * dx * (1.0 / r);
      py[r] = py[r - 1] * dy * (1.0 / r);
      pz[r] = pz[r - 1] * dz * (1.0 / r);
    }
    static_for<0, NTL>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      acc[l2l_tab<P>.n[t]] += L[l2l_tab<P>.src[t]] *
                              (px[l2l_tab<P>.ka[t]] * py[l2l_tab<P>.kb[t]] * pz[l2l_tab<P>.kc[t]]);
    });
  };
  // parent first, up to the root.  In fp64 up to order 4 the next ancestor's
  // data is loaded while the current one is shifted (two register sets: the
  // chain of dependent loads up the tree overlaps the arithmetic; 10^6
  // clustered particles: 67 -> 50 us).  Above order 4 the second set would
  // spill, and in fp32 it ran 8 % slower.
  double LA[K], cA[3];
  int64_t upA = -1;
  int64_t q = parent[a];
  if constexpr (P <= 4 && sizeof(T) == 8) {
    double LB[K], cB[3];
    int64_t upB = -1;
    if (q >= 0) fetch(q, LA, cA, upA);
    while (q >= 0) {
      const int64_t q1 = upA;
      if (q1 >= 0) fetch(q1, LB, cB, upB);
      shift_add(LA, cA);
      if (q1 < 0) break;
      const int64_t q2 = upB;
      if (q2 >= 0) fetch(q2, LA, cA, upA);
      shift_add(LB, cB);
      q = q2;
    }
  } else {
    for (; q >= 0; q = upA) {
      fetch(q, LA, cA, upA);
      shift_add(LA, cA);
    }
  }
  T* Oa = out + a * K;
#pragma unroll
  for (int k = 0; k < K; k++) Oa[k] = (T)acc[k];
}

// dst row r = src row r for the listed rows (row_bytes a multiple of 4)
__global__ void k_copy_rows(const int32_t* rows, int64_t n, int64_t words, const uint32_t* src,
                            uint32_t* dst) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= n * words) return;
  const int64_t i = g / words, w = g - i * words;
  const int64_t r = rows[i];
  dst[r * words + w] = src[r * words + w];
}

hipError_t launch_copy_rows(const int32_t* rows, int64_t n, int64_t row_bytes, const void* src,
                            void* dst, hipStream_t st) {
  const int64_t words = row_bytes / 4;
  if (n <= 0 || words <= 0) return hipSuccess;
  const int64_t tot = n * words;
  k_copy_rows<<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(rows, n, words,
                                                             (const uint32_t*)src, (uint32_t*)dst);
  return hipGetLastError();
}

template <typename T>
static bool l2l_pull_dispatch(int order, const int32_t* leaves, int64_t n_leaves,
                              const int32_t* parent, const double* centre, const void* local,
                              const int64_t* toff, const void* part, void* out, hipStream_t st) {
  const unsigned g = (unsigned)((n_leaves + 255) / 256);
  switch (order) {
#define L2LP(P)                                                                              \
  case P:                                                                                    \
    k_l2l_pull<T, P><<<g, 256, 0, st>>>(leaves, n_leaves, parent, centre, (const T*)local,    \
                                        toff, (const T*)part, (T*)out);                      \
    return true;
    L2LP(0) L2LP(1) L2LP(2) L2LP(3) L2LP(4) L2LP(5) L2LP(6)
#undef L2LP
    default:
      return false;
  }
}

bool launch_l2l_pull(int dtype, int order, const int32_t* leaves, int64_t n_leaves,
                     const int32_t* parent, const double* centre, const void* local,
                     const int64_t* toff, const void* part, void* out, hipStream_t st) {
  if (order > 6) return false;
  if (n_leaves <= 0) return true;
  return dtype == FMM_F64 ? l2l_pull_dispatch<double>(order, leaves, n_leaves, parent, centre,
                                                      local, toff, part, out, st)
                          : l2l_pull_dispatch<float>(order, leaves, n_leaves, parent, centre,
                                                     local, toff, part, out, st);
}

template <typename T>
static bool l2l_reg_dispatch(int order, int64_t lvl_begin, int64_t lvl_count, const int32_t* parent,
                             const double* centre, void* local, const uint8_t* skip_leaves,
                             hipStream_t st) {
  unsigned g = (unsigned)((lvl_count + 255) / 256);
  switch (order) {
#define L2LR(P)                                                                             \
  case P:                                                                                   \
    k_l2l_reg<T, P><<<g, 256, 0, st>>>(lvl_begin, lvl_count, parent, centre, (T*)local,     \
                                       skip_leaves);                                        \
    return true;
    L2LR(0) L2LR(1) L2LR(2) L2LR(3) L2LR(4) L2LR(5) L2LR(6)
#undef L2LR
    case 7:  // fp64 only
    case 8:
      if constexpr (std::is_same<T, double>::value) {
        if (order == 7)
          k_l2l_reg<T, 7><<<g, 256, 0, st>>>(lvl_begin, lvl_count, parent, centre, (T*)local,
                                             skip_leaves);
        else
          k_l2l_reg<T, 8><<<g, 256, 0, st>>>(lvl_begin, lvl_count, parent, centre, (T*)local,
                                             skip_leaves);
        return true;
      }
      return false;
    default:
      return false;
  }
}

template <typename T>
static bool p2m_reg_dispatch(int order, const void* pts, const int32_t* leaves, int64_t n_leaves,
                             const int32_t* begin, const int32_t* count, const double* centre,
                             void* mpole, hipStream_t st) {
  unsigned g = (unsigned)((n_leaves + 255) / 256);
  switch (order) {
#define P2MR(P)                                                                                  \
  case P:                                                                                        \
    k_p2m_reg<T, P><<<g, 256, 0, st>>>((const P4<T>*)pts, leaves, n_leaves, begin, count, centre, \
                                       (T*)mpole);                                               \
    return true;
    P2MR(0) P2MR(1) P2MR(2) P2MR(3) P2MR(4) P2MR(5) P2MR(6)
#undef P2MR
    case 7:
    case 8:  // fp64 only
      if constexpr (std::is_same<T, double>::value) {
        if (order == 7)
          k_p2m_reg<T, 7><<<g, 256, 0, st>>>((const P4<T>*)pts, leaves, n_leaves, begin, count,
                                             centre, (T*)mpole);
        else
          k_p2m_reg<T, 8><<<g, 256, 0, st>>>((const P4<T>*)pts, leaves, n_leaves, begin, count,
                                             centre, (T*)mpole);
        return true;
      }
      return false;
    default:
      return false;
  }
}

template <typename T>
static bool m2m_reg_dispatch(int order, int64_t lvl_begin, int64_t lvl_count,
                             const int32_t* first_child, const uint8_t* n_child,
                             const double* centre, void* mpole, hipStream_t st) {
  unsigned g = (unsigned)((lvl_count * 8 + 255) / 256);
  switch (order) {
#define M2MR(P)                                                                       \
  case P:                                                                             \
    k_m2m_reg<T, P><<<g, 256, 0, st>>>(lvl_begin, lvl_count, first_child, n_child, centre, \
                                       (T*)mpole);                                    \
    return true;
    M2MR(0) M2MR(1) M2MR(2) M2MR(3) M2MR(4) M2MR(5) M2MR(6)
#undef M2MR
    case 7:  // fp64 only
    case 8:
      if constexpr (std::is_same<T, double>::value) {
        if (order == 7)
          k_m2m_reg<T, 7><<<g, 256, 0, st>>>(lvl_begin, lvl_count, first_child, n_child, centre,
                                             (T*)mpole);
        else
          k_m2m_reg<T, 8><<<g, 256, 0, st>>>(lvl_begin, lvl_count, first_child, n_child, centre,
                                             (T*)mpole);
        return true;
      }
      return false;
    default:
      return false;
  }
}

template <typename T>
static bool m2m_top_dispatch(int order, const M2MLevels& lv, int l_top,
                             const int32_t* first_child, const uint8_t* n_child,
                             const double* centre, void* mpole, hipStream_t st) {
  switch (order) {
#define M2MT(P)                                                                          \
  case P:                                                                                \
    k_m2m_top<T, P><<<1, m2m_top_threads<P>(), 0, st>>>(lv, l_top, first_child, n_child, \
                                                        centre, (T*)mpole);              \
    return true;
    M2MT(0) M2MT(1) M2MT(2) M2MT(3) M2MT(4) M2MT(5) M2MT(6)
#undef M2MT
    case 7:  // fp64 only
    case 8:
      if constexpr (std::is_same<T, double>::value) {
        if (order == 7)
          k_m2m_top<T, 7><<<1, m2m_top_threads<7>(), 0, st>>>(lv, l_top, first_child, n_child,
                                                              centre, (T*)mpole);
        else
          k_m2m_top<T, 8><<<1, m2m_top_threads<8>(), 0, st>>>(lv, l_top, first_child, n_child,
                                                              centre, (T*)mpole);
        return true;
      }
      return false;
    default:
      return false;
  }
}

// ---------------- P2M: one wave per leaf, lanes over coefficients ----------------
// Particles are staged 64 at a time: lane j tabulates (-s_j)^a / a! per axis in
// LDS, then lane m accumulates m_j * ex[a] ey[b] ez[c] over the staged particles
// in particle order.
template <typename T>
__global__ void __launch_bounds__(EX_THREADS)
    k_p2m(int order, int K, const P4<T>* pts, const int32_t* leaves, int64_t n_leaves,
          const int32_t* begin, const int32_t* count, const double* centre, T* mpole) {
  __shared__ double tab[EX_WAVES][WAVE][3][PP];
  __shared__ double ms[EX_WAVES][WAVE];
  const int lane = __lane_id(), w = threadIdx.x / WAVE;
  for (int64_t li = (int64_t)blockIdx.x * EX_WAVES + w; li < n_leaves;
       li += (int64_t)gridDim.x * EX_WAVES) {
    const int32_t node = leaves[li];
    const double c[3] = {centre[3 * node], centre[3 * node + 1], centre[3 * node + 2]};
    double acc[KSLOTS] = {};  // coefficients lane, lane + 64, ...
    const int32_t j0 = begin[node], j1 = j0 + count[node];
    for (int32_t jb = j0; jb < j1; jb += WAVE) {
      const int nj = min(WAVE, j1 - jb);
      if (lane < nj) {
        const P4<T> p = pts[jb + lane];
        const double xs[3] = {c[0] - (double)p.x, c[1] - (double)p.y, c[2] - (double)p.z};
        for (int ax = 0; ax < 3; ax++) {
          double v = 1.0;
          tab[w][lane][ax][0] = 1.0;
          for (int q = 1; q <= order; q++) {
            v = v * xs[ax] * c_inv_int[q];
            tab[w][lane][ax][q] = v;
          }
        }
        ms[w][lane] = (double)p.m;
      }
      __builtin_amdgcn_wave_barrier();
      for (int r = 0; r < KSLOTS; r++) {
        const int m = lane + WAVE * r;
        if (m >= K) break;
        const int a = c_mi.a[m], b = c_mi.b[m], cc = c_mi.c[m];
        double s = acc[r];
        for (int j = 0; j < nj; j++) s += ms[w][j] * tab[w][j][0][a] * tab[w][j][1][b] * tab[w][j][2][cc];
        acc[r] = s;
      }
      __builtin_amdgcn_wave_barrier();
    }
    for (int r = 0; r < KSLOTS; r++) {
      const int m = lane + WAVE * r;
      if (m < K) mpole[(int64_t)node * K + m] = (T)acc[r];
    }
  }
}

hipError_t launch_p2m(int dtype, int order, const void* pts, const int32_t* leaves,
                      int64_t n_leaves, const int32_t* begin, const int32_t* count,
                      const double* centre, void* mpole, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  if (n_leaves == 0) return hipSuccess;
  if (dtype == FMM_F64 ? p2m_reg_dispatch<double>(order, pts, leaves, n_leaves, begin, count,
                                                  centre, mpole, st)
                       : p2m_reg_dispatch<float>(order, pts, leaves, n_leaves, begin, count,
                                                 centre, mpole, st))
    return hipGetLastError();
  int64_t blocks = std::min<int64_t>((n_leaves + EX_WAVES - 1) / EX_WAVES, 65535);
  if (dtype == FMM_F64)
    k_p2m<double><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, (const P4<double>*)pts, leaves,
                                                            n_leaves, begin, count, centre,
                                                            (double*)mpole);
  else
    k_p2m<float><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, (const P4<float>*)pts, leaves,
                                                           n_leaves, begin, count, centre,
                                                           (float*)mpole);
  return hipGetLastError();
}

// ---------------- M2M: one wave per parent, lanes over coefficients ----------------
// Mt_m(P) = sum_children sum_{k<=m} Mt_k(child) (-d)^(m-k) / (m-k)!, d = c_child - c_P;
// the children's moments and power tables are staged in LDS, children and
// terms are added in a fixed order.
template <typename T>
__global__ void __launch_bounds__(EX_THREADS)
    k_m2m(int order, int K, int64_t lvl_begin, int64_t lvl_count, const int32_t* first_child,
          const uint8_t* n_child, const double* centre, T* mpole) {
  __shared__ double mc[EX_WAVES][MAXCH][ncoef(FMM_MAX_ORDER)];
  __shared__ double tab[EX_WAVES][MAXCH][3][PP];
  const int lane = __lane_id(), w = threadIdx.x / WAVE;
  const int64_t RS = K;
  for (int64_t pi = (int64_t)blockIdx.x * EX_WAVES + w; pi < lvl_count;
       pi += (int64_t)gridDim.x * EX_WAVES) {
    const int64_t P = lvl_begin + pi;
    const int nc = n_child[P];
    if (nc == 0) continue;  // leaf: moments come from P2M
    const int64_t fc = first_child[P];
    for (int q = lane; q < nc * K; q += WAVE) {
      const int ch = q / K, k = q - ch * K;
      mc[w][ch][k] = (double)mpole[(fc + ch) * RS + k];
    }
    if (lane < 3 * nc) {
      const int ch = lane / 3, ax = lane - 3 * ch;
      const double nd = centre[3 * P + ax] - centre[3 * (fc + ch) + ax];  // -d
      double v = 1.0;
      tab[w][ch][ax][0] = 1.0;
      for (int q = 1; q <= order; q++) {
        v = v * nd * c_inv_int[q];
        tab[w][ch][ax][q] = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
    for (int m = lane; m < K; m += WAVE) {
      const int ma = c_mi.a[m], mb = c_mi.b[m], mcc = c_mi.c[m];
      double acc = 0.0;
      for (int ch = 0; ch < nc; ch++)
        for (int i = 0; i <= ma; i++)
          for (int j = 0; j <= mb; j++) {
            const double exy = tab[w][ch][0][ma - i] * tab[w][ch][1][mb - j];
            for (int k = 0; k <= mcc; k++)
              acc += mc[w][ch][mi_index(i, j, k)] * exy * tab[w][ch][2][mcc - k];
          }
      mpole[P * RS + m] = (T)acc;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

static hipError_t launch_m2m_level(int dtype, int order, int64_t lvl_begin, int64_t lvl_count,
                                   const int32_t* first_child, const uint8_t* n_child,
                                   const double* centre, void* mpole, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  if (lvl_count == 0) return hipSuccess;
  if (dtype == FMM_F64 ? m2m_reg_dispatch<double>(order, lvl_begin, lvl_count, first_child,
                                                  n_child, centre, mpole, st)
                       : m2m_reg_dispatch<float>(order, lvl_begin, lvl_count, first_child,
                                                 n_child, centre, mpole, st))
    return hipGetLastError();
  int64_t blocks = std::min<int64_t>((lvl_count + EX_WAVES - 1) / EX_WAVES, 65535);
  if (dtype == FMM_F64)
    k_m2m<double><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, lvl_begin, lvl_count,
                                                            first_child, n_child, centre,
                                                            (double*)mpole);
  else
    k_m2m<float><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, lvl_begin, lvl_count,
                                                           first_child, n_child, centre,
                                                           (float*)mpole);
  return hipGetLastError();
}

hipError_t launch_m2m_levels(int dtype, int order, const int64_t* level_off, int depth,
                             const int32_t* first_child, const uint8_t* n_child,
                             const double* centre, void* mpole, hipStream_t st) {
  // the levels from the root down whose parents all fit the one-block pass
  int l_top = -1;
  while (l_top + 1 < depth && level_off[l_top + 2] - level_off[l_top + 1] <= M2M_TOP_MAX) l_top++;
  for (int l = depth - 1; l > l_top; l--) {
    const hipError_t e = launch_m2m_level(dtype, order, level_off[l], level_off[l + 1] - level_off[l],
                                          first_child, n_child, centre, mpole, st);
    if (e != hipSuccess) return e;
  }
  if (l_top < 0) return hipSuccess;
  M2MLevels lv{};
  for (int l = 0; l <= l_top + 1; l++) lv.off[l] = level_off[l];
  if (dtype == FMM_F64 ? m2m_top_dispatch<double>(order, lv, l_top, first_child, n_child, centre,
                                                  mpole, st)
                       : m2m_top_dispatch<float>(order, lv, l_top, first_child, n_child, centre,
                                                 mpole, st))
    return hipGetLastError();
  for (int l = l_top; l >= 0; l--) {  // orders without register kernels
    const hipError_t e = launch_m2m_level(dtype, order, level_off[l], level_off[l + 1] - level_off[l],
                                          first_child, n_child, centre, mpole, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------- L2L: one wave per child, lanes over coefficients ----------------
// L_n(child) += sum_{|n|+|k|<=p} L_(n+k)(parent) d^k / k!, d = c_child - c_parent
template <typename T>
__global__ void __launch_bounds__(EX_THREADS)
    k_l2l(int order, int K, int64_t lvl_begin, int64_t lvl_count, const int32_t* parent,
          const double* centre, T* local) {
  __shared__ double lp[EX_WAVES][ncoef(FMM_MAX_ORDER)];
  __shared__ double tab[EX_WAVES][3][PP];
  const int lane = __lane_id(), w = threadIdx.x / WAVE;
  for (int64_t ci = (int64_t)blockIdx.x * EX_WAVES + w; ci < lvl_count;
       ci += (int64_t)gridDim.x * EX_WAVES) {
    const int64_t a = lvl_begin + ci;
    const int64_t P = parent[a];
    for (int k = lane; k < K; k += WAVE) lp[w][k] = (double)local[P * K + k];
    if (lane < 3) {
      const double d = centre[3 * a + lane] - centre[3 * P + lane];
      double v = 1.0;
      tab[w][lane][0] = 1.0;
      for (int q = 1; q <= order; q++) {
        v = v * d * c_inv_int[q];
        tab[w][lane][q] = v;
      }
    }
    __builtin_amdgcn_wave_barrier();
    for (int n = lane; n < K; n += WAVE) {
      const int na = c_mi.a[n], nb = c_mi.b[n], nc = c_mi.c[n];
      const int rem = order - (na + nb + nc);
      double acc = 0.0;
      for (int i = 0; i <= rem; i++)
        for (int j = 0; i + j <= rem; j++) {
          const double exy = tab[w][0][i] * tab[w][1][j];
          for (int k = 0; i + j + k <= rem; k++)
            acc += lp[w][mi_index(na + i, nb + j, nc + k)] * exy * tab[w][2][k];
        }
      local[a * K + n] = (T)((double)local[a * K + n] + acc);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_l2l(int dtype, int order, int64_t lvl_begin, int64_t lvl_count,
                      const int32_t* parent, const double* centre, void* local,
                      const uint8_t* skip_leaves, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  if (lvl_count == 0) return hipSuccess;
  if (dtype == FMM_F64 ? l2l_reg_dispatch<double>(order, lvl_begin, lvl_count, parent, centre,
                                                  local, skip_leaves, st)
                       : l2l_reg_dispatch<float>(order, lvl_begin, lvl_count, parent, centre,
                                                 local, skip_leaves, st))
    return hipGetLastError();
  if (skip_leaves) return hipErrorInvalidValue;  // only with the register kernels
  int64_t blocks = std::min<int64_t>((lvl_count + EX_WAVES - 1) / EX_WAVES, 65535);
  if (dtype == FMM_F64)
    k_l2l<double><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, lvl_begin, lvl_count, parent,
                                                            centre, (double*)local);
  else
    k_l2l<float><<<(unsigned)blocks, EX_THREADS, 0, st>>>(order, K, lvl_begin, lvl_count, parent,
                                                           centre, (float*)local);
  return hipGetLastError();
}

// ---------------- L2P: one thread per particle (sorted order) ----------------
// phi = sum_n L_n dx^n / n!,  a_alpha = -sum_{n_alpha >= 1} L_n dx^(n - e_alpha) / (n - e_alpha)!
template <typename T, int P>
__global__ void k_l2p(int64_t n, const P4<T>* pts, const int32_t* leaf_of, const double* centre,
                      const T* local, P4<T>* far) {
  constexpr int K = Tabs<P>::K;
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t leaf = leaf_of[k];
  const P4<T> p = pts[k];
  const T dx = (T)((double)p.x - centre[3 * leaf]);
  const T dy = (T)((double)p.y - centre[3 * leaf + 1]);
  const T dz = (T)((double)p.z - centre[3 * leaf + 2]);
  T px[P + 1], py[P + 1], pz[P + 1];  // x^i / i!
  px[0] = py[0] = pz[0] = (T)1;
#pragma unroll
  for (int i = 1; i <= P; i++) {
    px[i] = px[i - 1] * dx * (T)(1.0 / i);
    py[i] = py[i - 1] * dy * (T)(1.0 / i);
    pz[i] = pz[i - 1] * dz * (T)(1.0 / i);
  }
  const T* L = local + (int64_t)leaf * K;
  T phi = 0, ax = 0, ay = 0, az = 0;
  static_for<0, K>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int a = tabs<P>.a[i], b = tabs<P>.b[i], c = tabs<P>.c[i];
    const T l = L[i];
    phi += l * px[a] * py[b] * pz[c];
    if constexpr (a > 0) ax -= l * px[a - 1] * py[b] * pz[c];
    if constexpr (b > 0) ay -= l * px[a] * py[b - 1] * pz[c];
    if constexpr (c > 0) az -= l * px[a] * py[b] * pz[c - 1];
  });
  P4<T> o;
  o.x = phi;
  o.y = ax;
  o.z = ay;
  o.m = az;
  far[k] = o;
}

template <typename T>
static void l2p_dispatch(int order, unsigned g, hipStream_t st, int64_t n, const P4<T>* pts,
                         const int32_t* leaf_of, const double* centre, const T* local, P4<T>* far) {
  switch (order) {
#define L2P_CASE(P) \
  case P:           \
    k_l2p<T, P><<<g, 256, 0, st>>>(n, pts, leaf_of, centre, local, far); \
    break;
    L2P_CASE(0) L2P_CASE(1) L2P_CASE(2) L2P_CASE(3) L2P_CASE(4)
    L2P_CASE(5) L2P_CASE(6) L2P_CASE(7) L2P_CASE(8) L2P_CASE(9) L2P_CASE(10)
#undef L2P_CASE
    default:
      break;
  }
}

hipError_t launch_l2p(int dtype, int order, int64_t n, const void* pts, const int32_t* leaf_of,
                      const double* centre, const void* local, void* far, hipStream_t st) {
  unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == FMM_F64)
    l2p_dispatch<double>(order, g, st, n, (const P4<double>*)pts, leaf_of, centre,
                         (const double*)local, (P4<double>*)far);
  else
    l2p_dispatch<float>(order, g, st, n, (const P4<float>*)pts, leaf_of, centre,
                        (const float*)local, (P4<float>*)far);
  return hipGetLastError();
}

// ---------------- VJP: sensitivity records, their moments, far-field parts ----------------
// rec[k] = (sorted particle k, its sensitivities pb, ab from the caller's order)
template <typename T>
__global__ void k_vjp_gather(int64_t n, const P4<T>* pts, const int32_t* perm, const T* pb,
                             const T* ab, P8<T>* rec) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int64_t i = perm[k];
  P8<T> r;
  r.p = pts[k];
  r.c.x = pb[i];
  r.c.y = ab[3 * i];
  r.c.z = ab[3 * i + 1];
  r.c.m = ab[3 * i + 2];
  rec[k] = r;
}

hipError_t launch_vjp_gather(int dtype, int64_t n, const void* pts, const int32_t* perm,
                             const void* pb, const void* ab, void* rec, hipStream_t st) {
  const unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == FMM_F64)
    k_vjp_gather<double><<<g, 256, 0, st>>>(n, (const P4<double>*)pts, perm, (const double*)pb,
                                            (const double*)ab, (P8<double>*)rec);
  else
    k_vjp_gather<float><<<g, 256, 0, st>>>(n, (const P4<float>*)pts, perm, (const float*)pb,
                                           (const float*)ab, (P8<float>*)rec);
  return hipGetLastError();
}

// Moments of the sensitivity sources, one wave per leaf, lanes over
// coefficients.  A monopole pb and a point dipole ab at x = c + s (the
// dipole's potential is ab . grad_y G(y - x), G = -1/r) have the scaled
// moments
//   Mt_m = pb (-s)^m / m! + sum_a ab_a (-s)^(m - e_a) / (m - e_a)!,
// so with the staged tables tab[a][q] = (-s_a)^q / q! every term is a product
// of three table entries.
template <typename T>
__global__ void __launch_bounds__(EX_THREADS)
    k_p2m_dip(int order, int K, const P8<T>* rec, const int32_t* leaves, int64_t n_leaves,
              const int32_t* begin, const int32_t* count, const double* centre, T* mpole) {
  __shared__ double tab[EX_WAVES][WAVE][3][PP];
  __shared__ double wq[EX_WAVES][WAVE][4];  // pb, abx, aby, abz
  const int lane = __lane_id(), w = threadIdx.x / WAVE;
  for (int64_t li = (int64_t)blockIdx.x * EX_WAVES + w; li < n_leaves;
       li += (int64_t)gridDim.x * EX_WAVES) {
    const int32_t node = leaves[li];
    const double c[3] = {centre[3 * node], centre[3 * node + 1], centre[3 * node + 2]};
    double acc[KSLOTS] = {};  // coefficients lane, lane + 64, ...
    const int32_t j0 = begin[node], j1 = j0 + count[node];
    for (int32_t jb = j0; jb < j1; jb += WAVE) {
      const int nj = min(WAVE, j1 - jb);
      if (lane < nj) {
        const P8<T> r = rec[jb + lane];
        const double xs[3] = {c[0] - (double)r.p.x, c[1] - (double)r.p.y, c[2] - (double)r.p.z};
        for (int ax = 0; ax < 3; ax++) {
          double v = 1.0;
          tab[w][lane][ax][0] = 1.0;
          for (int q = 1; q <= order; q++) {
            v = v * xs[ax] * c_inv_int[q];
            tab[w][lane][ax][q] = v;
          }
        }
        wq[w][lane][0] = (double)r.c.x;
        wq[w][lane][1] = (double)r.c.y;
        wq[w][lane][2] = (double)r.c.z;
        wq[w][lane][3] = (double)r.c.m;
      }
      __builtin_amdgcn_wave_barrier();
      for (int rr = 0; rr < KSLOTS; rr++) {
        const int m = lane + WAVE * rr;
        if (m >= K) break;
        const int a = c_mi.a[m], b = c_mi.b[m], cc = c_mi.c[m];
        double s = acc[rr];
        for (int j = 0; j < nj; j++) {
          const double tx = tab[w][j][0][a], ty = tab[w][j][1][b], tz = tab[w][j][2][cc];
          double v = wq[w][j][0] * tx * ty * tz;
          if (a > 0) v += wq[w][j][1] * tab[w][j][0][a - 1] * ty * tz;
          if (b > 0) v += wq[w][j][2] * tx * tab[w][j][1][b - 1] * tz;
          if (cc > 0) v += wq[w][j][3] * tx * ty * tab[w][j][2][cc - 1];
          s += v;
        }
        acc[rr] = s;
      }
      __builtin_amdgcn_wave_barrier();
    }
    for (int rr = 0; rr < KSLOTS; rr++) {
      const int m = lane + WAVE * rr;
      if (m < K) mpole[(int64_t)node * K + m] = (T)acc[rr];
    }
  }
}

// The same moments for orders <= 6, one thread per leaf, all in registers.
template <typename T, int P>
__global__ void __launch_bounds__(256)
    k_p2m_dip_reg(const P8<T>* rec, const int32_t* leaves, int64_t n_leaves, const int32_t* begin,
                  const int32_t* count, const double* centre, T* mpole) {
  constexpr int K = Tabs<P>::K;
  const int64_t li = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (li >= n_leaves) return;
  const int32_t node = leaves[li];
  const double cx = centre[3 * node], cy = centre[3 * node + 1], cz = centre[3 * node + 2];
  double acc[K];
#pragma unroll
  for (int k = 0; k < K; k++) acc[k] = 0.0;
  const int32_t j0 = begin[node], j1 = j0 + count[node];
  for (int32_t j = j0; j < j1; j++) {
    const P8<T> r = rec[j];
    const double sx = cx - (double)r.p.x, sy = cy - (double)r.p.y, sz = cz - (double)r.p.z;  // -s
    const double q = (double)r.c.x, bx = (double)r.c.y, by = (double)r.c.z, bz = (double)r.c.m;
    double px[P + 1], py[P + 1], pz[P + 1];
    px[0] = py[0] = pz[0] = 1.0;
#pragma unroll
    for (int t = 1; t <= P; t++) {
      px[t] = px[t - 1] * sx * (1.0 / t);
      py[t] = py[t - 1] * sy * (1.0 / t);
      pz[t] = pz[t - 1] * sz * (1.0 / t);
    }
    static_for<0, K>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int a = tabs<P>.a[k], b = tabs<P>.b[k], c = tabs<P>.c[k];
      double v = q * px[a] * py[b] * pz[c];
      if constexpr (a > 0) v += bx * px[a - 1] * py[b] * pz[c];
      if constexpr (b > 0) v += by * px[a] * py[b - 1] * pz[c];
      if constexpr (c > 0) v += bz * px[a] * py[b] * pz[c - 1];
      acc[k] += v;
    });
  }
  T* out = mpole + (int64_t)node * K;
#pragma unroll
  for (int k = 0; k < K; k++) out[k] = (T)acc[k];
}

template <typename T>
static bool p2m_dip_reg_dispatch(int order, const void* rec, const int32_t* leaves,
                                 int64_t n_leaves, const int32_t* begin, const int32_t* count,
                                 const double* centre, void* mpole, hipStream_t st) {
  unsigned g = (unsigned)((n_leaves + 255) / 256);
  switch (order) {
#define P2MDR(P)                                                                          \
  case P:                                                                                 \
    k_p2m_dip_reg<T, P><<<g, 256, 0, st>>>((const P8<T>*)rec, leaves, n_leaves, begin, count, \
                                           centre, (T*)mpole);                            \
    return true;
    P2MDR(0) P2MDR(1) P2MDR(2) P2MDR(3) P2MDR(4) P2MDR(5) P2MDR(6)
#undef P2MDR
    default:
      return false;
  }
}

hipError_t launch_p2m_dip(int dtype, int order, const void* rec, const int32_t* leaves,
                          int64_t n_leaves, const int32_t* begin, const int32_t* count,
                          const double* centre, void* mpole, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  if (n_leaves == 0) return hipSuccess;
  if (dtype == FMM_F64 ? p2m_dip_reg_dispatch<double>(order, rec, leaves, n_leaves, begin, count,
                                                      centre, mpole, st)
                       : p2m_dip_reg_dispatch<float>(order, rec, leaves, n_leaves, begin, count,
                                                     centre, mpole, st))
    return hipGetLastError();
  int64_t blocks = std::min<int64_t>((n_leaves + EX_WAVES - 1) / EX_WAVES, 65535);
  if (dtype == FMM_F64)
    k_p2m_dip<double><<<(unsigned)blocks, EX_THREADS, 0, st>>>(
        order, K, (const P8<double>*)rec, leaves, n_leaves, begin, count, centre, (double*)mpole);
  else
    k_p2m_dip<float><<<(unsigned)blocks, EX_THREADS, 0, st>>>(
        order, K, (const P8<float>*)rec, leaves, n_leaves, begin, count, centre, (float*)mpole);
  return hipGetLastError();
}

// Far-field parts of the VJP at the particles, one thread per particle:
//   from the forward's leaf locals L:   a = -grad phi,  H = Hess phi
//     (H_ab = sum_n L_(n + e_a + e_b) dx^n / n!, the next higher derivative);
//   from the sensitivity locals B:      Psi and grad Psi;
// out[k] = (Psi, -pb a - H ab + m grad Psi) in sorted order.
template <typename T, int P>
__global__ void k_l2p_vjp(int64_t n, const P8<T>* rec, const int32_t* leaf_of,
                          const double* centre, const T* local, const T* blocal, P4<T>* out) {
  constexpr int K = Tabs<P>::K;
  int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t leaf = leaf_of[k];
  const P8<T> r = rec[k];
  const T dx = (T)((double)r.p.x - centre[3 * leaf]);
  const T dy = (T)((double)r.p.y - centre[3 * leaf + 1]);
  const T dz = (T)((double)r.p.z - centre[3 * leaf + 2]);
  T px[P + 1], py[P + 1], pz[P + 1];  // x^i / i!
  px[0] = py[0] = pz[0] = (T)1;
#pragma unroll
  for (int i = 1; i <= P; i++) {
    px[i] = px[i - 1] * dx * (T)(1.0 / i);
    py[i] = py[i - 1] * dy * (T)(1.0 / i);
    pz[i] = pz[i - 1] * dz * (T)(1.0 / i);
  }
  const T* L = local + (int64_t)leaf * K;
  const T* B = blocal + (int64_t)leaf * K;
  T ax = 0, ay = 0, az = 0;
  T hxx = 0, hyy = 0, hzz = 0, hxy = 0, hxz = 0, hyz = 0;
  T ps = 0, gx = 0, gy = 0, gz = 0;
  static_for<0, K>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int a = tabs<P>.a[i], b = tabs<P>.b[i], c = tabs<P>.c[i];
    const T l = L[i], q = B[i];
    ps += q * px[a] * py[b] * pz[c];
    if constexpr (a > 0) {
      ax -= l * px[a - 1] * py[b] * pz[c];
      gx += q * px[a - 1] * py[b] * pz[c];
    }
    if constexpr (b > 0) {
      ay -= l * px[a] * py[b - 1] * pz[c];
      gy += q * px[a] * py[b - 1] * pz[c];
    }
    if constexpr (c > 0) {
      az -= l * px[a] * py[b] * pz[c - 1];
      gz += q * px[a] * py[b] * pz[c - 1];
    }
    if constexpr (a > 1) hxx += l * px[a - 2] * py[b] * pz[c];
    if constexpr (b > 1) hyy += l * px[a] * py[b - 2] * pz[c];
    if constexpr (c > 1) hzz += l * px[a] * py[b] * pz[c - 2];
    if constexpr (a > 0 && b > 0) hxy += l * px[a - 1] * py[b - 1] * pz[c];
    if constexpr (a > 0 && c > 0) hxz += l * px[a - 1] * py[b] * pz[c - 1];
    if constexpr (b > 0 && c > 0) hyz += l * px[a] * py[b - 1] * pz[c - 1];
  });
  const T pb = r.c.x, bx = r.c.y, by = r.c.z, bz = r.c.m, m = r.p.m;
  P4<T> o;
  o.x = ps;
  o.y = -pb * ax - (hxx * bx + hxy * by + hxz * bz) + m * gx;
  o.z = -pb * ay - (hxy * bx + hyy * by + hyz * bz) + m * gy;
  o.m = -pb * az - (hxz * bx + hyz * by + hzz * bz) + m * gz;
  out[k] = o;
}

template <typename T>
static void l2p_vjp_dispatch(int order, unsigned g, hipStream_t st, int64_t n, const P8<T>* rec,
                             const int32_t* leaf_of, const double* centre, const T* local,
                             const T* blocal, P4<T>* out) {
  switch (order) {
#define L2PV_CASE(P) \
  case P:            \
    k_l2p_vjp<T, P><<<g, 256, 0, st>>>(n, rec, leaf_of, centre, local, blocal, out); \
    break;
    L2PV_CASE(0) L2PV_CASE(1) L2PV_CASE(2) L2PV_CASE(3) L2PV_CASE(4)
    L2PV_CASE(5) L2PV_CASE(6) L2PV_CASE(7) L2PV_CASE(8) L2PV_CASE(9) L2PV_CASE(10)
#undef L2PV_CASE
    default:
      break;
  }
}

hipError_t launch_l2p_vjp(int dtype, int order, int64_t n, const void* rec, const int32_t* leaf_of,
                          const double* centre, const void* local, const void* blocal, void* out,
                          hipStream_t st) {
  unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == FMM_F64)
    l2p_vjp_dispatch<double>(order, g, st, n, (const P8<double>*)rec, leaf_of, centre,
                             (const double*)local, (const double*)blocal, (P4<double>*)out);
  else
    l2p_vjp_dispatch<float>(order, g, st, n, (const P8<float>*)rec, leaf_of, centre,
                            (const float*)local, (const float*)blocal, (P4<float>*)out);
  return hipGetLastError();
}

// ---------------- helpers ----------------
__global__ void k_fill_zero(uint32_t* p, size_t n_words) {
  bookkeeping_priority();
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  size_t w = (bytes + 3) / 4;
  if (w == 0) return hipSuccess;
  size_t blocks = (w + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  k_fill_zero<<<(unsigned)blocks, 256, 0, st>>>((uint32_t*)p, w);
  return hipGetLastError();
}

// scaled moments -> raw moments M_m = (-1)^|m| m! Mt_m; locals copied as fp64
template <typename T>
__global__ void k_export(int K, int64_t total, const T* mpole, const T* local, double* mp,
                         double* lc) {
  int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int m = (int)(gid % K);
  const int a = c_mi.a[m], b = c_mi.b[m], c = c_mi.c[m];
  double f = 1.0;
  for (int i = 2; i <= a; i++) f *= i;
  for (int i = 2; i <= b; i++) f *= i;
  for (int i = 2; i <= c; i++) f *= i;
  if ((a + b + c) & 1) f = -f;
  if (mp) mp[gid] = (double)mpole[gid] * f;
  if (lc) lc[gid] = (double)local[gid];
}

hipError_t launch_export_expansions(int dtype, int order, int64_t n_nodes, const void* mpole,
                                    const void* local, double* mp_out, double* lc_out,
                                    hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  int64_t total = n_nodes * K;
  if (total == 0) return hipSuccess;
  unsigned g = (unsigned)((total + 255) / 256);
  if (dtype == FMM_F64)
    k_export<double><<<g, 256, 0, st>>>(K, total, (const double*)mpole, (const double*)local,
                                        mp_out, lc_out);
  else
    k_export<float><<<g, 256, 0, st>>>(K, total, (const float*)mpole, (const float*)local, mp_out,
                                       lc_out);
  return hipGetLastError();
}

}  // namespace mbg
