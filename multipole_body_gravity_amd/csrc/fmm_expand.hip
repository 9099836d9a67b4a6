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

__device__ __forceinline__ double pow_over_fact(double x, int n) {
  double r = 1.0;
  for (int i = 1; i <= n; i++) r = r * x / (double)i;
  return r;
}

// ---------------- P2M: one thread per (leaf, coefficient) ----------------
template <typename T>
__global__ void k_p2m(int K, const P4<T>* pts, const int32_t* leaves, int64_t n_leaves,
                      const int32_t* begin, const int32_t* count, const double* centre, T* mpole) {
  int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gid >= n_leaves * K) return;
  const int64_t li = gid / K;
  const int m = (int)(gid - li * K);
  const int32_t node = leaves[li];
  const int a = c_mi.a[m], b = c_mi.b[m], c = c_mi.c[m];
  const double cx = centre[3 * node], cy = centre[3 * node + 1], cz = centre[3 * node + 2];
  double acc = 0.0;
  const int32_t j0 = begin[node], j1 = j0 + count[node];
  for (int32_t j = j0; j < j1; j++) {
    const P4<T> p = pts[j];
    const double sx = cx - (double)p.x, sy = cy - (double)p.y, sz = cz - (double)p.z;  // -s
    acc += (double)p.m * pow_over_fact(sx, a) * pow_over_fact(sy, b) * pow_over_fact(sz, c);
  }
  mpole[(int64_t)node * K + m] = (T)acc;
}

hipError_t launch_p2m(int dtype, int order, const void* pts, const int32_t* leaves,
                      int64_t n_leaves, const int32_t* begin, const int32_t* count,
                      const double* centre, void* mpole, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  int64_t nt = n_leaves * K;
  if (nt == 0) return hipSuccess;
  unsigned g = (unsigned)((nt + 255) / 256);
  if (dtype == FMM_F64)
    k_p2m<double><<<g, 256, 0, st>>>(K, (const P4<double>*)pts, leaves, n_leaves, begin, count,
                                     centre, (double*)mpole);
  else
    k_p2m<float><<<g, 256, 0, st>>>(K, (const P4<float>*)pts, leaves, n_leaves, begin, count,
                                    centre, (float*)mpole);
  return hipGetLastError();
}

// ---------------- M2M: one thread per (parent, coefficient) ----------------
template <typename T>
__global__ void k_m2m(int K, int64_t lvl_begin, int64_t lvl_count, const int32_t* first_child,
                      const uint8_t* n_child, const double* centre, T* mpole) {
  int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gid >= lvl_count * K) return;
  const int64_t pi = gid / K;
  const int m = (int)(gid - pi * K);
  const int64_t P = lvl_begin + pi;
  const int nc = n_child[P];
  if (nc == 0) return;  // leaf: moments come from P2M
  const int ma = c_mi.a[m], mb = c_mi.b[m], mc = c_mi.c[m];
  double acc = 0.0;
  const int32_t fc = first_child[P];
  for (int ci = 0; ci < nc; ci++) {
    const int64_t ch = fc + ci;
    // -d = c_P - c_child
    const double nx = centre[3 * P] - centre[3 * ch], ny = centre[3 * P + 1] - centre[3 * ch + 1],
                 nz = centre[3 * P + 2] - centre[3 * ch + 2];
    const T* Mc = mpole + ch * K;
    for (int i = 0; i <= ma; i++) {
      const double ex = pow_over_fact(nx, ma - i);
      for (int j = 0; j <= mb; j++) {
        const double exy = ex * pow_over_fact(ny, mb - j);
        for (int k = 0; k <= mc; k++)
          acc += (double)Mc[mi_index(i, j, k)] * exy * pow_over_fact(nz, mc - k);
      }
    }
  }
  mpole[P * K + m] = (T)acc;
}

hipError_t launch_m2m(int dtype, int order, int64_t lvl_begin, int64_t lvl_count,
                      const int32_t* first_child, const uint8_t* n_child, const double* centre,
                      void* mpole, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  int64_t nt = lvl_count * K;
  if (nt == 0) return hipSuccess;
  unsigned g = (unsigned)((nt + 255) / 256);
  if (dtype == FMM_F64)
    k_m2m<double><<<g, 256, 0, st>>>(K, lvl_begin, lvl_count, first_child, n_child, centre,
                                     (double*)mpole);
  else
    k_m2m<float><<<g, 256, 0, st>>>(K, lvl_begin, lvl_count, first_child, n_child, centre,
                                    (float*)mpole);
  return hipGetLastError();
}

// ---------------- L2L: one thread per (child, coefficient) ----------------
// L_n(child) += sum_{|n|+|k|<=p} L_(n+k)(parent) d^k / k!, d = c_child - c_parent
template <typename T>
__global__ void k_l2l(int order, int K, int64_t lvl_begin, int64_t lvl_count, const int32_t* parent,
                      const double* centre, T* local) {
  int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gid >= lvl_count * K) return;
  const int64_t ci = gid / K;
  const int n = (int)(gid - ci * K);
  const int64_t a = lvl_begin + ci;
  const int64_t P = parent[a];
  const int na = c_mi.a[n], nb = c_mi.b[n], nc = c_mi.c[n];
  const int rem = order - (na + nb + nc);
  const double dx = centre[3 * a] - centre[3 * P], dy = centre[3 * a + 1] - centre[3 * P + 1],
               dz = centre[3 * a + 2] - centre[3 * P + 2];
  const T* Lp = local + P * K;
  double acc = 0.0;
  for (int i = 0; i <= rem; i++) {
    const double ex = pow_over_fact(dx, i);
    for (int j = 0; i + j <= rem; j++) {
      const double exy = ex * pow_over_fact(dy, j);
      for (int k = 0; i + j + k <= rem; k++)
        acc += (double)Lp[mi_index(na + i, nb + j, nc + k)] * exy * pow_over_fact(dz, k);
    }
  }
  local[a * K + n] = (T)((double)local[a * K + n] + acc);
}

hipError_t launch_l2l(int dtype, int order, int64_t lvl_begin, int64_t lvl_count,
                      const int32_t* parent, const double* centre, void* local, hipStream_t st) {
  hipError_t e = ensure_table();
  if (e != hipSuccess) return e;
  const int K = ncoef(order);
  int64_t nt = lvl_count * K;
  if (nt == 0) return hipSuccess;
  unsigned g = (unsigned)((nt + 255) / 256);
  if (dtype == FMM_F64)
    k_l2l<double><<<g, 256, 0, st>>>(order, K, lvl_begin, lvl_count, parent, centre,
                                     (double*)local);
  else
    k_l2l<float><<<g, 256, 0, st>>>(order, K, lvl_begin, lvl_count, parent, centre,
                                    (float*)local);
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
    L2P_CASE(5) L2P_CASE(6) L2P_CASE(7) L2P_CASE(8)
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

// ---------------- helpers ----------------
__global__ void k_fill_zero(uint32_t* p, size_t n_words) {
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
