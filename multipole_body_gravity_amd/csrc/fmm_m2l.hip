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
// Work split: one wave per target cell; lane l takes sources l, l+64, ... of the
// target's list, accumulates a private partial local expansion, and the 64
// partials are summed by a fixed butterfly, so the result does not depend on
// scheduling.  Each target is written once (every level in one launch).
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

// Derivatives of 1/|r| up to total degree P, graded layout.  Every index is a
// compile-time constant, so the whole table lives in registers.
template <typename T, int P>
__device__ __forceinline__ void dtensor(T x, T y, T z, T (&D)[Tabs<P>::K]) {
  constexpr int NR = Tabs<P>::NR;
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
    if constexpr (ax < 0) {
      R[e] = g[tabs<P>.rlev[e]];
    } else {
      const T u = ax == 0 ? x : (ax == 1 ? y : z);
      constexpr int s1 = tabs<P>.rs1[e];
      constexpr int s2 = tabs<P>.rs2[e];
      if constexpr (s2 >= 0) {
        R[e] = u * R[s1] + (T)tabs<P>.rc2[e] * R[s2];
      } else {
        R[e] = u * R[s1];
      }
    }
  });
  static_for<0, Tabs<P>::K>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    D[k] = R[tabs<P>.roff[0] + k];
  });
}

template <typename T, int P>
__global__ void __launch_bounds__(M2L_THREADS)
    k_m2l(int64_t n_nodes, const int64_t* __restrict__ off, const int32_t* __restrict__ src,
          const double* __restrict__ centre, const T* __restrict__ mpole, T* __restrict__ local) {
  constexpr int K = Tabs<P>::K;
  constexpr int NT = Tabs<P>::NT;
  const int lane = __lane_id();
  const int64_t wid = (int64_t)blockIdx.x * (M2L_THREADS / WAVE) + threadIdx.x / WAVE;
  const int64_t nw = (int64_t)gridDim.x * (M2L_THREADS / WAVE);
  for (int64_t a = wid; a < n_nodes; a += nw) {
    const int64_t e0 = off[a], e1 = off[a + 1];
    const double cax = centre[3 * a], cay = centre[3 * a + 1], caz = centre[3 * a + 2];
    T acc[K];
#pragma unroll
    for (int k = 0; k < K; k++) acc[k] = (T)0;
    for (int64_t e = e0 + lane; e < e1; e += WAVE) {
      const int64_t b = src[e];
      // the source's moments are loaded first; the derivative tensor, which
      // needs only the centres, is built while they are in flight
      const T* Mb = mpole + b * K;
      T M[K];
#pragma unroll
      for (int k = 0; k < K; k++) M[k] = Mb[k];
      const T rx = (T)(cax - centre[3 * b]);
      const T ry = (T)(cay - centre[3 * b + 1]);
      const T rz = (T)(caz - centre[3 * b + 2]);
      T D[K];
      dtensor<T, P>(rx, ry, rz, D);
      static_for<0, NT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        acc[tabs<P>.tn[t]] += M[tabs<P>.tm[t]] * D[tabs<P>.tk[t]];
      });
    }
    T* La = local + a * K;
    static_for<0, K>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      const T v = wave_sum(acc[n]);
      if (lane == (n & (WAVE - 1))) La[n] = -v;  // G = 1: L = -sum
    });
  }
}

template <typename T>
static void m2l_dispatch(int order, unsigned g, hipStream_t st, int64_t n_nodes, const int64_t* off,
                         const int32_t* src, const double* centre, const T* mpole, T* local) {
  switch (order) {
#define M2L_CASE(P) \
  case P:           \
    k_m2l<T, P><<<g, M2L_THREADS, 0, st>>>(n_nodes, off, src, centre, mpole, local); \
    break;
    M2L_CASE(0) M2L_CASE(1) M2L_CASE(2) M2L_CASE(3) M2L_CASE(4)
    M2L_CASE(5) M2L_CASE(6) M2L_CASE(7) M2L_CASE(8)
#undef M2L_CASE
    default:
      break;
  }
}

hipError_t launch_m2l(int dtype, int order, int64_t n_nodes, const int64_t* off,
                      const int32_t* src, const double* centre, const void* mpole, void* local,
                      hipStream_t st) {
  int64_t blocks = (n_nodes + (M2L_THREADS / WAVE) - 1) / (M2L_THREADS / WAVE);
  if (blocks > 65535) blocks = 65535;
  if (blocks < 1) blocks = 1;
  unsigned g = (unsigned)blocks;
  if (dtype == FMM_F64)
    m2l_dispatch<double>(order, g, st, n_nodes, off, src, centre, (const double*)mpole,
                         (double*)local);
  else
    m2l_dispatch<float>(order, g, st, n_nodes, off, src, centre, (const float*)mpole,
                        (float*)local);
  return hipGetLastError();
}

}  // namespace mbg
