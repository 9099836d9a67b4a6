// fmm_p2p.hip -- near field between leaf cells, plus the final combine.
//
// jz-fmm project page: the direct sum Phi(x_i) = -G sum_{j != i} m_j/|x_i - x_j|
// with the self term omitted ("From particle pairs to node pairs"), applied to
// the leaf pairs the walk did not accept ("Combining near and far
// interactions": at the leaves, add the remaining nearby interactions
// directly).  The far field computed by L2P is added here and the result is
// written in the caller's particle order.
//
// Work split: one wave per target leaf.  A leaf of tc <= 64 targets is spread
// over the 64 lanes as tc targets x floor(64/tc) source slices; each lane walks
// its slice of every source leaf in order, and the slices of one target are
// summed in a fixed order through LDS.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int P2P_THREADS = 256;
constexpr int P2P_WAVES = P2P_THREADS / WAVE;

__device__ __forceinline__ double p2p_rsqrt(double x) {
  double y = __builtin_amdgcn_rsq(x);
  double e = fma(-x * y, y, 1.0);
  return fma(y * e, fma(e, 0.375, 0.5), y);
}
__device__ __forceinline__ float p2p_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

template <typename T>
__global__ void __launch_bounds__(P2P_THREADS)
    k_p2p(const int32_t* __restrict__ leaves, int64_t n_leaves, const int32_t* __restrict__ begin,
          const int32_t* __restrict__ count, const int64_t* __restrict__ off,
          const int32_t* __restrict__ src, const P4<T>* __restrict__ pts,
          const P4<T>* __restrict__ far, const int32_t* __restrict__ perm, T* __restrict__ phi,
          T* __restrict__ acc) {
  __shared__ T part[P2P_WAVES][4][WAVE];
  const int lane = __lane_id();
  const int w = threadIdx.x / WAVE;
  for (int64_t li = (int64_t)blockIdx.x * P2P_WAVES + w; li < n_leaves;
       li += (int64_t)gridDim.x * P2P_WAVES) {
    const int32_t a = leaves[li];
    const int32_t tb = begin[a], tn = count[a];
    const int64_t e0 = off[a], e1 = off[a + 1];
    for (int32_t t0 = 0; t0 < tn; t0 += WAVE) {
      const int tc = min(WAVE, tn - t0);
      const int nsl = WAVE / tc;
      const int t = lane % tc, sl = lane / tc;
      const bool active = sl < nsl;
      const int32_t i = tb + t0 + t;
      const P4<T> pi = pts[i];
      T fp = 0, fx = 0, fy = 0, fz = 0;
      if (active) {
        for (int64_t e = e0; e < e1; e++) {
          const int32_t b = src[e];
          const int32_t j1 = begin[b] + count[b];
          for (int32_t j = begin[b] + sl; j < j1; j += nsl) {
            const P4<T> pj = pts[j];
            const T dx = pi.x - pj.x, dy = pi.y - pj.y, dz = pi.z - pj.z;
            const T r2 = dx * dx + dy * dy + dz * dz;
            T rinv = p2p_rsqrt(r2);
            rinv = (j == i) ? (T)0 : rinv;  // self term omitted
            const T mr = pj.m * rinv;
            const T mr3 = mr * rinv * rinv;
            fp -= mr;
            fx -= mr3 * dx;
            fy -= mr3 * dy;
            fz -= mr3 * dz;
          }
        }
      }
      part[w][0][lane] = fp;
      part[w][1][lane] = fx;
      part[w][2][lane] = fy;
      part[w][3][lane] = fz;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0);
      if (lane < tc) {
        T s0 = 0, s1 = 0, s2 = 0, s3 = 0;
        for (int s = 0; s < nsl; s++) {
          s0 += part[w][0][s * tc + lane];
          s1 += part[w][1][s * tc + lane];
          s2 += part[w][2][s * tc + lane];
          s3 += part[w][3][s * tc + lane];
        }
        const P4<T> f = far[i];
        const int64_t o = perm[i];
        phi[o] = f.x + s0;
        acc[3 * o] = f.y + s1;
        acc[3 * o + 1] = f.z + s2;
        acc[3 * o + 2] = f.m + s3;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

hipError_t launch_p2p(int dtype, const int32_t* leaves, int64_t n_leaves, const int32_t* begin,
                      const int32_t* count, const int64_t* off, const int32_t* src,
                      const void* pts, const void* far, const int32_t* perm, void* phi,
                      void* acc, hipStream_t st) {
  if (n_leaves == 0) return hipSuccess;
  int64_t blocks = (n_leaves + P2P_WAVES - 1) / P2P_WAVES;
  if (blocks > 65535) blocks = 65535;
  if (dtype == FMM_F64)
    k_p2p<double><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        leaves, n_leaves, begin, count, off, src, (const P4<double>*)pts, (const P4<double>*)far,
        perm, (double*)phi, (double*)acc);
  else
    k_p2p<float><<<(unsigned)blocks, P2P_THREADS, 0, st>>>(
        leaves, n_leaves, begin, count, off, src, (const P4<float>*)pts, (const P4<float>*)far,
        perm, (float*)phi, (float*)acc);
  return hipGetLastError();
}

}  // namespace mbg
