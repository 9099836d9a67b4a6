// fmm_lattice.hip -- the integer-lattice kick-drift-kick update.
//
// jz-fmm project page, "Why reversibility matters": positions and velocities
// live on an integer lattice while the force calculation stays floating point,
// and undoing an update subtracts exactly the integer increment that the
// forward update added.  With x = q dx, v = u dv (q, u int64) and s = +1
// (forward) or -1 (backward):
//   kick:   u += s rint(a (dt/2) / dv)
//   drift:  q += s rint(u (dt dv / dx))
// Each increment is one fp64 product rounded half to even, so it depends only
// on the integer state and the (bitwise reproducible) force.
#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

// |increment| above this (or non-finite) cannot be held: flag it
constexpr double LAT_MAX = 4611686018427387904.0;  // 2^62

template <typename T>
__global__ void k_lat_pos(int64_t n3, const int64_t* __restrict__ q, double dx,
                          T* __restrict__ pos) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n3) pos[i] = (T)((double)q[i] * dx);
}

template <typename T>
__global__ void k_lat_kick(int64_t n3, int64_t* __restrict__ u, const T* __restrict__ acc,
                           double c, int64_t s, int* __restrict__ flag) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n3) return;
  const double k = rint((double)acc[i] * c);
  if (!(fabs(k) < LAT_MAX)) {
    atomicOr(flag, 1);
    return;
  }
  u[i] += s * (int64_t)k;
}

__global__ void k_lat_drift(int64_t n3, int64_t* __restrict__ q, const int64_t* __restrict__ u,
                            double c, int64_t s, int* __restrict__ flag) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n3) return;
  const double k = rint((double)u[i] * c);
  if (!(fabs(k) < LAT_MAX)) {
    atomicOr(flag, 1);
    return;
  }
  q[i] += s * (int64_t)k;
}

hipError_t launch_lat_pos(int dtype, int64_t n, const int64_t* q, double dx, void* pos,
                          hipStream_t st) {
  const int64_t n3 = 3 * n;
  const unsigned g = (unsigned)((n3 + 255) / 256);
  if (dtype == FMM_F64)
    k_lat_pos<double><<<g, 256, 0, st>>>(n3, q, dx, (double*)pos);
  else
    k_lat_pos<float><<<g, 256, 0, st>>>(n3, q, dx, (float*)pos);
  return hipGetLastError();
}

hipError_t launch_lat_kick(int dtype, int64_t n, int64_t* u, const void* acc, double c, int s,
                           int* flag, hipStream_t st) {
  const int64_t n3 = 3 * n;
  const unsigned g = (unsigned)((n3 + 255) / 256);
  if (dtype == FMM_F64)
    k_lat_kick<double><<<g, 256, 0, st>>>(n3, u, (const double*)acc, c, (int64_t)s, flag);
  else
    k_lat_kick<float><<<g, 256, 0, st>>>(n3, u, (const float*)acc, c, (int64_t)s, flag);
  return hipGetLastError();
}

hipError_t launch_lat_drift(int64_t n, int64_t* q, const int64_t* u, double c, int s, int* flag,
                            hipStream_t st) {
  const int64_t n3 = 3 * n;
  const unsigned g = (unsigned)((n3 + 255) / 256);
  k_lat_drift<<<g, 256, 0, st>>>(n3, q, u, c, (int64_t)s, flag);
  return hipGetLastError();
}

}  // namespace mbg
