// fmm_direct.hip -- direct summation at chosen targets, the reference for
// accuracy measurements of the multipole evaluation.
//
// jz-fmm project page, "From particle pairs to node pairs": the potential of
// particle i is -G sum_{j != i} m_j / |x_i - x_j| and the acceleration its
// negative gradient (G = 1; the self term omitted by index).  Every sum runs
// in fp64 whatever the input precision, so that the result serves as a
// reference for both precisions.
//
// Work split: a block of 256 threads holds 256 targets (one per thread) and
// sums one slice of the sources, staged 256 at a time in LDS; the slices'
// partial sums are added per target in slice order by a second kernel, so the
// result has a fixed summation order.
#include <mutex>

#include "fmm_device.h"
#include "fmm_internal.h"

namespace mbg {

constexpr int DT_THREADS = 256;
constexpr int DT_SLICES = 64;  // source slices (blocks per 256 targets)

__device__ __forceinline__ double direct_rsqrt(double x) {
  // hardware estimate and two Newton steps: well below the rounding of the sums
  double y = __builtin_amdgcn_rsq(x);
  y = fma(0.5 * y, fma(-x * y, y, 1.0), y);
  return fma(0.5 * y, fma(-x * y, y, 1.0), y);
}

template <typename T>
__global__ void __launch_bounds__(DT_THREADS)
    k_direct_part(const T* __restrict__ pos, const T* __restrict__ mass, int64_t n,
                  const int64_t* __restrict__ targets, int64_t n_targets,
                  double* __restrict__ part) {
  __shared__ double sx[DT_THREADS], sy[DT_THREADS], sz[DT_THREADS], sm[DT_THREADS];
  const int64_t t = (int64_t)blockIdx.x * DT_THREADS + threadIdx.x;
  const int slice = blockIdx.y;
  const int64_t per = (n + DT_SLICES - 1) / DT_SLICES;
  const int64_t j0 = (int64_t)slice * per, j1 = min(n, j0 + per);
  int64_t it = -1;
  double xi = 0.0, yi = 0.0, zi = 0.0;
  bool bad = false;
  if (t < n_targets) {
    it = targets[t];
    bad = it < 0 || it >= n;  // out of range: NaN results, nothing read
    if (!bad) {
      xi = (double)pos[3 * it];
      yi = (double)pos[3 * it + 1];
      zi = (double)pos[3 * it + 2];
    }
  }
  double ph = 0.0, ax = 0.0, ay = 0.0, az = 0.0;
  for (int64_t b = j0; b < j1; b += DT_THREADS) {
    const int64_t j = b + threadIdx.x;
    if (j < j1) {
      sx[threadIdx.x] = (double)pos[3 * j];
      sy[threadIdx.x] = (double)pos[3 * j + 1];
      sz[threadIdx.x] = (double)pos[3 * j + 2];
      sm[threadIdx.x] = (double)mass[j];
    }
    __syncthreads();
    const int nb = (int)min((int64_t)DT_THREADS, j1 - b);
    for (int k = 0; k < nb; k++) {
      if (b + k == it) continue;  // self term omitted
      const double dx = xi - sx[k], dy = yi - sy[k], dz = zi - sz[k];
      const double r2 = dx * dx + dy * dy + dz * dz;
      const double rinv = direct_rsqrt(r2);
      const double mr = sm[k] * rinv;
      const double mr3 = mr * rinv * rinv;
      ph -= mr;
      ax -= mr3 * dx;
      ay -= mr3 * dy;
      az -= mr3 * dz;
    }
    __syncthreads();
  }
  if (bad) ph = ax = ay = az = __builtin_nan("");
  if (t < n_targets) {
    double* o = part + 4 * ((int64_t)slice * n_targets + t);
    o[0] = ph;
    o[1] = ax;
    o[2] = ay;
    o[3] = az;
  }
}

template <typename T>
__global__ void k_direct_sum(const double* __restrict__ part, int64_t n_targets,
                             T* __restrict__ phi, T* __restrict__ acc) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= n_targets) return;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int q = 0; q < DT_SLICES; q++)
    for (int c = 0; c < 4; c++) s[c] += part[4 * ((int64_t)q * n_targets + t) + c];
  phi[t] = (T)s[0];
  acc[3 * t] = (T)s[1];
  acc[3 * t + 1] = (T)s[2];
  acc[3 * t + 2] = (T)s[3];
}

// Workspace of the allocation-free variant: the slices' partial sums of up to
// FMM_DIRECT_NOALLOC_MAX_TARGETS targets (8 MiB), one copy per device, held
// until the process ends.  Host code never passes this name to a kernel: it
// is a host-side stand-in, and the device address comes from
// hipGetSymbolAddress (per device, on the first call there).
static __device__ __align__(256) double scratch[(size_t)DT_SLICES * FMM_DIRECT_NOALLOC_MAX_TARGETS * 4];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
double* scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// The device address of `scratch` on the current device (looked up once).
hipError_t scratch_address(double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = static_cast<double*>(ptr);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

// Both kernels on `st` over the workspace `part`.
hipError_t direct_launch(const void* pos, const void* mass, int64_t n, const int64_t* targets,
                         int64_t n_targets, int dtype, void* phi, void* acc, double* part,
                         hipStream_t st) {
  const dim3 grid((unsigned)((n_targets + DT_THREADS - 1) / DT_THREADS), DT_SLICES);
  const unsigned g2 = (unsigned)((n_targets + 255) / 256);
  if (dtype == FMM_F64) {
    k_direct_part<double><<<grid, DT_THREADS, 0, st>>>((const double*)pos, (const double*)mass, n,
                                                       targets, n_targets, part);
    k_direct_sum<double><<<g2, 256, 0, st>>>(part, n_targets, (double*)phi, (double*)acc);
  } else {
    k_direct_part<float><<<grid, DT_THREADS, 0, st>>>((const float*)pos, (const float*)mass, n,
                                                      targets, n_targets, part);
    k_direct_sum<float><<<g2, 256, 0, st>>>(part, n_targets, (float*)phi, (float*)acc);
  }
  return hipGetLastError();
}

}  // namespace mbg

using namespace mbg;

extern "C" int fmm_direct(const void* pos, const void* mass, int64_t n, const int64_t* targets,
                          int64_t n_targets, int dtype, void* phi, void* acc, void* stream) {
  if (!pos || !mass || !targets || !phi || !acc || n < 1 || n_targets < 0 ||
      (dtype != FMM_F32 && dtype != FMM_F64))
    return FMM_ERR_ARG;
  if (n_targets == 0) return FMM_OK;
  hipStream_t st = (hipStream_t)stream;
  double* part = nullptr;
  const size_t bytes = (size_t)DT_SLICES * (size_t)n_targets * 4 * sizeof(double);
  if (hipMalloc(&part, bytes) != hipSuccess) return FMM_ERR_OOM;
  hipError_t e = direct_launch(pos, mass, n, targets, n_targets, dtype, phi, acc, part, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  (void)hipFree(part);
  return e == hipSuccess ? FMM_OK : FMM_ERR_HIP;
}

extern "C" int fmm_direct_noalloc(const void* pos, const void* mass, int64_t n,
                                  const int64_t* targets, int64_t n_targets, int dtype, void* phi,
                                  void* acc, void* stream) {
  if (!pos || !mass || !targets || !phi || !acc || n < 1 || n_targets < 0 ||
      n_targets > FMM_DIRECT_NOALLOC_MAX_TARGETS || (dtype != FMM_F32 && dtype != FMM_F64))
    return FMM_ERR_ARG;
  if (n_targets == 0) return FMM_OK;
  double* part = nullptr;
  // every slot of the workspace that the sums read is written first by the
  // partial kernel of the same call: nothing needs clearing
  if (scratch_address(&part) != hipSuccess) return FMM_ERR_HIP;
  const hipError_t e = direct_launch(pos, mass, n, targets, n_targets, dtype, phi, acc, part,
                                     (hipStream_t)stream);
  return e == hipSuccess ? FMM_OK : FMM_ERR_HIP;
}
