// fmm_probe.hip -- measured vector peaks of the device, the denominators
// against which the benchmark states the achieved fraction of the fp64 and
// fp32 vector rates next to the published ones.
//
// Each lane runs CHAINS independent multiply-add chains (enough to hide the
// instruction latency) for a fixed number of iterations; the grid fills every
// compute unit several times over.  The chains' results are written out so
// that no work can be dropped.  fp32 is measured as this library compiles it:
// without packed two-wide operations, so its ceiling is the fp64 rate.
#include <chrono>

#include "fmm_internal.h"

namespace mbg {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_CHAINS = 16;
constexpr int PROBE_ITERS = 4096;

template <typename T>
__global__ void __launch_bounds__(PROBE_THREADS) k_fma_probe(T a, T b, T* __restrict__ out) {
  T x[PROBE_CHAINS];
  const T seed = (T)(threadIdx.x + blockIdx.x) * (T)1e-7;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; c++) x[c] = seed + (T)c;
  for (int i = 0; i < PROBE_ITERS; i++) {
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; c++) x[c] = fma(x[c], a, b);
  }
  T s = 0;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; c++) s += x[c];
  out[blockIdx.x * PROBE_THREADS + threadIdx.x] = s;
}

template <typename T>
hipError_t time_probe(int blocks, T* out, hipStream_t st, double* tflops) {
  hipEvent_t e0, e1;
  hipError_t e = hipEventCreate(&e0);
  if (e != hipSuccess) return e;
  e = hipEventCreate(&e1);
  if (e != hipSuccess) {
    (void)hipEventDestroy(e0);
    return e;
  }
  // a = 1 - 2^-20, b = 2^-30: the chains stay finite and never denormal
  const T a = (T)(1.0 - 1.0 / 1048576.0), b = (T)(1.0 / 1073741824.0);
  float best = 1e30f;
  for (int rep = 0; rep < 4 && e == hipSuccess; rep++) {  // the first run warms up
    e = hipEventRecord(e0, st);
    if (e == hipSuccess) {
      k_fma_probe<T><<<blocks, PROBE_THREADS, 0, st>>>(a, b, out);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, st);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && rep > 0 && ms < best) best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e == hipSuccess) {
    const double flops = 2.0 * PROBE_CHAINS * PROBE_ITERS * (double)blocks * PROBE_THREADS;
    *tflops = flops / (best * 1e-3) / 1e12;
  }
  return e;
}

}  // namespace mbg

using namespace mbg;

extern "C" int fmm_measure_peaks(double* fp64_tflops, double* fp32_tflops, void* stream) {
  if (!fp64_tflops || !fp32_tflops) return FMM_ERR_ARG;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return FMM_ERR_HIP;
  const int blocks = 32 * ncu;  // 8 waves per SIMD
  double* out = nullptr;
  if (hipMalloc(&out, (size_t)blocks * PROBE_THREADS * sizeof(double)) != hipSuccess)
    return FMM_ERR_OOM;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = time_probe<double>(blocks, out, st, fp64_tflops);
  if (e == hipSuccess) e = time_probe<float>(blocks, (float*)out, st, fp32_tflops);
  (void)hipFree(out);
  return e == hipSuccess ? FMM_OK : FMM_ERR_HIP;
}
