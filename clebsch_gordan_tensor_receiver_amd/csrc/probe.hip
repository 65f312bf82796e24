// Achievable-peak probes of the device (cgtp_measure_peak): a plain fused-multiply-add
// throughput kernel in fp32 and fp64 and a streaming device copy, timed with HIP events.  They
// give the measured ceilings that the convolution kernels' algorithmic rates are compared with,
// beside the published ones (vector FMA 78.6 TFLOP/s without packed fp32, 8 TB/s HBM).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "cgtp.h"
#include "errors.hpp"

namespace {

constexpr int kChains = 16;       // independent FMA chains per lane
constexpr int kProbeBlock = 256;  // four waves per workgroup

// Every lane runs kChains independent chains v = v * a + b for `iters` steps.  a and b are kernel
// arguments, so nothing folds at compile time; the sum is stored (to out[0]) only when it equals
// `sentinel` (never: every chain tends to 1 for a = 0.999, b = 0.001), which keeps the chains live
// without a store per lane.
template <typename T>
__global__ void __launch_bounds__(kProbeBlock) fma_probe(T a, T b, int iters, T sentinel, T* out) {
  T v[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) v[k] = T(threadIdx.x & 7) + T(k);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) v[k] = fma(v[k], a, b);
  }
  T s = T(0);
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += v[k];
  if (s == sentinel) out[0] = s;
}

// Grid-stride copy in 16-byte units.
__global__ void __launch_bounds__(kProbeBlock) copy_probe(const float4* __restrict__ src, float4* __restrict__ dst,
                                                          size_t n) {
  const size_t stride = (size_t)gridDim.x * kProbeBlock;
  for (size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

cgtp_status_t hip_fail(const char* what, hipError_t e) {
  return cgtp::set_error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

cgtp_status_t cgtp_measure_peak(int kind, void* dst, const void* src, size_t bytes, int reps, void* stream,
                                double* best, double* median) {
  if (kind < 0 || kind > 2 || reps < 1 || !best || !dst)
    return cgtp::set_error(CGTP_ERR_INVALID_ARG, "kind must be 0..2, reps >= 1, best and dst non-null");
  if (kind == 2 && (!src || bytes == 0 || bytes % 16 != 0))
    return cgtp::set_error(CGTP_ERR_INVALID_ARG, "the copy needs src and a size that is a positive multiple of 16");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail("device query", e);
  // Eight workgroups of four waves per compute unit: eight waves per SIMD.
  const unsigned grid = unsigned(std::max(ncu, 1)) * 8u;
  const int iters = 8192;
  hipEvent_t a, b;
  if ((e = hipEventCreate(&a)) != hipSuccess) return hip_fail("hipEventCreate", e);
  if ((e = hipEventCreate(&b)) != hipSuccess) {
    (void)hipEventDestroy(a);
    return hip_fail("hipEventCreate", e);
  }
  auto run = [&]() {
    if (kind == 0)
      hipLaunchKernelGGL(fma_probe<float>, dim3(grid), dim3(kProbeBlock), 0, s, 0.999f, 0.001f, iters, -1.0f,
                         static_cast<float*>(dst));
    else if (kind == 1)
      hipLaunchKernelGGL(fma_probe<double>, dim3(grid), dim3(kProbeBlock), 0, s, 0.999, 0.001, iters, -1.0,
                         static_cast<double*>(dst));
    else
      hipLaunchKernelGGL(copy_probe, dim3(grid * 4), dim3(kProbeBlock), 0, s, static_cast<const float4*>(src),
                         static_cast<float4*>(dst), bytes / 16);
    return hipGetLastError();
  };
  std::vector<double> rates;
  cgtp_status_t st = CGTP_OK;
  // Two untimed launches raise the clocks, then reps timed ones.
  for (int r = -2; r < reps && st == CGTP_OK; ++r) {
    if ((e = hipEventRecord(a, s)) != hipSuccess || (e = run()) != hipSuccess || (e = hipEventRecord(b, s)) != hipSuccess ||
        (e = hipEventSynchronize(b)) != hipSuccess) {
      st = hip_fail("probe launch", e);
      break;
    }
    float ms = 0.0f;
    if ((e = hipEventElapsedTime(&ms, a, b)) != hipSuccess) {
      st = hip_fail("hipEventElapsedTime", e);
      break;
    }
    if (r < 0 || ms <= 0.0f) continue;
    double work = kind == 2 ? 2.0 * double(bytes) / 1e9                                              // GB
                            : 2.0 * kChains * double(iters) * double(grid) * kProbeBlock / 1e12;  // TFLOP
    rates.push_back(work / (double(ms) * 1e-3));
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (st != CGTP_OK) return st;
  if (rates.empty()) return cgtp::set_error(CGTP_ERR_HIP, "no timed launch gave a positive duration");
  std::sort(rates.begin(), rates.end());
  *best = rates.back();
  if (median) *median = rates[rates.size() / 2];
  return cgtp::set_error(CGTP_OK, "");
}

}  // extern "C"
