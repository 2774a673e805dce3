// Measurement support: a shader-clock sampler and wall-clock timestamps (include/sparsp_measure.h).
#include "sparsp.h"
#include "sparsp_internal.h"
#include "sparsp_measure.h"

namespace {

__device__ __forceinline__ uint64_t shader_clock() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

// Lane 0 takes sample i once the wall clock has advanced i * interval ticks from the first sample.  Every
// wait ends: the wall clock runs at a constant rate, and the last sample is due n * interval ticks after the
// start.
__global__ __launch_bounds__(64) void clock_sampler_kernel(uint64_t* samples, int n, uint32_t interval) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock();
  for (int i = 0; i < n; ++i) {
    const uint64_t due = t0 + (uint64_t)i * interval;
    uint64_t w = wall_clock();
    while (w < due) {
      __builtin_amdgcn_s_sleep(2);
      w = wall_clock();
    }
    const uint64_t c = shader_clock();
    samples[2 * i] = c;
    samples[2 * i + 1] = w;
  }
}

__global__ void wall_timestamp_kernel(uint64_t* out) {
  if (threadIdx.x == 0) *out = wall_clock();
}

}  // namespace

extern "C" {

int32_t sparsp_clock_sampler(uint64_t* samples, int32_t n_samples, int32_t interval_ticks, void* stream) {
  if (!samples || n_samples < 2 || interval_ticks < 1) return SPARSP_ERR_INVALID;
  if ((uint64_t)n_samples * (uint64_t)interval_ticks > (1ull << 32)) return SPARSP_ERR_INVALID;
  hipLaunchKernelGGL(clock_sampler_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), samples,
                     n_samples, (uint32_t)interval_ticks);
  return hipGetLastError() == hipSuccess ? SPARSP_OK : SPARSP_ERR_HIP;
}

int32_t sparsp_wall_timestamp(uint64_t* out, void* stream) {
  if (!out) return SPARSP_ERR_INVALID;
  hipLaunchKernelGGL(wall_timestamp_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), out);
  return hipGetLastError() == hipSuccess ? SPARSP_OK : SPARSP_ERR_HIP;
}

int32_t sparsp_wall_clock_khz(int32_t* khz) {
  if (!khz) return SPARSP_ERR_INVALID;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SPARSP_ERR_HIP;
  if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate <= 0)
    return SPARSP_ERR_HIP;
  *khz = rate;
  return SPARSP_OK;
}

}  // extern "C"
