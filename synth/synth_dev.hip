/*
 * Device fill of seeded synthetic arrays (test and benchmark infrastructure,
 * not part of the optimizer library).  Uses the same definition as the host
 * fill (synth_core.h); with contraction disabled the values are bit-identical.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_QUAL static __host__ __device__ inline
#include "synth_core.h"

namespace {

__global__ void __launch_bounds__(256) fill_normal_kernel(uint64_t key, int64_t offset, int64_t n,
                                                          double mean, double std, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = synth_normal_f32(key, (uint64_t)(offset + j), mean, std);
}

__global__ void __launch_bounds__(256) fill_uniform_kernel(uint64_t key, int64_t offset, int64_t n,
                                                           double lo, double hi, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
    out[j] = synth_uniform_f32(key, (uint64_t)(offset + j), lo, hi);
}

int grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

extern "C" int synth_dev_fill_normal(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                                     double mean, double std, float* out, void* stream_handle) {
  if (n <= 0) return 0;
  if (!out) return 1;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream_handle, synth_key(seed, stream), offset, n, mean, std, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int synth_dev_fill_uniform(uint64_t seed, uint64_t stream, int64_t offset, int64_t n,
                                      double lo, double hi, float* out, void* stream_handle) {
  if (n <= 0) return 0;
  if (!out) return 1;
  hipLaunchKernelGGL(fill_uniform_kernel, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream_handle, synth_key(seed, stream), offset, n, lo, hi, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
