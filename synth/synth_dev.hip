// Seeded synthetic inputs, device side: fills HBM buffers with exactly the
// bytes synth_host.c produces for the same (seed, stream, index); see
// philox.h.  Inputs only: nothing here belongs to the shard step under test.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYNTH_FN __host__ __device__ static inline
#include "philox.h"

namespace {

__global__ void __launch_bounds__(256)
fill_bf16_kernel(uint16_t* __restrict__ out, int64_t n, uint64_t seed,
                 uint32_t sa, uint32_t sb, uint64_t i0, double c) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
       j += stride)
    out[j] = synth_normal_bf16(seed, sa, sb, i0 + (uint64_t)j, c);
}

__global__ void __launch_bounds__(256)
fill_f32_kernel(float* __restrict__ out, int64_t n, uint64_t seed,
                uint32_t sa, uint32_t sb, uint64_t i0, double c) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n;
       j += stride)
    out[j] = synth_normal_f32(seed, sa, sb, i0 + (uint64_t)j, c);
}

unsigned grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

extern "C" int synth_dev_fill_bf16(void* out, int64_t n, uint64_t seed,
                                   uint32_t sa, uint32_t sb, uint64_t i0,
                                   double c, hipStream_t stream) {
  if (n <= 0) return 0;
  if (out == nullptr) return -1;
  hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, stream,
                     static_cast<uint16_t*>(out), n, seed, sa, sb, i0, c);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int synth_dev_fill_f32(void* out, int64_t n, uint64_t seed,
                                  uint32_t sa, uint32_t sb, uint64_t i0,
                                  double c, hipStream_t stream) {
  if (n <= 0) return 0;
  if (out == nullptr) return -1;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, stream,
                     static_cast<float*>(out), n, seed, sa, sb, i0, c);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
