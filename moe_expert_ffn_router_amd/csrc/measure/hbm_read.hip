// HBM read calibration (measurement library, not part of the layer): a plain
// streaming read of `bytes` bytes (grid-strided 16-byte loads, 256-thread
// workgroups), each thread folding what it read into one word written to
// `sink`.  It does none of the layer's arithmetic; its time for a given byte
// count is what a pure read of those bytes costs on this chip, the practical
// ceiling the bandwidth-bound kernels are held to.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_measure.h"

namespace {

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t step = (size_t)gridDim.x * 256;
  uint32_t a = 0;
#pragma unroll 8
  for (; i < n16; i += step) {
    const uint4 v = src[i];
    a ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = a;
}

}  // namespace

extern "C" int moe_measure_hbm_read(const void* src, int64_t bytes, int32_t grid, uint32_t* sink,
                                    void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || grid < 1 || grid > 65536) return 1;
  if (reinterpret_cast<uintptr_t>(src) % 16) return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hbm_read_kernel<<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), (size_t)bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
