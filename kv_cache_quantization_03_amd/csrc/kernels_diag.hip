// Streaming-read ceiling for the roofline comparisons: plain 16-byte loads
// over a buffer, grid-stride, one XOR word per block so the loads stay.
#include "kernels_common.h"

namespace tq {

namespace {
constexpr int kDiagBlocks = 2048;  // 8 per CU
constexpr int kDiagThreads = 256;

__global__ __launch_bounds__(kDiagThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kDiagThreads / kWave];
  uint32_t x = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kDiagThreads + threadIdx.x; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kDiagThreads) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), m, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kDiagThreads / kWave; ++w) y ^= part[w];
    sink[blockIdx.x] = y;
  }
}
}  // namespace

int diag_stream_blocks() { return kDiagBlocks; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kDiagBlocks), dim3(kDiagThreads), 0, s,
                     static_cast<const uint4*>(src), static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace tq
