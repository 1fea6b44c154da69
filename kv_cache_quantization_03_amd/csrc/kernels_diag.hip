// Streaming ceiling for the roofline comparisons (measurement helper, not part
// of the method): one launch that reads a buffer and writes another, shaped
// like the bandwidth-bound kernels' own traffic, with as many bytes in flight
// as the hardware takes.  Each thread issues four independent 16-byte
// non-temporal loads before it uses any (a block covers 16 KiB), so no load
// waits for another; the write blocks store 16 KiB each with 16-byte stores.
// One XOR word per read block goes to sink so the loads are not removed.
#include "kernels_common.h"

namespace tq {

namespace {
constexpr int kDiagThreads = 256;
constexpr int kDiagLoads = 4;
constexpr size_t kDiagBlockBytes = size_t{kDiagThreads} * kDiagLoads * 16;  // 16 KiB per block

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kDiagThreads) void stream_kernel(const u4* __restrict__ src, int64_t n16_read,
                                                              u4* __restrict__ dst, int64_t n16_write,
                                                              int64_t read_blocks, uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kDiagThreads / kWave];
  if (static_cast<int64_t>(blockIdx.x) < read_blocks) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kDiagThreads * kDiagLoads + threadIdx.x;
    u4 v[kDiagLoads];
#pragma unroll
    for (int j = 0; j < kDiagLoads; ++j) {
      const int64_t i = base + static_cast<int64_t>(j) * kDiagThreads;
      v[j] = i < n16_read ? __builtin_nontemporal_load(&src[i]) : u4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kDiagLoads; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), m, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t y = 0;
      for (int w = 0; w < kDiagThreads / kWave; ++w) y ^= part[w];
      sink[blockIdx.x] = y;
    }
  } else {
    const int64_t base = (static_cast<int64_t>(blockIdx.x) - read_blocks) * kDiagThreads * kDiagLoads + threadIdx.x;
    const u4 w = {blockIdx.x, threadIdx.x, 0x9E3779B9u, 0x7F4A7C15u};
#pragma unroll
    for (int j = 0; j < kDiagLoads; ++j) {
      const int64_t i = base + static_cast<int64_t>(j) * kDiagThreads;
      if (i < n16_write) __builtin_nontemporal_store(w, &dst[i]);
    }
  }
}
}  // namespace

int64_t diag_stream_sink_words(size_t read_bytes) {
  return static_cast<int64_t>((read_bytes + kDiagBlockBytes - 1) / kDiagBlockBytes);
}

hipError_t launch_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes, uint32_t* sink,
                         hipStream_t s) {
  const int64_t rb = diag_stream_sink_words(read_bytes);
  const int64_t wb = static_cast<int64_t>((write_bytes + kDiagBlockBytes - 1) / kDiagBlockBytes);
  if (rb + wb == 0) return hipSuccess;
  hipLaunchKernelGGL(stream_kernel, dim3(static_cast<unsigned>(rb + wb)), dim3(kDiagThreads), 0, s,
                     static_cast<const u4*>(src), static_cast<int64_t>(read_bytes / 16), static_cast<u4*>(dst),
                     static_cast<int64_t>(write_bytes / 16), rb, sink);
  return hipGetLastError();
}

}  // namespace tq
