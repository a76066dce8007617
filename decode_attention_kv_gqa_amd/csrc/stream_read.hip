// A plain streaming read of a device buffer on gfx950: the practical HBM
// read rate of the machine, which the attention kernels' rates are set
// beside.  Not part of the decode path.
//
// Every workgroup walks a grid-stride share of the buffer in 16-byte
// non-temporal loads, four per lane in flight (the best of the launch shapes
// measured on MI355X for a 277 MB buffer: 6.9-7.0 TB/s at 512 workgroups),
// and folds every word it read into an XOR that it stores to sink[workgroup]
// at the end: the loads cannot be dropped, and the XOR of the sink words is
// the XOR of the whole buffer, which the caller can check.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 4;   // 16-byte loads per lane between waits

__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* __restrict__ src,
                                                        size_t n16, uint32_t* __restrict__ sink) {
  const size_t step = (size_t)gridDim.x * kThreads * kInFlight;
  uint32_t x = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads * kInFlight + threadIdx.x; i < n16; i += step) {
    u32x4 w[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const size_t j = i + (size_t)u * kThreads;
      w[u] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= w[u][0] ^ w[u][1] ^ w[u][2] ^ w[u][3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) y ^= part[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

extern "C" int gqa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                     int workgroups, void* stream) {
  if (!src || !sink) return GQA_ERR_NULL;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 || workgroups < 1)
    return GQA_ERR_SHAPE;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)workgroups), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4*>(src),
                     bytes / 16, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}
