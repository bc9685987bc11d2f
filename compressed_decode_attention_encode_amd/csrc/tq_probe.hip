// Streaming-read probe: one pass of 16-byte loads over a device buffer, folded into a
// single word so that no load can be dropped (measurement helper, not the method).
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // independent 16-byte loads in flight per thread

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // a store that practically never happens, but that the compiler cannot rule out
  if (acc == 0x9E3779B9u) sink[0] = acc ^ (uint32_t)i;
}

}  // namespace

extern "C" int tq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || ((uintptr_t)src & 15) || bytes == 0 || (bytes & 15)) return TQ_ERR_INVALID;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return TQ_ERR_HIP;
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + (size_t)kThreads * kUnroll - 1) / ((size_t)kThreads * kUnroll);
  const size_t cap = (size_t)cus * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, n16, sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
