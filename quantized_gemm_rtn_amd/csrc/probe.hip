// Measurement aid, not part of the product: a plain streaming read, the context
// against which the decode kernels' HBM rate is judged (what one launch of a
// read-only kernel reaches at the same byte count). Built into libwq_probe.so,
// declared in include/wq_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wq_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads per thread in flight, like the decode kernels' window

// Block b reads the kThreads * kUnroll 16-byte chunks starting at chunk
// b * kThreads * kUnroll (coalesced: consecutive threads read consecutive chunks),
// all loads issued before any is used. The XOR of the loaded words keeps the loads
// alive; it is stored only if it equals a constant, so the kernel writes (almost)
// nothing.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  uint4 v[kUnroll];
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int64_t c = base + (int64_t)i * kThreads;
    v[i] = src[c < n16 ? c : n16 - 1];
  }
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) a ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (a == 0x9E3779B9u) sink[0] = a;
}

}  // namespace

extern "C" int wq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return -1;
  if (bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return -2;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int64_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return -2;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
