// Down-projection of the low-rank high-precision branch for gfx950.
//
// The SVDQuant section of the DeepCompressor README keeps the weights' outliers in
// a high-precision low-rank branch next to the 4-bit residual, and fuses that
// branch into the low-bit kernel rather than running it as a separate pass over
// the activations. With W = L2 . L1 + R (L1 [r, K], L2 [N, r], fp16), the product
// needs t = x . L1^T first; the linear kernels then add t . L2^T to each output
// tile before its single store. This file computes t:
//
//  lowrank_down_kernel: one block per 16 rows of x, 16 components of the rank and
//    chunk of 32 steps of 32 input channels; each of its four waves takes every
//    fourth step of the chunk, with all its loads issued up front, and feeds one
//    16x16x32 fp16 MFMA per step (x rows in A, rows of L1 in B, fp32
//    accumulation). The waves' tiles are summed through LDS in a fixed order and
//    stored as the chunk's fp32 partial.
//  lowrank_finish_kernel: t = fp16 of the fixed-order sum of the chunks' partials
//    (one rounding, since t is an MFMA operand of the up-projection).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

constexpr int kLrChunkSteps = 32;  // 32-channel steps per K chunk
constexpr int kLrStepsPerWave = kLrChunkSteps / 4;

size_t lowrank_partial_bytes(int64_t M, int64_t K, int64_t r) {
  const int64_t chunks = (K / 32 + kLrChunkSteps - 1) / kLrChunkSteps;
  return ((size_t)chunks * M * r * 4 + 255) / 256 * 256;
}

__global__ void __launch_bounds__(256)
lowrank_down_kernel(const f16* __restrict__ x, int M, int K, const f16* __restrict__ L1, int r,
                    float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & 15, h = lane >> 4;
  const int j0 = blockIdx.x * 16, m0 = blockIdx.y * 16, chunk = blockIdx.z;
  const int s0 = chunk * kLrChunkSteps, s1 = min(K / 32, s0 + kLrChunkSteps);
  // lane (h, q): row m0 + q of x (rows past M read row M - 1, never stored) and
  // component j0 + q of L1 (r is a multiple of 32), channels 32 s + 8 h .. + 7
  const f16* xr = x + (size_t)min(m0 + q, M - 1) * K + 8 * h;
  const f16* lr = L1 + (size_t)(j0 + q) * K + 8 * h;
  uint4 av[kLrStepsPerWave], bv[kLrStepsPerWave];
#pragma unroll
  for (int i = 0; i < kLrStepsPerWave; ++i) {
    const int s = min(s0 + wave + 4 * i, s1 - 1);  // steps past the chunk reload its last one, unused
    av[i] = *reinterpret_cast<const uint4*>(xr + 32 * s);
    bv[i] = *reinterpret_cast<const uint4*>(lr + 32 * s);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kLrStepsPerWave; ++i)
    if (s0 + wave + 4 * i < s1)  // wave-uniform
      acc = mfma_16x16x32(as_f16x8(av[i]), as_f16x8(bv[i]), acc);
  __shared__ f32x4 red[3][64];
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += red[w][lane];
  // D[4 h + i][q]: row m0 + 4 h + i, component j0 + q
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * h + i;
    if (m < M) part[((size_t)chunk * M + m) * r + j0 + q] = acc[i];
  }
}

__global__ void __launch_bounds__(256)
lowrank_finish_kernel(const float* __restrict__ part, int chunks, int64_t Mr, f16* __restrict__ t) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < Mr; i += stride) {
    float v = part[i];
    for (int c = 1; c < chunks; ++c) v += part[(size_t)c * Mr + i];
    t[i] = (f16)v;
  }
}

hipError_t launch_lowrank_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* L1, int64_t r,
                               float* part, uint16_t* t, hipStream_t stream) {
  const int chunks = (int)((K / 32 + kLrChunkSteps - 1) / kLrChunkSteps);
  constexpr int64_t kRowsPerLaunch = 65535 * 16;  // gridDim.y limit
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const dim3 grid((unsigned)(r / 16), (unsigned)((mc + 15) / 16), (unsigned)chunks);
    hipLaunchKernelGGL(lowrank_down_kernel, grid, dim3(256), 0, stream, reinterpret_cast<const f16*>(x) + m * K,
                       (int)mc, (int)K, reinterpret_cast<const f16*>(L1), (int)r, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t Mr = mc * r;
    const int64_t blocks = (Mr + 255) / 256 < 1024 ? (Mr + 255) / 256 : 1024;
    hipLaunchKernelGGL(lowrank_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, chunks, Mr,
                       reinterpret_cast<f16*>(t) + m * r);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
