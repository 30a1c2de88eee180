// Decode kernel (M <= 16 rows per tile) of the W4A16 linear for gfx950, with the
// sparse outlier term fused into the same output tile.
//
// y[m, n] = sum_k x[m, k] (q[n, k] - z[n, g]) s[n, g]  +  sum_e val_e x[m, col_e]
//
// Weight-only quantization pays off on memory-bound token generation (AWQ paper,
// section 2), and its speed comes from dequantizing packed 4-bit weights on the
// fly inside the product, without an fp16 copy of W in DRAM (AWQ paper, section
// 1). At M <= 16 the kernel streams N*K/2 bytes of codes once and is bound by
// HBM bandwidth.
//
// Mapping (one 16-column tile of N per block, KW waves splitting K):
//  - Lane l = 16h + r supplies weights of output channel n0 + r and activations of
//    row m0 + r, for the 32 input channels [128g + 32h, 128g + 32h + 32) of each
//    group g: a 128-bit load of four packed words per lane, so the four lanes of
//    one channel read 64 contiguous bytes per group and a wave reads 16 rows.
//  - Each word becomes eight (q - z) values exact in fp16 and feeds one
//    16x16x32 fp16 MFMA with fp32 accumulation (x in rows, W in columns; rows
//    beyond M are zero). The group's fp32 partial is scaled by s once per group,
//    so the scale costs one multiply-add per group instead of one per weight.
//  - Sparse term: each lane walks the CSR row of its column (entries split across
//    the block's waves) and adds val * x in fp32 into the same accumulators.
//  - The KW partial tiles are summed through LDS in a fixed order (no atomics, so
//    results are deterministic) and stored once.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

template <int KW, int U>
__global__ void __launch_bounds__(64 * KW)
gemv_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
            const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
            const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
            const f16* __restrict__ val, void* __restrict__ y, int y_f32) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int G = K >> 7;
  const int n_ld = min(n0 + r, N - 1);  // ragged N: load a valid row, never store it
  const uint32_t* wrow = packed + (size_t)n_ld * (size_t)(K >> 3) + 4 * h;
  const f16* srow = scales + (size_t)n_ld * G;
  const f16* zrow = zeros + (size_t)n_ld * G;
  const bool xv = (m0 + r) < M;
  const f16* xrow = x + (size_t)(xv ? m0 + r : 0) * (size_t)K + 32 * h;
  const int g_lo = (G * wave) / KW, g_hi = (G * (wave + 1)) / KW;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int g = g_lo;
  for (; g + U <= g_hi; g += U) {
    uint4 wv[U];
    f16 sv[U], zv[U];
    uint4 xa[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wv[u] = *reinterpret_cast<const uint4*>(wrow + (size_t)(g + u) * 16);
      sv[u] = srow[g + u];
      zv[u] = zrow[g + u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        xa[u][t] = xv ? *reinterpret_cast<const uint4*>(xrow + (size_t)(g + u) * 128 + 8 * t)
                      : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const f16 zb = (f16)1024.0f + zv[u];
      const f16x2 bias = {zb, zb};
      const uint32_t wds[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        part = mfma_16x16x32(as_f16x8(perm_x8(xa[u][t])), codes_minus_zero(wds[t], bias), part);
      acc += (float)sv[u] * part;
    }
  }
  for (; g < g_hi; ++g) {
    const uint4 wv = *reinterpret_cast<const uint4*>(wrow + (size_t)g * 16);
    const f16 zb = (f16)1024.0f + zrow[g];
    const f16x2 bias = {zb, zb};
    const uint32_t wds[4] = {wv.x, wv.y, wv.z, wv.w};
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 xa = xv ? *reinterpret_cast<const uint4*>(xrow + (size_t)g * 128 + 8 * t)
                          : make_uint4(0u, 0u, 0u, 0u);
      part = mfma_16x16x32(as_f16x8(perm_x8(xa)), codes_minus_zero(wds[t], bias), part);
    }
    acc += (float)srow[g] * part;
  }

  // Sparse outlier term for column n = n0 + r and rows m0 + 4h + i.
  const int n = n0 + r;
  if (row_ptr != nullptr && n < N) {
    const int e1 = row_ptr[n + 1];
    for (int e = row_ptr[n] + wave; e < e1; e += KW) {
      const int c = col[e];
      const float v = (float)val[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * h + i;
        if (m < M) acc[i] += v * (float)x[(size_t)m * K + c];
      }
    }
  }

  if constexpr (KW > 1) {
    __shared__ f32x4 red[KW - 1][64];
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < KW - 1; ++w) acc += red[w][lane];
  }
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * h + i;
    if (m < M) {
      const size_t o = (size_t)m * N + n;
      if (y_f32)
        static_cast<float*>(y)[o] = acc[i];
      else
        static_cast<f16*>(y)[o] = (f16)acc[i];
    }
  }
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  constexpr int KW = 4, U = 4;
  constexpr int64_t kRowsPerLaunch = 65535 * 16;  // gridDim.y limit
  const size_t ysz = y_f32 ? 4 : 2;
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((mc + 15) / 16));
    hipLaunchKernelGGL((gemv_kernel<KW, U>), grid, dim3(64 * KW), 0, stream,
                       reinterpret_cast<const f16*>(x) + m * K, (int)mc, (int)K, packed,
                       reinterpret_cast<const f16*>(scales), reinterpret_cast<const f16*>(zeros), (int)N, row_ptr,
                       col, reinterpret_cast<const f16*>(val), static_cast<char*>(y) + (size_t)(m * N) * ysz,
                       y_f32);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
