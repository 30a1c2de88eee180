// Prefill kernel (large M) of the W4A16 linear for gfx950: a tiled fp16 MFMA GEMM
// whose weight tiles are dequantized from packed INT4 into LDS, with the sparse
// outlier term added into the same fp32 accumulators.
//
// At large batch the weight-only product turns compute-bound once the weights are
// dequantized to fp16 (MixQ news item: weight-only quantization can fall behind
// fp16 at many concurrent requests), and dequantization on the slower vector
// units can cost a large share of the runtime (QServe, DeepCompressor README).
// Here every weight is dequantized once per block into an fp16 LDS tile shared by
// all waves of the block, so the vector work per weight is amortized over BM rows
// of activations.
//
// Block tile BM x BN, K step 64 (half a quantization group, so one (s, z) per
// weight row per step), WM x WN waves each owning a (BM/WM) x (BN/WN) tile of
// 16x16 fp32 accumulators fed by v_mfma_f32_16x16x32_f16.
//  - Activation tile: 128-bit global loads, each chunk of eight reordered (perm_x8)
//    to match the dequantized weight order, stored to LDS.
//  - Weight tile: one 128-bit load of four packed words per thread, dequantized
//    to fp16 (q - z) * s (one rounding) and stored to LDS in the same order.
//  - LDS rows are padded to 72 halves (144 B) so the 16-byte fragment reads of 16
//    consecutive rows fall in distinct banks. Two LDS stages: the global loads of
//    step s+1 are in flight while step s computes; one barrier per step.
//  - Sparse term: each lane follows the CSR rows of its columns with a cursor; an
//    entry whose column falls in the current K step reads its activations from the
//    LDS tile already there, so no extra global traffic and no atomics.
#include "wq_device.h"
#include "wq_launch.h"

#include <climits>

namespace wq {

constexpr int kBK = 64;
constexpr int kLdsStride = 72;  // halves per LDS row (64 + 8 padding)

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
            const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
            const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
            const f16* __restrict__ val, void* __restrict__ y, int y_f32) {
  constexpr int T = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MT = TM / 16, NT = TN / 16;
  constexpr int XV = BM * (kBK / 8) / T;   // 128-bit activation loads per thread per step
  constexpr int WV = BN * (kBK / 32) / T;  // 128-bit weight loads per thread per step
  static_assert(XV * T == BM * (kBK / 8) && WV * T == BN * (kBK / 32) && WV >= 1, "tile/thread mismatch");
  constexpr int STAGE = (BM + BN) * kLdsStride;  // halves per LDS stage

  extern __shared__ __align__(16) f16 smem[];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int G = K >> 7;
  const size_t KW8 = (size_t)(K >> 3);

  // producer coordinates
  int x_row[XV], x_ch[XV];
  bool x_ok[XV];
#pragma unroll
  for (int i = 0; i < XV; ++i) {
    const int idx = t + i * T;
    x_row[i] = idx >> 3;
    x_ch[i] = idx & 7;
    x_ok[i] = (m0 + x_row[i]) < M;
  }
  int w_row[WV], w_hf[WV], w_n[WV];
#pragma unroll
  for (int i = 0; i < WV; ++i) {
    const int idx = t + i * T;
    w_row[i] = idx >> 1;
    w_hf[i] = idx & 1;
    w_n[i] = min(n0 + w_row[i], N - 1);
  }

  uint4 xr[XV], wr[WV];
  f16 sr[WV], zr[WV];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XV; ++i)
      xr[i] = x_ok[i] ? *reinterpret_cast<const uint4*>(x + (size_t)(m0 + x_row[i]) * K + k0 + 8 * x_ch[i])
                      : make_uint4(0u, 0u, 0u, 0u);
    const int g = k0 >> 7;
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      wr[i] = *reinterpret_cast<const uint4*>(packed + (size_t)w_n[i] * KW8 + (k0 >> 3) + 4 * w_hf[i]);
      sr[i] = scales[(size_t)w_n[i] * G + g];
      zr[i] = zeros[(size_t)w_n[i] * G + g];
    }
  };
  auto store_step = [&](f16* st) {
    f16* xs = st;
    f16* ws = st + BM * kLdsStride;
#pragma unroll
    for (int i = 0; i < XV; ++i)
      *reinterpret_cast<uint4*>(xs + x_row[i] * kLdsStride + 8 * x_ch[i]) = perm_x8(xr[i]);
#pragma unroll
    for (int i = 0; i < WV; ++i) {
      const f16 zb = (f16)1024.0f + zr[i];
      const f16x2 bias = {zb, zb};
      const f16x2 s2 = {sr[i], sr[i]};
      f16* dst = ws + w_row[i] * kLdsStride + 32 * w_hf[i];
      *reinterpret_cast<uint4*>(dst + 0) = dequant_word(wr[i].x, bias, s2);
      *reinterpret_cast<uint4*>(dst + 8) = dequant_word(wr[i].y, bias, s2);
      *reinterpret_cast<uint4*>(dst + 16) = dequant_word(wr[i].z, bias, s2);
      *reinterpret_cast<uint4*>(dst + 24) = dequant_word(wr[i].w, bias, s2);
    }
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = {0.f, 0.f, 0.f, 0.f};

  // sparse cursors, one per accumulator column of this lane
  int cur[NT], cend[NT], ccol[NT];
  float cval[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = n0 + wn * TN + j * 16 + (lane & 15);
    cur[j] = 0;
    cend[j] = 0;
    if (row_ptr != nullptr && n < N) {
      cur[j] = row_ptr[n];
      cend[j] = row_ptr[n + 1];
    }
    ccol[j] = cur[j] < cend[j] ? col[cur[j]] : INT_MAX;
    cval[j] = cur[j] < cend[j] ? (float)val[cur[j]] : 0.f;
  }

  const int nk = K / kBK;
  load_step(0);
  store_step(smem);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int k0 = s * kBK;
    f16* st = smem + (s & 1) * STAGE;
    if (s + 1 < nk) load_step(k0 + kBK);
    const f16* xs = st;
    const f16* ws = st + BM * kLdsStride;
#pragma unroll
    for (int kc = 0; kc < kBK; kc += 32) {
      f16x8 a[MT], b[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(xs + (wm * TM + i * 16 + (lane & 15)) * kLdsStride + kc +
                                               8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(ws + (wn * TN + j * 16 + (lane & 15)) * kLdsStride + kc +
                                               8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
    }
    // sparse entries whose column lies in [k0, k0 + 64)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      while (ccol[j] < k0 + kBK) {
        const int kk = ccol[j] - k0;
        const int slot = (kk & ~7) | perm_slot(kk & 7);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i][j][q] += cval[j] * (float)xs[(wm * TM + i * 16 + 4 * (lane >> 4) + q) * kLdsStride + slot];
        ++cur[j];
        ccol[j] = cur[j] < cend[j] ? col[cur[j]] : INT_MAX;
        cval[j] = cur[j] < cend[j] ? (float)val[cur[j]] : 0.f;
      }
    }
    if (s + 1 < nk) store_step(smem + ((s + 1) & 1) * STAGE);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wn * TN + j * 16 + (lane & 15);
      if (n >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * TM + i * 16 + 4 * (lane >> 4) + q;
        if (m < M) {
          const size_t o = (size_t)m * N + n;
          if (y_f32)
            static_cast<float*>(y)[o] = acc[i][j][q];
          else
            static_cast<f16*>(y)[o] = (f16)acc[i][j][q];
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_gemm_tile(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                                   const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                   const int32_t* row_ptr, const int32_t* col, const uint16_t* val, void* y,
                                   int y_f32, hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)(BM + BN) * kLdsStride * sizeof(f16);
  auto kern = gemm_kernel<BM, BN, WM, WN>;
  static bool attr_done = false;  // a benign race: setting the same attribute twice is harmless
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  constexpr int64_t kRowsPerLaunch = (int64_t)65535 * BM;  // gridDim.y limit
  const size_t ysz = y_f32 ? 4 : 2;
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((mc + BM - 1) / BM));
    hipLaunchKernelGGL(kern, grid, dim3(64 * WM * WN), lds, stream, reinterpret_cast<const f16*>(x) + m * K,
                       (int)mc, (int)K, packed, reinterpret_cast<const f16*>(scales),
                       reinterpret_cast<const f16*>(zeros), (int)N, row_ptr, col,
                       reinterpret_cast<const f16*>(val), static_cast<char*>(y) + (size_t)(m * N) * ysz, y_f32);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  return launch_gemm_tile<128, 128, 2, 2>(x, M, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32,
                                          stream);
}

}  // namespace wq
