// Act-order layers through a channel permutation, for gfx950.
//
// The GPTQ-R rows (GPTQ with reordering) of the DeepCompressor README perplexity
// table quantize the input channels in a permuted order, so that a group of 128
// consecutive channels in that order is a scattered set of channels in the
// original one (a per-channel group index). Here such a layer is kept in the
// permuted channel order: channel i of its codes, metadata and CSR columns is
// input channel perm[i]. Then the quantizer and the product of the plain layout
// apply unchanged, to W and to x with their columns gathered through perm:
//   y = x . W^T = x[:, perm] . W[:, perm]^T.
//
//  gather_cols_kernel<T>: dst[r, i] = src[r, perm[i]] for a row-major [rows, K]
//    matrix of fp16 (x) or fp32 (W), eight output channels per thread: eight
//    indices from one 32-byte load of perm, eight element loads (from cache: a
//    row of x is a few KB), one 16- or 32-byte store. Indices outside [0, K) are
//    clamped, so a wrong perm gives wrong values, never a wild read. Used for W
//    (offline) and for batches of at most 16 rows: there, staging whole rows in
//    LDS measured slower (fewer blocks, each with a long serial copy).
//  gather_rows_lds_kernel: larger batches of fp16 rows. Element loads scattered
//    over a row make every load instruction touch up to 64 cache lines, so each
//    block copies R whole rows (contiguous in memory) into LDS with 16-byte loads,
//    then gathers from LDS through perm (read once per R rows) and stores 16
//    bytes per eight channels. R rows of K halves fit in 64 KB. When the row
//    blocks alone cannot fill the GPU, blockIdx.y splits a row's output channels
//    over several blocks, each staging the whole row.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

template <typename T>
__global__ void __launch_bounds__(256)
gather_cols_kernel(const T* __restrict__ src, int64_t rows, int64_t K, const int32_t* __restrict__ perm,
                   T* __restrict__ dst) {
  const int64_t chunks = K >> 3;  // K is a multiple of 8
  const int64_t total = rows * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / chunks, c = i - r * chunks;
    const int4 p0 = *reinterpret_cast<const int4*>(perm + 8 * c);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + 8 * c + 4);
    const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    const T* row = src + r * K;
    T v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = row[min(max(idx[e], 0), (int)K - 1)];
    T* out = dst + r * K + 8 * c;
    if constexpr (sizeof(T) == 2) {
      uint4 w;
      uint32_t* wd = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wd[e] = (uint32_t)__builtin_bit_cast(uint16_t, v[2 * e]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, v[2 * e + 1]) << 16);
      *reinterpret_cast<uint4*>(out) = w;
    } else {
      *reinterpret_cast<float4*>(out) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(out + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

__global__ void __launch_bounds__(256)
gather_rows_lds_kernel(const f16* __restrict__ src, int64_t M, int K, const int32_t* __restrict__ perm, int R,
                       f16* __restrict__ dst) {
  extern __shared__ __align__(16) f16 rows_lds[];  // R x K
  const int chunks = K >> 3;
  const int per = (chunks + gridDim.y - 1) / gridDim.y;  // output chunks of this block's slice
  const int c_lo = blockIdx.y * per, c_hi = min(chunks, c_lo + per);
  for (int64_t m0 = (int64_t)blockIdx.x * R; m0 < M; m0 += (int64_t)gridDim.x * R) {
    const int rows = (int)(M - m0 < R ? M - m0 : R);
    const uint4* s4 = reinterpret_cast<const uint4*>(src + m0 * K);
    for (int i = threadIdx.x; i < rows * chunks; i += 256) reinterpret_cast<uint4*>(rows_lds)[i] = s4[i];
    __syncthreads();
    for (int c = c_lo + threadIdx.x; c < c_hi; c += 256) {
      const int4 p0 = *reinterpret_cast<const int4*>(perm + 8 * c);
      const int4 p1 = *reinterpret_cast<const int4*>(perm + 8 * c + 4);
      const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      int ix[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ix[e] = min(max(idx[e], 0), K - 1);
      for (int r = 0; r < rows; ++r) {
        const f16* row = rows_lds + r * K;
        uint4 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, row[ix[0]]) | ((uint32_t)__builtin_bit_cast(uint16_t, row[ix[1]]) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, row[ix[2]]) | ((uint32_t)__builtin_bit_cast(uint16_t, row[ix[3]]) << 16);
        w.z = (uint32_t)__builtin_bit_cast(uint16_t, row[ix[4]]) | ((uint32_t)__builtin_bit_cast(uint16_t, row[ix[5]]) << 16);
        w.w = (uint32_t)__builtin_bit_cast(uint16_t, row[ix[6]]) | ((uint32_t)__builtin_bit_cast(uint16_t, row[ix[7]]) << 16);
        *reinterpret_cast<uint4*>(dst + (m0 + r) * K + 8 * c) = w;
      }
    }
    __syncthreads();  // the next rows overwrite the LDS
  }
}

template <typename T>
static hipError_t launch_gather(const T* src, int64_t rows, int64_t K, const int32_t* perm, T* dst,
                                hipStream_t stream) {
  const int64_t total = rows * (K / 8);
  int64_t blocks = (total + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks);
  hipLaunchKernelGGL(gather_cols_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, stream, src, rows, K, perm, dst);
  return hipGetLastError();
}

hipError_t launch_gather_cols_f16(const uint16_t* src, int64_t rows, int64_t K, const int32_t* perm, uint16_t* dst,
                                  hipStream_t stream) {
  constexpr int64_t kLdsBytes = 65536;
  constexpr int64_t kCus = 256;  // compute units of an MI355X
  if (rows <= 16 || 2 * K > kLdsBytes)
    return launch_gather(reinterpret_cast<const f16*>(src), rows, K, perm, reinterpret_cast<f16*>(dst), stream);
  // rows per block: as many as fit in 64 KB, up to 8, while the grid keeps a block per CU
  int64_t R = kLdsBytes / (2 * K);
  R = R > 8 ? 8 : R;
  R = R > rows / kCus ? rows / kCus : R;
  R = R < 1 ? 1 : R;
  int64_t blocks = (rows + R - 1) / R;
  blocks = blocks > 65536 ? 65536 : blocks;
  // column slices: enough blocks for every CU, each slice at least 256 chunks
  int64_t splits = (kCus + blocks - 1) / blocks;
  const int64_t most = K / 8 / 256;
  splits = splits > most ? most : splits;
  splits = splits < 1 ? 1 : splits;
  hipLaunchKernelGGL(gather_rows_lds_kernel, dim3((unsigned)blocks, (unsigned)splits), dim3(256),
                     (size_t)(R * K * 2), stream,
                     reinterpret_cast<const f16*>(src), rows, (int)K, perm, (int)R, reinterpret_cast<f16*>(dst));
  return hipGetLastError();
}

hipError_t launch_gather_cols_f32(const float* src, int64_t rows, int64_t K, const int32_t* perm, float* dst,
                                  hipStream_t stream) {
  return launch_gather(src, rows, K, perm, dst, stream);
}

}  // namespace wq
