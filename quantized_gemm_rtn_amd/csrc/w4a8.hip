// W4A8 product with fp16 outlier channels, for gfx950.
//
// The MixQ news item runs the bulk of a layer with 8-bit activations on integer
// matrix units and keeps a few activation channels, the outliers (the same
// channels from one decode step to the next), in high precision, adding the two
// products in registers. Here the weights stay the INT4 g128 layer of the other
// entry points, and per row (token) of x:
//   s_x = fl32(amax / 127) over the non-outlier channels (1 when amax is 0),
//   xq  = clamp(rint(fl32(x / s_x)), -127, 127), 0 on the outlier channels,
//   y[m, n] = s_x[m] * sum_g s[n, g] * sum_{k in g} xq[m, k] * (q[n, k] - z[n, g])
//           + sum_j x[m, o_j] * w_hat[n, o_j].
//
//  act_int8_kernel: one block per row: amax (outlier channels skipped), then the
//    INT8 values, written in the order the weights' nibbles unpack to: in each 16
//    channels, bytes hold channels 0,2,4,6,1,3,5,7, 8,10,12,14,9,11,13,15 (masking a
//    code word with 0x0F0F0F0F gives its even codes as bytes, shifting it by 4 the
//    odd ones); the fp16 outlier values, padded with zeros to 16 per row.
//  outlier_weights_kernel: w_hat of the outlier channels, fp16 [N][16] (zeros
//    past n_out), the B operand of one fp16 MFMA per output tile.
//  w4a8_gemm_kernel: 128 x 128 output tiles, four waves of 2 x 2 tiles of
//    32x32x32 INT8 MFMAs. Per group of 128 channels the block stages the group's
//    activations and codes in LDS with coalesced loads (the next group's loads in
//    flight during this group's MFMAs, two LDS buffers); a lane reads 64 bytes of
//    xq per row tile and 8 code words per column tile (channels 64 h .. 64 h + 63
//    of the group for lane half h, so the k positions of A and B agree lane by
//    lane), subtracts the zero-point from the code bytes
//    ((b | 0x80) - z, then ^ 0x80: no borrow crosses bytes since b + 128 > z), and
//    sums four MFMAs exactly in int32; the group's sum is scaled by s[n, g] into
//    fp32. The epilogue multiplies by s_x of the row and adds the outlier product.
//
// Arithmetic that decides an integer (s_x, xq) is IEEE float32 with correctly
// rounded division and round-half-even, as in the definition; the file is built
// with -ffp-contract=off.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxOutliers = 16;

// bit e set: channel 16 c + e is an outlier (one pass over the list per 16 channels)
__device__ __forceinline__ uint32_t outlier_bits(int c, const int* o, int n_out) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kMaxOutliers; ++j) m |= (j < n_out && (o[j] >> 4) == c) ? 1u << (o[j] & 15) : 0u;
  return m;
}

__global__ void __launch_bounds__(256)
act_int8_kernel(const f16* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ outliers, int n_out,
                int8_t* __restrict__ xq, float* __restrict__ sx, f16* __restrict__ xo) {
  __shared__ float red[4];
  __shared__ int o[kMaxOutliers];
  // indices out of [0, K) are clamped here, once, for the mask and the gather alike
  if (threadIdx.x < kMaxOutliers)
    o[threadIdx.x] = (int)threadIdx.x < n_out ? min(max(outliers[threadIdx.x], 0), K - 1) : -1;
  __syncthreads();
  int ol[kMaxOutliers];
#pragma unroll
  for (int j = 0; j < kMaxOutliers; ++j) ol[j] = o[j];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunks = K >> 4;  // 16 channels per thread and pass
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const f16* row = x + m * K;
    float amax = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += 256) {
      const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * c);
      const uint4 b = *reinterpret_cast<const uint4*>(row + 16 * c + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const uint32_t om = outlier_bits(c, ol, n_out);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = fabsf((float)__builtin_bit_cast(f16, (uint16_t)(w[e >> 1] >> (16 * (e & 1)))));
        if (!((om >> e) & 1u)) amax = fmaxf(amax, v);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 1.0f;
    if (threadIdx.x == 0) sx[m] = s;
    if (threadIdx.x < kMaxOutliers)
      xo[m * kMaxOutliers + threadIdx.x] =
          (int)threadIdx.x < n_out ? row[ol[threadIdx.x]] : (f16)0.0f;
    for (int c = threadIdx.x; c < chunks; c += 256) {
      const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * c);
      const uint4 b = *reinterpret_cast<const uint4*>(row + 16 * c + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const uint32_t om = outlier_bits(c, ol, n_out);
      int qv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = (float)__builtin_bit_cast(f16, (uint16_t)(w[e >> 1] >> (16 * (e & 1))));
        float t = fminf(fmaxf(rintf(__fdiv_rn(v, s)), -127.0f), 127.0f);
        qv[e] = ((om >> e) & 1u) ? 0 : (int)t;
      }
      // byte order of the 16 channels: 0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15
      constexpr int ord[16] = {0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15};
      uint32_t d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        d[j] = (uint32_t)(qv[ord[4 * j]] & 0xFF) | ((uint32_t)(qv[ord[4 * j + 1]] & 0xFF) << 8) |
               ((uint32_t)(qv[ord[4 * j + 2]] & 0xFF) << 16) | ((uint32_t)(qv[ord[4 * j + 3]] & 0xFF) << 24);
      *reinterpret_cast<uint4*>(xq + m * K + 16 * c) = make_uint4(d[0], d[1], d[2], d[3]);
    }
    __syncthreads();  // red[] is reused by the next row
  }
}

__global__ void __launch_bounds__(256)
outlier_weights_kernel(const uint32_t* __restrict__ packed, const f16* __restrict__ scales,
                       const f16* __restrict__ zeros, int64_t N, int K, const int32_t* __restrict__ outliers,
                       int n_out, f16* __restrict__ wo) {
  const int64_t total = N * kMaxOutliers;
  const int G = K >> 7;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t n = i / kMaxOutliers;
    const int j = (int)(i - n * kMaxOutliers);
    f16 v = (f16)0.0f;
    if (j < n_out) {
      const int k = min(max(outliers[j], 0), K - 1);
      const uint32_t code = (packed[n * (K >> 3) + (k >> 3)] >> (4 * (k & 7))) & 0xFu;
      const int g = k >> 7;
      const float s = (float)scales[n * G + g], z = (float)zeros[n * G + g];
      v = (f16)(((float)code - z) * s);
    }
    wo[i] = v;
  }
}

// Group tiles in LDS: activations 128 rows x 128 bytes (row stride 144 bytes) and
// codes 128 columns x 64 bytes (stride 80 bytes), two buffers. The strides put the
// 16-byte fragment reads of eight consecutive lanes (rows or columns 144 or 80
// bytes apart) in distinct banks.
constexpr int kW8AStride = 144, kW8BStride = 80;
constexpr int kW8ABytes = 128 * kW8AStride, kW8BBytes = 128 * kW8BStride;

// 32x32 fp32 / int32 MFMA results: register r of lane (c, h) (c = lane % 32,
// h = lane / 32) holds row 8 (r / 4) + 4 h + r % 4, column c.
__global__ void __launch_bounds__(256)
w4a8_gemm_kernel(const int8_t* __restrict__ xq, const float* __restrict__ sx, const f16* __restrict__ xo,
                 int M, int K, const uint32_t* __restrict__ packed, const f16* __restrict__ scales,
                 const f16* __restrict__ zeros, const f16* __restrict__ wo, int N, void* __restrict__ y,
                 int y_f32) {
  __shared__ __align__(16) char lds[2 * (kW8ABytes + kW8BBytes)];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 31, h = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int mb = blockIdx.y * 128, nb = blockIdx.x * 128;
  const int m0 = mb + wm * 64, n0 = nb + wn * 64;
  const int G = K >> 7;
  // staging: thread t copies 16-byte chunk (t + 256 i) & 7 of activation row (t + 256 i) >> 3
  // (i < 4) and chunk (t + 256 i) & 3 of code column (t + 256 i) >> 2 (i < 2): a wave's
  // load covers 8 whole rows, or the 64-byte groups of 16 columns. Rows past M and
  // columns past N reread the last one and are never stored.
  // (32-bit byte offsets: M K and N K / 2 are below 2^31; chunk i of a thread sits
  // 32 i rows or 64 i columns after chunk 0 in LDS)
  uint32_t ag[4], bg[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (t >> 3) + 32 * i;
    ag[i] = (uint32_t)min(mb + row, M - 1) * (uint32_t)K + 16u * (uint32_t)(t & 7);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cl = (t >> 2) + 64 * i;
    bg[i] = (uint32_t)min(nb + cl, N - 1) * (uint32_t)(K >> 1) + 16u * (uint32_t)(t & 3);
  }
  const int al0 = (t >> 3) * kW8AStride + 16 * (t & 7), bl0 = (t >> 2) * kW8BStride + 16 * (t & 3);
  const char* xqb = reinterpret_cast<const char*>(xq);
  const char* pkb = reinterpret_cast<const char*>(packed);
  // The staged data of the next group (plain scalars: held in arrays captured by a
  // lambda, the compiler moved them to LDS).
  uint4 p0, p1, p2, p3, p4, p5;
#define WQ_W8_FETCH(g, r0, r1, r2, r3, r4, r5)                          \
  r0 = *reinterpret_cast<const uint4*>(xqb + ag[0] + 128 * (g));        \
  r1 = *reinterpret_cast<const uint4*>(xqb + ag[1] + 128 * (g));        \
  r2 = *reinterpret_cast<const uint4*>(xqb + ag[2] + 128 * (g));        \
  r3 = *reinterpret_cast<const uint4*>(xqb + ag[3] + 128 * (g));        \
  r4 = *reinterpret_cast<const uint4*>(pkb + bg[0] + 64 * (g));         \
  r5 = *reinterpret_cast<const uint4*>(pkb + bg[1] + 64 * (g));
#define WQ_W8_STASH(buf, r0, r1, r2, r3, r4, r5)                        \
  {                                                                     \
    char* A_ = lds + (buf) * (kW8ABytes + kW8BBytes);                   \
    char* B_ = A_ + kW8ABytes;                                          \
    *reinterpret_cast<uint4*>(A_ + al0) = r0;                           \
    *reinterpret_cast<uint4*>(A_ + al0 + 32 * kW8AStride) = r1;         \
    *reinterpret_cast<uint4*>(A_ + al0 + 64 * kW8AStride) = r2;         \
    *reinterpret_cast<uint4*>(A_ + al0 + 96 * kW8AStride) = r3;         \
    *reinterpret_cast<uint4*>(B_ + bl0) = r4;                           \
    *reinterpret_cast<uint4*>(B_ + bl0 + 64 * kW8BStride) = r5;         \
  }
  int col[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) col[j] = min(n0 + 32 * j + c, N - 1);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  // group x's data: LDS buffer x & 1
  WQ_W8_FETCH(0, p0, p1, p2, p3, p4, p5);
  WQ_W8_STASH(0, p0, p1, p2, p3, p4, p5);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    if (g + 1 < G) {  // in flight during this group's MFMAs
      WQ_W8_FETCH(g + 1, p0, p1, p2, p3, p4, p5);
    }
    float sc[2];
    uint32_t zz[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sc[j] = (float)scales[(size_t)col[j] * G + g];
      zz[j] = (uint32_t)(int)(float)zeros[(size_t)col[j] * G + g] * 0x01010101u;
    }
    const char* A = lds + (g & 1) * (kW8ABytes + kW8BBytes);
    const char* B = A + kW8ABytes;
    // lane (c, h): channels 64 h .. 64 h + 63 of the group, 16 per step
    uint4 w[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const char* bp = B + (wn * 64 + 32 * j + c) * kW8BStride + 32 * h;
      w[j][0] = *reinterpret_cast<const uint4*>(bp);
      w[j][1] = *reinterpret_cast<const uint4*>(bp + 16);
    }
    i32x16 part[2][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      i32x4 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const i32x4*>(A + (wm * 64 + 32 * i + c) * kW8AStride + 64 * h + 16 * s);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t* wd = reinterpret_cast<const uint32_t*>(&w[j][0]);
        const uint32_t w0 = wd[2 * s], w1 = wd[2 * s + 1];
        const uint32_t d[4] = {w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
        for (int e = 0; e < 4; ++e) b[j][e] = (int)(((d[e] | 0x80808080u) - zz[j]) ^ 0x80808080u);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          part[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], s == 0 ? i32x16{} : part[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] += sc[j] * (float)part[i][j][r];
    // the other buffer was last read in the previous group, before its barrier
    // the other buffer was last read in the previous group, before its barrier
    if (g + 1 < G) WQ_W8_STASH((g + 1) & 1, p0, p1, p2, p3, p4, p5);
    __syncthreads();
  }
#undef WQ_W8_FETCH
#undef WQ_W8_STASH
  // epilogue: s_x of the row, plus the outlier channels' product (one fp16 MFMA).
  // The row scales of the lane's 32 rows are loaded together first; the output kind
  // is chosen once, and a wave inside M x N stores with no bounds test (tested per
  // element, the kind and the bounds compile to a branch per store).
  float sxv[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) sxv[i][r] = sx[min(m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3), M - 1)];
  const bool full = m0 + 64 <= M && n0 + 64 <= N;
  const auto epilogue = [&](auto* out, auto conv) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const f16x8 ao = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(
                                                     xo + (size_t)min(m0 + 32 * i + c, M - 1) * kMaxOutliers + 8 * h));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f16x8 bo =
            __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(wo + (size_t)col[j] * kMaxOutliers + 8 * h));
        const f32x16 o = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo, f32x16{}, 0, 0, 0);
        const int n = n0 + 32 * j + c;
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            out[(size_t)m * N + n] = conv(sxv[i][r] * acc[i][j][r] + o[r]);
          }
        } else if (n < N) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m < M) out[(size_t)m * N + n] = conv(sxv[i][r] * acc[i][j][r] + o[r]);
          }
        }
      }
    }
  };
  if (y_f32)
    epilogue(static_cast<float*>(y), [](float v) { return v; });
  else
    epilogue(static_cast<f16*>(y), [](float v) { return (f16)v; });
}

size_t w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const auto r256 = [](size_t b) { return (b + 255) / 256 * 256; };
  return r256((size_t)M * K) + r256((size_t)M * 4) + r256((size_t)M * kMaxOutliers * 2) +
         r256((size_t)N * kMaxOutliers * 2);
}

hipError_t launch_act_int8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                           int8_t* xq, float* sx, uint16_t* xo, hipStream_t stream) {
  const int64_t blocks = M < 65536 ? M : 65536;
  hipLaunchKernelGGL(act_int8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<const f16*>(x),
                     M, (int)K, outliers, (int)n_out, xq, sx, reinterpret_cast<f16*>(xo));
  return hipGetLastError();
}

hipError_t launch_w4a8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                       const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, void* y,
                       int y_f32, void* workspace, hipStream_t stream) {
  const auto r256 = [](size_t b) { return (b + 255) / 256 * 256; };
  char* ws = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws);
  float* sx = reinterpret_cast<float*>(ws + r256((size_t)M * K));
  uint16_t* xo = reinterpret_cast<uint16_t*>(ws + r256((size_t)M * K) + r256((size_t)M * 4));
  uint16_t* wo = reinterpret_cast<uint16_t*>(ws + r256((size_t)M * K) + r256((size_t)M * 4) +
                                             r256((size_t)M * kMaxOutliers * 2));
  hipError_t e = launch_act_int8(x, M, K, outliers, n_out, xq, sx, xo, stream);
  if (e != hipSuccess) return e;
  int64_t wblocks = (N * kMaxOutliers + 255) / 256;
  wblocks = wblocks > 65536 ? 65536 : wblocks;
  hipLaunchKernelGGL(outlier_weights_kernel, dim3((unsigned)wblocks), dim3(256), 0, stream, packed,
                     reinterpret_cast<const f16*>(scales), reinterpret_cast<const f16*>(zeros), N, (int)K, outliers,
                     (int)n_out, reinterpret_cast<f16*>(wo));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int64_t kRowsPerLaunch = 65535 * 128;  // gridDim.y limit
  const size_t ysz = y_f32 ? 4 : 2;
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    hipLaunchKernelGGL(w4a8_gemm_kernel, dim3((unsigned)((N + 127) / 128), (unsigned)((mc + 127) / 128)), dim3(256),
                       0, stream, xq + m * K, sx + m, reinterpret_cast<const f16*>(xo) + m * kMaxOutliers, (int)mc,
                       (int)K, packed, reinterpret_cast<const f16*>(scales), reinterpret_cast<const f16*>(zeros),
                       reinterpret_cast<const f16*>(wo), (int)N, static_cast<char*>(y) + (size_t)(m * N) * ysz,
                       y_f32);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
