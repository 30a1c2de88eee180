// Decode kernel for a single activation row (M = 1) of the W4A16 linear, with the
// sparse outlier term, for gfx950.
//
// At M = 1 the product is a stream of N*K/2 bytes of codes through a dot product
// with one activation row (AWQ paper, sections 1-2: weight-only quantization pays
// off on memory-bound generation, by dequantizing packed 4-bit weights on the fly).
// The MFMA kernels feed 16 channels to each matrix op and so read 16 rows x 64 bytes
// per load instruction; this kernel reads whole rows instead:
//  - A wave owns R = 4 consecutive output channels (rows of W, K/2 bytes each). Its
//    load instruction j reads 1 KB of one row, contiguous: lane l gets bytes
//    [1024 i + 16 l, + 16) of row r (step j = R i + r), the codes of input channels
//    [2048 i + 32 l, + 32). A lane keeps D steps in flight (a rolling prefetch).
//  - The block (four waves, 16 rows) stages x once in LDS, each run of eight channels
//    in the order the codes unpack to, odd channels pre-scaled by 1/16 (as in the
//    block-staged MFMA kernel). A lane reads the 32 activations of its chunk into
//    registers once per chunk and uses them for the wave's R rows.
//  - Each word unpacks in five instructions to 1024 + q (even channels) and
//    1024 + 16q (odd ones) and meets the activations in four v_dot2_f32_f16 (fp32
//    accumulation). The lane's 32 channels lie in one group, so the zero-point, the
//    1024 bias and the scale come off once per lane and step:
//        sum (q - z) x s = s (P - (1024 + z) S_even - (64 + z) S_odd),
//    with S_even, S_odd the lane's sums of its even and odd activations.
//  - Sparse term: the lanes of a wave split each of its rows' CSR entries (entry
//    e0 + l + 64 u for lane l) and add val * x into the same per-row accumulators;
//    each lane's first entry of each row is loaded in the prologue.
//  - Each row's 64 lane sums are reduced in a fixed order (xor butterfly); no atomics.
#include "gemv_kernels.h"

namespace wq {

constexpr int kDotRows = 4;   // R: rows per wave
constexpr int kDotWaves = 4;  // waves per block
constexpr int kDotDepth = 8;  // D: weight loads in flight per lane
constexpr int kDotChunk = 2048;  // input channels per load instruction (1 KB of codes)

// XV: 16-byte staging loads of x per thread (x has K / 8 of them, K <= 2048 XV)
template <int XV, bool SP>
__global__ void __launch_bounds__(64 * kDotWaves)
gemv_dot_kernel(const f16* __restrict__ x, int K, const uint32_t* __restrict__ packed,
                const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
                const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, const f16* __restrict__ val,
                void* __restrict__ y, int y_f32) {
  constexpr int R = kDotRows, D = kDotDepth, T = 64 * kDotWaves;
  extern __shared__ __align__(16) char smem[];
  const int G = K >> 7;
  // LDS: (s, 1024 + z) of the block's rows, sz[rows][G + 1] | x [K], permuted per 8,
  // odd channels / 16
  f16x2* sz = reinterpret_cast<f16x2*>(smem);
  f16* xs = reinterpret_cast<f16*>(smem + (size_t)kDotWaves * R * (G + 1) * 4);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nb = blockIdx.x * kDotWaves * R;  // first row of the block
  const int n0 = nb + wave * R;               // first row of the wave
  const int C = K / kDotChunk;  // chunks per row (K is a multiple of kDotChunk)
  const int J = R * C;          // steps of the wave, chunk-major: j = R i + r

  // per row: codes of this lane's 32 channels
  const uint32_t* wrow = packed + (size_t)min(n0, N - 1) * (size_t)(K >> 3) + 4 * lane;
  const size_t rstride = (size_t)(K >> 3);
  // CSR bounds of the wave's rows go out first
  int e0[R], e1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    e0[r] = e1[r] = 0;
    if constexpr (SP) {
      const int n = min(n0 + r, N - 1);
      e0[r] = row_ptr[n];
      e1[r] = row_ptr[n + 1];
    }
  }
  // step j's loads (j clamped into the wave's steps: loads are never conditional)
  uint4 wbuf[D];
  auto issue = [&](int slot, int j) {
    const int jj = min(j, J - 1);
    const int i = jj / R, r = jj - i * R;
    // ragged N: rows past N - 1 read row N - 1 (valid), and are never stored
    const size_t ro = (size_t)(min(n0 + r, N - 1) - min(n0, N - 1)) * rstride;
    wbuf[slot] = *reinterpret_cast<const uint4*>(wrow + ro + (size_t)i * (kDotChunk / 8));
  };
  // the block's (s, z), staged like the MFMA decode kernels, 16 rows at a time
  constexpr int SZB = kDotWaves * R / 16;
  static_assert(SZB * 16 == kDotWaves * R, "the block's rows are whole sets of 16");
  SzStage<8, T> szs[SZB];
#pragma unroll
  for (int b = 0; b < SZB; ++b) szs[b].load(scales, zeros, min(nb + 16 * b, N - 1), N, G, t);
  // x staging loads, then the first D steps of weights, then the staging stores (the
  // staging indices are clamped, not tested: a clamped thread rewrites the last vector)
  const int xvecs = K >> 3;
  uint4 xv[XV];
#pragma unroll
  for (int u = 0; u < XV; ++u) xv[u] = *reinterpret_cast<const uint4*>(x + 8 * min(t + u * T, xvecs - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);
  __builtin_amdgcn_sched_barrier(0);
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
#pragma unroll
  for (int u = 0; u < XV; ++u) {
    uint4 p = perm_x8(xv[u]);
    p.y = as_u32(as_f16x2(p.y) * sixteenth);
    p.w = as_u32(as_f16x2(p.w) * sixteenth);
    *reinterpret_cast<uint4*>(xs + 8 * min(t + u * T, xvecs - 1)) = p;
  }
#pragma unroll
  for (int b = 0; b < SZB; ++b)
    szs[b].store(sz + (size_t)16 * b * (G + 1), scales, zeros, min(nb + 16 * b, N - 1), N, G, t);
  // the lane's first CSR entry of each row (entry e0 + lane), behind the weights: the
  // rows' bounds have arrived with the staged activations, and the sum after the main
  // loop then waits for no global load (the 70B down-projection has 14 entries per
  // row, so one per lane covers nearly every row). Indices are clamped into the row,
  // or to entry 0 for an empty row (the kernel takes a CSR only with nnz >= 1).
  int hc[R];
  f16 hv[R];
  if constexpr (SP) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = max(min(e0[r] + lane, e1[r] - 1), 0);
      hc[r] = col[e];
      hv[r] = val[e];
    }
  }
  __syncthreads();
  const f16x2* szw = sz + (size_t)(wave * R) * (G + 1) + (lane >> 2);  // this lane's group column

  const uint32_t magic = magic_1024x2();
  const f16x2 ones = {(f16)1.0f, (f16)1.0f};
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  uint4 xa[4];
  float se = 0.f, so = 0.f;
  // step j in slot j % D
  auto step = [&](int j, int slot) {
    const int i = j / R, r = j - (j / R) * R;
    if (r == 0) {  // a new chunk: this lane's 32 activations and their sums
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xa[q] = *reinterpret_cast<const uint4*>(xs + (size_t)i * kDotChunk + 32 * lane + 8 * q);
      float e = 0.f, o = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e = __builtin_amdgcn_fdot2(as_f16x2(xa[q].x), ones, e, false);
        e = __builtin_amdgcn_fdot2(as_f16x2(xa[q].z), ones, e, false);
        o = __builtin_amdgcn_fdot2(as_f16x2(xa[q].y), ones, o, false);
        o = __builtin_amdgcn_fdot2(as_f16x2(xa[q].w), ones, o, false);
      }
      se = e;
      so = 16.0f * o;  // odd activations were stored / 16
    }
    const uint4 w = wbuf[slot];
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float p = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 b = codes_biased_x16(wd[q], magic);
      p = __builtin_amdgcn_fdot2(as_f16x2(b.x), as_f16x2(xa[q].x), p, false);
      p = __builtin_amdgcn_fdot2(as_f16x2(b.y), as_f16x2(xa[q].y), p, false);
      p = __builtin_amdgcn_fdot2(as_f16x2(b.z), as_f16x2(xa[q].z), p, false);
      p = __builtin_amdgcn_fdot2(as_f16x2(b.w), as_f16x2(xa[q].w), p, false);
    }
    (void)slot;
    const f16x2 sbz = szw[(size_t)r * (G + 1) + 16 * i];  // (s, 1024 + z) of group 16 i + lane / 4
    const float s = (float)sbz[0], c1 = (float)sbz[1];
    acc[r] += s * (p - c1 * se - (c1 - 960.0f) * so);
  };
  // windows of D steps (D a multiple of R, so a window starts a chunk): each step is
  // consumed and its slot refilled with the same step of the next window, kept next
  // to the consumption by a scheduling barrier; the last window refills nothing
  int j = 0;
  for (; j + D < J; j += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      step(j + d, d);
      issue(d, j + d + D);
      __builtin_amdgcn_sched_barrier(0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 | 0x0400);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (j + d < J) step(j + d, d);

  // sparse term: lane l takes entries e0 + l, e0 + l + 64, ... of each row (the
  // first from the registers loaded in the prologue)
  if constexpr (SP) {
    const auto add = [&](int r, int c, float v) {
      const f16 xc = xs[(c & ~7) | perm_slot(c & 7)];
      acc[r] += ((c & 1) ? 16.0f * v : v) * (float)xc;  // odd channels were stored / 16
    };
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (e0[r] + lane < e1[r]) add(r, hc[r], (float)hv[r]);
#pragma unroll
    for (int r = 0; r < R; ++r)
      for (int e = e0[r] + lane + 64; e < e1[r]; e += 64) add(r, col[e], (float)val[e]);
  }
  // fixed-order sum over the 64 lanes: DPP scans inside each 16-lane row (totals in
  // lanes 15, 31, 47, 63), then the four row totals in order; lane r stores row n0 + r
  float tot[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = row16_sum_to_last(acc[r]);
    tot[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  }
  if (lane < R) {
    const float v = lane == 0 ? tot[0] : lane == 1 ? tot[1] : lane == 2 ? tot[2] : tot[3];
    const int n = n0 + lane;
    if (n < N) {
      if (y_f32)
        static_cast<float*>(y)[n] = v;
      else
        static_cast<f16*>(y)[n] = (f16)v;
    }
  }
}

// the (s, z) staging takes 16-byte vectors of eight halves: G = K / 128 up to 256
bool gemv_dot_supported(int64_t M, int64_t K, const uint16_t* scales, const uint16_t* zeros) {
  return M == 1 && K % kDotChunk == 0 && K <= 32768 && reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(zeros) % 16 == 0;
}

hipError_t launch_gemv_dot(const uint16_t* x, int64_t K, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* zeros, int64_t N, const int32_t* row_ptr, const int32_t* col,
                           const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  const size_t lds = (size_t)kDotRows * kDotWaves * (K / 128 + 1) * 4 + (size_t)K * 2;
  const int64_t rows_per_block = (int64_t)kDotRows * kDotWaves;
  const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block));
  auto args = [&](auto kern) {
    if (lds > 65536) {
      const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * kDotWaves), lds, stream, reinterpret_cast<const f16*>(x), (int)K,
                       packed, reinterpret_cast<const f16*>(scales), reinterpret_cast<const f16*>(zeros), (int)N,
                       row_ptr, col, reinterpret_cast<const f16*>(val), y, y_f32);
    return hipGetLastError();
  };
  const int64_t xloads = (K / 8 + 64 * kDotWaves - 1) / (64 * kDotWaves);
  const bool sp = row_ptr != nullptr;
#define WQ_DOT(XV) \
  if (xloads <= XV) return sp ? args(gemv_dot_kernel<XV, true>) : args(gemv_dot_kernel<XV, false>);
  WQ_DOT(1) WQ_DOT(2) WQ_DOT(4) WQ_DOT(8) WQ_DOT(16)
#undef WQ_DOT
  return hipErrorInvalidValue;  // K above 32768: not supported (gemv_dot_supported)
}

}  // namespace wq
