// Decode kernels (M <= 16 rows per tile) of the W4A16 linear for gfx950, with the
// sparse outlier term fused into the same output tile.
//
// y[m, n] = sum_k x[m, k] (q[n, k] - z[n, g]) s[n, g]  +  sum_e val_e x[m, col_e]
//
// Weight-only quantization pays off on memory-bound token generation (AWQ paper,
// section 2), and its speed comes from dequantizing packed 4-bit weights on the
// fly inside the product, without an fp16 copy of W in DRAM (AWQ paper, section
// 1). At M <= 16 the kernel streams N*K/2 bytes of codes once and is bound by
// HBM bandwidth, so everything here serves two goals: keep enough weight bytes in
// flight, and keep the vector work per weight small enough to hide under them.
//
// Mapping (one 16-column tile of N per block, KW waves splitting K):
//  - Lane l = 16h + r reads output channel n0 + r, input channels
//    [128g + 32h, 128g + 32h + 32) of each group g: one 128-bit load of four packed
//    words, so a channel's four lanes read 64 contiguous bytes per group. Each wave
//    keeps D groups in flight (a rolling prefetch).
//  - The block first stages the fp16 scale and zero-point of its 16 channels for
//    all groups into LDS with wide loads.
//  - Each word feeds one 16x16x32 fp16 MFMA with fp32 accumulation (x rows in A,
//    W channels in B). Rows of A at or beyond M hold whatever valid data is at hand:
//    they only reach output rows that are never stored.
//  - The group's fp32 partial is scaled by s once per group.
//  - Sparse term: each lane walks the CSR row of its column (entries split across
//    the block's waves) and adds val * x in fp32 into the same accumulators.
//  - The KW partial tiles are summed through LDS in a fixed order (no atomics, so
//    results are deterministic) and stored once.
//
// Two kernels:
//  gemv_lds_kernel (M*K <= 32768): the block stages x[m0 .. m0+mrows) in LDS, in
//    the dequantized weight order, with odd input channels pre-scaled by 1/16, and
//    the per-(row, group) sums of x over even and odd channels. The weights are
//    then unpacked with five instructions per word as 1024 + q or 1024 + 16q (no
//    zero-point subtraction per weight); the zero-point and the 1024 bias come off
//    once per group:  sum (q - z) x = P - (1024 + z) S_even - (64 + z) S_odd.
//  gemv_stream_kernel: activations are too large for LDS; each group's activations
//    are prefetched together with its weights and the weights are unpacked to the
//    exact integers q - z.
//
// Every global load is unconditional, with its address clamped to valid memory: a
// load under a divergent branch makes the compiler wait for all outstanding loads
// where the branches join, which would serialize the stream. For the same reason
// staged values are loaded before the weight prefetch is issued and stored after.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

constexpr int kGemvWaves = 4;   // KW
constexpr int kGemvDepth = 8;   // D: groups in flight per lane (128-bit weight loads)
constexpr int kGemvDepthX = 4;  // D when each group also carries its activations
constexpr int kXLdsMaxHalves = 32768;
// sched_barrier mask: ALU, VALU, SALU, MFMA, LDS and transcendental instructions may
// be scheduled across it, vector memory instructions may not.
constexpr int kSchedAllButVmem = 0x0001 | 0x0002 | 0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 | 0x0400;

// ---------------------------------------------------------------------------
// Scale / zero-point staging: LDS sz[16][G + 1] = (s, 1024 + z) for the block's rows.
// The row stride G + 1 is odd (G is even whenever it matters), so the 16 lanes that
// read one group of 16 rows hit 16 different banks.
//   SZV = 8: rows as 16-byte vectors (G % 8 == 0, G <= 256): <= 2 loads per thread
//   SZV = 1: as halves (G <= 256): <= 16 loads per thread
//   SZV = 0: a plain loop (any G), run after the weight prefetch
template <int SZV, int T>
struct SzStage {
  static constexpr int C = SZV == 8 ? 2 : (SZV == 1 ? 16 : 0);
  uint4 v8s[SZV == 8 ? C : 1], v8z[SZV == 8 ? C : 1];
  uint16_t v1s[SZV == 1 ? C : 1], v1z[SZV == 1 ? C : 1];

  __device__ __forceinline__ void load(const f16* scales, const f16* zeros, int n0, int N, int G, int t) {
    const int nload = SZV ? 16 * G / SZV : 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int idx = min(t + i * T, nload - 1);
      const int e = idx * SZV;
      const int row = e / G, c = e - row * G;
      const size_t o = (size_t)min(n0 + row, N - 1) * G + c;
      if constexpr (SZV == 8) {
        v8s[i] = *reinterpret_cast<const uint4*>(scales + o);
        v8z[i] = *reinterpret_cast<const uint4*>(zeros + o);
      } else {
        v1s[i] = __builtin_bit_cast(uint16_t, scales[o]);
        v1z[i] = __builtin_bit_cast(uint16_t, zeros[o]);
      }
    }
  }
  // stores are unconditional too (clamped indices rewrite identical values), so the
  // compiler cannot sink a staging load behind the weight prefetch
  __device__ __forceinline__ void store(f16x2* sz, const f16* scales, const f16* zeros, int n0, int N, int G,
                                        int t) {
    const f16 k1024 = (f16)1024.0f;
    const int nload = SZV ? 16 * G / SZV : 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int idx = min(t + i * T, nload - 1);
      if constexpr (SZV == 8) {
        const f16x8 s8 = as_f16x8(v8s[i]), z8 = as_f16x8(v8z[i]);
        const int base = 8 * idx + (8 * idx) / G;  // row * (G + 1) + column
#pragma unroll
        for (int j = 0; j < 8; ++j) sz[base + j] = f16x2{s8[j], (f16)(k1024 + z8[j])};
      } else {
        sz[idx + idx / G] = f16x2{bits_to_f16(v1s[i]), (f16)(k1024 + bits_to_f16(v1z[i]))};
      }
    }
    if constexpr (SZV == 0) {
      for (int idx = t; idx < 16 * G; idx += T) {
        const int row = idx / G, c = idx - row * G;
        const size_t o = (size_t)min(n0 + row, N - 1) * G + c;
        sz[idx + row] = f16x2{scales[o], (f16)(k1024 + zeros[o])};
      }
    }
  }
};

// Fixed-order sum of the KW partial tiles through LDS and the single store.
template <int KW>
__device__ __forceinline__ void reduce_store(f32x4 acc, int wave, int lane, int m0, int mrows, int n, int N,
                                             void* y, int y_f32) {
  if constexpr (KW > 1) {
    __shared__ f32x4 red[KW - 1][64];
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < KW - 1; ++w) acc += red[w][lane];
  }
  if (n >= N) return;
  const int h = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * h + i;
    if (m < mrows) {
      const size_t o = (size_t)(m0 + m) * N + n;
      if (y_f32)
        static_cast<float*>(y)[o] = acc[i];
      else
        static_cast<f16*>(y)[o] = (f16)acc[i];
    }
  }
}

// ---------------------------------------------------------------------------
template <int KW, int D, int XC, int SZV, int MR>
__global__ void __launch_bounds__(64 * KW)
gemv_lds_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
                const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
                const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                const f16* __restrict__ val, void* __restrict__ y, int y_f32) {
  constexpr int T = 64 * KW;
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int G = K >> 7;
  const int mrows = min(16, M - m0);
  const int SR = MR == 1 ? 1 : 4 * ((mrows + 3) >> 2);  // rows of the x-sum tables
  // LDS: sz[16][G + 1] (s, 1024 + z) | xs[mrows][K] permuted, odd channels / 16 |
  //      sums of x over even / odd channels per (group, row)
  f16x2* sz = reinterpret_cast<f16x2*>(smem);
  f16* xs = reinterpret_cast<f16*>(smem + (size_t)16 * (G + 1) * 4);
  // x sums per group: [g][2][SR] (even rows then odd rows); with MR == 1, SR == 1
  // and the pair (even, odd) of row 0 is adjacent
  float* sab = reinterpret_cast<float*>(smem + (size_t)16 * (G + 1) * 4 + (size_t)mrows * K * 2);

  const int n_ld = min(n0 + r, N - 1);  // ragged N: load a valid row, never store it
  const uint32_t* wrow = packed + (size_t)n_ld * (size_t)(K >> 3) + 4 * h;
  const int g_lo = (G * wave) / KW, g_hi = (G * (wave + 1)) / KW;
  const int ng = g_hi - g_lo;

  // ---- prologue: staging loads, weight prefetch, staging stores
  SzStage<SZV, T> szs;
  szs.load(scales, zeros, n0, N, G, t);
  const int x_vecs = mrows * (K >> 3);
  uint4 xv[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int idx = min(t + i * T, x_vecs - 1);
    const int row = idx / (K >> 3), c8 = idx - row * (K >> 3);
    xv[i] = *reinterpret_cast<const uint4*>(x + (size_t)(m0 + row) * K + 8 * c8);
  }
  const int nfull = ng / D;
  const int g_first_valid = min(g_lo, G - 1);  // waves without groups still load valid memory
  uint4 wbuf[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int g = max(min(g_lo + i, g_hi - 1), g_first_valid);
    wbuf[i] = *reinterpret_cast<const uint4*>(wrow + (size_t)g * 16);
  }

  szs.store(sz, scales, zeros, n0, N, G, t);
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 ones = {(f16)1.0f, (f16)1.0f};
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int idx_raw = t + i * T;
    const int idx = min(idx_raw, x_vecs - 1);
    const uint4 p = perm_x8(xv[i]);  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
    // even-channel and odd-channel sums of this chunk, fp32 (products by 1 are exact)
    float se = __builtin_amdgcn_fdot2(as_f16x2(p.x), ones, 0.0f, false);
    se = __builtin_amdgcn_fdot2(as_f16x2(p.z), ones, se, false);
    float so = __builtin_amdgcn_fdot2(as_f16x2(p.y), ones, 0.0f, false);
    so = __builtin_amdgcn_fdot2(as_f16x2(p.w), ones, so, false);
    uint4 q = p;
    q.y = as_u32(as_f16x2(p.y) * sixteenth);
    q.w = as_u32(as_f16x2(p.w) * sixteenth);
    *reinterpret_cast<uint4*>(xs + 8 * idx) = q;
    // the 16 chunks of a group sit in 16 consecutive lanes: fixed-order butterfly
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      se += __shfl_xor(se, o, 16);
      so += __shfl_xor(so, o, 16);
    }
    if ((idx_raw & 15) == 0 && idx_raw < x_vecs) {
      const int row = idx_raw / (K >> 3), g = (idx_raw - row * (K >> 3)) >> 4;
      if constexpr (MR == 1) {
        sab[2 * g] = se;
        sab[2 * g + 1] = so;
      } else {
        sab[2 * g * SR + row] = se;
        sab[2 * g * SR + SR + row] = so;
      }
    }
  }
  __syncthreads();

  // ---- main loop over this wave's groups
  const int xr = min(r, mrows - 1);
  const f16* xl = xs + (size_t)xr * K + 32 * h;
  const f16x2* szr = sz + r * (G + 1);
  const int srow = min(4 * h, SR - 4);
  const uint32_t magic = magic_1024x2();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto group = [&](const uint4& w, int g) {
    const uint32_t wds[4] = {w.x, w.y, w.z, w.w};
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint4 xa = *reinterpret_cast<const uint4*>(xl + (size_t)g * 128 + 8 * tt);
      part = mfma_16x16x32(as_f16x8(xa), as_f16x8(codes_biased_x16(wds[tt], magic)), part);
    }
    const f16x2 sbz = szr[g];
    const float s = (float)sbz[0];
    const float c1 = (float)sbz[1];  // 1024 + z
    const float c2 = c1 - 960.0f;     // 64 + z
    // only the first MR rows of a lane's four can be stored (MR < 4 when M <= 2)
    if constexpr (MR == 1) {
      const float2 eo = *reinterpret_cast<const float2*>(sab + 2 * g * SR);
      acc[0] += s * (part[0] - c1 * eo.x - c2 * eo.y);
    } else {
      const f32x4 e = *reinterpret_cast<const f32x4*>(sab + 2 * g * SR + srow);
      const f32x4 o = *reinterpret_cast<const f32x4*>(sab + 2 * g * SR + SR + srow);
#pragma unroll
      for (int i = 0; i < MR; ++i) acc[i] += s * (part[i] - c1 * e[i] - c2 * o[i]);
    }
  };

  // blocks of D groups: each step consumes one buffered word, then refills the same
  // register with the same step of the next block (consume first, so the refill can
  // reuse the register and the loop carries no copy of an in-flight load)
  int gb = 0;
  const uint32_t* wnext = wrow + (size_t)(g_lo + D) * 16;
  for (int b = 0; b + 1 < nfull; ++b, gb += D, wnext += D * 16) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      group(wbuf[i], g_lo + gb + i);
      wbuf[i] = *reinterpret_cast<const uint4*>(wnext + i * 16);
      // keep the refill here: left alone, the scheduler sinks all refills to the end
      // of the block, and the wave then waits for every load before issuing more.
      // Only memory instructions are pinned; arithmetic may still overlap groups.
      __builtin_amdgcn_sched_barrier(kSchedAllButVmem);
    }
  }
  if (nfull > 0) {
#pragma unroll
    for (int i = 0; i < D; ++i) group(wbuf[i], g_lo + gb + i);
    gb += D;
  }
  for (; gb < ng; ++gb) group(*reinterpret_cast<const uint4*>(wrow + (size_t)(g_lo + gb) * 16), g_lo + gb);

  // ---- sparse outlier term for column n = n0 + r, activations from LDS
  const int n = n0 + r;
  if (row_ptr != nullptr && n < N) {
    const int e1 = row_ptr[n + 1];
    for (int e = row_ptr[n] + wave; e < e1; e += KW) {
      const int c = col[e];
      const float v = (float)val[e];
      const int cs = (c & ~7) | perm_slot(c & 7);
      const float unscale = (c & 1) ? 16.0f : 1.0f;  // odd channels were stored / 16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(4 * h + i, mrows - 1);
        acc[i] += v * ((float)xs[(size_t)m * K + cs] * unscale);
      }
    }
  }
  reduce_store<KW>(acc, wave, lane, m0, mrows, n, N, y, y_f32);
}

// ---------------------------------------------------------------------------
template <int KW, int D, int SZV>
__global__ void __launch_bounds__(64 * KW)
gemv_stream_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
                   const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
                   const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                   const f16* __restrict__ val, void* __restrict__ y, int y_f32) {
  constexpr int T = 64 * KW;
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int r = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int G = K >> 7;
  const int mrows = min(16, M - m0);
  f16x2* sz = reinterpret_cast<f16x2*>(smem);  // [16][G + 1]: (s, 1024 + z)

  const int n_ld = min(n0 + r, N - 1);
  const uint32_t* wrow = packed + (size_t)n_ld * (size_t)(K >> 3) + 4 * h;
  const int g_lo = (G * wave) / KW, g_hi = (G * (wave + 1)) / KW;
  const int ng = g_hi - g_lo;
  const int xr = min(r, mrows - 1);
  const f16* xrow = x + (size_t)(m0 + xr) * K + 32 * h;

  SzStage<SZV, T> szs;
  szs.load(scales, zeros, n0, N, G, t);
  // each group's activations travel with its weights (same prefetch unit, same order)
  const int nfull = ng / D;
  const int g_first_valid = min(g_lo, G - 1);
  uint4 wbuf[D];
  uint4 xbuf[D][4];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int g = max(min(g_lo + i, g_hi - 1), g_first_valid);
    wbuf[i] = *reinterpret_cast<const uint4*>(wrow + (size_t)g * 16);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xbuf[i][tt] = *reinterpret_cast<const uint4*>(xrow + (size_t)g * 128 + 8 * tt);
  }
  szs.store(sz, scales, zeros, n0, N, G, t);
  __syncthreads();

  const f16x2* szr = sz + r * (G + 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto group = [&](const uint4& w, const uint4* xg, int g) {
    const f16x2 sbz = szr[g];
    const f16x2 bias = {sbz[1], sbz[1]};
    const uint32_t wds[4] = {w.x, w.y, w.z, w.w};
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      part = mfma_16x16x32(as_f16x8(perm_x8(xg[tt])), codes_minus_zero(wds[tt], bias), part);
    acc += (float)sbz[0] * part;
  };

  int gb = 0;
  for (int b = 0; b + 1 < nfull; ++b, gb += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int g = g_lo + gb + i;
      group(wbuf[i], xbuf[i], g);
      wbuf[i] = *reinterpret_cast<const uint4*>(wrow + (size_t)(g + D) * 16);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        xbuf[i][tt] = *reinterpret_cast<const uint4*>(xrow + (size_t)(g + D) * 128 + 8 * tt);
      __builtin_amdgcn_sched_barrier(kSchedAllButVmem);  // keep the refill next to its consumption
    }
  }
  if (nfull > 0) {
#pragma unroll
    for (int i = 0; i < D; ++i) group(wbuf[i], xbuf[i], g_lo + gb + i);
    gb += D;
  }
  for (; gb < ng; ++gb) {
    const int g = g_lo + gb;
    const uint4 w = *reinterpret_cast<const uint4*>(wrow + (size_t)g * 16);
    uint4 xg[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xg[tt] = *reinterpret_cast<const uint4*>(xrow + (size_t)g * 128 + 8 * tt);
    group(w, xg, g);
  }

  const int n = n0 + r;
  if (row_ptr != nullptr && n < N) {
    const int e1 = row_ptr[n + 1];
    for (int e = row_ptr[n] + wave; e < e1; e += KW) {
      const int c = col[e];
      const float v = (float)val[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(4 * h + i, mrows - 1);
        acc[i] += v * (float)x[(size_t)(m0 + m) * K + c];
      }
    }
  }
  reduce_store<KW>(acc, wave, lane, m0, mrows, n, N, y, y_f32);
}

// ---------------------------------------------------------------------------
template <typename Kern>
static hipError_t launch_rows(Kern kern, size_t lds, const uint16_t* x, int64_t M, int64_t K,
                              const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                              const int32_t* row_ptr, const int32_t* col, const uint16_t* val, void* y, int y_f32,
                              hipStream_t stream, size_t* lds_set) {
  if (lds > 65536 && lds > *lds_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    *lds_set = lds;
  }
  constexpr int64_t kRowsPerLaunch = 65535 * 16;  // gridDim.y limit
  const size_t ysz = y_f32 ? 4 : 2;
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((mc + 15) / 16));
    hipLaunchKernelGGL(kern, grid, dim3(64 * kGemvWaves), lds, stream, reinterpret_cast<const f16*>(x) + m * K,
                       (int)mc, (int)K, packed, reinterpret_cast<const f16*>(scales),
                       reinterpret_cast<const f16*>(zeros), (int)N, row_ptr, col, reinterpret_cast<const f16*>(val),
                       static_cast<char*>(y) + (size_t)(m * N) * ysz, y_f32);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int XC, int SZV, int MR>
static hipError_t launch_lds(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                             const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  static size_t lds_set = 0;
  const int64_t G = K / kGroup, mrows = M < 16 ? M : 16, SR = MR == 1 ? 1 : 4 * ((mrows + 3) / 4);
  const size_t lds = (size_t)16 * (G + 1) * 4 + (size_t)mrows * K * 2 + (size_t)2 * G * SR * 4;
  return launch_rows(gemv_lds_kernel<kGemvWaves, kGemvDepth, XC, SZV, MR>, lds, x, M, K, packed, scales, zeros, N,
                     row_ptr, col, val, y, y_f32, stream, &lds_set);
}

template <int SZV>
static hipError_t launch_stream(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                                const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  static size_t lds_set = 0;
  const size_t lds = (size_t)16 * (K / kGroup + 1) * 4;
  return launch_rows(gemv_stream_kernel<kGemvWaves, kGemvDepthX, SZV>, lds, x, M, K, packed, scales, zeros, N,
                     row_ptr, col, val, y, y_f32, stream, &lds_set);
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  const int64_t G = K / kGroup;
  const int64_t mrows_max = M < 16 ? M : 16;
  // activations fit in LDS next to the scales: stage them once per block, with the
  // fewest staging registers that cover them
  const int64_t xloads = (mrows_max * K / 8 + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
  const int xc = mrows_max * K > kXLdsMaxHalves ? 0 : xloads <= 2 ? 2 : xloads <= 4 ? 4 : xloads <= 8 ? 8 : 16;
  // scales/zeros rows as 16-byte vectors when every row starts 16-byte aligned
  const bool vec = G % 8 == 0 && G <= 256 && reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(zeros) % 16 == 0;
  const int sv = vec ? 8 : (G <= 256 ? 1 : 0);
#define WQ_ARGS x, M, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32, stream
  // output rows a lane can hold: rows 4h .. 4h+3 of the tile, so M = 1, 2 need fewer
  const int mr = mrows_max == 1 ? 1 : (mrows_max == 2 ? 2 : 4);
#define WQ_LDS(XC, SV, MR) \
  if (xc == XC && sv == SV && mr == MR) return launch_lds<XC, SV, MR>(WQ_ARGS)
#define WQ_LDS_MR(XC, SV) WQ_LDS(XC, SV, 1); WQ_LDS(XC, SV, 2); WQ_LDS(XC, SV, 4)
  WQ_LDS_MR(2, 8); WQ_LDS_MR(4, 8); WQ_LDS_MR(8, 8); WQ_LDS_MR(16, 8);
  WQ_LDS_MR(2, 1); WQ_LDS_MR(4, 1); WQ_LDS_MR(8, 1); WQ_LDS_MR(16, 1);
  WQ_LDS_MR(2, 0); WQ_LDS_MR(4, 0); WQ_LDS_MR(8, 0); WQ_LDS_MR(16, 0);
#undef WQ_LDS_MR
  if (sv == 8) return launch_stream<8>(WQ_ARGS);
  if (sv == 1) return launch_stream<1>(WQ_ARGS);
  return launch_stream<0>(WQ_ARGS);
#undef WQ_LDS
#undef WQ_ARGS
}

}  // namespace wq
