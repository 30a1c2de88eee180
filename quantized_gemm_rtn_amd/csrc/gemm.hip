// Prefill kernel (large M) of the W4A16 linear for gfx950: a tiled fp16 MFMA GEMM
// with on-the-fly INT4 dequantization, and the sparse outlier term added into the
// same fp32 accumulators.
//
// At large batch the weight-only product turns compute-bound once the weights are
// dequantized to fp16 (MixQ news item: weight-only quantization can fall behind
// fp16 at many concurrent requests), and dequantization on the slower vector units
// can cost a large share of the runtime (QServe, DeepCompressor README). The design
// therefore keeps the vector work per MFMA small and away from the LDS:
//
//  - Block tile BM x BN, K step 64 (half a quantization group), WGM x WGN waves,
//    each owning a (BM/WGM) x (BN/WGN) tile of 32x32 fp32 accumulators fed by
//    v_mfma_f32_32x32x16_f16 (lane l supplies A[l%32][8(l/32)+j], B[8(l/32)+j][l%32]
//    and holds D[8(i/4) + 4(l/32) + i%4][l%32]).
//  - Weights go straight from global memory into MFMA B registers: one 128-bit load
//    of four packed words per lane and 32-column subtile per K step, dequantized in
//    registers to fp16 (q - z) * s (the subtraction is exact, one rounding in the
//    multiply). Each word of eight codes is exactly one lane's B operand for one
//    MFMA; its nibble order (0,4,1,5,2,6,3,7) is matched by reordering activations.
//  - Activations go through LDS (two stages, one barrier per K step): 128-bit global
//    loads, each chunk of eight reordered (perm_x8), rows padded to 72 halves so
//    fragment reads of 8 consecutive rows hit distinct banks. Rows beyond M are
//    loaded from row M-1 (valid memory) and only reach rows that are never stored.
//  - Sparse term: each lane follows the CSR rows of its columns with a cursor. An
//    entry whose input channel falls in the eight channels the lane is about to feed
//    to an MFMA is added (fp16) to that dequantized weight, so the same MFMA applies
//    it: no extra accumulators, no extra MFMAs, no atomics. For a layer split by the
//    quantizer the dense weight at an outlier position is exactly zero, so the sum
//    is the sparse value itself.
//  - Split K (when the tile grid alone cannot fill the GPU and a workspace is
//    given): each K slice writes fp32 partials, and a second kernel sums the slices
//    in a fixed order and stores y. Results stay deterministic.
//  - Tile order is XCD-aware: consecutive block ids go to different XCDs, so the
//    id is remapped to give each XCD a contiguous range of tiles sharing weight
//    columns in its L2.
#include "wq_device.h"
#include "wq_launch.h"

#include <climits>

namespace wq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_32x32x16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kBK = 64;
constexpr int kLdsStride = 72;  // halves per LDS row (64 + 8 padding)
constexpr int kNumXcd = 8;

struct GemmArgs {
  const f16* x;
  const uint32_t* packed;
  const f16* scales;
  const f16* zeros;
  const int32_t* row_ptr;
  const int32_t* col;
  const f16* val;
  int nnz;
  void* y;           // final output (no split) or fp32 partials [S][M][N]
  int M, N, K;
  int y_f32;         // output dtype when not split
  int ksplit;        // number of K slices (1: no split)
  int k_per_slice;   // multiple of kBK
  int tiles_m, tiles_n;
};

// Two waves per SIMD (two blocks per CU): the blocks run out of phase, so one
// block's waits on memory and barriers are covered by the other's MFMAs.
template <int BM, int BN, int WGM, int WGN, bool SPARSE>
__global__ void __launch_bounds__(64 * WGM * WGN, 2)
gemm_kernel(GemmArgs a) {
  constexpr int T = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int MT = WTM / 32, NT = WTN / 32;    // 32x32 subtiles per wave
  constexpr int XV = BM * (kBK / 8) / T;         // 128-bit activation loads per thread per step
  static_assert(XV * T == BM * (kBK / 8) && MT >= 1 && NT >= 1, "tile/thread mismatch");
  constexpr int STAGE = BM * kLdsStride;         // halves per LDS stage

  extern __shared__ __align__(16) f16 smem[];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K >> 7;
  const int KW8 = K >> 3;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a contiguous
  // range of logical tiles, M fastest, so tiles that share weight columns meet in
  // the same L2.
  const int ntile = a.tiles_m * a.tiles_n;
  const int nblk = ntile * a.ksplit;
  int bid = blockIdx.x;
  if (nblk % kNumXcd == 0) bid = (bid % kNumXcd) * (nblk / kNumXcd) + bid / kNumXcd;
  const int slice = bid / ntile;
  const int tile = bid - slice * ntile;
  const int m0 = (tile % a.tiles_m) * BM, n0 = (tile / a.tiles_m) * BN;
  const int kb = slice * a.k_per_slice;
  const int ke = min(K, kb + a.k_per_slice);

  // activation producer: thread t loads rows (t >> 3) + i * T/8, chunk t & 7 (rows
  // beyond M read row M-1). Offsets are 32-bit element offsets (N*K, M*K < 2^31).
  constexpr int XROWS = T / 8;
  const int xrow0 = t >> 3, xch = t & 7;
  int xoff[XV];
#pragma unroll
  for (int i = 0; i < XV; ++i) xoff[i] = min(m0 + xrow0 + i * XROWS, M - 1) * K + 8 * xch;
  const int xdst0 = xrow0 * kLdsStride + 8 * xch;
  // weight rows of this lane: column (l % 32) of each 32-wide subtile
  const int h = lane >> 5;
  int woff[NT], soff[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(n0 + wn * WTN + j * 32 + (lane & 31), N - 1);
    woff[j] = n * (int)KW8 + 4 * h;
    soff[j] = n * G;
  }

  uint4 xr[XV], wr[NT];
  f16 sr[NT], zr[NT];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XV; ++i) xr[i] = *reinterpret_cast<const uint4*>(a.x + xoff[i] + k0);
    const int g = k0 >> 7;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      wr[j] = *reinterpret_cast<const uint4*>(a.packed + woff[j] + (k0 >> 3));
      sr[j] = a.scales[soff[j] + g];
      zr[j] = a.zeros[soff[j] + g];
    }
  };
  auto store_x = [&](f16* st) {
#pragma unroll
    for (int i = 0; i < XV; ++i)
      *reinterpret_cast<uint4*>(st + xdst0 + i * XROWS * kLdsStride) = perm_x8(xr[i]);
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Sparse cursors, one per accumulator column of this lane. Entry cur (l0, w0) and
  // entry cur + 1 (l1, w1) sit in registers, refilled by unconditional loads at one
  // fixed point per K step; their validity (cur < cend) is applied where they are
  // compared, so no load result is consumed early. Only a third entry of one row
  // inside a single 64-wide K step (rare) takes a direct load; its value is moved
  // into place inside that branch, so no pending load crosses the branch join and
  // the compiler keeps exact wait counts for the weight and activation prefetches.
  int cur[NT], cend[NT], l0[NT], l1[NT];
  f16 w0[NT], w1[NT];
  bool have1[NT];
  auto refill = [&](int j) {
    const int i0 = max(min(cur[j], a.nnz - 1), 0), i1 = max(min(cur[j] + 1, a.nnz - 1), 0);
    l0[j] = a.col[i0];
    l1[j] = a.col[i1];
    w0[j] = a.val[i0];
    w1[j] = a.val[i1];
    have1[j] = true;
  };
  auto pop = [&](int j) {
    ++cur[j];
    if (have1[j]) {
      l0[j] = l1[j];
      w0[j] = w1[j];
      have1[j] = false;
    } else {
      const int i0 = max(min(cur[j], a.nnz - 1), 0);
      const int lt = a.col[i0];
      const uint32_t wt = __builtin_bit_cast(uint16_t, a.val[i0]);
      int lm;
      uint32_t wm;
      asm volatile("v_mov_b32 %0, %1" : "=v"(lm) : "v"(lt));
      asm volatile("v_mov_b32 %0, %1" : "=v"(wm) : "v"(wt));
      l0[j] = lm;
      w0[j] = __builtin_bit_cast(f16, (uint16_t)wm);
    }
  };
  auto c0 = [&](int j) { return cur[j] < cend[j] ? l0[j] : INT_MAX; };
  if constexpr (SPARSE) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wn * WTN + j * 32 + (lane & 31);
      int lo = 0, hi = 0;
      if (n < N) {
        lo = a.row_ptr[n];
        hi = a.row_ptr[n + 1];
      }
      cend[j] = hi;
      while (lo < hi) {  // first entry of this K slice (columns are ascending)
        const int mid = (lo + hi) >> 1;
        if (a.col[mid] < kb) lo = mid + 1; else hi = mid;
      }
      cur[j] = lo;
      refill(j);
    }
  }

  const int nk = (ke - kb) / kBK;
  if (nk > 0) {
    load_step(kb);
    store_x(smem);
  }
  __syncthreads();
  uint4 wc[NT];
  f16 sc[NT], zc[NT];
  for (int s = 0; s < nk; ++s) {
    const int k0 = kb + s * kBK;
    const f16* xs = smem + (s & 1) * STAGE;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      wc[j] = wr[j];
      sc[j] = sr[j];
      zc[j] = zr[j];
    }
    if (s + 1 < nk) load_step(k0 + kBK);
    // four k16 steps: word (4h + ks) of each lane's 128-bit weight load
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f16x8 av[MT], bv[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        av[i] = *reinterpret_cast<const f16x8*>(xs + (wm * WTM + i * 32 + (lane & 31)) * kLdsStride +
                                                8 * (4 * h + ks));
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const f16 zb = (f16)1024.0f + zc[j];
        const f16x2 bias = {zb, zb};
        const f16x2 s2 = {sc[j], sc[j]};
        const uint32_t w = ks == 0 ? wc[j].x : ks == 1 ? wc[j].y : ks == 2 ? wc[j].z : wc[j].w;
        uint4 d = dequant_word(w, bias, s2);
        // sparse entries of this column inside this lane's eight input channels
        // [kc, kc + 8) are added to the dequantized weight (entries below kc belong
        // to the other half-wave's channels and are skipped)
        if constexpr (SPARSE) {
          const int kc = k0 + 8 * (4 * h + ks);
          for (int c = c0(j); c < kc + 8; c = c0(j)) {
            if (c >= kc) {
              // selects, not a dynamic index: a runtime index into a register vector
              // would send it through scratch memory
              const int slot = perm_slot(c - kc);
              const int p = slot >> 1;
              const uint32_t pr = p == 0 ? d.x : p == 1 ? d.y : p == 2 ? d.z : d.w;
              const f16x2 cur2 = as_f16x2(pr);
              const f16 old = (slot & 1) ? cur2[1] : cur2[0];
              const uint32_t sb = __builtin_bit_cast(uint16_t, (f16)(old + w0[j]));
              const uint32_t nw = (slot & 1) ? ((pr & 0xFFFFu) | (sb << 16)) : ((pr & 0xFFFF0000u) | sb);
              d.x = p == 0 ? nw : d.x;
              d.y = p == 1 ? nw : d.y;
              d.z = p == 2 ? nw : d.z;
              d.w = p == 3 ? nw : d.w;
            }
            pop(j);
          }
        }
        bv[j] = as_f16x8(d);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma_32x32x16(av[i], bv[j], acc[i][j]);
    }
    // the rest of this K step's entries belong to the other half-wave
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        // the rest of this K step's entries belong to the other half-wave
        while (c0(j) < k0 + kBK) pop(j);
        refill(j);
      }
    }
    if (s + 1 < nk) store_x(smem + ((s + 1) & 1) * STAGE);
    __syncthreads();
  }

  // store: the final y, or this slice's fp32 partial tile
  const bool partial = a.ksplit > 1;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n0 + wn * WTN + j * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + wm * WTM + i * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
        if (m < M) {
          const size_t o = (size_t)m * N + n;
          if (partial)
            static_cast<float*>(a.y)[(size_t)slice * M * N + o] = acc[i][j][q];
          else if (a.y_f32)
            static_cast<float*>(a.y)[o] = acc[i][j][q];
          else
            static_cast<f16*>(a.y)[o] = (f16)acc[i][j][q];
        }
      }
    }
}

// y = sum over slices s = 0..S-1 of ws[s] (fixed order), in the output dtype.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ ws, int S, size_t MN, void* __restrict__ y, int y_f32) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += stride) {
    float v = ws[i];
    for (int s = 1; s < S; ++s) v += ws[(size_t)s * MN + i];
    if (y_f32)
      static_cast<float*>(y)[i] = v;
    else
      static_cast<f16*>(y)[i] = (f16)v;
  }
}

struct GemmPlan {
  int bm, bn;
  int ksplit, k_per_slice;
};

// Tile and split choice for M x N x K (shared by the launcher and the workspace query).
static GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  p.bm = M <= 64 ? 64 : 128;
  p.bn = 256;
  const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  const int64_t ksteps = K / kBK;
  int64_t s = 1;
  // split K while the grid is below two blocks per CU and each slice keeps >= 16 steps
  while (tiles * s * 2 <= 512 && ksteps / (s * 2) >= 16) s *= 2;
  p.ksplit = (int)s;
  p.k_per_slice = (int)(((ksteps + s - 1) / s) * kBK);
  return p;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(M, N, K);
  return p.ksplit > 1 ? (size_t)p.ksplit * M * N * 4 : 0;
}

template <int BM, int BN, int WGM, int WGN, bool SPARSE>
static hipError_t launch_tile(GemmArgs a, hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)BM * kLdsStride * sizeof(f16);
  auto kern = gemm_kernel<BM, BN, WGM, WGN, SPARSE>;
  static bool attr_done = false;  // setting the same attribute twice is harmless
  if (lds > 65536 && !attr_done) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int64_t nblk = (int64_t)a.tiles_m * a.tiles_n * a.ksplit;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * WGM * WGN), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, int64_t nnz, void* y, int y_f32, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  constexpr int64_t kRowsPerLaunch = (int64_t)1 << 20;  // keeps the block count within int range
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    GemmPlan p = plan_gemm(mc, N, K);
    const size_t need = p.ksplit > 1 ? (size_t)p.ksplit * mc * N * 4 : 0;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
      p.ksplit = 1;  // no (or too small) workspace: run unsplit
      p.k_per_slice = (int)K;
    }
    const size_t ysz = y_f32 ? 4 : 2;
    GemmArgs a;
    a.x = reinterpret_cast<const f16*>(x) + m * K;
    a.packed = packed;
    a.scales = reinterpret_cast<const f16*>(scales);
    a.zeros = reinterpret_cast<const f16*>(zeros);
    a.row_ptr = row_ptr;
    a.col = col;
    a.val = reinterpret_cast<const f16*>(val);
    a.nnz = row_ptr != nullptr ? nnz : 0;
    void* yout = static_cast<char*>(y) + (size_t)(m * N) * ysz;
    a.y = p.ksplit > 1 ? workspace : yout;
    a.M = (int)mc;
    a.N = (int)N;
    a.K = (int)K;
    a.y_f32 = y_f32;
    a.ksplit = p.ksplit;
    a.k_per_slice = p.k_per_slice;
    hipError_t e;
    const bool sp = row_ptr != nullptr;
    if (p.bm == 64)
      e = sp ? launch_tile<64, 256, 1, 4, true>(a, stream) : launch_tile<64, 256, 1, 4, false>(a, stream);
    else
      e = sp ? launch_tile<128, 256, 1, 4, true>(a, stream) : launch_tile<128, 256, 1, 4, false>(a, stream);
    if (e != hipSuccess) return e;
    if (p.ksplit > 1) {
      const size_t MN = (size_t)mc * N;
      const int64_t blocks = (int64_t)((MN + 255) / 256) < 4096 ? (int64_t)((MN + 255) / 256) : 4096;
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                         static_cast<const float*>(workspace), p.ksplit, MN, yout, y_f32);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace wq
