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
#include <type_traits>

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
  // low-rank branch: t [M][lr_r] and L2 [N][lr_r] fp16, lr_r = 0 for none
  const f16* lr_t;
  const f16* lr_up;
  int lr_r;
  // x^T [K][xt_mp] for a sparse term added in the slice sum (gemm_big_kernel<..., true>)
  f16* xt;
  int xt_mp;
};

// Up-projection of a low-rank branch for a wave's MT x NT subtiles of 32 x 32:
// acc[i][j] += t . L2^T with rows of t [M][r] in A and rows of L2 [N][r] in B, 16
// of the rank per 32x32x16 MFMA (the same output layout as the weights' MFMAs);
// added by the first K slice only. Rows past M or N read the last row and are
// never stored.
template <int MT, int NT>
__device__ __forceinline__ void lowrank_add32(f32x16 (&acc)[MT][NT], const f16* t, const f16* up, int r, int M,
                                              int N, int mbase, int nbase, int lane) {
  const int h = lane >> 5, c32 = lane & 31;
  for (int s = 0; s < r; s += 16) {
    f16x8 av[MT], bv[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      av[i] = as_f16x8(*reinterpret_cast<const uint4*>(t + (size_t)min(mbase + 32 * i + c32, M - 1) * r + s + 8 * h));
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bv[j] = as_f16x8(*reinterpret_cast<const uint4*>(up + (size_t)min(nbase + 32 * j + c32, N - 1) * r + s + 8 * h));
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = mfma_32x32x16(av[i], bv[j], acc[i][j]);
  }
}

// Stores a wave's MT x NT subtiles of 32 x 32 MFMA results (lane 32h + c holds
// column c of each, value q at row 8 (q / 4) + 4h + q % 4) into out [M, N] (y, or a K
// slice's fp32 partial), from row mw and column nw. The output kind is chosen by the
// caller, outside the loops, and a wave whose subtiles lie inside M x N stores with
// no bounds test: with the kind and the bounds tested per element, the unrolled
// stores compiled to about a thousand branches per wave, and per-block timestamps put
// the store of a 128 x 256 prefill tile at 10-19 us.
template <int MT, int NT, typename T, typename Conv>
__device__ __forceinline__ void store_subtiles(const f32x16 (&acc)[MT][NT], T* __restrict__ out, int mw, int nw,
                                               int M, int N, int lane, Conv conv) {
  const int h = lane >> 5, c = lane & 31;
  if (mw + 32 * MT <= M && nw + 32 * NT <= N) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        T* p = out + (size_t)(mw + 32 * i + 4 * h) * N + (nw + 32 * j + c);
#pragma unroll
        for (int q = 0; q < 16; ++q) p[(size_t)(8 * (q >> 2) + (q & 3)) * N] = conv(acc[i][j][q]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = nw + 32 * j + c;
        if (n >= N) continue;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = mw + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
          if (m < M) out[(size_t)m * N + n] = conv(acc[i][j][q]);
        }
      }
  }
}

// y (fp16 or fp32) or the fp32 partial of K slice `slice`, by the kind of output
template <int MT, int NT>
__device__ __forceinline__ void store_output(const f32x16 (&acc)[MT][NT], const GemmArgs& a, int slice, int mw,
                                             int nw, int lane) {
  const auto same = [](float v) { return v; };
  if (a.ksplit > 1)
    store_subtiles<MT, NT>(acc, static_cast<float*>(a.y) + (size_t)slice * a.M * a.N, mw, nw, a.M, a.N, lane, same);
  else if (a.y_f32)
    store_subtiles<MT, NT>(acc, static_cast<float*>(a.y), mw, nw, a.M, a.N, lane, same);
  else
    store_subtiles<MT, NT>(acc, static_cast<f16*>(a.y), mw, nw, a.M, a.N, lane, [](float v) { return (f16)v; });
}

// Two waves per SIMD (two blocks per CU): the blocks run out of phase, so one
// block's waits on memory and barriers are covered by the other's MFMAs.
// BITS = 3: 3-bit codes, 32 per three words (a lane reads one 12-byte run per K
// step instead of four words); G64: one (s, z) per 64 input channels, which is one
// per K step.
template <int BM, int BN, int WGM, int WGN, bool SPARSE, int BITS = 4, bool G64 = false>
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
  const int Gs = G64 ? K >> 6 : K >> 7;     // (s, z) per row
  const int RW = BITS == 4 ? K >> 3 : 3 * (K >> 5);  // words per row
  typedef typename std::conditional<BITS == 4, uint4, uint3>::type WT;

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
    woff[j] = n * RW + (BITS == 4 ? 4 : 3) * h;
    soff[j] = n * Gs;
  }

  uint4 xr[XV];
  WT wr[NT];
  f16 sr[NT], zr[NT];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XV; ++i) xr[i] = *reinterpret_cast<const uint4*>(a.x + xoff[i] + k0);
    const int g = G64 ? k0 >> 6 : k0 >> 7;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      wr[j] = *reinterpret_cast<const WT*>(a.packed + woff[j] + (BITS == 4 ? k0 >> 3 : 3 * (k0 >> 5)));
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

  const uint32_t magic = magic_1024x2();
  const int nk = (ke - kb) / kBK;
  if (nk > 0) {
    load_step(kb);
    store_x(smem);
  }
  __syncthreads();
  WT wc[NT];
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
        const f16 zb = (f16)1024.0f + zc[j], zn = -((f16)64.0f + zc[j]);
        const f16x2 bias = {zb, zb}, nbias16 = {zn, zn};
        const f16x2 s2 = {sc[j], sc[j]};
        uint4 d;
        if constexpr (BITS == 4) {
          const uint32_t w = ks == 0 ? wc[j].x : ks == 1 ? wc[j].y : ks == 2 ? wc[j].z : wc[j].w;
          d = dequant_word_x16(w, magic, bias, nbias16, s2);
        } else {
          d = dequant3(wc[j], ks, magic, bias, s2);
        }
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

  if (a.lr_r > 0 && slice == 0) lowrank_add32<MT, NT>(acc, a.lr_t, a.lr_up, a.lr_r, M, N, m0 + wm * WTM, n0 + wn * WTN, lane);
  // store: the final y, or this slice's fp32 partial tile
  store_output<MT, NT>(acc, a, slice, m0 + wm * WTM, n0 + wn * WTN, lane);
}

// ---------------------------------------------------------------------------
constexpr int kBigSS = 128;                // halves per super-step (one group)
constexpr int kXtPerThread = 2;            // transpose items per thread and super-step (XT)
constexpr int64_t kBigFillBlocks = 256;     // one block per compute unit
constexpr int kBigSzBytes = 2 * 2 * 256 * 4;  // (s, z) table: 2 buffers x 2 groups x 256 columns

// Dense kernel for large M. As launched: block tile 128 x 256, four waves side by
// side along N, each 128 x 64 (4 x 2 subtiles of 32 x 32), two blocks per compute
// unit. The two blocks on a CU meet at their own barriers, so they drift out of
// phase and each SIMD interleaves one wave's waits with the other's MFMAs. (The
// template also takes 256 x 256 tiles with eight or four waves, one block per CU.)
// K is consumed in super-steps of one quantization group (128), each split into
// eight MFMA sub-steps of 16.
//  - Weights, scales and zero-points of super-step s + 1 are loaded during the first
//    half of super-step s into the other of two register sets, a whole super-step
//    ahead of their use; activations of s + 1 go at the same time straight from
//    global memory into the other of two LDS stages (buffer loads to LDS), so they
//    occupy no registers and need no LDS store instructions.
//  - Within a super-step the A fragments and dequantized B operands of sub-step
//    ks + 1 are prepared while the MFMAs of sub-step ks run.
//  - Lane l = 32h + c of a wave supplies column c of each 32-wide subtile; in
//    sub-step ks it feeds the eight input channels 64 (ks / 4) + 32h + 8 (ks % 4)
//    of the group (word 8 (ks / 4) + 4h + ks % 4 of the column's 16 words), in
//    their natural order, matching activations kept in natural order in LDS.
//  - With XT, the block also writes its share of the activations' transpose
//    xt [K][Mp] (Mp: M rounded up to 8, rows M .. Mp - 1 zero) from the LDS stage of
//    each super-step: 128 / tiles_n (rounded up) input channels of the group for the
//    block's rows, so that the tiles_n blocks of a row tile and slice cover every
//    channel once. The slice sum then gathers the sparse term's activations from it.
template <int BM, int BN, int WGM, int WGN, int MINB, int WS, bool XT>
__global__ void __launch_bounds__(64 * WGM * WGN, MINB)
gemm_big_kernel(GemmArgs a) {
  constexpr int T = 64 * WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MT = WTM / 32, NT = WTN / 32;
  constexpr int XV = BM * (kBigSS / 8) / T;  // 16-byte activation loads per thread per super-step
  constexpr int XP = XV / 4;                  // ... per part
  constexpr int XR = T / 16;                  // rows between a thread's activation loads
  constexpr int STAGE = BM * kBigSS;          // rows of 256 bytes, 16-byte chunks swizzled
  static_assert((T == 256 || T == 512) && (BN == 256 || BN == 128) && XP * 4 == XV && (NT == 1 || NT == 2 || NT == 4) &&
                    MT >= NT,
                "tile/thread mismatch");

  extern __shared__ __align__(16) f16 smem[];
  // LDS: two activation stages | (s, z) table szl[buffer][group of the pair][column]
  uint32_t* szl = reinterpret_cast<uint32_t*>(smem + 2 * STAGE);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int h = lane >> 5, c32 = lane & 31;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K >> 7;  // even (the launcher sends odd G to the other kernel)

  const int ntile = a.tiles_m * a.tiles_n;
  const int nblk = ntile * a.ksplit;
  int bid = blockIdx.x;
  if (nblk % kNumXcd == 0) bid = (bid % kNumXcd) * (nblk / kNumXcd) + bid / kNumXcd;
  const int slice = bid / ntile;
  const int tile = bid - slice * ntile;
  const int m0 = (tile % a.tiles_m) * BM, n0 = (tile / a.tiles_m) * BN;
  const int tn = tile / a.tiles_m;
  // (block-uniform values, kept in scalar registers for the loads' scalar offsets)
  const int g0 = __builtin_amdgcn_readfirstlane(slice * (a.k_per_slice >> 7));            // even
  const int ng = __builtin_amdgcn_readfirstlane(min(G, g0 + (a.k_per_slice >> 7)) - g0);  // even

  // All loads go through buffer resources: a per-lane byte offset fixed for the
  // whole kernel (row or column) plus a per-super-step scalar offset (the group), so
  // no address arithmetic is left in the loop. Rows past M and columns past N read
  // zeros, which only reach outputs that are never stored (M*K and N*K are below
  // 2^31, so byte offsets fit in 32 bits).
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(a.x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t wrs = buffer_rsrc(a.packed, (uint32_t)N * (uint32_t)(K >> 1));
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(a.scales, (uint32_t)N * (uint32_t)G * 2u);
  const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(a.zeros, (uint32_t)N * (uint32_t)G * 2u);
  // activations go straight from global memory to LDS: load i of wave w fills the
  // 1 KB block b = i (T / 64) + w of a stage, rows 4b .. 4b + 3, lane l the 16 bytes
  // at position l & 15 of row 4b + (l >> 4). Chunk c (input channels 8c .. 8c + 7 of
  // the group) of row r sits at position c ^ (r & 15), so the 16 rows of a fragment
  // read fall in distinct banks. Rows beyond M reread row M - 1.
  const int xrow_l = 4 * wave + (lane >> 4);  // row in block 0; + XR i for load i
  const int xch = (lane & 15) ^ (xrow_l & 15);
  const uint32_t xvo = ((uint32_t)(m0 + xrow_l) * (uint32_t)K + 8u * (uint32_t)xch) * 2u;
  const uint32_t xstep = (uint32_t)XR * (uint32_t)K * 2u;
  // weights: load I of a super-step (I < 2 NT) gives lane 16q + c the 16 bytes q
  // (words 4q .. 4q+3) of column 16 I + c of the wave's tile, so one load reads 64
  // contiguous bytes of each of 16 columns; shuffle_w then moves them into the
  // lanes of the MFMA B operand
  const uint32_t wvo = (uint32_t)(n0 + wn * WTN + (lane & 15)) * (uint32_t)(K >> 1) + 16u * (uint32_t)(lane >> 4);
  const uint32_t wstep = 16u * (uint32_t)(K >> 1);  // 16 columns
  // (s, z) producer: thread t stages column n0 + (t & 255) for the two groups of a
  // pair (with 512 threads, two threads write the same value)
  const int tc = t & 255;
  const uint32_t szvo = ((uint32_t)(n0 + tc) * (uint32_t)G + (uint32_t)g0) * 2u;

  struct WSet {
    uint4 w[NT][2];
  };
  // weights: 2 WS register sets; the sets of WS consecutive super-steps are loaded
  // together (WS super-steps ahead of the first of them), so the 64 bytes a column
  // gives each group come from DRAM as WS neighbouring pieces rather than one piece
  // per super-step
  WSet wset[2 * WS];
  uint32_t sp = 0, zp = 0;  // staged (s, z) of a pair: fp16 pairs (group 2q, 2q + 1)
  // the loads of super-step g in four parts (part p: activation loads XP p ..
  // XP (p + 1) - 1 into stage xd, and the weights of loads p NT / 2 ..), issued over
  // the first four sub-steps (clamped past the slice)
  // activation loads XP p .. XP (p + 1) - 1 of super-step g into stage xd (clamped
  // past the slice)
  auto load_x_part = [&](f16* xd, int g, int p) {
    const uint32_t gg = (uint32_t)(g0 + min(g, ng - 1));
#pragma unroll
    for (int i = XP * p; i < XP * p + XP; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void*)(xd + (i * (T / 64) + wave) * 512), 16, xvo + i * xstep,
          (int)(256u * gg), 0, 0);
  };
  // weight loads I .. I + c - 1 of super-step g into W
  auto load_w = [&](WSet& W, int g, int I0, int c) {
    const uint32_t gg = (uint32_t)(g0 + min(g, ng - 1));
#pragma unroll
    for (int I = I0; I < I0 + c; ++I)
      W.w[I >> 1][I & 1] =
          __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wvo + I * wstep, (int)(64u * gg), 0));
  };
  // Loads 2j and 2j + 1 hold columns 32j .. 32j+15 and 32j+16 .. 32j+31 with 16-lane
  // row q holding words 4q .. 4q+3. The B operand of subtile j wants, in row R of the
  // wave, (column half R & 1, words 4 (R >> 1) ..) in its first register set and
  // (column half R & 1, words 8 + 4 (R >> 1) ..) in its second: a swap of odd and
  // even 16-lane rows between the two loads, then of the 32-lane halves between the
  // two results, per dword.
  auto shuffle_w = [&](WSet& W) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      uint32_t* x0 = reinterpret_cast<uint32_t*>(&W.w[j][0]);
      uint32_t* x1 = reinterpret_cast<uint32_t*>(&W.w[j][1]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto r16 = __builtin_amdgcn_permlane16_swap(x0[d], x1[d], false, false);
        const auto r32 = __builtin_amdgcn_permlane32_swap(r16[0], r16[1], false, false);
        x0[d] = r32[0];
        x1[d] = r32[1];
      }
    }
  };
  // (s, z) of the pair starting at super-step g (g even, clamped past the slice)
  auto load_sz = [&](int g) {
    const int so = 2 * min(g, ng - 2);
    sp = __builtin_amdgcn_raw_buffer_load_b32(srs, szvo, so, 0);
    zp = __builtin_amdgcn_raw_buffer_load_b32(zrs, szvo, so, 0);
  };
  auto store_sz = [&](int buf) {
    szl[(2 * buf) * 256 + tc] = (sp & 0xFFFFu) | (zp << 16);
    szl[(2 * buf + 1) * 256 + tc] = (sp >> 16) | (zp & 0xFFFF0000u);
  };
  auto read_sz = [&](uint32_t (&sz)[NT], int buf, int grp) {
#pragma unroll
    for (int j = 0; j < NT; ++j) sz[j] = szl[(2 * buf + grp) * 256 + wn * WTN + 32 * j + c32];
  };
  const uint32_t magic = magic_1024x2();
  // Transpose items of this thread (XT): the LDS offset of its value in a stage, its
  // byte offset in xt without the group's part (past the end when the item is not this
  // block's, so that the buffer store writes nothing), and whether its row is past M.
  // The block's items: cpb = 128 / tiles_n (rounded up) channels from tn cpb, those
  // below 128, times its rows below Mp; the launcher sends only shapes with
  // cpb BM <= kXtPerThread T, so a fixed number of items per thread covers them (no
  // loop, which would split the unrolled super-step).
  uint32_t xt_lds[kXtPerThread], xt_off[kXtPerThread];
  bool xt_zero[kXtPerThread];
  const __amdgpu_buffer_rsrc_t xtrs = buffer_rsrc(a.xt, XT ? (uint32_t)K * (uint32_t)a.xt_mp * 2u : 0u);
  if constexpr (XT) {
    const int cpb = (kBigSS + a.tiles_n - 1) / a.tiles_n;
#pragma unroll
    for (int i = 0; i < kXtPerThread; ++i) {
      const int q = t + i * T;
      const int cl = q / BM, r = q - cl * BM;
      const int ch = tn * cpb + cl, m = m0 + r;
      const bool mine = cl < cpb && ch < kBigSS && m < a.xt_mp;
      xt_lds[i] = (uint32_t)(r * kBigSS + ((((ch >> 3) & 15) ^ (r & 15)) << 3) + (ch & 7));
      xt_off[i] = mine ? ((uint32_t)ch * (uint32_t)a.xt_mp + (uint32_t)m) * 2u : 0x80000000u;
      xt_zero[i] = m >= M;
    }
  }
  // xt[g0 + g][ch][m] for the thread's items from stage xs (the swizzled layout above),
  // 64 consecutive rows per wave at 64-row tiles. Issued at the start of the super-step,
  // before its loads: the barrier's counted wait then still leaves only weight loads in
  // flight, whatever order loads and stores complete in. (Stored at the end of the
  // super-step instead, after the loads, the 70B layer at M = 512 took 1.2 us less,
  // but the wait would rely on stores being counted off in order with loads.)
  auto write_xt = [&](const f16* xs, int g) {
    const int so = __builtin_amdgcn_readfirstlane((g0 + g) * kBigSS * a.xt_mp * 2);
#pragma unroll
    for (int i = 0; i < kXtPerThread; ++i) {
      const f16 v = xs[xt_lds[i]];
      const unsigned short b = xt_zero[i] ? (unsigned short)0 : __builtin_bit_cast(unsigned short, v);
      __builtin_amdgcn_raw_buffer_store_b16(b, xtrs, (int)xt_off[i], so, 0);
    }
  };
  // A fragment of row r, chunk c = 8 (ks / 4) + 4h + ks % 4 (r & 15 == c32 & 15)
  auto read_a = [&](f16x8 (&av)[MT], const f16* xs, int ks) {
    const int c = (8 * (ks >> 2) + 4 * h + (ks & 3)) ^ (c32 & 15);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      av[i] = *reinterpret_cast<const f16x8*>(xs + (wm * WTM + 32 * i + c32) * kBigSS + 8 * c);
  };
  const f16x2 mul = {(f16)1.0f, (f16)0.0625f};
  auto deq_b = [&](const WSet& W, int j, int ks, uint32_t sz) {
    const f16x2 sz2 = as_f16x2(sz);  // (s, z)
    const f16x2 add = {-((f16)1024.0f + sz2[1]), -((f16)64.0f + sz2[1])}, s2 = {sz2[0], sz2[0]};
    const uint4& q = W.w[j][ks >> 2];
    const int c = ks & 3;
    const uint32_t w = c == 0 ? q.x : c == 1 ? q.y : c == 2 ? q.z : q.w;
    return as_f16x8(dequant_word_nat(w, magic, mul, add, s2));
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Super-step g = g_window + u (u = 0 .. 2 WS - 1, a constant after unrolling): its
  // weights are in set u and those of the next one in set u + 1; activations are read
  // from stage xs and the next ones loaded into stage xn (last read before the
  // barrier that ended the previous super-step). At u = 0 and u = WS the weights of
  // the other half of the sets (the next WS super-steps) are loaded. The A fragments
  // of sub-step ks + 1 are read during sub-step ks, and the B operand of the next
  // column (of the next sub-step, or of the next super-step after the last column) is
  // unpacked during the MFMAs of the current one. The (s, z) of pair q + 1 are loaded
  // in the second super-step of pair q - 1 and staged in the first of pair q, a
  // barrier before they are first read.
  f16x8 a0[MT], a1[MT];
  f16x8 bcur;
  uint32_t szc[NT], szn[NT];
  auto superstep = [&](int u, const f16* xs, f16* xn, int g) {
    const WSet& W = wset[u];
    WSet& Wn = wset[(u + 1) % (2 * WS)];
    const int pp = g & 1, buf = (g >> 1) & 1;
    constexpr int WPK = WS * 2 * NT / 4;  // weight loads per sub-step 0 .. 3 at a window start
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      f16x8 (&cur)[MT] = (ks & 1) ? a1 : a0;
      f16x8 (&nxt)[MT] = (ks & 1) ? a0 : a1;
      // (s, z) and activation loads first, weight loads after them: the barrier at the
      // end then waits for the activations only (the transpose's stores, older still,
      // with them)
      if constexpr (XT)
        if (ks == 0) write_xt(xs, g);
      if (ks == 0 && pp == 1) load_sz(g + 3);
      if (ks == 0) {
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) load_x_part(xn, g + 1, p2);
      }
      if (ks < 4 && (u == 0 || u == WS)) {
        // window loads: super-steps g + WS + v into sets (u + WS + v) mod 2 WS
#pragma unroll
        for (int q = ks * WPK; q < (ks + 1) * WPK; ++q) {
          const int v = q / (2 * NT), I = q % (2 * NT);
          load_w(wset[(u + WS + v) % (2 * WS)], g + WS + v, I, 1);
        }
      }
      if (ks == 4 && pp == 0) store_sz(buf ^ 1);
      if (ks == 6) read_sz(szn, pp == 0 ? buf : buf ^ 1, pp ^ 1);  // the next super-step's
      if (ks < 7) read_a(nxt, xs, ks + 1);
      if (ks == 7) shuffle_w(Wn);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const f16x8 bnext = j + 1 < NT ? deq_b(W, j + 1, ks, szc[j + 1])
                                       : (ks < 7 ? deq_b(W, 0, ks + 1, szc[0]) : deq_b(Wn, 0, 0, szn[0]));
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i][j] = mfma_32x32x16(cur[i], bcur, acc[i][j]);
        bcur = bnext;
      }

      // (two waves per SIMD interleave MFMAs and vector work by themselves; an
      // explicit per-MFMA interleaving here only cost registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      // Stage xn must be complete for every wave before the barrier: wait for this
      // wave's activation loads (and LDS reads), but not for the weight loads issued
      // after them, which stay in flight (s_waitcnt: vmcnt in bits 3:0 and 15:14,
      // expcnt 7 = no wait, lgkmcnt 0). A plain __syncthreads() would wait for all.
      constexpr int nw = WS * 2 * NT;
      if (u == 0 || u == WS)
        __builtin_amdgcn_s_waitcnt((nw & 15) | ((nw >> 4) << 14) | 0x70);
      else
        __builtin_amdgcn_s_waitcnt(0x70);
      __builtin_amdgcn_s_barrier();
    }
    read_a(a0, xn, 0);
#pragma unroll
    for (int j = 0; j < NT; ++j) szc[j] = szn[j];
  };

  if (ng > 0) {
    // prologue: (s, z) of pairs 0 (staged) and 1 (in registers), activations of
    // super-step 0, weights of super-steps 0 .. WS - 1 (ng is a multiple of 2 WS)
    load_sz(0);
    store_sz(0);
    load_sz(2);
#pragma unroll
    for (int p = 0; p < 4; ++p) load_x_part(smem, 0, p);
#pragma unroll
    for (int v = 0; v < WS; ++v) load_w(wset[v], v, 0, 2 * NT);
    shuffle_w(wset[0]);
    __syncthreads();
    read_a(a0, smem, 0);
    read_sz(szc, 0, 0);
    bcur = deq_b(wset[0], 0, 0, szc[0]);
    for (int g = 0; g < ng; g += 2 * WS) {
#pragma unroll
      for (int u = 0; u < 2 * WS; ++u)
        superstep(u, smem + (u & 1) * STAGE, smem + ((u + 1) & 1) * STAGE, g + u);
    }
  }

  if (a.lr_r > 0 && slice == 0) lowrank_add32<MT, NT>(acc, a.lr_t, a.lr_up, a.lr_r, M, N, m0 + wm * WTM, n0 + wn * WTN, lane);
  // store: the final y, or this slice's fp32 partial tile
  store_output<MT, NT>(acc, a, slice, m0 + wm * WTM, n0 + wn * WTN, lane);
}

// sum over slices s = 0..S-1 of ws[s * MN + o], in slice order. The loads go out B at
// a time (addresses clamped into the S slices, the extra terms added as +0, which
// leaves the sum unchanged): one load per iteration would wait for each slice in turn.
// B follows S (2, 4 or 8), so that few slices issue no extra loads.
template <int B>
__device__ __forceinline__ float slice_sum_b(const float* __restrict__ ws, int S, size_t MN, size_t o) {
  float v = 0.f;
  for (int s0 = 0; s0 < S; s0 += B) {
    float p[B];
#pragma unroll
    for (int u = 0; u < B; ++u) p[u] = ws[(size_t)min(s0 + u, S - 1) * MN + o];
#pragma unroll
    for (int u = 0; u < B; ++u) v += s0 + u < S ? p[u] : 0.f;
  }
  return v;
}
__device__ __forceinline__ float slice_sum(const float* __restrict__ ws, int S, size_t MN, size_t o) {
  if (S <= 2) return slice_sum_b<2>(ws, S, MN, o);
  if (S <= 4) return slice_sum_b<4>(ws, S, MN, o);
  return slice_sum_b<8>(ws, S, MN, o);
}

// y = sum over slices s = 0..S-1 of ws[s] (fixed order), in the output dtype.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ ws, int S, size_t MN, void* __restrict__ y, int y_f32) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += stride) {
    const float v = slice_sum(ws, S, MN, i);
    if (y_f32)
      static_cast<float*>(y)[i] = v;
    else
      static_cast<f16*>(y)[i] = (f16)v;
  }
}

// x [M][K] -> xt [K][Mp] (Mp: M rounded up to 8; rows M .. Mp-1 of xt are zero), in
// 64 x 64 tiles through LDS. The sparse term then reads, for an entry in input
// channel c, the activations of all rows as one contiguous run xt[c][0 .. M).
__global__ void __launch_bounds__(256) transpose_x_kernel(const f16* __restrict__ x, int M, int K,
                                                          f16* __restrict__ xt, int Mp) {
  __shared__ uint32_t tile[64][33];  // 64 rows x 64 halves, rows 33 dwords apart
  const int t = threadIdx.x;
  const int k0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 3, ch = q & 7;
    const int m = m0 + row;
    uint4 v = {0u, 0u, 0u, 0u};
    if (m < M) v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + k0 + 8 * ch);
    tile[row][4 * ch] = v.x;
    tile[row][4 * ch + 1] = v.y;
    tile[row][4 * ch + 2] = v.z;
    tile[row][4 * ch + 3] = v.w;
  }
  __syncthreads();
  const uint16_t* th = reinterpret_cast<const uint16_t*>(&tile[0][0]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;
    const int kk = q >> 3, mc = q & 7;
    const int m = m0 + 8 * mc;
    if (m >= Mp) continue;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)th[(8 * mc + 2 * j) * 66 + kk] | ((uint32_t)th[(8 * mc + 2 * j + 1) * 66 + kk] << 16);
    *reinterpret_cast<uint4*>(xt + (size_t)(k0 + kk) * Mp + m) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// VM consecutive fp16 values as floats (VM = 1, 2, 4, 8; p aligned to 2 VM bytes)
template <int VM>
__device__ __forceinline__ void load_halves(const f16* p, float (&o)[VM]) {
  if constexpr (VM == 8) {
    const f16x8 v = as_f16x8(*reinterpret_cast<const uint4*>(p));
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (float)v[j];
  } else if constexpr (VM == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const f16x2 a = as_f16x2(u.x), b = as_f16x2(u.y);
    o[0] = (float)a[0]; o[1] = (float)a[1]; o[2] = (float)b[0]; o[3] = (float)b[1];
  } else if constexpr (VM == 2) {
    const f16x2 a = as_f16x2(*reinterpret_cast<const uint32_t*>(p));
    o[0] = (float)a[0]; o[1] = (float)a[1];
  } else {
    o[0] = (float)p[0];
  }
}

// y = sum of the S fp32 K-slices + W_sparse x, for NC output channels per block and
// rows in chunks of 64 VM. Block b takes row chunks b % C, b % C + C, ... (C a
// divisor of 8) of channel block b / C: blocks are dealt to the 8 XCDs in turn, so
// every block on one XCD gathers from the same rows of xt, which then stay in that
// XCD's L2. Sparse term: wave w takes channels n0 + w and n0 + w + 8; each lane
// holds VM rows and adds, for every CSR entry (c, v) of the channel in order,
// v * xt[c][rows] (eight entries' loads in flight at once). The per-(row, channel)
// sums pass through LDS to the fixed-order slice sum.
template <int VM>
__global__ void __launch_bounds__(512)
splitk_sparse_reduce_kernel(const float* __restrict__ ws, int S, int M, int N, const f16* __restrict__ xt, int Mp,
                            const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                            const f16* __restrict__ val, void* __restrict__ y, int y_f32, int C) {
  constexpr int NC = 16, MC = 64 * VM, NW = 8;
  __shared__ float sp[NC][MC + 1];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // channel block: in each group of 16 / C channel blocks, position p runs on the
  // XCD of p mod (8 / C), so position p takes channel block 2 (p mod H) + p / H
  // (H = 8 / C): channel blocks 2j and 2j + 1, the two 64-byte halves of a row's
  // 128-byte lines of partial sums, are read through one L2 (blocks dealt to the
  // XCDs in turn would otherwise put them on two). The last group of fewer keeps
  // the plain order; with C == 8 the order is the plain one.
  int nb = blockIdx.x / C;
  const int nblk = gridDim.x / C, H = 8 / C, gs = 2 * H;
  if ((nb / gs) * gs + gs <= nblk) nb = (nb / gs) * gs + 2 * (nb % H) + (nb % gs) / H;
  const int n0 = nb * NC;
  const size_t MN = (size_t)M * N;
  for (int mb = (blockIdx.x % C) * MC; mb < M; mb += MC * C) {
    const int mrow = mb + VM * lane;
    const int mr = mrow < Mp ? mrow : 0;  // lanes past the padded rows read row 0
#pragma unroll
    for (int cc = 0; cc < NC / NW; ++cc) {
      const int nl = wave + NW * cc;
      const int n = n0 + nl;
      float acc[VM];
#pragma unroll
      for (int j = 0; j < VM; ++j) acc[j] = 0.f;
      if (n < N) {
        const int e0 = row_ptr[n], e1 = row_ptr[n + 1];
        // up to 64 entries at a time: lane l loads entry e + l's (column, value) in
        // one coalesced load each, and each entry reaches the whole wave through a
        // lane read (one vector memory instruction per entry, the gather, instead of
        // three)
        for (int e = e0; e < e1; e += 64) {
          const int el = min(e + lane, e1 - 1);
          const int lc = col[el];
          const int lv = (int)__builtin_bit_cast(uint16_t, val[el]);
          const int cnt = min(64, e1 - e);
          for (int u0 = 0; u0 < cnt; u0 += 8) {
            float xv[8][VM], v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const int uu = min(u0 + u, cnt - 1);
              const int c = __builtin_amdgcn_readlane(lc, uu);
              v[u] = (float)__builtin_bit_cast(f16, (uint16_t)__builtin_amdgcn_readlane(lv, uu));
              load_halves<VM>(xt + (size_t)c * Mp + mr, xv[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
              for (int j = 0; j < VM; ++j) acc[j] = u0 + u < cnt ? acc[j] + v[u] * xv[u][j] : acc[j];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < VM; ++j) sp[nl][VM * lane + j] = acc[j];
    }
    __syncthreads();
    for (int q = t; q < MC * NC; q += 64 * NW) {
      const int nl = q % NC, ml = q / NC;
      const int m = mb + ml, n = n0 + nl;
      if (m < M && n < N) {
        const size_t o = (size_t)m * N + n;
        float v = slice_sum(ws, S, MN, o);
        v += sp[nl][ml];
        if (y_f32)
          static_cast<float*>(y)[o] = v;
        else
          static_cast<f16*>(y)[o] = (f16)v;
      }
    }
    __syncthreads();
  }
}

struct GemmPlan {
  int bm, bn;
  // 0: gemm_kernel; 1: gemm_big_kernel 128 x 256; 2 (M <= 64): gemm_big_kernel 64 x 256
  // or 64 x 128 (bn) with weight windows of four or two super-steps
  int kind;
  int ksplit, k_per_slice;
  // the sparse term is added in the slice sum (of one slice or several), from
  // activations transposed into the workspace, instead of inside gemm_kernel
  bool sparse_in_reduce;
};

// Tile and split choice for M x N x K (shared by the launcher and the workspace query).
// Dense products take gemm_big_kernel above M = 128 (an even number of groups) and
// the M <= 64 kernels for M <= 64 (a multiple of four groups); the others take
// gemm_kernel (and so does a product with a CSR term unless its kernel splits K).
static GemmPlan plan_gemm_kind(int64_t M, int64_t N, int64_t K, bool sparse) {
  GemmPlan p;
  const int64_t G = K / 128;
  p.sparse_in_reduce = false;
  p.kind = sparse ? 0 : (M > 128 && G % 2 == 0 ? 1 : (M <= 64 && G % 4 == 0 ? 2 : 0));
  p.bm = p.kind == 1 ? 128 : (M <= 64 ? 64 : 128);
  p.bn = 256;
  int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  int64_t s = 1;
  if (p.kind != 0) {
    // split K while the grid is below two blocks per CU (large M) or one (M <= 64,
    // where longer slices amortize each block's first loads and partial stores better
    // than a second block per CU hides latency), and each slice keeps >= 8 groups;
    // slices are a multiple of two (large M) or four (M <= 64) groups
    const int64_t groups = K / 128;
    const auto split = [&](int64_t tl, int64_t target) {
      int64_t sp = 1;
      while (tl * sp * 2 <= target && groups / (sp * 2) >= 8) sp *= 2;
      return sp;
    };
    s = split(tiles, p.kind == 2 ? 256 : 512);
    // M <= 64 on a layer whose 64 x 256 tiles and slices leave CUs without a block:
    // 64 x 128 tiles instead (each wave one 32-column subtile), up to two blocks per
    // CU. Measured with the GEMM forced: 4096 x 4096 at M = 32 and 64 19.4 and 20.4
    // against 24.8 and 25.0 us. On the 70B down-projection, whose 256-wide grid has a
    // block on every CU, 128-wide tiles took 76.9 against 70.5 us at M = 64.
    if (p.kind == 2 && tiles * s < kBigFillBlocks) {
      p.bn = 128;
      tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
      s = split(tiles, 2 * kBigFillBlocks);
    }
    p.ksplit = (int)s;
    const int64_t q = p.kind == 1 ? 2 : 4;  // slices: a multiple of q groups
    const int64_t per = ((groups + s - 1) / s + q - 1) / q * q;
    p.k_per_slice = (int)(per * 128);
  } else {
    const int64_t ksteps = K / kBK;
    // split K while the grid is below two blocks per CU and each slice keeps >= 16 steps
    while (tiles * s * 2 <= 512 && ksteps / (s * 2) >= 16) s *= 2;
    p.ksplit = (int)s;
    p.k_per_slice = (int)(((ksteps + s - 1) / s) * kBK);
  }
  return p;
}

static size_t partials_bytes(const GemmPlan& p, int64_t M, int64_t N) {
  return p.ksplit > 1 || p.sparse_in_reduce ? ((size_t)p.ksplit * M * N * 4 + 255) / 256 * 256 : 0;
}

static int64_t padded_rows(int64_t M) { return (M + 7) / 8 * 8; }

static size_t plan_workspace(const GemmPlan& p, int64_t M, int64_t N, int64_t K) {
  return partials_bytes(p, M, N) + (p.sparse_in_reduce ? (size_t)K * padded_rows(M) * 2 : 0);
}

// A product with a CSR term takes the dense kernel of its shape when that is
// gemm_big_kernel, split or not: the sparse term then joins the slice sum (of one
// fp32 slice when K is not split). Other shapes take gemm_kernel, the term inside.
static GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool sparse) {
  if (sparse) {
    GemmPlan d = plan_gemm_kind(M, N, K, false);
    if (d.kind != 0) {
      d.sparse_in_reduce = true;
      return d;
    }
  }
  return plan_gemm_kind(M, N, K, sparse);
}

// the dense product's GEMM plan for this shape (given a full workspace)
GemmPlanInfo gemm_plan_info(int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(M, N, K, false);
  const int64_t bm = p.kind == 1 ? 128 : p.bm;
  GemmPlanInfo i;
  i.blocks = ((M + bm - 1) / bm) * ((N + p.bn - 1) / p.bn) * p.ksplit;
  i.ksplit = p.ksplit;
  i.big = p.kind != 0;
  i.bn = p.bn;
  return i;
}

// enough for the dense and the sparse plan of the shape, and for the tile kernel's
// plan (the one the other weight formats take)
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const size_t a = plan_workspace(plan_gemm(M, N, K, false), M, N, K);
  const size_t b = plan_workspace(plan_gemm(M, N, K, true), M, N, K);
  const size_t c = plan_workspace(plan_gemm_kind(M, N, K, true), M, N, K);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

// the workspace of the plan a 4-bit, 128-channel-group product of this shape takes
// with a full workspace, dense or with a CSR term
size_t gemm_plan_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sparse) {
  return plan_workspace(plan_gemm(M, N, K, sparse), M, N, K);
}

template <int BM, int BN, int WGM, int WGN, int MINB, int WS>
static hipError_t launch_big(GemmArgs a, hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)BM * kBigSS * sizeof(f16) + kBigSzBytes;
  auto kern = a.xt != nullptr ? gemm_big_kernel<BM, BN, WGM, WGN, MINB, WS, true>
                              : gemm_big_kernel<BM, BN, WGM, WGN, MINB, WS, false>;
  {
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int64_t nblk = (int64_t)a.tiles_m * a.tiles_n * a.ksplit;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * WGM * WGN), lds, stream, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, bool SPARSE, int BITS = 4, bool G64 = false>
static hipError_t launch_tile(GemmArgs a, hipStream_t stream) {
  constexpr size_t lds = 2 * (size_t)BM * kLdsStride * sizeof(f16);
  auto kern = gemm_kernel<BM, BN, WGM, WGN, SPARSE, BITS, G64>;
  if (lds > 65536) {
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  const int64_t nblk = (int64_t)a.tiles_m * a.tiles_n * a.ksplit;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * WGM * WGN), lds, stream, a);
  return hipGetLastError();
}

// tile kernel for a weight format other than 4-bit codes with 128-channel groups
static hipError_t launch_tile_fmt(const GemmArgs& a, int bm, bool sp, WFormat f, hipStream_t stream) {
#define WQ_TF(BM, SP, B, G6) \
  if (bm == BM && sp == SP && f.bits == B && f.g64 == G6) return launch_tile<BM, 256, 1, 4, SP, B, G6>(a, stream);
#define WQ_TF_F(BM, SP) WQ_TF(BM, SP, 4, true) WQ_TF(BM, SP, 3, false) WQ_TF(BM, SP, 3, true)
  WQ_TF_F(64, true) WQ_TF_F(64, false) WQ_TF_F(128, true) WQ_TF_F(128, false)
#undef WQ_TF_F
#undef WQ_TF
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, int64_t nnz, void* y, int y_f32, void* workspace,
                       size_t workspace_bytes, const LowRank& lr, hipStream_t stream, WFormat f) {
  constexpr int64_t kRowsPerLaunch = (int64_t)1 << 20;  // keeps the block count within int range
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const bool sp = row_ptr != nullptr;
    // the other weight formats run in the tile kernel (its K step of 64 channels is
    // one 64-channel group, or two 3-bit runs per lane pair), the CSR term inside it
    GemmPlan p = f.plain() ? plan_gemm(mc, N, K, sp) : plan_gemm_kind(mc, N, K, true);
    if (p.sparse_in_reduce && (workspace == nullptr || workspace_bytes < plan_workspace(p, mc, N, K)))
      p = plan_gemm_kind(mc, N, K, true);  // too small a workspace: the sparse term inside gemm_kernel
    const size_t need = plan_workspace(p, mc, N, K);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
      p.ksplit = 1;  // no (or too small) workspace: run unsplit
      p.k_per_slice = (int)K;
    }
    const bool sp_kernel = sp && !p.sparse_in_reduce;  // sparse term inside gemm_kernel
    const int64_t Mp = padded_rows(mc);
    f16* xt = p.sparse_in_reduce
                  ? reinterpret_cast<f16*>(static_cast<char*>(workspace) + partials_bytes(p, mc, N))
                  : nullptr;
    // the GEMM writes x^T itself when its blocks' shares fit (wide layers); else a launch
    const int64_t big_bm = p.kind == 1 ? 128 : 64, tn = (N + p.bn - 1) / p.bn;
    const bool xt_in_gemm = p.sparse_in_reduce && (kBigSS + tn - 1) / tn * big_bm <= kXtPerThread * 256 &&
                            (size_t)K * (size_t)Mp * 2 < ((size_t)1 << 31);
    if (p.sparse_in_reduce && !xt_in_gemm) {
      const dim3 tgrid((unsigned)(K / 64), (unsigned)((mc + 63) / 64));
      hipLaunchKernelGGL(transpose_x_kernel, tgrid, dim3(256), 0, stream, reinterpret_cast<const f16*>(x) + m * K,
                         (int)mc, (int)K, xt, (int)Mp);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const size_t ysz = y_f32 ? 4 : 2;
    GemmArgs a;
    a.x = reinterpret_cast<const f16*>(x) + m * K;
    a.packed = packed;
    a.scales = reinterpret_cast<const f16*>(scales);
    a.zeros = reinterpret_cast<const f16*>(zeros);
    a.row_ptr = sp_kernel ? row_ptr : nullptr;
    a.col = col;
    a.val = reinterpret_cast<const f16*>(val);
    a.nnz = sp_kernel ? nnz : 0;
    void* yout = static_cast<char*>(y) + (size_t)(m * N) * ysz;
    a.y = p.ksplit > 1 || p.sparse_in_reduce ? workspace : yout;
    a.M = (int)mc;
    a.N = (int)N;
    a.K = (int)K;
    a.y_f32 = p.sparse_in_reduce ? 1 : y_f32;  // one fp32 slice when not split
    a.ksplit = p.ksplit;
    a.k_per_slice = p.k_per_slice;
    a.lr_t = lr.r > 0 ? reinterpret_cast<const f16*>(lr.t) + m * lr.r : nullptr;
    a.lr_up = reinterpret_cast<const f16*>(lr.up);
    a.lr_r = (int)lr.r;
    a.xt = xt_in_gemm ? xt : nullptr;  // written by gemm_big_kernel<..., true>
    a.xt_mp = (int)Mp;
    hipError_t e;
    // weight windows of WS super-steps need slices and K of a multiple of 2 WS groups;
    // kind 2 has G and its slices (or the whole K) multiples of four groups, so WS is
    // four or two
    const int64_t per = p.k_per_slice / 128, G = K / 128;
    if (p.kind == 1)
      e = launch_big<128, 256, 1, 4, 2, 1>(a, stream);
    else if (p.kind == 2 && per % 8 == 0 && G % 8 == 0)
      e = p.bn == 128 ? launch_big<64, 128, 1, 4, 2, 4>(a, stream) : launch_big<64, 256, 1, 4, 2, 4>(a, stream);
    else if (p.kind == 2)
      e = p.bn == 128 ? launch_big<64, 128, 1, 4, 2, 2>(a, stream) : launch_big<64, 256, 1, 4, 2, 2>(a, stream);
    else if (!f.plain())
      e = launch_tile_fmt(a, p.bm, sp_kernel, f, stream);
    else if (p.bm == 64)
      e = sp_kernel ? launch_tile<64, 256, 1, 4, true>(a, stream) : launch_tile<64, 256, 1, 4, false>(a, stream);
    else
      e = sp_kernel ? launch_tile<128, 256, 1, 4, true>(a, stream) : launch_tile<128, 256, 1, 4, false>(a, stream);
    if (e != hipSuccess) return e;
    if (p.sparse_in_reduce) {
      // Up to 512 rows: one chunk per block (the gather's loads 2 VM bytes per lane).
      // More rows: chunks of 256 dealt to the XCDs (C of them, C a divisor of 8) when
      // such a chunk of xt (K x 256 halves) fits well inside one XCD's 4 MB L2, so
      // that the gather reads it from there rather than from the memory-side cache
      // (prefill layer with 0.45 % outliers: 378-383 against 407-410 us). Dealt at 64
      // or 128 rows per chunk, the 70B layer at M = 512 lost 7-90 us (eight times the
      // CSR walks, 2-byte loads), and its K = 28672 leaves no chunk inside one L2.
      int vm = mc > 256 ? 8 : mc > 128 ? 4 : mc > 64 ? 2 : 1;
      int C = 1;
      if (mc > 512 && K * 256 * 2 <= ((int64_t)5 << 19)) {
        vm = 4;
        const int64_t chunks = (mc + 255) / 256;
        C = chunks > 4 ? 8 : chunks > 2 ? 4 : 2;
      }
      const dim3 rgrid((unsigned)((N + 15) / 16 * C));
#define WQ_SPRED(VM)                                                                                         \
  if (vm == VM)                                                                                              \
  hipLaunchKernelGGL(splitk_sparse_reduce_kernel<VM>, rgrid, dim3(512), 0, stream,                          \
                     static_cast<const float*>(workspace), p.ksplit, (int)mc, (int)N, xt, (int)Mp, row_ptr, col, \
                     reinterpret_cast<const f16*>(val), yout, y_f32, C)
      WQ_SPRED(1);
      WQ_SPRED(2);
      WQ_SPRED(4);
      WQ_SPRED(8);
#undef WQ_SPRED
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else if (p.ksplit > 1) {
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
