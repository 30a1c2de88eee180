#pragma once
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
//  gemv_ring_kernel (activations too large for LDS): each group's activations are
//    prefetched with its weights, in whole-row pieces, and each wave passes them
//    through an LDS slot of its own into the fragment order of the MFMA. The weights
//    are unpacked to the exact integers q - z (nine instructions per word).
//
// Every global load is unconditional, with its address clamped to valid memory: a
// load under a divergent branch makes the compiler wait for all outstanding loads
// where the branches join, which would serialize the stream. For the same reason
// staged values are loaded before the weight prefetch is issued and stored after.
#include <type_traits>

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

constexpr int kGemvWaves = 4;   // KW
constexpr int kGemvDepth = 8;   // D: groups in flight per lane (128-bit weight loads)
constexpr int kGemvRingDepth = 4;  // D of gemv_ring_kernel
constexpr int kNumCu = 256;
constexpr int kGemvEarly = 2;   // weight groups issued before the wait on staged data (see below)
constexpr int kXLdsMaxHalves = 32768;
constexpr int kSparseBatch = 4;  // CSR entries per lane whose loads are in flight together
// SZV value of gemv_lds_kernel for scales and zero-points held in registers (see below)
constexpr int kSzInRegs = -1;
// sched_barrier mask between consecutive groups of a window: scalar, MFMA, LDS and
// transcendental instructions may be scheduled across it; vector memory and the
// other vector ALU instructions may not. The weight refills then stay next to the
// group that frees their register, and the unpacking of a word is not hoisted above
// earlier groups (which would move the wait for its load up with it).
constexpr int kSchedKeepGroups = 0x0004 | 0x0008 | 0x0080 | 0x0100 | 0x0200 | 0x0400;

// ---------------------------------------------------------------------------
// Scale / zero-point staging: LDS sz[16][G + 1] = (s, 1024 + z) for the block's rows.
// The row stride G + 1 is odd (G is even whenever it matters), so the 16 lanes that
// read one group of 16 rows hit 16 different banks.
//   SZV = 8, 4, 2: rows as vectors of SZV halves (G % SZV == 0, so no vector
//     crosses a row; G <= kSzMaxG): <= 2, 2, 4 loads per thread
//   SZV = 1: as halves (G <= 64): <= 4 loads per thread
//   SZV = 0: a plain loop (any G), run after the weight prefetch
template <int V> struct SzBits;
template <> struct SzBits<8> { typedef uint4 type; };
template <> struct SzBits<4> { typedef uint2 type; };
template <> struct SzBits<2> { typedef uint32_t type; };
template <> struct SzBits<1> { typedef uint16_t type; };
// the same bits as V halves, in a register type (indexing a bit-cast array would go
// through scratch memory)
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
template <int V> struct SzHalves;
template <> struct SzHalves<8> { typedef f16x8 type; };
template <> struct SzHalves<4> { typedef f16x4 type; };
template <> struct SzHalves<2> { typedef f16x2 type; };
template <> struct SzHalves<1> { typedef f16 type; };
template <int V>
__device__ __forceinline__ f16 sz_half(const typename SzHalves<V>::type& v, int j) {
  if constexpr (V == 1) {
    return v;
  } else {
    return v[j];
  }
}
// largest G each vector width is chosen for
template <int V> constexpr int kSzMaxG = V == 8 ? 256 : (V == 1 ? 64 : 128);

template <int SZV, int T>
struct SzStage {
  static constexpr int V = SZV > 0 ? SZV : 1;
  static constexpr int C = SZV == 0 ? 0 : (16 * kSzMaxG<V> / V + T - 1) / T;
  typedef typename SzBits<V>::type Vec;
  // single halves are held in 32-bit registers (arrays of 16-bit values stay in memory)
  typedef typename std::conditional<V == 1, uint32_t, Vec>::type Reg;
  Reg vs[C > 0 ? C : 1], vz[C > 0 ? C : 1];

  __device__ __forceinline__ void load(const f16* scales, const f16* zeros, int n0, int N, int G, int t) {
    const int nload = 16 * G / V;
    // the block's 16 rows are contiguous; past row N - 1 the last vector is repeated
    const size_t o0 = (size_t)n0 * G, o_last = (size_t)N * G - V;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int idx = min(t + i * T, nload - 1);
      const size_t o = min(o0 + (size_t)idx * V, o_last);
      vs[i] = *reinterpret_cast<const Vec*>(scales + o);
      vz[i] = *reinterpret_cast<const Vec*>(zeros + o);
    }
  }
  // stores are unconditional too (clamped indices rewrite identical values), so the
  // compiler cannot sink a staging load behind the weight prefetch
  __device__ __forceinline__ void store(f16x2* sz, const f16* scales, const f16* zeros, int n0, int N, int G,
                                        int t) {
    const f16 k1024 = (f16)1024.0f;
    const int nload = 16 * G / V;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int idx = min(t + i * T, nload - 1);
      typedef typename SzHalves<V>::type H;
      const H s = __builtin_bit_cast(H, (Vec)vs[i]), z = __builtin_bit_cast(H, (Vec)vz[i]);
      const int base = V * idx + (V * idx) / G;  // row * (G + 1) + column
#pragma unroll
      for (int j = 0; j < V; ++j) sz[base + j] = f16x2{sz_half<V>(s, j), (f16)(k1024 + sz_half<V>(z, j))};
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

// The first B CSR entries of a lane's share of a row (entries e0, e0 + KW, ... below
// e1), loaded in the prologue so that their latency hides under the weight stream.
// Loads are unconditional: indices are clamped into the row, or to entry 0 for an
// empty row (the product only takes this path with nnz >= 1), and values stay raw
// fp16 until use, since converting them would wait for the load on the spot.
template <int B, int KW>
struct SparseHead {
  int c[B];
  f16 v[B];
  __device__ __forceinline__ void load(const int32_t* col, const f16* val, int e0, int e1) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int eb = max(min(e0 + b * KW, e1 - 1), 0);
      c[b] = col[eb];
      v[b] = val[eb];
    }
  }
  // value of entry b, 0 past the row end
  __device__ __forceinline__ float weight(int b, int e0, int e1) const {
    return e0 + b * KW < e1 ? (float)v[b] : 0.0f;
  }
};

// Sum over each 16-lane row of the wave (fixed order, a Hillis-Steele scan with
// DPP row shifts that read 0 past the row start); the row total lands in its last
// lane. DPP moves cost a VALU slot, where a lane shuffle through LDS would cost a
// round trip per step.
__device__ __forceinline__ float row16_sum_to_last(float v) {
#define WQ_ROW_SHR(n) \
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + (n), 0xf, 0xf, true))
  WQ_ROW_SHR(1);
  WQ_ROW_SHR(2);
  WQ_ROW_SHR(4);
  WQ_ROW_SHR(8);
#undef WQ_ROW_SHR
  return v;
}

// Keeps the four registers of an MFMA result reserved until the group's epilogue
// has consumed it (acc depends on it), in accumulation registers. With fewer than
// four output rows stored, part[1..3] are never read; in blocks of more than 256
// threads the compiler then put the MFMA result in ordinary vector registers and
// handed the unread ones to other instructions while the MFMA could still be
// writing them, which corrupted an LDS address (wrong results, no fault). An
// accumulation-register operand here keeps them reserved and puts the MFMA in its
// accumulation-register form, as in 256-thread blocks. No instruction is emitted.
// The hazard was seen only in blocks of more than 256 threads, which no decode
// launch uses: kGemvMaxThreads caps the kernels that rely on this guard.
__device__ __forceinline__ void hold_accumulator(const f32x4& part, const f32x4& acc) {
  asm volatile("" ::"a"(part), "v"(acc));
}
constexpr int kGemvMaxThreads = 256;

// The 32 codes a lane reads per group of 128 input channels (input channels
// 32h .. 32h + 31 of the group for lane 16h + r): four words of 4-bit codes, or one
// 12-byte run of 3-bit codes. A row holds GW words per group.
template <int BITS> struct WRun;
template <> struct WRun<4> {
  typedef uint4 type;
  static constexpr int group_words = 16, lane_words = 4;
};
template <> struct WRun<3> {
  typedef uint3 type;
  static constexpr int group_words = 12, lane_words = 3;
};

// (1024 + q) pairs of MFMA step t (four steps per run), in perm_x8 order; 4-bit codes
// at odd positions carry a factor 16 (codes_biased_x16)
__device__ __forceinline__ uint4 step_biased(const uint4& w, int t, uint32_t magic) {
  return codes_biased_x16(t == 0 ? w.x : t == 1 ? w.y : t == 2 ? w.z : w.w, magic);
}
__device__ __forceinline__ uint4 step_biased(const uint3& w, int t, uint32_t magic) {
  return codes3_biased(w, t, magic);
}
// B operand of MFMA step t: exact q - z (SCALED = false) or fp16 (q - z) * s
// (bias = 1024 + z, nbias16 = -(64 + z), s in both halves)
template <bool SCALED>
__device__ __forceinline__ uint4 step_operand(const uint4& w, int t, uint32_t magic, f16x2 bias, f16x2 nbias16,
                                              f16x2 s) {
  const uint32_t x = t == 0 ? w.x : t == 1 ? w.y : t == 2 ? w.z : w.w;
  if constexpr (SCALED) {
    return dequant_word_x16(x, magic, bias, nbias16, s);
  } else {
    return codes_minus_zero_x16(x, magic, bias, nbias16);
  }
}
template <bool SCALED>
__device__ __forceinline__ uint4 step_operand(const uint3& w, int t, uint32_t magic, f16x2 bias, f16x2 nbias16,
                                              f16x2 s) {
  (void)nbias16;
  if constexpr (SCALED) {
    return dequant3(w, t, magic, bias, s);
  } else {
    return codes3_minus_zero(w, t, magic, bias);
  }
}

// (s, z) of a window of D groups in one load: 16 bytes for D = 8, 8 bytes for D = 4.
template <int D> struct SzVecOf;
template <> struct SzVecOf<8> { using type = uint4; };
template <> struct SzVecOf<4> { using type = uint2; };
template <int D> struct HalfWords { uint32_t w[D / 2]; };

// Half i of a vector of fp16 values; i is a compile-time constant after unrolling.
template <typename V>
__device__ __forceinline__ f16 half_of(const V& v, int i) {
  const auto a = __builtin_bit_cast(HalfWords<sizeof(V) / 2>, v);
  const uint32_t w = a.w[i >> 1];
  return bits_to_f16((uint16_t)((i & 1) ? w >> 16 : w & 0xffffu));
}

// A wave's ng groups are consumed in windows of D prefetched groups. Windows start
// at 0, D, 2D, ...; when D does not divide ng, the last window is moved back to end
// at group ng (so every load stays inside the wave's range and is prefetched like
// the others) and its first D - ng % D groups, already done, are skipped. With
// ng < D there is one window whose loads past ng repeat group ng - 1.
struct Windows {
  int n, nfull, last_lo, last_hi, ng, D;
  __device__ Windows(int ng_, int D_) : ng(ng_), D(D_) {
    nfull = ng / D;
    const int rem = ng - nfull * D;
    n = ng >= D ? nfull + (rem > 0) : (ng > 0);
    last_lo = ng >= D && rem > 0 ? D - rem : 0;
    last_hi = ng >= D ? D : ng;
  }
  // start of window b + 1, given the start gs of window b
  __device__ int next(int b, int gs) const { return b + 1 < nfull ? gs + D : ng - D; }
};

// Fixed-order sum of the KW partial tiles through LDS and the single store; with NT
// tiles per wave, tile j holds output channel n + 16j.
template <int KW, int NT>
__device__ __forceinline__ void reduce_store_tiles(f32x4 (&acc)[NT], int wave, int lane, int m0, int mrows, int n,
                                                   int N, void* y, int y_f32) {
  if constexpr (KW > 1) {
    __shared__ f32x4 red[KW - 1][NT][64];
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) red[wave - 1][j][lane] = acc[j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < KW - 1; ++w)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] += red[w][j][lane];
  }
  const int h = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int nj = n + 16 * j;
    if (nj >= N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * h + i;
      if (m < mrows) {
        const size_t o = (size_t)(m0 + m) * N + nj;
        if (y_f32)
          static_cast<float*>(y)[o] = acc[j][i];
        else
          static_cast<f16*>(y)[o] = (f16)acc[j][i];
      }
    }
  }
}

template <int KW>
__device__ __forceinline__ void reduce_store(f32x4 acc, int wave, int lane, int m0, int mrows, int n, int N,
                                             void* y, int y_f32) {
  f32x4 a[1] = {acc};
  reduce_store_tiles<KW, 1>(a, wave, lane, m0, mrows, n, N, y, y_f32);
}

// ---------------------------------------------------------------------------
// Up-projection of a low-rank branch for a wave's NT 16-channel tiles:
// acc[j] += t . L2^T, rows m0 .. m0 + 15 of t [M][r] in A and the tile's rows of
// L2 [N][r] in B, 32 of the rank per 16x16x32 MFMA (the same output layout as the
// weights' MFMAs); rows past M or N read the last row and are never stored.
//
// The operands of the first 32 components are loaded into registers at the end of
// the prologue (LrFirst), so their latency hides behind the main loop instead of
// following it; there, the test of r no longer waits (its argument is not among
// those preloaded into registers, and its load has landed by then), and plain loads
// leave the LDS accesses of the main loop free of waits (a load straight to LDS
// would make them wait for it).
template <int NT>
struct LrFirst {
  uint4 a, b[NT];
  __device__ __forceinline__ void load(const f16* t, const f16* up, int r, int M, int N, int m0, int n0, int lane) {
    const int q = lane & 15, h = lane >> 4;
    a = *reinterpret_cast<const uint4*>(t + (size_t)min(m0 + q, M - 1) * r + 8 * h);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      b[j] = *reinterpret_cast<const uint4*>(up + (size_t)min(n0 + 16 * j + q, N - 1) * r + 8 * h);
  }
};

// the sum itself, by the wave that loaded `first`: components 32 .. r - 1 from
// global memory, four steps' loads before their MFMAs
template <int NT>
__device__ __forceinline__ void lowrank_add16(f32x4 (&acc)[NT], const LrFirst<NT>& first, const f16* t, const f16* up,
                                              int r, int M, int N, int m0, int n0, int lane) {
  const int q = lane & 15, h = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = mfma_16x16x32(as_f16x8(first.a), as_f16x8(first.b[j]), acc[j]);
  const f16* ta = t + (size_t)min(m0 + q, M - 1) * r + 8 * h;
  const f16* ub[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) ub[j] = up + (size_t)min(n0 + 16 * j + q, N - 1) * r + 8 * h;
  for (int s = 32; s < r; s += 128) {
    uint4 a[4], b[4][NT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + 32 * u < r) {  // wave-uniform
        a[u] = *reinterpret_cast<const uint4*>(ta + s + 32 * u);
#pragma unroll
        for (int j = 0; j < NT; ++j) b[u][j] = *reinterpret_cast<const uint4*>(ub[j] + s + 32 * u);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + 32 * u < r)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = mfma_16x16x32(as_f16x8(a[u]), as_f16x8(b[u][j]), acc[j]);
  }
}

// G64: one (s, z) per 64 input channels. A lane's 32 channels of a group lie in one
// half of it, so each lane dequantizes (q - z) s into the operand with its own (s, z)
// (the 128-channel correction per group below cannot split the two halves): the
// activations are staged unscaled and without the sum tables, and (s, z) in LDS.
template <int KW, int D, int XC, int SZV, int MR, bool SP, int BITS = 4, bool G64 = false>
__global__ void __launch_bounds__(64 * KW)
gemv_lds_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
                const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
                const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                const f16* __restrict__ val, void* __restrict__ y, int y_f32, const f16* __restrict__ lr_t,
                const f16* __restrict__ lr_up, int lr_r) {
  constexpr int T = 64 * KW;
  static_assert(T <= kGemvMaxThreads, "MFMA results of larger blocks were clobbered (see hold_accumulator)");
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, in a scalar register
  const int r = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  static_assert(!G64 || SZV != kSzInRegs, "64-channel groups stage (s, z) in LDS");
  const int G = K >> 7;
  const int Gs = G64 ? 2 * G : G;  // (s, z) per row
  const int mrows = min(16, M - m0);
  const int SR = MR == 1 ? 1 : 4 * ((mrows + 3) >> 2);  // rows of the x-sum tables
  // LDS: sz[16][G + 1] (s, 1024 + z), unless SZV == kSzInRegs |
  //      xs[mrows][K] permuted, odd channels / 16 |
  //      sums of x over even / odd channels per (group, row)
  const size_t sz_bytes = SZV == kSzInRegs ? 0 : (size_t)16 * (Gs + 1) * 4;
  f16x2* sz = reinterpret_cast<f16x2*>(smem);
  f16* xs = reinterpret_cast<f16*>(smem + sz_bytes);
  // x sums per group: [g][2][SR] (even rows then odd rows); with MR == 1, SR == 1
  // and the pair (even, odd) of row 0 is adjacent
  float* sab = reinterpret_cast<float*>(smem + sz_bytes + (size_t)mrows * K * 2);

  const int n_ld = min(n0 + r, N - 1);  // ragged N: load a valid row, never store it
  using WT = typename WRun<BITS>::type;
  constexpr int GW = WRun<BITS>::group_words;
  const uint32_t* wrow = packed + (size_t)n_ld * (size_t)(G * GW) + WRun<BITS>::lane_words * h;
  const int g_lo = (G * wave) / KW, g_hi = (G * (wave + 1)) / KW;
  const int ng = g_hi - g_lo;

  // ---- prologue: staging loads, weight prefetch, staging stores
  // CSR bounds of the lane's row go out first: the wait on the staging loads covers them
  int sp_e0 = 0, sp_e1 = 0;
  if constexpr (SP) {
    sp_e0 = row_ptr[n_ld] + wave;
    sp_e1 = row_ptr[n_ld + 1];
  }
  SzStage<SZV == kSzInRegs ? 8 : SZV, T> szs;
  if constexpr (SZV != kSzInRegs) szs.load(scales, zeros, n0, N, Gs, t);
  // the block's rows of x are contiguous in memory and in LDS
  const int x_vecs = mrows * (K >> 3);
  const f16* xblk = x + (size_t)m0 * K;
  uint4 xv[XC];
#pragma unroll
  for (int i = 0; i < XC; ++i) xv[i] = *reinterpret_cast<const uint4*>(xblk + 8 * min(t + i * T, x_vecs - 1));
  // in-register mode: each lane loads the (s, z) of its row for a window of D groups
  // as two D-half vectors, issued with the window's weights
  using SzVec = typename SzVecOf<D>::type;
  const f16* s_row = scales + (size_t)n_ld * G + g_lo;
  const f16* z_row = zeros + (size_t)n_ld * G + g_lo;
  SzVec sv = {}, zv = {};
  WT wbuf[D];
  auto prefetch = [&](int i) {
    const int g = g_lo + min(i, max(ng - 1, 0));
    wbuf[i] = *reinterpret_cast<const WT*>(wrow + (size_t)g * GW);
  };
  // The staging loads stay ahead of the weight loads (waits count loads in issue
  // order). The first D0 weight groups go out before the wait on the staging loads,
  // the others after it. Every block starts at once and its activations come from
  // HBM too, so they queue behind the weight loads already issued: per-wave
  // timestamps on the 7B decode layer put the end of the staging at 2.7 us (median)
  // of a 6.5 us launch with all eight groups issued first. Two groups first keep
  // the stream going while the activations arrive sooner (6.65 -> 6.46 us there,
  // 8.0 -> 7.5 us at M = 2).
  constexpr int D0 = kGemvEarly < D ? kGemvEarly : D;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SZV == kSzInRegs) {
    sv = *reinterpret_cast<const SzVec*>(s_row);
    zv = *reinterpret_cast<const SzVec*>(z_row);
  }
#pragma unroll
  for (int i = 0; i < D0; ++i) prefetch(i);
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (SZV != kSzInRegs) szs.store(sz, scales, zeros, n0, N, Gs, t);
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
    if constexpr (BITS == 4 && !G64) {  // odd positions meet codes carrying a factor 16
      q.y = as_u32(as_f16x2(p.y) * sixteenth);
      q.w = as_u32(as_f16x2(p.w) * sixteenth);
    }
    // unconditional (clamped lanes rewrite the values of the last vector), so the
    // compiler cannot sink a staging load behind the weight prefetch
    *reinterpret_cast<uint4*>(xs + 8 * idx) = q;
    // the 16 chunks of a group sit in one 16-lane row; its total lands in lane 15
    se = row16_sum_to_last(se);
    so = row16_sum_to_last(so);
    if (!G64 && (idx_raw & 15) == 15 && idx_raw < x_vecs) {
      if constexpr (MR == 1) {  // a single row
        const int g = idx_raw >> 4;
        sab[2 * g] = se;
        sab[2 * g + 1] = so;
      } else {
        const int row = idx_raw / (K >> 3), g = (idx_raw - row * (K >> 3)) >> 4;
        sab[2 * g * SR + row] = se;
        sab[2 * g * SR + SR + row] = so;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = D0; i < D; ++i) prefetch(i);
  SparseHead<kSparseBatch, KW> sph;
  if constexpr (SP) sph.load(col, val, sp_e0, sp_e1);
  LrFirst<1> lr_first;
  if (lr_r > 0 && wave == 0) lr_first.load(lr_t, lr_up, lr_r, M, N, m0, n0, lane);
  __syncthreads();

  // ---- main loop over this wave's groups
  const int xr = min(r, mrows - 1);
  const f16* xl = xs + (size_t)xr * K + 32 * h;
  const f16x2* szr = sz + r * (Gs + 1);
  const int srow = min(4 * h, SR - 4);
  const uint32_t magic = magic_1024x2();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // group g of the wave, the i-th of its window (i selects the in-register (s, z))
  auto group = [&](const WT& w, int g, int i) {
    // the four LDS reads go out together, so their latency is paid once per group
    uint4 xa[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xa[tt] = *reinterpret_cast<const uint4*>(xl + (size_t)g * 128 + 8 * tt);
    __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);  // DS reads first
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
    if constexpr (G64) {
      // lanes h = 0, 1 and h = 2, 3 fall in the two halves of the group
      const f16x2 sbz = szr[2 * g + (h >> 1)];
      const f16x2 bias = {sbz[1], sbz[1]};
      const f16 nb = (f16)960.0f - sbz[1];  // -(64 + z)
      const f16x2 nbias16 = {nb, nb};
      const f16x2 s2 = {sbz[0], sbz[0]};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        part = mfma_16x16x32(as_f16x8(xa[tt]), as_f16x8(step_operand<true>(w, tt, magic, bias, nbias16, s2)), part);
#pragma unroll
      for (int i = 0; i < MR; ++i) acc[i] += part[i];
      hold_accumulator(part, acc);
      return;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      part = mfma_16x16x32(as_f16x8(xa[tt]), as_f16x8(step_biased(w, tt, magic)), part);
    float s, c1;  // c1 = 1024 + z
    if constexpr (SZV == kSzInRegs) {
      s = (float)half_of(sv, i);
      c1 = (float)half_of(zv, i) + 1024.0f;
    } else {
      const f16x2 sbz = szr[g];
      s = (float)sbz[0];
      c1 = (float)sbz[1];
    }
    const float c2 = BITS == 4 ? c1 - 960.0f : c1;  // 64 + z for the codes carrying 16
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
    hold_accumulator(part, acc);
  };

  // windows of D groups: each step consumes one buffered word, then refills the same
  // register with the same step of the next window (consume first, so the refill can
  // reuse the register and the loop carries no copy of an in-flight load).
  // In-register mode: the next window's (s, z) are loaded right after its first
  // weight word, so they arrive before that word is consumed; the current window's
  // are kept until its last group.
  const Windows win(ng, D);
  int gs = 0;
  for (int b = 0; b + 1 < win.n; ++b) {
    const int gs_next = win.next(b, gs);
    const uint32_t* wn = wrow + (size_t)(g_lo + gs_next) * GW;
    SzVec sn = sv, zn = zv;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      group(wbuf[i], g_lo + gs + i, i);
      wbuf[i] = *reinterpret_cast<const WT*>(wn + i * GW);
      if constexpr (SZV == kSzInRegs) {
        if (i == 0) {
          sn = *reinterpret_cast<const SzVec*>(s_row + gs_next);
          zn = *reinterpret_cast<const SzVec*>(z_row + gs_next);
        }
      }
      // keep the refill here: left alone, the scheduler sinks all refills to the end
      // of the window, and the wave then waits for every load before issuing more.
      __builtin_amdgcn_sched_barrier(kSchedKeepGroups);
    }
    sv = sn;
    zv = zn;
    gs = gs_next;
  }
  if (win.last_lo == 0 && win.last_hi == D) {  // a full last window, without branches
#pragma unroll
    for (int i = 0; i < D; ++i) group(wbuf[i], g_lo + gs + i, i);
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i >= win.last_lo && i < win.last_hi) group(wbuf[i], g_lo + gs + i, i);
  }

  // ---- sparse outlier term for column n = n0 + r (entries split over the KW
  // waves), activations from LDS
  const int n = n0 + r;
  if constexpr (SP) {
    const auto add = [&](int c, float v) {
      const int cs = (c & ~7) | perm_slot(c & 7);
      const float vu = BITS == 4 && !G64 && (c & 1) ? 16.0f * v : v;  // odd channels were stored / 16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(4 * h + i, mrows - 1);
        acc[i] += vu * (float)xs[(size_t)m * K + cs];
      }
    };
#pragma unroll
    for (int b = 0; b < kSparseBatch; ++b) add(sph.c[b], sph.weight(b, sp_e0, sp_e1));
    // the rest of the row, kSparseBatch entries per pass
    for (int e = sp_e0 + kSparseBatch * KW; e < sp_e1; e += kSparseBatch * KW) {
      SparseHead<kSparseBatch, KW> more;
      more.load(col, val, e, sp_e1);
#pragma unroll
      for (int b = 0; b < kSparseBatch; ++b) add(more.c[b], more.weight(b, e, sp_e1));
    }
  }
  // low-rank branch, once per output tile (wave 0, before the waves' sum)
  if (lr_r > 0 && wave == 0) {
    f32x4 a1[1] = {acc};
    lowrank_add16<1>(a1, lr_first, lr_t, lr_up, lr_r, M, N, m0, n0, lane);
    acc = a1[0];
  }
  reduce_store<KW>(acc, wave, lane, m0, mrows, n, N, y, y_f32);
}

// ---------------------------------------------------------------------------
// Each wave passes the activations of each of its groups through a slot of LDS of
// its own, right before use: the staging loads read whole rows (16 lanes x 16 bytes
// cover one row's 256 bytes of a group, four rows per load), where the fragment
// order of the MFMA would need four scattered 16-byte pieces per row and step.
// Rows of the slot are 272 bytes apart, so the 16 rows of a fragment read fall in
// distinct banks. One wave writes and reads its slot, and LDS instructions of a
// wave execute in order, so no barrier is involved.
// SZV == kSzInRegs (128-channel groups, windows starting at multiples of D): each
// lane loads the (s, z) of its rows for a window of D groups as two vectors,
// issued with the window's weights, and the block stages nothing.
template <int KW, int D, int XL, int NT, int SZV, bool SP, int BITS = 4, bool G64 = false>
__global__ void __launch_bounds__(64 * KW)
gemv_ring_kernel(const f16* __restrict__ x, int M, int K, const uint32_t* __restrict__ packed,
                 const f16* __restrict__ scales, const f16* __restrict__ zeros, int N,
                 const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                 const f16* __restrict__ val, void* __restrict__ y, int y_f32, const f16* __restrict__ lr_t,
                 const f16* __restrict__ lr_up, int lr_r) {
  constexpr int T = 64 * KW;
  static_assert(T <= kGemvMaxThreads, "MFMA results of larger blocks were clobbered (see hold_accumulator)");
  constexpr bool kRegs = SZV == kSzInRegs;
  static_assert(!kRegs || (!G64 && (D == 4 || D == 8)), "in-register (s, z): 128-channel groups, 4 or 8 groups");
  constexpr int R = 4 * XL;          // rows staged per group
  constexpr int kRowHalves = 136;    // 128 + 8
  extern __shared__ __align__(16) char smem[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * 16 * NT, m0 = blockIdx.y * 16;
  const int G = K >> 7;
  const int Gs = G64 ? 2 * G : G;  // (s, z) per row: one per 64 or per 128 input channels
  const int mrows = min(16, M - m0);
  f16x2* sz = reinterpret_cast<f16x2*>(smem);  // NT x [16][Gs + 1]: (s, 1024 + z), unless kRegs
  f16* slot = reinterpret_cast<f16*>(smem + (kRegs ? 0 : (size_t)NT * 16 * (Gs + 1) * 4)) + wave * (R * kRowHalves);

  using WT = typename WRun<BITS>::type;
  constexpr int GW = WRun<BITS>::group_words;
  const uint32_t* wrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
    wrow[j] = packed + (size_t)min(n0 + 16 * j + r, N - 1) * (size_t)(G * GW) + WRun<BITS>::lane_words * h;
  const int g_lo = (G * wave) / KW, g_hi = (G * (wave + 1)) / KW;
  const int ng = g_hi - g_lo;
  // staging: lane (h, r) loads chunk r (input channels 8r .. 8r+7 of a group) of
  // rows h, h + 4, ..., h + 4(XL-1); rows past M repeat the last row
  const f16* xst[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) xst[j] = x + (size_t)(m0 + min(h + 4 * j, mrows - 1)) * K + 8 * r;

  // CSR bounds of the lane's rows go out first: the wait on the staging loads covers
  // them (ragged N: a valid row is walked and never stored)
  int sp_e0[NT], sp_e1[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    sp_e0[j] = sp_e1[j] = 0;
    if constexpr (SP) {
      const int nr = min(n0 + 16 * j + r, N - 1);
      sp_e0[j] = row_ptr[nr] + wave;
      sp_e1[j] = row_ptr[nr + 1];
    }
  }
  SzStage<kRegs ? 8 : SZV, T> szs[NT];
  using SzVec = typename SzVecOf<(D == 4 || D == 8) ? D : 8>::type;
  const f16* s_row[NT];
  const f16* z_row[NT];
  SzVec sv[NT], zv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if constexpr (kRegs) {
      const size_t o = (size_t)min(n0 + 16 * j + r, N - 1) * G + g_lo;
      s_row[j] = scales + o;
      z_row[j] = zeros + o;
      sv[j] = *reinterpret_cast<const SzVec*>(s_row[j]);
      zv[j] = *reinterpret_cast<const SzVec*>(z_row[j]);
    } else {
      szs[j].load(scales, zeros, min(n0 + 16 * j, N - 1), N, Gs, t);
    }
  }
  const int g_first_valid = min(g_lo, G - 1);
  WT wbuf[D][NT];
  uint4 xbuf[D][XL];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int g = max(min(g_lo + i, g_hi - 1), g_first_valid);
#pragma unroll
    for (int j = 0; j < NT; ++j) wbuf[i][j] = *reinterpret_cast<const WT*>(wrow[j] + (size_t)g * GW);
#pragma unroll
    for (int j = 0; j < XL; ++j) xbuf[i][j] = *reinterpret_cast<const uint4*>(xst[j] + (size_t)g * 128);
  }
  if constexpr (!kRegs) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
      szs[j].store(sz + j * 16 * (Gs + 1), scales, zeros, min(n0 + 16 * j, N - 1), N, Gs, t);
    __syncthreads();
  }
  // the first CSR entries of each row, behind the initial weight prefetch
  constexpr int HB = kSparseBatch / NT;
  SparseHead<HB, KW> sph[NT];
  if constexpr (SP) {
#pragma unroll
    for (int j = 0; j < NT; ++j) sph[j].load(col, val, sp_e0[j], sp_e1[j]);
  }
  LrFirst<NT> lr_first;
  if (lr_r > 0 && wave == 0) lr_first.load(lr_t, lr_up, lr_r, M, N, m0, n0, lane);

  const f16x2* szr = sz + r * (Gs + 1);
  const uint32_t magic = magic_1024x2();
  const f16* frag = slot + min(r, R - 1) * kRowHalves + 32 * h;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f16 k1024 = (f16)1024.0f;
  // group g, position i of its window
  auto group = [&](const WT* w, const uint4* xg, int g, int i) {
#pragma unroll
    for (int j = 0; j < XL; ++j) *reinterpret_cast<uint4*>(slot + (h + 4 * j) * kRowHalves + 8 * r) = perm_x8(xg[j]);
    uint4 xa[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) xa[tt] = *reinterpret_cast<const uint4*>(frag + 8 * tt);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      // with 64-channel groups, lanes h = 0, 1 and h = 2, 3 fall in different groups,
      // so the scale goes into the operand; otherwise it scales the group's sum
      f16x2 sbz;
      if constexpr (kRegs) {
        sbz = f16x2{half_of(sv[j], i), (f16)(k1024 + half_of(zv[j], i))};
      } else {
        sbz = szr[j * 16 * (Gs + 1) + (G64 ? 2 * g + (h >> 1) : g)];
      }
      const f16x2 bias = {sbz[1], sbz[1]};
      const f16 nb = (f16)960.0f - sbz[1];  // -(64 + z)
      const f16x2 nbias16 = {nb, nb};
      const f16x2 s2 = {sbz[0], sbz[0]};
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        part = mfma_16x16x32(as_f16x8(xa[tt]), as_f16x8(step_operand<G64>(w[j], tt, magic, bias, nbias16, s2)), part);
      if constexpr (G64)
        acc[j] += part;
      else
        acc[j] += (float)sbz[0] * part;
      hold_accumulator(part, acc[j]);
    }
  };

  const Windows win(ng, D);
  int gs = 0;
  for (int b = 0; b + 1 < win.n; ++b) {
    const int gs_next = win.next(b, gs);
    SzVec sn[NT], zn[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      sn[j] = sv[j];
      zn[j] = zv[j];
    }
#pragma unroll
    for (int i = 0; i < D; ++i) {
      group(wbuf[i], xbuf[i], g_lo + gs + i, i);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        wbuf[i][j] = *reinterpret_cast<const WT*>(wrow[j] + (size_t)(g_lo + gs_next + i) * GW);
#pragma unroll
      for (int j = 0; j < XL; ++j)
        xbuf[i][j] = *reinterpret_cast<const uint4*>(xst[j] + (size_t)(g_lo + gs_next + i) * 128);
      // in-register mode: the next window's (s, z) right after its first weights
      if constexpr (kRegs) {
        if (i == 0) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            sn[j] = *reinterpret_cast<const SzVec*>(s_row[j] + gs_next);
            zn[j] = *reinterpret_cast<const SzVec*>(z_row[j] + gs_next);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(kSchedKeepGroups);  // keep the refill next to its consumption
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      sv[j] = sn[j];
      zv[j] = zn[j];
    }
    gs = gs_next;
  }
  // activations of the first CSR entries, gathered before the last window so that
  // its groups cover their latency
  f16 spx[NT][HB][4];
  if constexpr (SP) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int b = 0; b < HB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) spx[j][b][i] = x[(size_t)(m0 + min(4 * h + i, mrows - 1)) * K + sph[j].c[b]];
  }
  if (win.last_lo == 0 && win.last_hi == D) {
#pragma unroll
    for (int i = 0; i < D; ++i) group(wbuf[i], xbuf[i], g_lo + gs + i, i);
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i >= win.last_lo && i < win.last_hi) group(wbuf[i], xbuf[i], g_lo + gs + i, i);
  }

  if constexpr (SP) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int b = 0; b < HB; ++b) {
        const float v = sph[j].weight(b, sp_e0[j], sp_e1[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] += v * (float)spx[j][b][i];
      }
      // the rest of the row, kSparseBatch entries per pass, their loads in flight together
      for (int e = sp_e0[j] + HB * KW; e < sp_e1[j]; e += kSparseBatch * KW) {
        SparseHead<kSparseBatch, KW> more;
        more.load(col, val, e, sp_e1[j]);
        f16 xv[kSparseBatch][4];
#pragma unroll
        for (int b = 0; b < kSparseBatch; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) xv[b][i] = x[(size_t)(m0 + min(4 * h + i, mrows - 1)) * K + more.c[b]];
#pragma unroll
        for (int b = 0; b < kSparseBatch; ++b) {
          const float v = more.weight(b, e, sp_e1[j]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] += v * (float)xv[b][i];
        }
      }
    }
  }
  // low-rank branch, once per output tile (wave 0, before the waves' sum)
  if (lr_r > 0 && wave == 0) lowrank_add16<NT>(acc, lr_first, lr_t, lr_up, lr_r, M, N, m0, n0, lane);
  reduce_store_tiles<KW, NT>(acc, wave, lane, m0, mrows, n0 + r, N, y, y_f32);
}

// ---------------------------------------------------------------------------
// One launch per 65535 row tiles (the grid's y limit) of a decode kernel.
template <typename Kern>
inline hipError_t launch_rows(Kern kern, size_t lds, int cols, const uint16_t* x, int64_t M, int64_t K,
                              const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                              const int32_t* row_ptr, const int32_t* col, const uint16_t* val, void* y, int y_f32,
                              const LowRank& lr, hipStream_t stream) {
  if (lds > 65536) {
    const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
  }
  constexpr int64_t kRowsPerLaunch = 65535 * 16;  // gridDim.y limit
  const size_t ysz = y_f32 ? 4 : 2;
  for (int64_t m = 0; m < M; m += kRowsPerLaunch) {
    const int64_t mc = M - m < kRowsPerLaunch ? M - m : kRowsPerLaunch;
    const dim3 grid((unsigned)((N + cols - 1) / cols), (unsigned)((mc + 15) / 16));
    hipLaunchKernelGGL(kern, grid, dim3(64 * kGemvWaves), lds, stream, reinterpret_cast<const f16*>(x) + m * K,
                       (int)mc, (int)K, packed, reinterpret_cast<const f16*>(scales),
                       reinterpret_cast<const f16*>(zeros), (int)N, row_ptr, col, reinterpret_cast<const f16*>(val),
                       static_cast<char*>(y) + (size_t)(m * N) * ysz, y_f32,
                       lr.r > 0 ? reinterpret_cast<const f16*>(lr.t) + m * lr.r : nullptr,
                       reinterpret_cast<const f16*>(lr.up), (int)lr.r);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace wq
