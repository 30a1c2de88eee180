// Down-projection of the low-rank high-precision branch for gfx950.
//
// The SVDQuant section of the DeepCompressor README keeps the weights' outliers in
// a high-precision low-rank branch next to the 4-bit residual, and fuses that
// branch into the low-bit kernel rather than running it as a separate pass over
// the activations. With W = L2 . L1 + R (L1 [r, K], L2 [N, r], fp16), the product
// needs t = x . L1^T first; the linear kernels then add t . L2^T to each output
// tile before its single store. This file computes t, with one of two kernels:
//
//  lowrank_down_dot_kernel (at most 16 rows, decode): the product is r dot-product
//    sets over K, so each pair (component, group of at most four rows) gets a block
//    of its own (r * ceil(M / 4) blocks, each reading its row of L1 once, where a
//    16-component MFMA tile would put sixteen rows of L1 through one CU; more rows
//    per block make each wave issue more loads one after another, which costs more
//    than reading the row of L1 again from L2). The block's waves split K in
//    512-channel steps, accumulate x . L1[j] with fp16 dot2 into fp32 per row, sum
//    their lanes by recursive halving (each exchange hands half of a lane's rows to
//    its partner) and their waves through LDS in wave order, and store fp16 t.
//  lowrank_down_kernel (more rows): one block per 16 rows of x, CT = 32 (or 16)
//    components of the rank and chunk of at most 128 steps of 32 input channels
//    (the chunks are sized so that the grid has about a block per CU); each of its
//    sixteen waves takes every sixteenth step of the chunk, with all its loads
//    issued up front, and feeds CT / 16 16x16x32 fp16 MFMAs per step (x rows in A,
//    rows of L1 in B, fp32 accumulation), so each row of x is read once per CT
//    components. Blocks of 16 components are used where K fits one chunk and the
//    32-component tiles give at least half of the CUs but not all of them a block:
//    twice the blocks, each with two thirds of the loads, and still no partials. The waves'
//    tiles are summed through LDS in a fixed order; with a single chunk the block
//    rounds the sum to fp16 t itself, else it stores the chunk's fp32 partial and
//  lowrank_finish_kernel: t = fp16 of the sum of the chunks' partials in chunk
//    order, a thread per element with eight chunks' loads in flight at a time.
// t is rounded once, to fp16, because it is an MFMA operand of the up-projection.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

constexpr int kLrWaves = 16;
constexpr int kLrStepsPerWave = 8;
constexpr int kLrChunkSteps = kLrWaves * kLrStepsPerWave;  // 32-channel steps per K chunk

constexpr int64_t kLrTargetBlocks = 256;  // about one block per CU

// Steps per chunk and number of chunks for M rows: one chunk (no partials) when
// the row and component tiles alone give half the CUs a block and K fits one
// chunk; otherwise enough chunks for about a block per CU, but at least one step
// for each of a block's waves.
struct LrPlan {
  int steps, chunks, ct;  // ct: components per block (32 or 16)
};
static LrPlan lowrank_plan(int64_t M, int64_t K, int64_t r) {
  const int64_t nsteps = K / 32, tiles32 = ((M + 15) / 16) * (r / 32);
  const int ct = nsteps <= kLrChunkSteps && tiles32 >= kLrTargetBlocks / 2 && tiles32 < kLrTargetBlocks ? 16 : 32;
  const int64_t tiles = ct == 16 ? 2 * tiles32 : tiles32;
  int64_t chunks = (nsteps + kLrChunkSteps - 1) / kLrChunkSteps;
  if (!(chunks == 1 && tiles >= kLrTargetBlocks / 2)) {
    const int64_t want = (kLrTargetBlocks + tiles - 1) / tiles;
    const int64_t cap = nsteps / kLrWaves > chunks ? nsteps / kLrWaves : chunks;
    chunks = want > chunks ? want : chunks;
    chunks = chunks < cap ? chunks : cap;
  }
  const int64_t steps = (nsteps + chunks - 1) / chunks;
  return LrPlan{(int)steps, (int)((nsteps + steps - 1) / steps), ct};
}

constexpr int64_t kLrRowsPerLaunch = 65535 * 16;  // gridDim.y limit

// enough for the partials of every launch: a full one and the remainder
size_t lowrank_partial_bytes(int64_t M, int64_t K, int64_t r) {
  if (M <= 16) return 0;  // the dot kernel writes t directly
  size_t most = 0;
  for (const int64_t rows : {M < kLrRowsPerLaunch ? M : kLrRowsPerLaunch, M % kLrRowsPerLaunch}) {
    if (rows == 0) continue;
    const LrPlan p = lowrank_plan(rows, K, r);
    const size_t b = p.chunks > 1 ? ((size_t)p.chunks * rows * r * 4 + 255) / 256 * 256 : 0;
    most = b > most ? b : most;
  }
  return most;
}

template <int CT>
__global__ void __launch_bounds__(64 * kLrWaves)
lowrank_down_kernel(const f16* __restrict__ x, int M, int K, const f16* __restrict__ L1, int r, int cs,
                    float* __restrict__ part, f16* __restrict__ t) {
  static_assert(CT == 16 || CT == 32, "16 or 32 components per block");
  constexpr int U = CT / 16;  // 16x16 tiles per block
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & 15, h = lane >> 4;
  const int j0 = blockIdx.x * CT, m0 = blockIdx.y * 16, chunk = blockIdx.z;
  const int s0 = chunk * cs, s1 = min(K / 32, s0 + cs);  // cs <= kLrChunkSteps
  // lane (h, q): row m0 + q of x (rows past M read row M - 1, never stored) and
  // components j0 + 16 u + q of L1 (r is a multiple of 32), channels
  // 32 s + 8 h .. + 7
  const f16* xr = x + (size_t)min(m0 + q, M - 1) * K + 8 * h;
  const f16* lr0 = L1 + (size_t)(j0 + q) * K + 8 * h;
  // a wave's steps: s0 + wave + 16 i below s1 (a wave-uniform test: steps past the
  // chunk load nothing, where clamped reloads of one address would contend)
  uint4 av[kLrStepsPerWave], bv[kLrStepsPerWave][U];
#pragma unroll
  for (int i = 0; i < kLrStepsPerWave; ++i) {
    const int s = s0 + wave + kLrWaves * i;
    if (s < s1) {
      av[i] = *reinterpret_cast<const uint4*>(xr + 32 * s);
#pragma unroll
      for (int u = 0; u < U; ++u) bv[i][u] = *reinterpret_cast<const uint4*>(lr0 + (size_t)16 * u * K + 32 * s);
    }
  }
  f32x4 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kLrStepsPerWave; ++i)
    if (s0 + wave + kLrWaves * i < s1) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = mfma_16x16x32(as_f16x8(av[i]), as_f16x8(bv[i][u]), acc[u]);
    }
  __shared__ f32x4 red[kLrWaves - 1][U][64];
  if (wave > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) red[wave - 1][u][lane] = acc[u];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kLrWaves - 1; ++w)
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] += red[w][u][lane];
  // D[4 h + i][q] of tile u: row m0 + 4 h + i, component j0 + 16 u + q
  const bool single = gridDim.z == 1;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * h + i;
      if (m < M) {
        const size_t o = (size_t)m * r + j0 + 16 * u + q;
        if (single)
          t[o] = (f16)acc[u][i];
        else
          part[(size_t)chunk * M * r + o] = acc[u][i];
      }
    }
}

__global__ void __launch_bounds__(256)
lowrank_finish_kernel(const float* __restrict__ part, int chunks, int64_t Mr, f16* __restrict__ t) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < Mr; i += stride) {
    float v = 0.f;
    for (int c0 = 0; c0 < chunks; c0 += 8) {
      float p[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) p[u] = part[(size_t)min(c0 + u, chunks - 1) * Mr + i];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < chunks) v = c0 + u == 0 ? p[u] : v + p[u];
    }
    t[i] = (f16)v;
  }
}

constexpr int kDotMaxWaves = 16;

template <int MR>
__global__ void __launch_bounds__(64 * kDotMaxWaves)
lowrank_down_dot_kernel(const f16* __restrict__ x, int M, int K, const f16* __restrict__ L1, int r,
                        f16* __restrict__ t) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int j = blockIdx.x, m0 = blockIdx.y * MR;
  const int nsteps = (K + 511) >> 9;
  const f16* lrow = L1 + (size_t)j * K + 8 * lane;
  const f16* xrow[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) xrow[m] = x + (size_t)min(m0 + m, M - 1) * K + 8 * lane;  // rows past M: unused
  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;
  constexpr int SB = 4;  // steps per batch of loads
  for (int s0 = wave; s0 < nsteps; s0 += W * SB) {
    // lane's channels in step s: 512 s + 8 lane .. + 7 (K is a multiple of 128, so
    // a lane's eight are all in range or all out)
    uint4 b[SB];
    bool ok[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int c = 512 * (s0 + W * u);
      ok[u] = s0 + W * u < nsteps && c + 8 * lane < K;
      b[u] = ok[u] ? *reinterpret_cast<const uint4*>(lrow + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      uint4 a[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u)
        a[u] = ok[u] ? *reinterpret_cast<const uint4*>(xrow[m] + 512 * (s0 + W * u)) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w}, bv[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, av[e]), __builtin_bit_cast(f16x2, bv[e]), acc[m],
                                          false);
      }
    }
  }
  // lanes: at the exchange with offset o the lane with bit o set keeps the upper
  // half of its rows and the partner the lower, each adding the other's copy; after
  // log2(MR) exchanges lane l holds row l >> (6 - log2(MR)), and the remaining
  // offsets sum that row over the lanes that share it.
  constexpr int LM = MR == 1 ? 0 : (MR == 2 ? 1 : 2);
  static_assert(1 << LM == MR, "rows per block: 1, 2 or 4");
#pragma unroll
  for (int step = 0, cnt = MR; step < 6; ++step, cnt = cnt > 1 ? cnt / 2 : 1) {
    const int o = 32 >> step;
    if (cnt > 1) {
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < cnt / 2; ++i) {
        const float give = upper ? acc[i] : acc[i + cnt / 2];
        const float keep = upper ? acc[i + cnt / 2] : acc[i];
        acc[i] = keep + __shfl_xor(give, o);
      }
    } else {
      acc[0] += __shfl_xor(acc[0], o);
    }
  }
  // waves: through LDS, summed in wave order by wave 0
  __shared__ float red[kDotMaxWaves][MR];
  if ((lane & ((64 >> LM) - 1)) == 0) red[wave][lane >> (6 - LM)] = acc[0];
  __syncthreads();
  if (wave == 0 && lane < MR && m0 + lane < M) {
    float v = red[0][lane];
    for (int w = 1; w < W; ++w) v += red[w][lane];
    t[(size_t)(m0 + lane) * r + j] = (f16)v;
  }
}

template <int MR>
static hipError_t launch_dot(const uint16_t* x, int64_t M, int64_t K, const uint16_t* L1, int64_t r, uint16_t* t,
                             hipStream_t stream) {
  const int64_t nsteps = (K + 511) / 512;
  int64_t w = (nsteps + 1) / 2;  // about two steps per wave
  w = w < 1 ? 1 : (w > kDotMaxWaves ? kDotMaxWaves : w);
  hipLaunchKernelGGL(lowrank_down_dot_kernel<MR>, dim3((unsigned)r, (unsigned)((M + MR - 1) / MR)),
                     dim3((unsigned)(64 * w)), 0, stream,
                     reinterpret_cast<const f16*>(x), (int)M, (int)K, reinterpret_cast<const f16*>(L1), (int)r,
                     reinterpret_cast<f16*>(t));
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* L1, int64_t r,
                               float* part, uint16_t* t, hipStream_t stream) {
  if (M <= 16) {
    if (M == 1) return launch_dot<1>(x, M, K, L1, r, t, stream);
    if (M == 2) return launch_dot<2>(x, M, K, L1, r, t, stream);
    return launch_dot<4>(x, M, K, L1, r, t, stream);
  }
  for (int64_t m = 0; m < M; m += kLrRowsPerLaunch) {
    const int64_t mc = M - m < kLrRowsPerLaunch ? M - m : kLrRowsPerLaunch;
    const LrPlan p = lowrank_plan(mc, K, r);
    const int chunks = p.chunks;
    f16* tm = reinterpret_cast<f16*>(t) + m * r;
    const dim3 grid((unsigned)(r / p.ct), (unsigned)((mc + 15) / 16), (unsigned)chunks);
    if (p.ct == 16)
      hipLaunchKernelGGL(lowrank_down_kernel<16>, grid, dim3(64 * kLrWaves), 0, stream,
                         reinterpret_cast<const f16*>(x) + m * K, (int)mc, (int)K, reinterpret_cast<const f16*>(L1),
                         (int)r, p.steps, part, tm);
    else
      hipLaunchKernelGGL(lowrank_down_kernel<32>, grid, dim3(64 * kLrWaves), 0, stream,
                         reinterpret_cast<const f16*>(x) + m * K, (int)mc, (int)K, reinterpret_cast<const f16*>(L1),
                         (int)r, p.steps, part, tm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (chunks > 1) {
      const int64_t Mr = mc * r;
      const int64_t blocks = (Mr + 255) / 256 < 1024 ? (Mr + 255) / 256 : 1024;
      hipLaunchKernelGGL(lowrank_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, chunks, Mr, tm);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace wq
