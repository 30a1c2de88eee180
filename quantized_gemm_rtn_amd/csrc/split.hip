// Dense-and-sparse split for gfx950: the sparse_k weights of largest |w| move to
// an fp16 CSR matrix and read as +0 in the dense part (SqueezeLLM explainer,
// sections 2.2-2.3: W = W_dense + W_sparse with a small fraction of the weights
// kept in fp16; here chosen by magnitude, ties by lower flat index).
//
// Exact and deterministic:
//  1. Radix select on the 31-bit key bits(|w|) (for finite floats, integer order
//     of these bits is the order of |w|): three histogram passes of 11, 11 and 9
//     bits find the threshold key T of the sparse_k-th largest |w| and the count
//     of keys above it. Integer histogram counts do not depend on the order in
//     which they are added.
//  2. Per row: keys above T and keys equal to T.
//  3. One scan over rows: the equal keys are taken in ascending flat index until
//     sparse_k is reached (rows in order, columns in order inside a row), giving
//     each row's count and row_ptr.
//  4. Per row, in column order: write col/val and a selection bitmap that the
//     quantizer reads to treat the moved entries as +0.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

constexpr int kBins = 2048;

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t split_workspace_bytes(int64_t N, int64_t K) {
  size_t b = align256(kBins * 4) + align256(16 * 4) + 3 * align256((size_t)N * 4);
  b += align256((size_t)N * (size_t)K / 8);  // one bit per weight
  return b;
}

SplitWorkspace split_workspace_carve(void* base, int64_t N, int64_t K) {
  char* p = static_cast<char*>(base);
  SplitWorkspace w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256(kBins * 4);
  w.state = reinterpret_cast<uint32_t*>(p);
  p += align256(16 * 4);
  w.cnt_gt = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)N * 4);
  w.cnt_eq = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)N * 4);
  w.take_eq = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)N * 4);
  w.mask = reinterpret_cast<uint32_t*>(p);
  (void)K;
  return w;
}

__device__ __forceinline__ uint32_t abs_key(float v) { return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu; }

__global__ void __launch_bounds__(256) split_init_kernel(uint32_t* hist, uint32_t* state, uint32_t k) {
  for (int i = threadIdx.x; i < kBins; i += 256) hist[i] = 0;
  if (threadIdx.x == 0) {
    state[0] = 0;  // prefix of T found so far
    state[1] = 0;  // bits of T that are fixed
    state[2] = k;  // entries still to select among keys matching the prefix
    state[3] = 0;  // keys known to be above T
  }
}

__global__ void __launch_bounds__(256)
split_hist_kernel(const float* __restrict__ W, int64_t nvec, const uint32_t* __restrict__ state,
                  uint32_t* __restrict__ hist, int shift, uint32_t digit_mask) {
  __shared__ uint32_t lh[kBins];
  for (int i = threadIdx.x; i < kBins; i += 256) lh[i] = 0;
  __syncthreads();
  const uint32_t prefix = state[0], pmask = state[1];
  const float4* W4 = reinterpret_cast<const float4*>(W);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
    const float4 v = W4[i];
    const uint32_t k[4] = {abs_key(v.x), abs_key(v.y), abs_key(v.z), abs_key(v.w)};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((k[j] & pmask) == prefix) atomicAdd(&lh[(k[j] >> shift) & digit_mask], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += 256)
    if (lh[i]) atomicAdd(&hist[i], lh[i]);
}

// One block: find the digit holding the k-th largest key among those matching the
// prefix, extend the prefix, and clear the histogram for the next pass.
__global__ void __launch_bounds__(256)
split_select_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ state, int shift, uint32_t digit_mask) {
  __shared__ uint32_t h[kBins];
  __shared__ uint32_t part[256];
  const int t = threadIdx.x;
  for (int i = t; i < kBins; i += 256) {
    h[i] = hist[i];
    hist[i] = 0;
  }
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += h[8 * t + j];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    const uint32_t k = state[2];
    uint32_t above = 0;
    int tt = 255;
    for (; tt > 0; --tt) {
      if (above + part[tt] >= k) break;
      above += part[tt];
    }
    int d = 8 * tt + 7;
    for (; d > 8 * tt; --d) {
      if (above + h[d] >= k) break;
      above += h[d];
    }
    state[0] |= (uint32_t)d << shift;
    state[1] |= digit_mask << shift;
    state[2] = k - above;
    state[3] += above;
  }
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ void __launch_bounds__(256)
split_rowcount_kernel(const float* __restrict__ W, int64_t K, const uint32_t* __restrict__ state,
                      uint32_t* __restrict__ cnt_gt, uint32_t* __restrict__ cnt_eq) {
  __shared__ uint32_t sg[4], se[4];
  const int64_t n = blockIdx.x;
  const uint32_t T = state[0];
  const float4* row = reinterpret_cast<const float4*>(W + n * K);
  uint32_t gt = 0, eq = 0;
  for (int64_t i = threadIdx.x; i < K / 4; i += 256) {
    const float4 v = row[i];
    const uint32_t k[4] = {abs_key(v.x), abs_key(v.y), abs_key(v.z), abs_key(v.w)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gt += k[j] > T;
      eq += k[j] == T;
    }
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sg[w] = gt;
    se[w] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    cnt_gt[n] = sg[0] + sg[1] + sg[2] + sg[3];
    cnt_eq[n] = se[0] + se[1] + se[2] + se[3];
  }
}

// Exclusive scan over a 1024-thread block; returns the block total in `total`.
__device__ uint32_t block_excl_scan_1024(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (t == 0) {
    uint32_t a = 0;
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = sh[i];
      sh[i] = a;
      a += c;
    }
    sh[16] = a;
  }
  __syncthreads();
  const uint32_t r = x - v + sh[w];
  total = sh[16];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024)
split_scan_kernel(int64_t N, const uint32_t* __restrict__ state, const uint32_t* __restrict__ cnt_gt,
                  const uint32_t* __restrict__ cnt_eq, uint32_t* __restrict__ take_eq,
                  int32_t* __restrict__ row_ptr) {
  __shared__ uint32_t sh[17];
  const uint32_t need = state[2];  // keys equal to T that are selected, in flat order
  uint32_t carry_eq = 0, carry_nnz = 0;
  for (int64_t base = 0; base < N; base += 1024) {
    const int64_t n = base + threadIdx.x;
    const uint32_t ce = n < N ? cnt_eq[n] : 0u;
    const uint32_t cg = n < N ? cnt_gt[n] : 0u;
    uint32_t tot;
    const uint32_t before = carry_eq + block_excl_scan_1024(ce, sh, tot);
    carry_eq += tot;
    const uint32_t take = before >= need ? 0u : min(ce, need - before);
    const uint32_t nnz = cg + take;
    const uint32_t pos = carry_nnz + block_excl_scan_1024(nnz, sh, tot);
    carry_nnz += tot;
    if (n < N) {
      take_eq[n] = take;
      row_ptr[n] = (int32_t)pos;
    }
  }
  if (threadIdx.x == 0) row_ptr[N] = (int32_t)carry_nnz;
}

__global__ void __launch_bounds__(256)
split_compact_kernel(const float* __restrict__ W, int64_t K, const uint32_t* __restrict__ state,
                     const uint32_t* __restrict__ take_eq, const int32_t* __restrict__ row_ptr,
                     int32_t* __restrict__ col, uint16_t* __restrict__ val, uint32_t* __restrict__ mask) {
  __shared__ uint32_t wq_eq[4], wq_sel[4];
  const int64_t n = blockIdx.x;
  const uint32_t T = state[0];
  const uint32_t take = take_eq[n];
  const uint32_t base = (uint32_t)row_ptr[n];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t below = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  uint32_t run_eq = 0, run_sel = 0;
  for (int64_t k0 = 0; k0 < K; k0 += 256) {
    const int64_t k = k0 + t;
    const bool valid = k < K;
    const float v = valid ? W[n * K + k] : 0.0f;
    const uint32_t key = abs_key(v);
    const bool gt = valid && key > T;
    const bool eq = valid && key == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wq_eq[w] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_rank = run_eq + (uint32_t)__popcll(beq & below);
    for (int i = 0; i < w; ++i) eq_rank += wq_eq[i];
    const bool sel = gt || (eq && eq_rank < take);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wq_sel[w] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t pos = base + run_sel + (uint32_t)__popcll(bsel & below);
    for (int i = 0; i < w; ++i) pos += wq_sel[i];
    if (sel) {
      col[pos] = (int32_t)k;
      val[pos] = __builtin_bit_cast(uint16_t, (f16)v);
    }
    if (lane == 0 && k0 + 64 * w < K) {
      const int64_t word = (n * K + k0 + 64 * w) >> 5;
      mask[word] = (uint32_t)bsel;
      mask[word + 1] = (uint32_t)(bsel >> 32);
    }
    run_eq += wq_eq[0] + wq_eq[1] + wq_eq[2] + wq_eq[3];
    run_sel += wq_sel[0] + wq_sel[1] + wq_sel[2] + wq_sel[3];
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) fill_zero_i32_kernel(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

hipError_t launch_fill_zero_i32(int32_t* p, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_split(const float* W, int64_t N, int64_t K, int64_t sparse_k, int32_t* row_ptr,
                        int32_t* col, uint16_t* val, const SplitWorkspace& ws, hipStream_t stream) {
  const int64_t nvec = N * K / 4;
  int64_t hb = (nvec + 255) / 256;
  if (hb > 2048) hb = 2048;
  hipLaunchKernelGGL(split_init_kernel, dim3(1), dim3(256), 0, stream, ws.hist, ws.state, (uint32_t)sparse_k);
  const int shifts[3] = {20, 9, 0};
  const uint32_t masks[3] = {0x7FFu, 0x7FFu, 0x1FFu};
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL(split_hist_kernel, dim3((unsigned)hb), dim3(256), 0, stream, W, nvec, ws.state, ws.hist,
                       shifts[p], masks[p]);
    hipLaunchKernelGGL(split_select_kernel, dim3(1), dim3(256), 0, stream, ws.hist, ws.state, shifts[p], masks[p]);
  }
  hipLaunchKernelGGL(split_rowcount_kernel, dim3((unsigned)N), dim3(256), 0, stream, W, K, ws.state, ws.cnt_gt,
                     ws.cnt_eq);
  hipLaunchKernelGGL(split_scan_kernel, dim3(1), dim3(1024), 0, stream, N, ws.state, ws.cnt_gt, ws.cnt_eq,
                     ws.take_eq, row_ptr);
  hipLaunchKernelGGL(split_compact_kernel, dim3((unsigned)N), dim3(256), 0, stream, W, K, ws.state, ws.take_eq,
                     row_ptr, col, val, ws.mask);
  return hipGetLastError();
}

}  // namespace wq
