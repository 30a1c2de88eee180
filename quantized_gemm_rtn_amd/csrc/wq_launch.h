// Host-side launchers of the gfx950 kernels (internal; the public ABI is include/wq.h).
// Each returns the hipError_t of its launches; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Raises kernel `kern`'s dynamic-LDS limit to `bytes` on the current device, once:
// hipFuncSetAttribute costs tens of microseconds of host time per call, so the
// (kernel, device) pairs already raised are remembered (under a mutex).
hipError_t set_dynamic_lds(const void* kern, size_t bytes);

// Workspace carved up by the outlier split.
struct SplitWorkspace {
  uint32_t* hist;     // [2048] radix histogram
  uint32_t* state;    // [16]   select state: prefix, prefix mask, k remaining, count above
  uint32_t* cnt_gt;   // [N]    per row: keys above the threshold
  uint32_t* cnt_eq;   // [N]    per row: keys equal to the threshold
  uint32_t* take_eq;  // [N]    per row: equal keys that are selected
  uint32_t* mask;     // [N*K/32] selection bitmap
};
size_t split_workspace_bytes(int64_t N, int64_t K);
SplitWorkspace split_workspace_carve(void* base, int64_t N, int64_t K);

hipError_t launch_split(const float* W, int64_t N, int64_t K, int64_t sparse_k, int32_t* row_ptr,
                        int32_t* col, uint16_t* val, const SplitWorkspace& ws, hipStream_t stream);
hipError_t launch_fill_zero_i32(int32_t* p, int64_t n, hipStream_t stream);
// dst[r, i] = src[r, perm[i]] for a row-major [rows, K] matrix (K a multiple of 8)
hipError_t launch_gather_cols_f16(const uint16_t* src, int64_t rows, int64_t K, const int32_t* perm, uint16_t* dst,
                                  hipStream_t stream);
hipError_t launch_gather_cols_f32(const float* src, int64_t rows, int64_t K, const int32_t* perm, float* dst,
                                  hipStream_t stream);

// W4A8 with fp16 outlier channels (at most 16): workspace = xq | s_x | xo | w_hat of the outliers
size_t w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_act_int8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                           int8_t* xq, float* sx, uint16_t* xo, hipStream_t stream);
hipError_t launch_w4a8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                       const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, void* y,
                       int y_f32, void* workspace, hipStream_t stream);

hipError_t launch_quantize(const float* W, const uint32_t* mask, int64_t N, int64_t K, int64_t group, int bits,
                           uint8_t* codes, uint16_t* scales, uint16_t* zeros, hipStream_t stream);
hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, hipStream_t stream);

// The up-projection of a low-rank branch, added to every output tile before its
// store: t [M, r] fp16 (the down-projection x . L1^T) and L2 [N, r] fp16; r = 0: none.
struct LowRank {
  const uint16_t* t = nullptr;
  const uint16_t* up = nullptr;
  int64_t r = 0;
};

// The down-projection t = fp16(x . L1^T) of a low-rank branch (r a multiple of 32),
// through fp32 partials of K chunks in `part` (lowrank_partial_bytes(M, K, r)).
size_t lowrank_partial_bytes(int64_t M, int64_t K, int64_t r);
hipError_t launch_lowrank_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* L1, int64_t r,
                               float* part, uint16_t* t, hipStream_t stream);

// Weight format of a product: 4-bit codes (eight per word) or 3-bit codes (32 per
// three words, the layout of wq_pack_bits), with one (s, z) per 128 or per 64 input
// channels ([N, K/128] or [N, K/64] metadata).
struct WFormat {
  int bits = 4;
  bool g64 = false;
  bool plain() const { return bits == 4 && !g64; }
};

// mfma_only: never the single-row kernel (the MFMA decode kernels at every M)
hipError_t launch_gemv(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, void* y, int y_f32, const LowRank& lr,
                       hipStream_t stream, WFormat f = WFormat{}, bool mfma_only = false);
// the same for the formats other than 4-bit with 128-channel groups (no low-rank branch)
hipError_t launch_gemv_fmt(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                           const int32_t* col, const uint16_t* val, void* y, int y_f32, WFormat f,
                           hipStream_t stream);
// the single-row decode kernel (whole rows per wave, VALU dot products): for M = 1,
// K a multiple of 2048 up to 32768, 4-bit codes with 128-channel groups, 16-byte
// aligned scales and zeros
bool gemv_dot_supported(int64_t M, int64_t K, const uint16_t* scales, const uint16_t* zeros);
hipError_t launch_gemv_dot(const uint16_t* x, int64_t K, const uint32_t* packed, const uint16_t* scales,
                           const uint16_t* zeros, int64_t N, const int32_t* row_ptr, const int32_t* col,
                           const uint16_t* val, void* y, int y_f32, hipStream_t stream);
// packing of 3-bit codes: [N, K] bytes -> [N, 3K/32] words (K a multiple of 32)
hipError_t launch_pack3(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, hipStream_t stream);
// The GEMM splits K through `workspace` (fp32 partials) when its tile grid alone
// cannot fill the GPU and the workspace holds gemm_workspace_bytes(M, N, K);
// otherwise it runs unsplit.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
// ... of the plan one product takes (4-bit codes, 128-channel groups; a CSR term or
// not); at most gemm_workspace_bytes(M, N, K)
size_t gemm_plan_workspace_bytes(int64_t M, int64_t N, int64_t K, bool sparse);
// the dense GEMM's plan for M x N x K: blocks of its launch (split K included), K
// slices, whether it is gemm_big_kernel, and its tile width (256, or 128 for M <= 64
// where 256-wide tiles would leave compute units without a block)
struct GemmPlanInfo {
  int64_t blocks;
  int ksplit;
  bool big;
  int bn;
};
GemmPlanInfo gemm_plan_info(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, int64_t nnz, void* y, int y_f32, void* workspace,
                       size_t workspace_bytes, const LowRank& lr, hipStream_t stream, WFormat f = WFormat{});

}  // namespace wq
