// C ABI of the W4A16 group-quantized linear (declared in include/wq.h).
//
// Every entry point validates all of its arguments on the host before it makes
// any HIP call, so a bad call returns a negative status and launches nothing
// (and the validation is testable on a machine without a GPU).
#include "../../include/wq.h"
#include "wq_launch.h"

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

// Scratch of wq_linear_sparse_noalloc, in each GPU's memory for the life of the
// process: the split-K partial sums and the transposed activations of the GEMM.
// In host code this name only stands in for the symbol: kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[WQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kGroup = 128;
constexpr int64_t kMax32 = (int64_t)1 << 31;  // element counts must stay below 2^31
constexpr int64_t kMaxRank = 256;             // rank of the low-rank branch: multiples of 32 up to this
constexpr int64_t kMaxOutliers = 16;          // fp16 outlier channels of the W4A8 product

// t [M][r] fp16 of the low-rank branch, at the start of its workspace
size_t lowrank_t_bytes(int64_t M, int64_t r) { return ((size_t)M * r * 2 + 255) / 256 * 256; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// The HIP error of this thread's last failed launch (hipSuccess if none): a
// launcher reads and clears HIP's own error state, so the cause is kept here for
// wq_last_hip_error().
thread_local hipError_t last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return WQ_OK;
  last_hip_error = e;
  return WQ_ERR_HIP;
}

// Device address of `scratch` on each GPU, looked up once per device (with that
// device current) on its first no-allocation call.
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_address[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_address[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_address[dev] = p;
  }
  *out = scratch_address[dev];
  return hipSuccess;
}

// group: the (s, z) slot width the products read, 128 (every product) or 64 (the
// entry points that take 64-channel groups pass allow_g64)
int check_linear_args(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, const uint16_t* scales,
                      const uint16_t* zeros, int64_t N, int32_t group, const int32_t* row_ptr,
                      const int32_t* col, const uint16_t* val, int64_t nnz, void* y, int32_t y_dtype,
                      int32_t kernel, bool allow_g64 = false) {
  // M = 0 (an empty batch) is valid and computes nothing; x and y may then be NULL
  if (!packed || !scales || !zeros) return WQ_ERR_NULL;
  if (M != 0 && (!x || !y)) return WQ_ERR_NULL;
  if (row_ptr == nullptr && nnz != 0) return WQ_ERR_NULL;
  if (nnz > 0 && (!col || !val)) return WQ_ERR_NULL;
  if (group != kGroup && !(allow_g64 && group == 64)) return WQ_ERR_UNSUPPORTED;
  if (y_dtype != WQ_F16 && y_dtype != WQ_F32) return WQ_ERR_UNSUPPORTED;
  if (kernel != WQ_KERNEL_AUTO && kernel != WQ_KERNEL_GEMV && kernel != WQ_KERNEL_GEMM &&
      kernel != WQ_KERNEL_GEMV_MFMA)
    return WQ_ERR_UNSUPPORTED;
  if (M < 0 || N < 1 || K < kGroup || K % kGroup != 0) return WQ_ERR_SHAPE;
  if (nnz < 0 || nnz >= kMax32) return WQ_ERR_SHAPE;
  if (N >= kMax32 / K || M >= kMax32 / K || M >= kMax32 / N) return WQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(y, 4))
    return WQ_ERR_ALIGN;
  if ((row_ptr && !aligned(row_ptr, 4)) || (col && !aligned(col, 4)) || (val && !aligned(val, 2)))
    return WQ_ERR_ALIGN;
  return WQ_OK;
}

int check_quantize_args(const float* W, int64_t N, int64_t K, int32_t group, int64_t sparse_k, uint8_t* codes,
                        uint16_t* scales, uint16_t* zeros, int32_t* row_ptr, int32_t* col, uint16_t* val,
                        void* workspace, size_t workspace_bytes) {
  if (!W || !codes || !scales || !zeros) return WQ_ERR_NULL;
  if (sparse_k > 0 && (!row_ptr || !col || !val)) return WQ_ERR_NULL;
  if (N < 1 || K < kGroup || K % kGroup != 0 || N >= kMax32 / K) return WQ_ERR_SHAPE;
  // quantization group: 64, a multiple of 128 that divides K, or -1 for one group per row
  const int64_t g = group == -1 ? K : group;
  if (g != 64 && (g < kGroup || g % kGroup != 0 || K % g != 0)) return WQ_ERR_UNSUPPORTED;
  if (sparse_k < 0 || sparse_k > N * K) return WQ_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2)) return WQ_ERR_ALIGN;
  if ((row_ptr && !aligned(row_ptr, 4)) || (col && !aligned(col, 4)) || (val && !aligned(val, 2)))
    return WQ_ERR_ALIGN;
  if (sparse_k > 0) {
    const size_t need = wq::split_workspace_bytes(N, K);
    if (!workspace || workspace_bytes < need) return WQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return WQ_ERR_ALIGN;
  }
  return WQ_OK;
}

// the permuted copy of W or x at the start of an act-order workspace
size_t act_order_copy_bytes(int64_t rows, int64_t K, size_t elem) { return ((size_t)rows * K * elem + 255) / 256 * 256; }

// (kernel, device) -> the dynamic-LDS limit already set there
std::mutex lds_mutex;
std::map<std::pair<const void*, int>, size_t> lds_limit;

}  // namespace

hipError_t wq::set_dynamic_lds(const void* kern, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(lds_mutex);
  const auto key = std::make_pair(kern, dev);
  const auto it = lds_limit.find(key);
  if (it != lds_limit.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) lds_limit[key] = bytes;
  return e;
}

extern "C" {

int wq_last_hip_error(void) { return (int)last_hip_error; }

const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "a required pointer is NULL";
    case WQ_ERR_SHAPE: return "a size is out of range or inconsistent";
    case WQ_ERR_ALIGN: return "a pointer is not sufficiently aligned";
    case WQ_ERR_UNSUPPORTED: return "unsupported group size, dtype or kernel choice";
    case WQ_ERR_HIP: return "a HIP kernel launch failed";
    case WQ_ERR_WORKSPACE: return "workspace missing or too small";
    case WQ_ERR_SCRATCH: return "the product needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

size_t wq_quantize_workspace_bytes(int64_t N, int64_t K, int64_t sparse_k) {
  if (N < 1 || K < kGroup || K % kGroup != 0 || N >= kMax32 / K) return 0;
  if (sparse_k <= 0) return 0;
  return wq::split_workspace_bytes(N, K);
}

int wq_quantize_rtn_bits(const float* W, int64_t N, int64_t K, int32_t group, int32_t bits, int64_t sparse_k,
                         uint8_t* codes, uint16_t* scales, uint16_t* zeros, int32_t* row_ptr, int32_t* col,
                         uint16_t* val, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_quantize_args(W, N, K, group, sparse_k, codes, scales, zeros, row_ptr, col, val, workspace,
                                     workspace_bytes);
  if (rc != WQ_OK) return rc;
  if (bits < 2 || bits > 4) return WQ_ERR_UNSUPPORTED;
  const int64_t g = group == -1 ? K : group;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  if (sparse_k > 0) {
    const wq::SplitWorkspace ws = wq::split_workspace_carve(workspace, N, K);
    e = wq::launch_split(W, N, K, sparse_k, row_ptr, col, val, ws, s);
    if (e == hipSuccess) e = wq::launch_quantize(W, ws.mask, N, K, g, bits, codes, scales, zeros, s);
  } else {
    if (row_ptr) e = wq::launch_fill_zero_i32(row_ptr, N + 1, s);
    if (e == hipSuccess) e = wq::launch_quantize(W, nullptr, N, K, g, bits, codes, scales, zeros, s);
  }
  return hip_status(e);
}

int wq_quantize_rtn(const float* W, int64_t N, int64_t K, int32_t group, int64_t sparse_k, uint8_t* codes,
                    uint16_t* scales, uint16_t* zeros, int32_t* row_ptr, int32_t* col, uint16_t* val,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return wq_quantize_rtn_bits(W, N, K, group, 4, sparse_k, codes, scales, zeros, row_ptr, col, val, workspace,
                              workspace_bytes, stream);
}

int wq_pack(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, void* stream) {
  return wq_pack_bits(codes, N, K, 4, packed, stream);
}

int wq_pack_bits(const uint8_t* codes, int64_t N, int64_t K, int32_t bits, uint32_t* packed, void* stream) {
  if (!codes || !packed) return WQ_ERR_NULL;
  if (bits != 3 && bits != 4) return WQ_ERR_UNSUPPORTED;
  const int64_t unit = bits == 4 ? 8 : 32;
  if (N < 1 || K < unit || K % unit != 0 || N >= kMax32 / K) return WQ_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(packed, bits == 4 ? 16 : 4)) return WQ_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  return hip_status(bits == 4 ? wq::launch_pack(codes, N, K, packed, s) : wq::launch_pack3(codes, N, K, packed, s));
}

size_t wq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) return 0;
  if (N >= kMax32 / K || M >= kMax32 / K || M >= kMax32 / N) return 0;
  return wq::gemm_workspace_bytes(M, N, K);
}

// The decode kernels re-read the weights once per 16 rows (their time steps up at
// M = 17, 33 and 49), the GEMM reads them once but needs a grid that fills the GPU.
// Measured (decode kernel / GEMM, us, both forced):
//  - 8192 x 28672 (64 x 256 tiles, a block on every CU): the GEMM from M = 20
//    (77.3 / 64.1; at M = 16 49.7 / 63.4);
//  - 4096 x 4096 with its CSR and 11008 x 4096 (64 x 128 tiles, four K slices):
//    the decode kernel to M = 32 (15.6 / 19.4, 18.9 / 22.1), the GEMM from M = 40
//    (20.3 / 19.9, 27.9 / 22.6);
//  - 8192 x 3584 (28 groups, two K slices): the decode kernel to M = 48
//    (22.3 / 23.6), the GEMM at M = 64 (27.8 / 24.6).
// Shapes that take the tile GEMM (a group count that is not a multiple of four)
// keep the rule measured before these tiles: the decode kernel while the GEMM's
// grid has fewer than 128 blocks.
int wq_auto_kernel(int64_t M, int64_t N, int64_t K) {
  if (M <= 16) return WQ_KERNEL_GEMV;
  if (M > 64 || N < 1 || K < kGroup || K % kGroup != 0) return WQ_KERNEL_GEMM;
  const wq::GemmPlanInfo p = wq::gemm_plan_info(M, N, K);
  if (!p.big) return p.blocks < 128 ? WQ_KERNEL_GEMV : WQ_KERNEL_GEMM;
  if (p.bn == 256) return WQ_KERNEL_GEMM;
  if (M <= 32) return WQ_KERNEL_GEMV;
  if (M <= 48 && p.ksplit < 4) return WQ_KERNEL_GEMV;
  return WQ_KERNEL_GEMM;
}

int wq_linear_sparse_bits(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, int32_t bits,
                          const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                          const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz, void* y,
                          int32_t y_dtype, int32_t kernel, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_linear_args(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                   kernel, true);
  if (rc != WQ_OK) return rc;
  if (bits != 3 && bits != 4) return WQ_ERR_UNSUPPORTED;
  if (bits == 3 && !aligned(packed, 4)) return WQ_ERR_ALIGN;
  if (M == 0) return WQ_OK;
  if (kernel == WQ_KERNEL_AUTO) kernel = wq_auto_kernel(M, N, K);
  const int y_f32 = y_dtype == WQ_F32;
  const int32_t* rp = nnz > 0 ? row_ptr : nullptr;  // nnz == 0: the dense product
  wq::WFormat f;
  f.bits = bits;
  f.g64 = group == 64;
  hipError_t e;
  if (kernel == WQ_KERNEL_GEMV || kernel == WQ_KERNEL_GEMV_MFMA)
    e = wq::launch_gemv(x, M, K, packed, scales, zeros, N, rp, col, val, y, y_f32, wq::LowRank{},
                        as_stream(stream), f, kernel == WQ_KERNEL_GEMV_MFMA);
  else
    e = wq::launch_gemm(x, M, K, packed, scales, zeros, N, rp, col, val, nnz, y, y_f32,
                        workspace != nullptr && aligned(workspace, 16) ? workspace : nullptr, workspace_bytes,
                        wq::LowRank{}, as_stream(stream), f);
  return hip_status(e);
}

int wq_linear_sparse_kernel(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                            const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                            const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz,
                            void* y, int32_t y_dtype, int32_t kernel, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return wq_linear_sparse_bits(x, M, K, packed, 4, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                               kernel, workspace, workspace_bytes, stream);
}

size_t wq_linear_lowrank_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) return 0;
  if (N >= kMax32 / K || M >= kMax32 / K || M >= kMax32 / N) return 0;
  if (r < 32 || r % 32 != 0 || r > kMaxRank) return 0;
  return lowrank_t_bytes(M, r) + wq::lowrank_partial_bytes(M, K, r) + wq::gemm_workspace_bytes(M, N, K);
}

int wq_linear_lowrank(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, const uint16_t* scales,
                      const uint16_t* zeros, int64_t N, int32_t group, const int32_t* row_ptr, const int32_t* col,
                      const uint16_t* val, int64_t nnz, const uint16_t* L1, const uint16_t* L2, int64_t r, void* y,
                      int32_t y_dtype, int32_t kernel, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_linear_args(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                   kernel);
  if (rc != WQ_OK) return rc;
  if (!L1 || !L2) return WQ_ERR_NULL;
  if (r < 1) return WQ_ERR_SHAPE;
  if (r % 32 != 0 || r > kMaxRank) return WQ_ERR_UNSUPPORTED;
  if (!aligned(L1, 16) || !aligned(L2, 16)) return WQ_ERR_ALIGN;
  if (M == 0) return WQ_OK;
  const size_t need = wq_linear_lowrank_workspace_bytes(M, N, K, r);
  if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need) return WQ_ERR_WORKSPACE;
  // workspace: t | down-projection partials | the GEMM's split-K workspace
  char* ws = static_cast<char*>(workspace);
  uint16_t* t = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + lowrank_t_bytes(M, r));
  char* gws = ws + lowrank_t_bytes(M, r) + wq::lowrank_partial_bytes(M, K, r);
  const size_t gws_bytes = workspace_bytes - (size_t)(gws - ws);
  if (kernel == WQ_KERNEL_AUTO) kernel = wq_auto_kernel(M, N, K);
  const int y_f32 = y_dtype == WQ_F32;
  const int32_t* rp = nnz > 0 ? row_ptr : nullptr;  // nnz == 0: no sparse term
  const wq::LowRank lr{t, L2, r};
  hipError_t e = wq::launch_lowrank_down(x, M, K, L1, r, part, t, as_stream(stream));
  if (e != hipSuccess) return hip_status(e);
  if (kernel == WQ_KERNEL_GEMV || kernel == WQ_KERNEL_GEMV_MFMA)
    e = wq::launch_gemv(x, M, K, packed, scales, zeros, N, rp, col, val, y, y_f32, lr, as_stream(stream));
  else
    e = wq::launch_gemm(x, M, K, packed, scales, zeros, N, rp, col, val, nnz, y, y_f32, gws, gws_bytes, lr,
                        as_stream(stream));
  return hip_status(e);
}

int wq_linear_sparse(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, const uint16_t* scales,
                     const uint16_t* zeros, int64_t N, int32_t group, const int32_t* row_ptr, const int32_t* col,
                     const uint16_t* val, int64_t nnz, void* y, int32_t y_dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!row_ptr) return WQ_ERR_NULL;
  return wq_linear_sparse_kernel(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                 WQ_KERNEL_AUTO, workspace, workspace_bytes, stream);
}

int wq_linear_sparse_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                             const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz, void* y,
                             int32_t y_dtype, void* stream) {
  const int rc = check_linear_args(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                   WQ_KERNEL_AUTO);
  if (rc != WQ_OK) return rc;
  if (M == 0) return WQ_OK;
  const int kernel = wq_auto_kernel(M, N, K);
  const size_t need = kernel == WQ_KERNEL_GEMM ? wq::gemm_plan_workspace_bytes(M, N, K, nnz > 0) : 0;
  if (need > WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERR_SCRATCH;
  const int y_f32 = y_dtype == WQ_F32;
  const int32_t* rp = nnz > 0 ? row_ptr : nullptr;
  hipError_t e;
  if (kernel == WQ_KERNEL_GEMV) {
    e = wq::launch_gemv(x, M, K, packed, scales, zeros, N, rp, col, val, y, y_f32, wq::LowRank{},
                        as_stream(stream));
  } else {
    void* ws = nullptr;
    e = scratch_of_current_device(&ws);
    if (e == hipSuccess)
      e = wq::launch_gemm(x, M, K, packed, scales, zeros, N, rp, col, val, nnz, y, y_f32, ws, need, wq::LowRank{},
                          as_stream(stream));
  }
  return hip_status(e);
}

int wq_linear(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, const uint16_t* scales,
              const uint16_t* zeros, int64_t N, int32_t group, void* y, int32_t y_dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  return wq_linear_sparse_kernel(x, M, K, packed, scales, zeros, N, group, nullptr, nullptr, nullptr, 0, y,
                                 y_dtype, WQ_KERNEL_AUTO, workspace, workspace_bytes, stream);
}

size_t wq_quantize_act_order_workspace_bytes(int64_t N, int64_t K, int64_t sparse_k) {
  if (N < 1 || K < kGroup || K % kGroup != 0 || N >= kMax32 / K) return 0;
  return act_order_copy_bytes(N, K, 4) + wq_quantize_workspace_bytes(N, K, sparse_k);
}

int wq_quantize_rtn_act_order(const float* W, int64_t N, int64_t K, int32_t group, const int32_t* perm,
                              int64_t sparse_k, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                              int32_t* row_ptr, int32_t* col, uint16_t* val, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!perm) return WQ_ERR_NULL;
  if (group == 64) return WQ_ERR_UNSUPPORTED;  // the act-order product reads 128-channel metadata
  // W's own checks stand in for those of the permuted copy, which lives in the workspace
  const size_t copy = act_order_copy_bytes(N, K, 4);
  char* ws = static_cast<char*>(workspace);
  const size_t inner_bytes = workspace_bytes > copy ? workspace_bytes - copy : 0;
  int rc = check_quantize_args(W, N, K, group, sparse_k, codes, scales, zeros, row_ptr, col, val,
                               ws ? ws + copy : nullptr, inner_bytes);
  if (rc != WQ_OK) return rc;
  if (!aligned(perm, 16)) return WQ_ERR_ALIGN;
  if (!ws || workspace_bytes < wq_quantize_act_order_workspace_bytes(N, K, sparse_k)) return WQ_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return WQ_ERR_ALIGN;
  float* Wp = reinterpret_cast<float*>(ws);
  const hipError_t e = wq::launch_gather_cols_f32(W, N, K, perm, Wp, as_stream(stream));
  if (e != hipSuccess) return hip_status(e);
  return wq_quantize_rtn(Wp, N, K, group, sparse_k, codes, scales, zeros, row_ptr, col, val,
                         sparse_k > 0 ? ws + copy : nullptr, inner_bytes, stream);
}

int wq_quantize_act_int8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                         int8_t* xq, float* sx, uint16_t* xo, void* stream) {
  if (n_out > 0 && !outliers) return WQ_ERR_NULL;
  if (M != 0 && (!x || !xq || !sx || !xo)) return WQ_ERR_NULL;
  if (n_out < 0 || n_out > kMaxOutliers) return WQ_ERR_UNSUPPORTED;
  if (M < 0 || K < kGroup || K % kGroup != 0 || M >= kMax32 / K) return WQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(sx, 4) || !aligned(xo, 16) || !aligned(outliers, 4))
    return WQ_ERR_ALIGN;
  if (M == 0) return WQ_OK;
  return hip_status(wq::launch_act_int8(x, M, K, outliers, n_out, xq, sx, xo, as_stream(stream)));
}

size_t wq_linear_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) return 0;
  if (N >= kMax32 / K || M >= kMax32 / K || M >= kMax32 / N) return 0;
  return wq::w4a8_workspace_bytes(M, N, K);
}

int wq_linear_w4a8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                   const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                   void* y, int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_out > 0 && !outliers) return WQ_ERR_NULL;
  const int rc = check_linear_args(x, M, K, packed, scales, zeros, N, group, nullptr, nullptr, nullptr, 0, y,
                                   y_dtype, WQ_KERNEL_AUTO);
  if (rc != WQ_OK) return rc;
  if (n_out < 0 || n_out > kMaxOutliers) return WQ_ERR_UNSUPPORTED;
  if (!aligned(outliers, 4)) return WQ_ERR_ALIGN;
  if (M == 0) return WQ_OK;
  if (!workspace || workspace_bytes < wq_linear_w4a8_workspace_bytes(M, N, K)) return WQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_w4a8(x, M, K, outliers, n_out, packed, scales, zeros, N, y, y_dtype == WQ_F32,
                                   workspace, as_stream(stream)));
}

size_t wq_linear_act_order_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < kGroup || K % kGroup != 0) return 0;
  if (N >= kMax32 / K || M >= kMax32 / K || M >= kMax32 / N) return 0;
  return act_order_copy_bytes(M, K, 2) + wq::gemm_workspace_bytes(M, N, K);
}

int wq_linear_act_order(const uint16_t* x, int64_t M, int64_t K, const int32_t* perm, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                        const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz, void* y,
                        int32_t y_dtype, int32_t kernel, void* workspace, size_t workspace_bytes, void* stream) {
  if (!perm) return WQ_ERR_NULL;
  const int rc = check_linear_args(x, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                   kernel);
  if (rc != WQ_OK) return rc;
  if (!aligned(perm, 16)) return WQ_ERR_ALIGN;
  if (M == 0) return WQ_OK;
  if (!workspace || workspace_bytes < wq_linear_act_order_workspace_bytes(M, N, K)) return WQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return WQ_ERR_ALIGN;
  // workspace: x with its columns in the layer's order | the GEMM's split-K workspace
  char* ws = static_cast<char*>(workspace);
  const size_t copy = act_order_copy_bytes(M, K, 2);
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  const hipError_t e = wq::launch_gather_cols_f16(x, M, K, perm, xp, as_stream(stream));
  if (e != hipSuccess) return hip_status(e);
  return wq_linear_sparse_kernel(xp, M, K, packed, scales, zeros, N, group, row_ptr, col, val, nnz, y, y_dtype,
                                 kernel, ws + copy, workspace_bytes - copy, stream);
}

}  // extern "C"
