/*
 * wq.h - C ABI of the MI355X (gfx950) W4A16 group-quantized linear layer.
 *
 * The layer computes y = x . dequant(Wq)^T + W_sparse . x, the dense-and-sparse
 * product of the SqueezeLLM explainer (sections 2.2-2.3: W = W_dense + W_sparse,
 * W x = W_dense x + W_sparse x), where the dense part holds asymmetric INT4
 * round-to-nearest codes with one fp16 scale and zero-point per group of 128
 * input channels (the "W4A16 g128" rows of the DeepCompressor README perplexity
 * table; RTN as the calibration-free baseline in the AWQ paper, section 2), packed
 * eight codes per 32-bit word and dequantized on the fly inside the product (AWQ
 * paper, section 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller. The library
 *    never allocates or frees memory, launches its kernels on `stream` (a
 *    hipStream_t; NULL = the default stream, which must belong to the current
 *    device) and never synchronizes: results are ready when work queued after
 *    them on `stream` runs. Calls that share output or workspace buffers must not
 *    overlap.
 *  - State: none between calls, except (a) each GPU's scratch array of
 *    wq_linear_sparse_noalloc and its device address, looked up under a mutex on
 *    the first such call on that GPU, (b) a per-thread copy of the last HIP
 *    launch error (wq_last_hip_error), and (c) the record, under a mutex, of the
 *    kernels whose dynamic-LDS limit was already raised on each device (setting
 *    it costs tens of microseconds per call). Every entry point other than
 *    wq_linear_sparse_noalloc is reentrant and thread-safe.
 *  - fp16 values travel as uint16_t bit patterns. All arrays are row-major and
 *    contiguous.
 *  - Every argument is validated on the host BEFORE any HIP call; a failed
 *    validation returns a negative wq_status and launches nothing. A failed
 *    kernel launch returns WQ_ERR_HIP; the library has already read (and so
 *    cleared) HIP's own error state, and wq_last_hip_error() returns the cause.
 *  - Preconditions the device does not check: inputs are finite; a group's
 *    range (max - min) is at most 15 * 65504 and every |w| of a sparse entry at
 *    most 65504, so scales and sparse values fit fp16; INT4 codes are <= 15.
 *  - Integer sizes: 1 <= N, 0 <= M, K a positive multiple of 128, N*K < 2^31.
 *    M = 0 (an empty batch) returns WQ_OK without launching anything; x and y
 *    may then be NULL.
 *  - Alignment: W, x, codes and packed must be 16-byte aligned, the output y of a
 *    linear product 4-byte aligned (WQ_ERR_ALIGN).
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_ERR_NULL = -1,        /* a required pointer is NULL                        */
  WQ_ERR_SHAPE = -2,       /* a size is out of range or inconsistent            */
  WQ_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned                  */
  WQ_ERR_UNSUPPORTED = -4, /* group size other than 128, unknown dtype / kernel */
  WQ_ERR_HIP = -5,         /* a kernel launch failed                            */
  WQ_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required        */
  WQ_ERR_SCRATCH = -7      /* needs more than WQ_NOALLOC_SCRATCH_BYTES          */
} wq_status;

/* Bytes of the scratch array wq_linear_sparse_noalloc keeps on each GPU. */
#define WQ_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

typedef enum { WQ_F16 = 0, WQ_F32 = 1 } wq_dtype;

/* Kernel choice for the linear entry points. AUTO uses the decode GEMV for
 * M <= 16, and up to M = 64 also when the GEMM's launch for the shape would have
 * fewer than 128 blocks (a small layer, whose GEMM cannot fill the GPU), the MFMA
 * GEMM otherwise; the others force one kernel at any M. */
typedef enum { WQ_KERNEL_AUTO = 0, WQ_KERNEL_GEMV = 1, WQ_KERNEL_GEMM = 2, WQ_KERNEL_GEMV_MFMA = 3 } wq_kernel;
/* WQ_KERNEL_GEMV picks among the decode kernels by shape: for a single row of a long
 * layer (M = 1, K a multiple of 2048 from 12288 to 32768, 4-bit codes, 128-channel
 * groups, no low-rank branch) the single-row kernel, whole rows per wave on the
 * vector units; else the MFMA decode kernels. WQ_KERNEL_GEMV_MFMA forces the MFMA decode kernels (for
 * measuring one against the other). */

/* Bytes of device workspace wq_quantize_rtn needs (0 when sparse_k == 0).
 * Returns 0 for invalid sizes as well; wq_quantize_rtn reports those. */
size_t wq_quantize_workspace_bytes(int64_t N, int64_t K, int64_t sparse_k);

/*
 * wq_quantize_rtn - offline dense-and-sparse split plus RTN group quantization.
 *
 *  W        [N, K] float32, the weights (output channel n, input channel k).
 *  group    input channels per quantization group: 64, 128, a larger multiple of
 *           128 that divides K, or -1 for one group per row (the default of the
 *           group-size option in the SqueezeLLM explainer, section 5.3, which notes
 *           that smaller groups cost metadata and may gain accuracy);
 *           WQ_ERR_UNSUPPORTED otherwise. The metadata is written in the layout the
 *           linear entry points read: [N, K/64] for group = 64 (products with
 *           group = 64), else one (s, z) per 128 channels, [N, K/128], a coarser
 *           group's (s, z) repeated in each of its 128-channel slots (products with
 *           group = 128).
 *  sparse_k number of entries moved to the sparse fp16 part, 0 <= sparse_k <= N*K.
 *           They are the sparse_k entries of largest |w| (ties: lower flat index
 *           n*K + k first); the SqueezeLLM explainer (section 2.2) keeps such a
 *           small fraction (0.05 % / 0.45 %) of the weights in fp16, chosen there by
 *           a Hessian sensitivity that needs calibration data, here by magnitude.
 *           The dense part is W with those entries set to +0.
 *  codes    [N, K] uint8 out: q = clamp(rint(w / s) + z, 0, 15) for the dense part.
 *  scales   [N, K/128] ([N, K/64] for group = 64) fp16 out:
 *           s = fp16(max(fl32(fl32(max - min) / 15), 2^-14)), max and min over the group.
 *  zeros    the same shape, fp16 out: z = clamp(rint(-min / s), 0, 15), an integer.
 *           (All float32 steps are IEEE, correctly rounded, half-to-even.)
 *  row_ptr  [N+1] int32 out, col [sparse_k] int32 out, val [sparse_k] fp16 out:
 *           the sparse part in CSR, rows = output channels, columns ascending.
 *           Required when sparse_k > 0; when sparse_k == 0 they may be NULL, and a
 *           non-NULL row_ptr is filled with zeros.
 *  workspace device scratch of at least wq_quantize_workspace_bytes(N, K, sparse_k)
 *           bytes (may be NULL when that is 0). Its contents on entry do not matter.
 */
int wq_quantize_rtn(const float* W, int64_t N, int64_t K, int32_t group, int64_t sparse_k,
                    uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                    int32_t* row_ptr, int32_t* col, uint16_t* val,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_quantize_rtn_bits - wq_quantize_rtn with codes of `bits` bits, 2 <= bits <= 4
 * (WQ_ERR_UNSUPPORTED otherwise): qmax = 2^bits - 1 replaces 15 in the formulas
 * above (the SqueezeLLM explainer quantizes to 3 or 4 bits). The codes, at most
 * qmax, are written and packed exactly as 4-bit codes, so every product entry
 * point takes the layer unchanged (the storage and traffic stay those of INT4).
 * wq_quantize_rtn is wq_quantize_rtn_bits with bits = 4.
 */
int wq_quantize_rtn_bits(const float* W, int64_t N, int64_t K, int32_t group, int32_t bits, int64_t sparse_k,
                         uint8_t* codes, uint16_t* scales, uint16_t* zeros, int32_t* row_ptr, int32_t* col,
                         uint16_t* val, void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_pack - 4-bit packing (AWQ paper, section 1): eight consecutive codes along K
 * per 32-bit word, code k = 8t + i in bits [4i, 4i + 4) of word t.
 *  codes  [N, K] uint8 in (only the low 4 bits of each byte are used).
 *  packed [N, K/8] uint32 out.
 */
int wq_pack(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, void* stream);

/*
 * wq_pack_bits - wq_pack for bits = 4, or the 3-bit packing for bits = 3 (the
 * SqueezeLLM explainer's 3-bit models, section 1; packing is what turns a smaller
 * code into fewer bytes, AWQ paper, section 1; no page gives a 3-bit layout, so
 * this one is defined here): every run of 32 consecutive codes (k = 32u .. 32u + 31,
 * K a multiple of 32) takes three words, 3u .. 3u + 2, with no bit unused. Code pair
 * P = 4t + p (t, p = 0..3) is (lo = code 32u + 8t + p, hi = code 32u + 8t + p + 4);
 * pairs 0..14 sit in word 3u + P / 5, lo at bits [3i, 3i + 3) and hi at bits
 * [16 + 3i, 16 + 3i + 3) with i = P % 5; pair 15 puts bit b of code 32u + 27 at
 * bit 15 and bit b of code 32u + 31 at bit 31 of word 3u + b.
 *  codes  [N, K] uint8 in (only the low 3 bits of each byte are used for bits = 3).
 *  packed [N, K/8] (bits = 4) or [N, 3K/32] (bits = 3) uint32 out, 4-byte aligned
 *         for bits = 3. bits other than 3 or 4: WQ_ERR_UNSUPPORTED.
 */
int wq_pack_bits(const uint8_t* codes, int64_t N, int64_t K, int32_t bits, uint32_t* packed, void* stream);

/* Bytes of device workspace with which the linear entry points may split the K
 * dimension of the prefill GEMM across blocks (fp32 partial sums, reduced in a
 * fixed order), for shapes whose output tiles alone cannot fill the GPU, and, for a
 * product with a CSR term, hold the activations transposed ([K, M rounded up to 8]
 * fp16) and, when K is not split, one fp32 partial of y, so that the sparse term
 * joins that fixed-order sum. 0 when neither is planned. A call given less (or
 * NULL) runs unsplit, the sparse term inside the GEMM: same results up to rounding
 * order, slower. */
size_t wq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * wq_linear - y = x . dequant(packed, scales, zeros)^T with on-the-fly
 * dequantization w_hat[n, k] = (q[n, k] - z[n, k/128]) * s[n, k/128].
 *  x       [M, K] fp16 activations.
 *  packed  [N, K/8] uint32 codes as written by wq_pack.
 *  group   128, or 64 for a layer quantized with 64-channel groups.
 *  scales, zeros [N, K/group] fp16 as written by wq_quantize_rtn.
 *  y       [M, N] out, fp16 (y_dtype = WQ_F16, one rounding of the fp32
 *          accumulator) or float32 (WQ_F32). Accumulation is fp32.
 *  workspace: device scratch (16-byte aligned) of wq_linear_workspace_bytes(M, N, K)
 *          bytes, or NULL; contents on entry do not matter. Calls sharing it must
 *          not overlap.
 *  Results are deterministic: no atomics, fixed reduction order.
 */
int wq_linear(const uint16_t* x, int64_t M, int64_t K,
              const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
              int64_t N, int32_t group, void* y, int32_t y_dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_linear_sparse - wq_linear plus the sparse term W_sparse . x (SqueezeLLM
 * explainer, section 2.3), added to the same fp32 accumulators before the one
 * store of y:  y[m, n] += sum over CSR entries e of row n of val[e] * x[m, col[e]].
 *  row_ptr [N+1], col [nnz] int32 and val [nnz] fp16 as written by
 *  wq_quantize_rtn (row_ptr[0] == 0, row_ptr[N] == nnz, columns in [0, K)).
 *  nnz == 0 is valid and equals wq_linear (col / val may then be NULL).
 */
int wq_linear_sparse(const uint16_t* x, int64_t M, int64_t K,
                     const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int32_t group,
                     const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz,
                     void* y, int32_t y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_linear_sparse_bits - wq_linear_sparse_kernel for a layer of 3- or 4-bit codes
 * (bits), packed by wq_pack_bits with the same bits ([N, 3K/32] words for bits = 3,
 * the SqueezeLLM explainer's 3-bit models, section 1), with 64- or 128-channel groups
 * (group, the metadata [N, K/group] of wq_quantize_rtn). A 3-bit layer moves 0.375
 * bytes of codes per weight instead of 0.5. Every format runs in the decode kernels
 * (M <= 16) and in the tile GEMM above; only 4-bit codes with 128-channel groups take
 * the large-M GEMM. row_ptr may be NULL when nnz == 0.
 *  bits other than 3 or 4, or group other than 64 or 128: WQ_ERR_UNSUPPORTED.
 */
int wq_linear_sparse_bits(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed, int32_t bits,
                          const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                          const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz,
                          void* y, int32_t y_dtype, int32_t kernel,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_linear_sparse_kernel - wq_linear_sparse with an explicit kernel choice
 * (wq_kernel), used to measure both kernels on either side of the M crossover.
 * row_ptr may be NULL (then nnz must be 0): this is the dense product.
 */
int wq_linear_sparse_kernel(const uint16_t* x, int64_t M, int64_t K,
                            const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
                            int64_t N, int32_t group,
                            const int32_t* row_ptr, const int32_t* col, const uint16_t* val,
                            int64_t nnz, void* y, int32_t y_dtype, int32_t kernel,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * wq_linear_sparse_noalloc - wq_linear_sparse (kernel chosen by M; row_ptr may be
 * NULL when nnz == 0, the dense product) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace and allocates nothing: the fp32 partial sums
 * and transposed activations of the GEMM go to a scratch array of
 * WQ_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory from the
 * first such call on that GPU (the current device) until the process ends.
 *  - A product whose GEMM plan would need more (its split-K partial sums; with a
 *    CSR term also the transposed activations and, when K is not split, one fp32
 *    partial of y; at most wq_linear_workspace_bytes(M, N, K)) returns
 *    WQ_ERR_SCRATCH and launches nothing.
 *  - Every call on one GPU uses the same scratch: calls that can run at the same
 *    time on one GPU (other streams, other host threads) race and give wrong
 *    results. Queue them on one stream, or use wq_linear_sparse with separate
 *    workspaces. Nothing in the scratch needs to start at zero: each call writes
 *    what it later reads.
 *  - Results are identical to wq_linear_sparse given a full workspace.
 */
int wq_linear_sparse_noalloc(const uint16_t* x, int64_t M, int64_t K,
                             const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
                             int64_t N, int32_t group,
                             const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz,
                             void* y, int32_t y_dtype, void* stream);

/* Bytes of device workspace wq_linear_lowrank needs: t = x . L1^T [M, r] fp16,
 * for M > 16 the fp32 partials of the K chunks it is summed over, and the split-K
 * workspace of wq_linear_workspace_bytes(M, N, K). 0 for invalid sizes (r must be
 * a multiple of 32 up to 256). */
size_t wq_linear_lowrank_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r);

/*
 * wq_linear_lowrank - wq_linear_sparse_kernel plus a rank-r high-precision branch
 * (SVDQuant section of the DeepCompressor README: a low-rank branch holds the
 * weights' outliers while the residual is quantized, fused with the low-bit
 * kernel rather than run as a separate pass):
 *   y = x . dequant(packed)^T + W_sparse . x + (x . L1^T) . L2^T,
 * i.e. W = L2 . L1 + residual.
 *  L1  [r, K] fp16, the down-projection (one row per component), 16-byte aligned.
 *  L2  [N, r] fp16, the up-projection, 16-byte aligned.
 *  r   a multiple of 32 up to 256 (WQ_ERR_UNSUPPORTED otherwise; < 1: WQ_ERR_SHAPE).
 *  row_ptr / col / val / nnz as in wq_linear_sparse; row_ptr may be NULL when
 *  nnz == 0 (no sparse term). kernel as in wq_linear_sparse_kernel.
 *  workspace: required, wq_linear_lowrank_workspace_bytes(M, N, K, r) bytes,
 *  16-byte aligned (WQ_ERR_WORKSPACE otherwise); contents on entry do not matter.
 * t = x . L1^T is accumulated in fp32 and rounded once to fp16 (it is an MFMA
 * operand); each output tile then adds t . L2^T to its fp32 accumulators before
 * the one store of y. Deterministic, like the other linear entry points.
 */
int wq_linear_lowrank(const uint16_t* x, int64_t M, int64_t K,
                      const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros,
                      int64_t N, int32_t group,
                      const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz,
                      const uint16_t* L1, const uint16_t* L2, int64_t r,
                      void* y, int32_t y_dtype, int32_t kernel,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Act-order layers (the GPTQ-R rows, GPTQ with reordering, of the DeepCompressor
 * README perplexity table): the input channels are quantized in a permuted order,
 * so a group is a scattered set of original channels (a per-channel group index
 * g_idx[perm[i]] = i / group). Such a layer is kept in the permuted order: channel
 * i of its codes, scales, zeros and CSR columns is input channel perm[i].
 *  perm  [K] int32, 16-byte aligned, a permutation of 0..K-1. Not checked: an
 *        index outside [0, K) is clamped (wrong values, never an invalid read).
 */

/* Bytes of device workspace wq_quantize_rtn_act_order needs: W with its columns
 * permuted (N*K float32, rounded up to 256 bytes) plus wq_quantize_workspace_bytes.
 * 0 for invalid sizes. */
size_t wq_quantize_act_order_workspace_bytes(int64_t N, int64_t K, int64_t sparse_k);

/*
 * wq_quantize_rtn_act_order - wq_quantize_rtn of W[:, perm] (column i of the copy is
 * column perm[i] of W): the same split, groups, codes, metadata and CSR, all in the
 * permuted channel order (CSR columns are positions in that order; ties of |w| go
 * to the lower flat index in that order). group = 64 is WQ_ERR_UNSUPPORTED here (the
 * act-order product reads 128-channel metadata).
 *  workspace  required, 256-byte aligned, wq_quantize_act_order_workspace_bytes.
 */
int wq_quantize_rtn_act_order(const float* W, int64_t N, int64_t K, int32_t group, const int32_t* perm,
                              int64_t sparse_k, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                              int32_t* row_ptr, int32_t* col, uint16_t* val, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of device workspace wq_linear_act_order needs: x with its columns permuted
 * (M*K fp16, rounded up to 256 bytes) plus wq_linear_workspace_bytes(M, N, K). */
size_t wq_linear_act_order_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * wq_linear_act_order - wq_linear_sparse_kernel for a layer in permuted channel
 * order: y = x[:, perm] . dequant(packed)^T + W_sparse' x[:, perm], which equals
 * x . W^T for W in the original order. x is in the original channel order; its
 * columns are gathered through perm into the workspace, then the product runs as
 * in wq_linear_sparse_kernel (row_ptr may be NULL when nnz == 0).
 *  workspace  required for M >= 1, 256-byte aligned, wq_linear_act_order_workspace_bytes.
 */
int wq_linear_act_order(const uint16_t* x, int64_t M, int64_t K, const int32_t* perm, const uint32_t* packed,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                        const int32_t* row_ptr, const int32_t* col, const uint16_t* val, int64_t nnz, void* y,
                        int32_t y_dtype, int32_t kernel, void* workspace, size_t workspace_bytes, void* stream);

/*
 * W4A8 with fp16 outlier channels (the MixQ news item: most activation channels
 * in 8 bits on integer matrix units, a few fixed outlier channels in high
 * precision, the two products added in registers). The weights are the INT4 g128
 * layer of the other entry points. Per row m of x, over the channels that are not
 * outliers:  s_x[m] = fl32(amax / 127) (1 when amax is 0),
 *            xq[m, k] = clamp(rint(fl32(x[m, k] / s_x[m])), -127, 127),
 * and  y[m, n] = s_x[m] * sum_k xq[m, k] * w_hat[n, k] + sum_j x[m, o_j] * w_hat[n, o_j],
 * with w_hat = (q - z) * s. INT8 sums are exact (int32) per group of 128 channels;
 * the rest is fp32 (the outlier weights w_hat are rounded once to fp16, an MFMA
 * operand).
 *  outliers  [n_out] int32 channel indices, distinct, in [0, K) (not checked: an
 *            index out of range is clamped), 0 <= n_out <= 16 (WQ_ERR_UNSUPPORTED
 *            otherwise); may be NULL when n_out == 0.
 */

/*
 * wq_quantize_act_int8 - the activation step alone.
 *  xq  [M, K] int8 out, 16-byte aligned, in the order the products read it: in
 *      each 16 consecutive channels c0..c15 the bytes hold c0, c2, c4, c6, c1, c3,
 *      c5, c7, c8, c10, c12, c14, c9, c11, c13, c15; 0 on outlier channels.
 *  sx  [M] float32 out.   xo  [M, 16] fp16 out, 16-byte aligned: x[m, o_j] for
 *      j < n_out, then zeros.
 */
int wq_quantize_act_int8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                         int8_t* xq, float* sx, uint16_t* xo, void* stream);

/* Bytes of device workspace wq_linear_w4a8 needs (xq, s_x, the outlier
 * activations and the outlier weights). 0 for invalid sizes. */
size_t wq_linear_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * wq_linear_w4a8 - y as above. x [M, K] fp16, packed/scales/zeros as in wq_linear
 * (group must be 128), y [M, N] fp16 or float32 (y_dtype).
 *  workspace  required for M >= 1, 256-byte aligned, wq_linear_w4a8_workspace_bytes.
 * Three launches: the activation step, the outlier weights, the INT8 MFMA product.
 */
int wq_linear_w4a8(const uint16_t* x, int64_t M, int64_t K, const int32_t* outliers, int64_t n_out,
                   const uint32_t* packed, const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group,
                   void* y, int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* The kernel WQ_KERNEL_AUTO picks for an M x N x K product (WQ_KERNEL_GEMV or
 * WQ_KERNEL_GEMM; see wq_kernel). */
int wq_auto_kernel(int64_t M, int64_t N, int64_t K);

/* A static, NUL-terminated description of a wq_status value. */
const char* wq_status_string(int status);

/* The hipError_t (as int) of the calling thread's last launch that returned
 * WQ_ERR_HIP, or 0 (hipSuccess) if there was none. */
int wq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
