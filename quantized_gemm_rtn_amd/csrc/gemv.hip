// Launchers of the decode kernels (gemv_kernels.h) for 4-bit layers with one
// (s, z) per 128 input channels; gemv_fmt.hip has those of the other weight formats.
#include "gemv_kernels.h"

namespace wq {

constexpr int64_t kDotMinK = 12288;  // the single-row kernel from this K on (see launch_gemv)

template <int XC, int SZV, int MR, bool SP>
static hipError_t launch_lds(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                             const int32_t* col, const uint16_t* val, void* y, int y_f32, const LowRank& lr,
                             hipStream_t stream) {
  const int64_t G = K / kGroup, mrows = M < 16 ? M : 16, SR = MR == 1 ? 1 : 4 * ((mrows + 3) / 4);
  const size_t lds = (SZV == kSzInRegs ? 0 : (size_t)16 * (G + 1) * 4) + (size_t)mrows * K * 2 +
                     (size_t)2 * G * SR * 4;
  return launch_rows(gemv_lds_kernel<kGemvWaves, kGemvDepth, XC, SZV, MR, SP>, lds, 16, x, M, K, packed, scales, zeros, N,
                     row_ptr, col, val, y, y_f32, lr, stream);
}

template <int XL, int NT, int SZV, bool SP>
static hipError_t launch_ring(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                              const int32_t* col, const uint16_t* val, void* y, int y_f32, const LowRank& lr,
                              hipStream_t stream) {
  const size_t lds = (SZV == kSzInRegs ? 0 : (size_t)NT * 16 * (K / kGroup + 1) * 4) +
                     (size_t)kGemvWaves * 4 * XL * 136 * 2;
  return launch_rows(gemv_ring_kernel<kGemvWaves, kGemvRingDepth, XL, NT, SZV, SP>, lds, 16 * NT, x, M, K, packed,
                     scales, zeros, N, row_ptr, col, val, y, y_f32, lr, stream);
}

hipError_t launch_gemv(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                       const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                       const int32_t* col, const uint16_t* val, void* y, int y_f32, const LowRank& lr,
                       hipStream_t stream, WFormat f, bool mfma_only) {
  if (!f.plain()) return launch_gemv_fmt(x, M, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32, f, stream);
  // one activation row of a long layer: whole rows per wave and VALU dot products
  // (gemv_dot.hip). Measured at M = 1 (single-row against MFMA kernel, us): K = 4096
  // 7.0 / 6.7, 8192 11.1 / 9.8, 14336 14.7 / 15.3, 28672 26.6 / 30.0.
  if (!mfma_only && lr.r == 0 && K >= kDotMinK && gemv_dot_supported(M, K, scales, zeros))
    return launch_gemv_dot(x, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32, stream);
  const int64_t G = K / kGroup;
  // a CSR is passed only with nnz >= 1: its kernels may read entry 0 of an empty row
  const bool sp = row_ptr != nullptr;
  const int64_t mrows_max = M < 16 ? M : 16;
  // scales/zeros rows as vectors of 8, 4 or 2 halves when G is a multiple of the
  // width and every row starts aligned to it
  const auto aligned = [&](uintptr_t b) {
    return reinterpret_cast<uintptr_t>(scales) % b == 0 && reinterpret_cast<uintptr_t>(zeros) % b == 0;
  };
  const int sv = G % 8 == 0 && G <= kSzMaxG<8> && aligned(16)  ? 8
                 : G % 4 == 0 && G <= kSzMaxG<4> && aligned(8) ? 4
                 : G % 2 == 0 && G <= kSzMaxG<2> && aligned(4) ? 2
                 : G <= kSzMaxG<1>                             ? 1
                                                               : 0;
  const bool vec = sv == 8;
  // scales and zero-points in registers, two loads per window of D groups, when each
  // wave has exactly one window (4096 input channels): there they skip the block's
  // LDS staging (headline layer 6.43 against 6.85 us). With more windows each one
  // reloads them inside the weight stream, and staging the block's (s, z) once with
  // the activations is faster for one row (70B down-projection with the MFMA kernel
  // 28.6 against 30.5 us, with a rank-32 branch 31.8 against 33.6; K = 8192 11.3
  // against 11.6) and for two rows at K = 8192 (13.5 against 14.1 us), but not for two
  // rows from K = 12288 on (22.8 against 22.2 us, K = 16384 28.6 against 28.0).
  static_assert(kGemvDepth == 4 || kGemvDepth == 8, "in-register (s, z) windows hold 4 or 8 groups");
  const bool in_regs = vec && G % (kGemvDepth * kGemvWaves) == 0 &&
                       (G == kGemvDepth * kGemvWaves || (mrows_max == 2 && G >= 96));
  const int sz_mode = in_regs ? kSzInRegs : sv;
  // output rows a lane can hold: rows 4h .. 4h+3 of the tile, so M = 1, 2 need fewer
  const int mr = mrows_max == 1 ? 1 : (mrows_max == 2 ? 2 : 4);
  // activations fit in LDS next to the scales: stage them once per block, with the
  // fewest staging registers that cover them
  const int64_t xloads = (mrows_max * K / 8 + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
  // (from M = 3 on, staging per wave and group is faster, even where x would fit)
  const int xc = mrows_max * K > kXLdsMaxHalves || mrows_max > 2 ? 0
                 : xloads <= 1 ? 1 : xloads <= 2 ? 2 : xloads <= 4 ? 4 : xloads <= 8 ? 8 : 16;
#define WQ_ARGS x, M, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32, lr, stream
#define WQ_LDS(XC, SV, MR)                                 \
  if (xc == XC && sz_mode == SV && mr == MR) {             \
    if (sp) return launch_lds<XC, SV, MR, true>(WQ_ARGS);  \
    return launch_lds<XC, SV, MR, false>(WQ_ARGS);         \
  }
#define WQ_LDS_MR(XC, SV) WQ_LDS(XC, SV, 1); WQ_LDS(XC, SV, 2)
  WQ_LDS_MR(1, kSzInRegs); WQ_LDS_MR(2, kSzInRegs); WQ_LDS_MR(4, kSzInRegs); WQ_LDS_MR(8, kSzInRegs);
  WQ_LDS_MR(16, kSzInRegs);
  WQ_LDS_MR(1, 8); WQ_LDS_MR(2, 8); WQ_LDS_MR(4, 8); WQ_LDS_MR(8, 8); WQ_LDS_MR(16, 8);
  WQ_LDS_MR(1, 4); WQ_LDS_MR(2, 4); WQ_LDS_MR(4, 4); WQ_LDS_MR(8, 4); WQ_LDS_MR(16, 4);
  WQ_LDS_MR(1, 2); WQ_LDS_MR(2, 2); WQ_LDS_MR(4, 2); WQ_LDS_MR(8, 2); WQ_LDS_MR(16, 2);
  WQ_LDS_MR(1, 1); WQ_LDS_MR(2, 1); WQ_LDS_MR(4, 1); WQ_LDS_MR(8, 1); WQ_LDS_MR(16, 1);
  WQ_LDS_MR(1, 0); WQ_LDS_MR(2, 0); WQ_LDS_MR(4, 0); WQ_LDS_MR(8, 0); WQ_LDS_MR(16, 0);
#undef WQ_LDS_MR
  const int xl = mrows_max <= 4 ? 1 : (mrows_max <= 8 ? 2 : 4);
  // two 16-channel tiles per wave share each staged activation fragment, as long as
  // the grid still has a block for every CU and spreads evenly over them (the CU with
  // the most blocks at most 15 % above the mean: 344 pairs of 11008 channels on 256
  // CUs, 1.49x, run faster as 688 single tiles)
  const int64_t pairs = ((N + 31) / 32) * ((M + 15) / 16);
  const int nt = pairs >= kNumCu && (pairs + kNumCu - 1) / kNumCu * kNumCu * 100 <= 115 * pairs ? 2 : 1;
  // per-wave staging with (s, z) in registers, loaded per window of D groups with its
  // weights, when each wave has at most two windows (up to 4096 input channels):
  // 4096 x 4096 at M = 16, 8 and 4 9.7, 7.3 and 6.7 against 10.2, 7.6 and 7.1 us,
  // the 11008 x 4096 layer at M = 16 13.4 against 13.5. On the 70B down-projection
  // (14 windows per wave) the reloads inside the weight stream cost more than the
  // block's staging saves: 43.3 against 38.4 us at M = 8.
  const bool ring_regs = vec && G % (kGemvRingDepth * kGemvWaves) == 0 && G <= 2 * kGemvRingDepth * kGemvWaves;
#define WQ_RING_SV(XL, NT, SP)                                   \
  if (ring_regs) return launch_ring<XL, NT, kSzInRegs, SP>(WQ_ARGS); \
  if (sv == 8) return launch_ring<XL, NT, 8, SP>(WQ_ARGS);       \
  if (sv == 4) return launch_ring<XL, NT, 4, SP>(WQ_ARGS);       \
  if (sv == 2) return launch_ring<XL, NT, 2, SP>(WQ_ARGS);       \
  if (sv == 1) return launch_ring<XL, NT, 1, SP>(WQ_ARGS);       \
  return launch_ring<XL, NT, 0, SP>(WQ_ARGS);
#define WQ_RING(XL, NT)            \
  if (xl == XL && nt == NT) {      \
    if (sp) { WQ_RING_SV(XL, NT, true) } \
    WQ_RING_SV(XL, NT, false)      \
  }
  WQ_RING(1, 1);
  WQ_RING(2, 1);
  WQ_RING(4, 1);
  WQ_RING(1, 2);
  WQ_RING(2, 2);
  WQ_RING(4, 2);
#undef WQ_RING
#undef WQ_RING_SV
  return hipErrorInvalidValue;  // not reached
#undef WQ_LDS
#undef WQ_ARGS
}

}  // namespace wq
