// Launchers of the decode kernels (gemv_kernels.h) for the weight formats other
// than 4-bit codes with 128-channel groups: 3-bit codes (the SqueezeLLM explainer's
// 3-bit models, section 1), whose layer moves 0.375 instead of 0.5 bytes per
// weight, and one (s, z) per 64 input channels (a smaller group than the default,
// section 5.3 of the same page). Fewer variants are built than for the 4-bit
// layer: (s, z) staged as vectors of eight halves or by the plain loop, and the
// block-staged kernel for one or two rows.
#include "gemv_kernels.h"

namespace wq {

template <int XC, int SZV, int MR, bool SP>
static hipError_t launch_lds3(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                              const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                              const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  const int64_t G = K / kGroup, mrows = M < 16 ? M : 16, SR = MR == 1 ? 1 : 4 * ((mrows + 3) / 4);
  const size_t lds = (SZV == kSzInRegs ? 0 : (size_t)16 * (G + 1) * 4) + (size_t)mrows * K * 2 +
                     (size_t)2 * G * SR * 4;
  return launch_rows(gemv_lds_kernel<kGemvWaves, kGemvDepth, XC, SZV, MR, SP, 3>, lds, 16, x, M, K, packed, scales,
                     zeros, N, row_ptr, col, val, y, y_f32, LowRank{}, stream);
}

// block-staged activations with one (s, z) per 64 input channels, dequantized into
// the operand per lane (3- or 4-bit codes)
template <int XC, int MR, bool SP, int BITS>
static hipError_t launch_lds_g64(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                                 const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                                 const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  const int64_t Gs = 2 * (K / kGroup), mrows = M < 16 ? M : 16;
  const size_t lds = (size_t)16 * (Gs + 1) * 4 + (size_t)mrows * K * 2;
  return launch_rows(gemv_lds_kernel<kGemvWaves, kGemvDepth, XC, 8, MR, SP, BITS, true>, lds, 16, x, M, K, packed,
                     scales, zeros, N, row_ptr, col, val, y, y_f32, LowRank{}, stream);
}

template <int XL, int NT, int SZV, bool SP, int BITS, bool G64>
static hipError_t launch_ring_fmt(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                                  const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                                  const int32_t* col, const uint16_t* val, void* y, int y_f32, hipStream_t stream) {
  const int64_t Gs = (G64 ? 2 : 1) * (K / kGroup);
  const size_t lds = (SZV == kSzInRegs ? 0 : (size_t)NT * 16 * (Gs + 1) * 4) + (size_t)kGemvWaves * 4 * XL * 136 * 2;
  return launch_rows(gemv_ring_kernel<kGemvWaves, kGemvRingDepth, XL, NT, SZV, SP, BITS, G64>, lds, 16 * NT, x, M, K,
                     packed, scales, zeros, N, row_ptr, col, val, y, y_f32, LowRank{}, stream);
}

hipError_t launch_gemv_fmt(const uint16_t* x, int64_t M, int64_t K, const uint32_t* packed,
                           const uint16_t* scales, const uint16_t* zeros, int64_t N, const int32_t* row_ptr,
                           const int32_t* col, const uint16_t* val, void* y, int y_f32, WFormat f,
                           hipStream_t stream) {
  const int64_t G = K / kGroup, Gs = f.g64 ? 2 * G : G;
  const bool sp = row_ptr != nullptr;
  const int64_t mrows_max = M < 16 ? M : 16;
  const bool aligned16 = reinterpret_cast<uintptr_t>(scales) % 16 == 0 && reinterpret_cast<uintptr_t>(zeros) % 16 == 0;
  const int sv = Gs % 8 == 0 && Gs <= kSzMaxG<8> && aligned16 ? 8 : 0;
#define WQ_ARGS x, M, K, packed, scales, zeros, N, row_ptr, col, val, y, y_f32, stream
  // block-staged activations for one or two rows of a 3-bit layer with 128-channel
  // groups, as for 4-bit codes
  if (f.bits == 3 && !f.g64 && sv == 8 && mrows_max <= 2 && mrows_max * K <= kXLdsMaxHalves) {
    const int64_t xloads = (mrows_max * K / 8 + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
    const int xc = xloads <= 1 ? 1 : xloads <= 2 ? 2 : xloads <= 4 ? 4 : xloads <= 8 ? 8 : 16;
    const int szm = G % (kGemvDepth * kGemvWaves) == 0 ? kSzInRegs : 8;
    const int mr = mrows_max == 1 ? 1 : 2;
#define WQ_LDS3(XC, SZ, MR)                                  \
  if (xc == XC && szm == SZ && mr == MR) {                   \
    if (sp) return launch_lds3<XC, SZ, MR, true>(WQ_ARGS);   \
    return launch_lds3<XC, SZ, MR, false>(WQ_ARGS);          \
  }
#define WQ_LDS3_X(XC) WQ_LDS3(XC, kSzInRegs, 1) WQ_LDS3(XC, kSzInRegs, 2) WQ_LDS3(XC, 8, 1) WQ_LDS3(XC, 8, 2)
    WQ_LDS3_X(1) WQ_LDS3_X(2) WQ_LDS3_X(4) WQ_LDS3_X(8) WQ_LDS3_X(16)
#undef WQ_LDS3_X
#undef WQ_LDS3
  }
  // one or two rows with 64-channel groups: the same staging, (q - z) s per lane
  if (f.g64 && sv == 8 && mrows_max <= 2 && mrows_max * K <= kXLdsMaxHalves) {
    const int64_t xloads = (mrows_max * K / 8 + 64 * kGemvWaves - 1) / (64 * kGemvWaves);
    const int xc = xloads <= 1 ? 1 : xloads <= 2 ? 2 : xloads <= 4 ? 4 : 8;
    const int mr = mrows_max == 1 ? 1 : 2;
#define WQ_LG(XC, MR, B)                                      \
  if (xc == XC && mr == MR && f.bits == B) {                  \
    if (sp) return launch_lds_g64<XC, MR, true, B>(WQ_ARGS);  \
    return launch_lds_g64<XC, MR, false, B>(WQ_ARGS);         \
  }
#define WQ_LG_X(XC) WQ_LG(XC, 1, 4) WQ_LG(XC, 2, 4) WQ_LG(XC, 1, 3) WQ_LG(XC, 2, 3)
    WQ_LG_X(1) WQ_LG_X(2) WQ_LG_X(4) WQ_LG_X(8)
#undef WQ_LG_X
#undef WQ_LG
  }
  const int xl = mrows_max <= 4 ? 1 : (mrows_max <= 8 ? 2 : 4);
  const int64_t pairs = ((N + 31) / 32) * ((M + 15) / 16);
  const int nt = pairs >= kNumCu && (pairs + kNumCu - 1) / kNumCu * kNumCu * 100 <= 115 * pairs ? 2 : 1;
  // 3-bit codes with 128-channel groups: (s, z) in registers where each wave has at
  // most two windows, as for 4-bit codes
  const bool ring_regs = f.bits == 3 && !f.g64 && sv == 8 && G % (kGemvRingDepth * kGemvWaves) == 0 &&
                         G <= 2 * kGemvRingDepth * kGemvWaves;
#define WQ_RR(XL, NT)                                                              \
  if (ring_regs && xl == XL && nt == NT) {                                         \
    if (sp) return launch_ring_fmt<XL, NT, kSzInRegs, true, 3, false>(WQ_ARGS);    \
    return launch_ring_fmt<XL, NT, kSzInRegs, false, 3, false>(WQ_ARGS);           \
  }
  WQ_RR(1, 1) WQ_RR(2, 1) WQ_RR(4, 1) WQ_RR(1, 2) WQ_RR(2, 2) WQ_RR(4, 2)
#undef WQ_RR
#define WQ_RF(XL, NT, SZ, B, G6)                                          \
  if (xl == XL && nt == NT && sv == SZ && f.bits == B && f.g64 == G6) {    \
    if (sp) return launch_ring_fmt<XL, NT, SZ, true, B, G6>(WQ_ARGS);     \
    return launch_ring_fmt<XL, NT, SZ, false, B, G6>(WQ_ARGS);            \
  }
#define WQ_RF_F(XL, NT, SZ) WQ_RF(XL, NT, SZ, 4, true) WQ_RF(XL, NT, SZ, 3, false) WQ_RF(XL, NT, SZ, 3, true)
#define WQ_RF_S(XL, NT) WQ_RF_F(XL, NT, 8) WQ_RF_F(XL, NT, 0)
  WQ_RF_S(1, 1) WQ_RF_S(2, 1) WQ_RF_S(4, 1) WQ_RF_S(1, 2) WQ_RF_S(2, 2) WQ_RF_S(4, 2)
#undef WQ_RF_S
#undef WQ_RF_F
#undef WQ_RF
#undef WQ_ARGS
  return hipErrorInvalidValue;  // an unsupported format
}

}  // namespace wq
