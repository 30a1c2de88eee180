// RTN group quantizer and INT4 packer for gfx950.
//
// Quantizer (asymmetric INT4, one scale and zero-point per 128 input channels;
// round-to-nearest is the calibration-free baseline of the AWQ paper, section 2,
// and the LLM Compressor article's FAQ; "W4A16 g128" in the DeepCompressor README
// perplexity table): per group, mn/mx -> s = fp16(max(fl32(mx - mn) / qmax, 2^-14)),
// z = clamp(rint(-mn / s), 0, qmax), q = clamp(rint(w / s) + z, 0, qmax), with
// qmax = 15 for INT4 codes (7 or 3 for the 3- and 2-bit codes the SqueezeLLM
// explainer also uses, kept in the same 4-bit packing).
//
// The codes are integers decided by float32 arithmetic, so this file must round
// exactly like the definition: IEEE float32 division correctly rounded
// (__fdiv_rn), rintf = round half to even (v_rndne_f32), fp16 conversion to
// nearest even, and no contraction (the translation unit is built with
// -ffp-contract=off; nothing here would contract anyway).
//
// The quantizer is HBM-bound (4 B read + 1 B written per weight); one wave owns
// one group at a time: per 128 weights a 512-byte coalesced load (two floats per
// lane), a butterfly min/max across the wave, and a 128-byte store of codes.
//
// Coarser groups (a multiple of 128 channels, up to one group per row, which the
// group-size option in section 5.3 of the SqueezeLLM explainer has as its default)
// take the
// min/max over all their 128-channel chunks and then code each chunk; the (s, z) of
// such a group is written to every 128-channel slot of the [N, K/128] metadata,
// the layout the linear kernels read, so their products need no change. With 128
// the weights stay in registers between the two passes; coarser groups reload them
// (from cache).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

// Groups of 64 channels (a smaller group, which the same section of the SqueezeLLM
// explainer says trades metadata for accuracy) are quantized two per wave: lanes
// 0..31 hold one group and lanes 32..63 the next, the min/max butterfly stays
// within each half, and the metadata is [N, K/64].
//
// MODE 0: groups of 128 (gc == 1 at compile time); 1: coarser groups; 2: groups of 64
template <int MODE>
__global__ void __launch_bounds__(256)
rtn_quantize_kernel(const float* __restrict__ W, const uint32_t* __restrict__ mask, int64_t N, int64_t K,
                    int64_t gc_arg, float qmax, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                    uint16_t* __restrict__ zeros) {
  constexpr bool COARSE = MODE == 1;
  const int lane = threadIdx.x & 63;
  const int64_t gc = COARSE ? gc_arg : 1;
  const int64_t G = K / kGroup;  // 128-channel metadata slots per row
  const int64_t Gq = G / gc;     // quantization groups per row (gc slots each)
  const int64_t total = N * Gq;
  const int64_t stride = (int64_t)gridDim.x * 4;
  // two weights of a 128-channel chunk; entries moved to the sparse part count as
  // +0 in the dense part
  const auto load = [&](int64_t off) {
    float2 v = *reinterpret_cast<const float2*>(W + off);
    if (mask != nullptr) {
      const uint32_t mw = mask[off >> 5];
      const uint32_t b = (uint32_t)(off & 31);
      if ((mw >> b) & 1u) v.x = 0.0f;
      if ((mw >> (b + 1)) & 1u) v.y = 0.0f;
    }
    return v;
  };
  for (int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); gid < total; gid += stride) {
    const int64_t n = gid / Gq;
    const int64_t g0 = (gid - n * Gq) * gc;  // first metadata slot of the group
    const int64_t off0 = n * K + g0 * kGroup + 2 * lane;
    const float2 v0 = load(off0);
    float mn = fminf(v0.x, v0.y);
    float mx = fmaxf(v0.x, v0.y);
    for (int64_t c = 1; c < gc; ++c) {
      const float2 v = load(off0 + c * kGroup);
      mn = fminf(mn, fminf(v.x, v.y));
      mx = fmaxf(mx, fmaxf(v.x, v.y));
    }
#pragma unroll
    for (int o = MODE == 2 ? 16 : 32; o >= 1; o >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, o));
      mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    float d = __fdiv_rn(mx - mn, qmax);
    d = fmaxf(d, 0x1p-14f);
    const f16 s16 = (f16)d;
    const float s = (float)s16;
    float zf = rintf(__fdiv_rn(-mn, s));
    zf = fminf(fmaxf(zf, 0.0f), qmax);
    const int zi = (int)zf;  // an integer, so a -0 never reaches the stored fp16
    for (int64_t c = 0; c < gc; ++c) {
      const int64_t off = off0 + c * kGroup;
      const float2 v = c == 0 ? v0 : load(off);
      float t0 = rintf(__fdiv_rn(v.x, s)) + (float)zi;
      float t1 = rintf(__fdiv_rn(v.y, s)) + (float)zi;
      t0 = fminf(fmaxf(t0, 0.0f), qmax);
      t1 = fminf(fmaxf(t1, 0.0f), qmax);
      const uint32_t q0 = (uint32_t)t0, q1 = (uint32_t)t1;
      *reinterpret_cast<uint16_t*>(codes + off) = (uint16_t)(q0 | (q1 << 8));
      if (MODE == 2 ? (lane & 31) == 0 : lane == 0) {
        // with groups of 64, slot 2 (g0 + c) + (lane >> 5) of a [N, K/64] row
        const int64_t slot = MODE == 2 ? n * 2 * G + 2 * (g0 + c) + (lane >> 5) : n * G + g0 + c;
        scales[slot] = __builtin_bit_cast(uint16_t, s16);
        zeros[slot] = __builtin_bit_cast(uint16_t, (f16)(float)zi);
      }
    }
  }
}

// Eight codes (one per byte, low nibble used) -> one word, code i in bits [4i, 4i+4).
__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t* __restrict__ codes, int64_t nwords, uint32_t* __restrict__ packed) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) {
    const uint2 c = *reinterpret_cast<const uint2*>(codes + 8 * i);
    const uint32_t lo = c.x & 0x0F0F0F0Fu, hi = c.y & 0x0F0F0F0Fu;
    packed[i] = (lo & 0xFu) | ((lo >> 4) & 0xF0u) | ((lo >> 8) & 0xF00u) | ((lo >> 12) & 0xF000u) |
                ((hi & 0xFu) << 16) | ((hi << 12) & 0xF00000u) | ((hi << 8) & 0xF000000u) |
                ((hi << 4) & 0xF0000000u);
  }
}

// 32 codes (one per byte, low three bits used) -> three words, in the layout of
// wq_pack_bits: pair P = 4t + p = (code 8t + p, code 8t + p + 4); pairs 0..14 five to a
// word at bits 3i and 16 + 3i (i = P % 5), pair 15's bits in bit 15 (code 27) and
// bit 31 (code 31) of each word.
__global__ void __launch_bounds__(256)
pack3_kernel(const uint8_t* __restrict__ codes, int64_t nruns, uint32_t* __restrict__ packed) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nruns; i += stride) {
    const uint4 c0 = *reinterpret_cast<const uint4*>(codes + 32 * i);
    const uint4 c1 = *reinterpret_cast<const uint4*>(codes + 32 * i + 16);
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const auto code = [&](int k) { return (cw[k >> 2] >> (8 * (k & 3))) & 7u; };
    uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
    for (int P = 0; P < 15; ++P) {
      const int lo = 8 * (P >> 2) + (P & 3);
      w[P / 5] |= (code(lo) << (3 * (P % 5))) | (code(lo + 4) << (16 + 3 * (P % 5)));
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) w[b] |= (((code(27) >> b) & 1u) << 15) | (((code(31) >> b) & 1u) << 31);
    packed[3 * i] = w[0];
    packed[3 * i + 1] = w[1];
    packed[3 * i + 2] = w[2];
  }
}

static int64_t clamp_blocks(int64_t want) { return want < 1 ? 1 : (want > 65536 ? 65536 : want); }

hipError_t launch_quantize(const float* W, const uint32_t* mask, int64_t N, int64_t K, int64_t group, int bits,
                           uint8_t* codes, uint16_t* scales, uint16_t* zeros, hipStream_t stream) {
  const float qmax = (float)((1 << bits) - 1);
  const int64_t groups = N * (K / group);
  const int64_t blocks = clamp_blocks((groups + 3) / 4);
  if (group == kGroup)
    hipLaunchKernelGGL(rtn_quantize_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream, W, mask, N, K,
                       (int64_t)1, qmax, codes, scales, zeros);
  else if (group == 64)  // one wave per pair of groups
    hipLaunchKernelGGL(rtn_quantize_kernel<2>, dim3((unsigned)clamp_blocks((groups / 2 + 3) / 4)), dim3(256), 0,
                       stream, W, mask, N, K, (int64_t)1, qmax, codes, scales, zeros);
  else
    hipLaunchKernelGGL(rtn_quantize_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, W, mask, N, K,
                       group / kGroup, qmax, codes, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_pack3(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, hipStream_t stream) {
  const int64_t nruns = N * (K / 32);
  const int64_t blocks = clamp_blocks((nruns + 255) / 256);
  hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, nruns, packed);
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* codes, int64_t N, int64_t K, uint32_t* packed, hipStream_t stream) {
  const int64_t nwords = N * (K / 8);
  const int64_t blocks = clamp_blocks((nwords + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, nwords, packed);
  return hipGetLastError();
}

}  // namespace wq
