// Device-side helpers shared by the gfx950 kernels of the W4A16 linear.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;

// One CDNA4 matrix-core step: a 16x32 fp16 tile times a 32x16 fp16 tile added to
// a 16x16 fp32 tile. Lane l supplies A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16]
// for j = 0..7 and receives D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }

// Buffer resource of a device array of `bytes` bytes: loads through it take a 32-bit
// byte offset in a vector register plus one in a scalar register, and loads past the
// end of the array return zeros (the third-dword value gfx9 expects for raw data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Dequantization order inside one 32-bit word.
//
// fp16 0x6400 is 1024.0 and its ten mantissa bits have weight 1, so OR-ing a
// 4-bit code q into the low mantissa gives exactly 1024 + q. Masking a word with
// 0x000F000F therefore yields two halves at once: codes 0 and 4, then (after
// shifting by 4, 8, 12) codes 1/5, 2/6, 3/7. The eight values of a word thus come
// out in the order 0,4,1,5,2,6,3,7. A contraction over K does not care about the
// order inside a chunk of eight, as long as the activations are fed in the same
// order: perm_x8 reorders eight consecutive activations to match.

// Eight consecutive fp16 values x0..x7 (two per dword) reordered to
// x0,x4,x1,x5,x2,x6,x3,x7, the order codes_biased produces.
__device__ __forceinline__ uint4 perm_x8(uint4 v) {
  uint4 o;
  o.x = (v.x & 0xFFFFu) | (v.z << 16);
  o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
  o.z = (v.y & 0xFFFFu) | (v.w << 16);
  o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
  return o;
}

// v_and_or_b32 with the mask in a scalar register and the OR operand in a vector
// register: (a & mask) | b in one instruction (the compiler otherwise emits an AND
// and an OR, since this VOP3 form takes no literal operands on gfx9).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(b));
  return r;
}

// fp16 0x6400 (1024.0) in both halves, materialized in a vector register.
__device__ __forceinline__ uint32_t magic_1024x2() {
  uint32_t r;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(r));
  return r;
}

// Five-instruction unpacking of a word into four fp16 pairs, in the order of
// perm_x8: (1024+q0, 1024+q4), (1024+16q1, 1024+16q5), (1024+q2, 1024+q6),
// (1024+16q3, 1024+16q7). Codes at bits 4..7 of a half are left in place, so they
// carry a factor 16 (still exact: 1024 + 16q < 2048); the activations they meet
// are pre-scaled by 1/16.
__device__ __forceinline__ uint4 codes_biased_x16(uint32_t w, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  uint4 r;
  r.x = and_or(w, 0x000F000Fu, magic);
  r.y = and_or(w, 0x00F000F0u, magic);
  r.z = and_or(w8, 0x000F000Fu, magic);
  r.w = and_or(w8, 0x00F000F0u, magic);
  return r;
}

// fp16 (q - z) * s for the eight codes of a word, in the order of perm_x8, from the
// five-instruction unpacking: (1024 + q) - (1024 + z), and (1024 + 16q) / 16 - (64 + z)
// in one fused multiply-add, are both exact, so every value is rounded once, in the
// multiply by s: the same values as dequant_word, in 13 instructions instead of 19.
// bias = 1024 + z and nbias16 = -(64 + z) in both halves.
__device__ __forceinline__ uint4 dequant_word_x16(uint32_t w, uint32_t magic, f16x2 bias, f16x2 nbias16, f16x2 s) {
  const uint4 b = codes_biased_x16(w, magic);
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 a0 = (as_f16x2(b.x) - bias) * s;
  const f16x2 a1 = __builtin_elementwise_fma(as_f16x2(b.y), sixteenth, nbias16) * s;
  const f16x2 a2 = (as_f16x2(b.z) - bias) * s;
  const f16x2 a3 = __builtin_elementwise_fma(as_f16x2(b.w), sixteenth, nbias16) * s;
  return uint4{as_u32(a0), as_u32(a1), as_u32(a2), as_u32(a3)};
}

// Exact fp16 (q - z) for the eight codes of a word, in the order of perm_x8, from the
// five-instruction unpacking: (1024 + q) - (1024 + z) and (1024 + 16q) / 16 - (64 + z)
// (nine instructions; bias = 1024 + z, nbias16 = -(64 + z) in both halves).
__device__ __forceinline__ uint4 codes_minus_zero_x16(uint32_t w, uint32_t magic, f16x2 bias, f16x2 nbias16) {
  const uint4 b = codes_biased_x16(w, magic);
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 a0 = as_f16x2(b.x) - bias;
  const f16x2 a1 = __builtin_elementwise_fma(as_f16x2(b.y), sixteenth, nbias16);
  const f16x2 a2 = as_f16x2(b.z) - bias;
  const f16x2 a3 = __builtin_elementwise_fma(as_f16x2(b.w), sixteenth, nbias16);
  return uint4{as_u32(a0), as_u32(a1), as_u32(a2), as_u32(a3)};
}

// fp16 (q - z) * s for the eight codes of a word in their natural order (q0, q1),
// (q2, q3), (q4, q5), (q6, q7): byte b of the word copied into both halves, masked
// to (q_2b, 16 q_2b+1) and biased by 1024, then (1, 1/16) * v + (-(1024 + z),
// -(64 + z)) is exactly q - z, rounded once in the multiply by s (sixteen
// instructions). mul = (1, 1/16), add = (-(1024 + z), -(64 + z)), s in both halves.
__device__ __forceinline__ uint4 dequant_word_nat(uint32_t w, uint32_t magic, f16x2 mul, f16x2 add, f16x2 s) {
  uint32_t r[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t t = __builtin_amdgcn_perm(w, w, 0x0c000c00u | (0x00010001u * b));
    const f16x2 v = as_f16x2(and_or(t, 0x00F0000Fu, magic));
    r[b] = as_u32(__builtin_elementwise_fma(v, mul, add) * s);
  }
  return uint4{r[0], r[1], r[2], r[3]};
}

// ---------------------------------------------------------------------------
// 3-bit codes. A run of 32 consecutive codes is packed into three words (the
// layout of wq_pack_bits): code pair P = 4t + p (t, p = 0..3) is (8t + p, 8t + p + 4),
// the pair that register p of MFMA step t holds in the perm_x8 order above; pairs
// 0..14 sit five to a word (pair P in word P / 5 at bits 3i and 16 + 3i, i = P % 5),
// pair 15 in the top bit of each half-word (bit b of code 27 at bit 15 of word b,
// of code 31 at bit 31). So a lane that loads one run (12 bytes) holds the B
// operands of four MFMA steps, like the four words of a 4-bit run, and each pair
// comes out as (1024 + q_lo, 1024 + q_hi) in two instructions (six for pair 15).
__device__ __forceinline__ uint32_t pair3_biased(const uint3& w, int P, uint32_t magic) {
  if (P < 15) {
    const uint32_t x = P < 5 ? w.x : (P < 10 ? w.y : w.z);
    const int i = P % 5;
    return and_or(i ? x >> (3 * i) : x, 0x00070007u, magic);
  }
  uint32_t v = and_or(w.x >> 15, 0x00010001u, magic);
  v = and_or(w.y >> 14, 0x00020002u, v);
  return and_or(w.z >> 13, 0x00040004u, v);
}

// The four fp16 pairs (1024 + q) of MFMA step t (codes 8t .. 8t + 7 in perm_x8 order).
__device__ __forceinline__ uint4 codes3_biased(const uint3& w, int t, uint32_t magic) {
  return uint4{pair3_biased(w, 4 * t, magic), pair3_biased(w, 4 * t + 1, magic), pair3_biased(w, 4 * t + 2, magic),
               pair3_biased(w, 4 * t + 3, magic)};
}

// Exact fp16 q - z of MFMA step t (bias = 1024 + z in both halves).
__device__ __forceinline__ uint4 codes3_minus_zero(const uint3& w, int t, uint32_t magic, f16x2 bias) {
  const uint4 b = codes3_biased(w, t, magic);
  return uint4{as_u32(as_f16x2(b.x) - bias), as_u32(as_f16x2(b.y) - bias), as_u32(as_f16x2(b.z) - bias),
               as_u32(as_f16x2(b.w) - bias)};
}

// fp16 (q - z) * s of MFMA step t: the subtraction is exact, the multiply rounds once.
__device__ __forceinline__ uint4 dequant3(const uint3& w, int t, uint32_t magic, f16x2 bias, f16x2 s) {
  const uint4 b = codes3_biased(w, t, magic);
  return uint4{as_u32((as_f16x2(b.x) - bias) * s), as_u32((as_f16x2(b.y) - bias) * s),
               as_u32((as_f16x2(b.z) - bias) * s), as_u32((as_f16x2(b.w) - bias) * s)};
}

// Slot of element j (0..7) of a chunk of eight after perm_x8.
__device__ __forceinline__ int perm_slot(int j) { return ((j & 3) << 1) | (j >> 2); }

__device__ __forceinline__ f16 bits_to_f16(uint16_t b) { return __builtin_bit_cast(f16, b); }

}  // namespace wq
