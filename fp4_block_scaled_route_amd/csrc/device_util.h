// Device helpers shared by the gfx950 NVFP4 kernels: exact E2M1/E4M3 decode
// into fp16, round-to-nearest-even encoders, per-row power-of-two shifts.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over `bytes` bytes at `base` (gfx9-family descriptor:
// stride 0, 32-bit data format word).  Loads beyond `bytes` return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Same, with the non-temporal cache hint (streamed data read once).
__device__ __forceinline__ u32x4 buf_load16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// 16-byte load and store that bypass the L1 and L2 caches (cache policy sc0
// sc1: system coherent): data one workgroup hands to another on a different
// XCD within a launch, without a device-wide fence (which writes back and
// invalidates the whole L2).
constexpr int kCoherent = 1 | 16;
__device__ __forceinline__ u32x4 buf_load16_coherent(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCoherent));
}
__device__ __forceinline__ void buf_store16_coherent(u32x4 v, rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r,
                                         voff, 0, kCoherent);
}

// 8 E2M1 codes (element e in nibble e of `w`) times one E4M3 block scale,
// as 8 fp16.  Exact: |E2M1 * E4M3| lies in {0} U [2^-10, 2688] and needs at
// most 5 significant bits, which fp16 holds.  The hardware converter applies
// only the exponent of its scale operand, so the block scale is multiplied in
// afterwards with one packed fp16 multiply per pair of elements.
__device__ __forceinline__ f16x8 decode8(uint32_t w, f16 s) {
  f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  const f16x2 ss = {s, s};
  a0 *= ss;
  a1 *= ss;
  a2 *= ss;
  a3 *= ss;
  return (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// Four E4M3 scale bytes -> four fp16 values (exact: E4M3 fits fp16).
__device__ __forceinline__ void scales4(uint32_t s, f16 (&out)[4]) {
  f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
  f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

__device__ __forceinline__ float e4m3_to_float(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// Round-to-nearest-even E4M3FN byte of a non-negative float, saturating at
// 448 (0x7E).  Normal range: keep 3 mantissa bits with RNE on the 20 dropped
// bits; subnormal range (< 2^-6): the byte is RNE(v * 2^9).
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
  const int e = (int)(b >> 23) - 127;
  if (e < -6) return (uint32_t)__builtin_rintf(__uint_as_float(b) * 512.0f);  // 0..8; 8 = 2^-6
  const uint32_t mant = b & 0x7FFFFFu;
  const uint32_t keep = mant >> 20, rem = mant & 0xFFFFFu;
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) code += 1;
  return code > 0x7Eu ? 0x7Eu : code;
}

// Round-to-nearest-even E2M1 code of a float, saturating at 6; the sign bit
// is the float's sign bit.  Thresholds are the midpoints between the
// magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; at a midpoint the even code wins.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Power-of-two shift that maps a row whose max |value| has the fp32 bit
// pattern `mbits` into [2^14, 2^15): exact fp16 staging of bf16/fp32 rows.
// Zero rows, and rows whose max is inf/NaN, get shift 0.
// NVFP4 quantization of one 16-element block with global scale gs (every step
// one correctly rounded fp32 operation, in this order): scale byte =
// RNE_E4M3(amax_blk / (6 * gs)); codes = RNE_E2M1(x * (1 / (E4M3(byte) * gs)))
// packed two per byte, element 2j in the low nibble.  gs == 0 or a zero scale
// gives zero codes.  Returns the scale byte.
__device__ __forceinline__ uint32_t quant_block16_sw(const float (&xv)[16], float gs, uint2& packed) {
  float ab = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) ab = fmaxf(ab, __builtin_fabsf(xv[e]));
  uint32_t sbyte = 0;
  packed = make_uint2(0u, 0u);
  if (gs != 0.0f) {
    sbyte = e4m3_encode_nonneg(ab / (6.0f * gs));
    const float scale = e4m3_to_float(sbyte) * gs;
    if (scale != 0.0f) {
      const float r = 1.0f / scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        packed.x |= e2m1_encode(xv[e] * r) << (4 * e);
        packed.y |= e2m1_encode(xv[8 + e] * r) << (4 * e);
      }
    }
  }
  return sbyte;
}

// E4M3 byte of a non-negative float, RNE, saturating at 448: the hardware
// converter on the value clamped to 448.  Equal to e4m3_encode_nonneg for
// every non-negative fp32 input (all 2^31 non-negative bit patterns compared
// on MI355X; a NaN clamps to 448 in both).
__device__ __forceinline__ uint32_t e4m3_encode_hw(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(v, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// The same block quantization with the hardware converters: the E2M1
// converter (scale operand 1.0) rounds to nearest even and saturates at 6
// exactly as e2m1_encode for every fp32 input that is not a NaN (all 2^32
// bit patterns compared on MI355X).  Blocks holding an infinity or a NaN, and
// scales whose reciprocal is not finite, take the software encoders, so that
// no NaN ever reaches the converter: the result is bit-identical to
// quant_block16_sw for every input.
__device__ __forceinline__ uint32_t quant_block16(const float (&xv)[16], float gs, uint2& packed) {
  uint32_t im = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) im = max(im, __float_as_uint(xv[e]) & 0x7FFFFFFFu);
  if (im >= 0x7F800000u) return quant_block16_sw(xv, gs, packed);
  packed = make_uint2(0u, 0u);
  if (gs == 0.0f) return 0u;
  const uint32_t sbyte = e4m3_encode_hw(__uint_as_float(im) / (6.0f * gs));
  const float scale = e4m3_to_float(sbyte) * gs;
  if (scale == 0.0f) return sbyte;
  const float r = 1.0f / scale;
  if (!(r <= 3.402823466e38f)) return quant_block16_sw(xv, gs, packed);
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xv[0] * r, xv[1] * r, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xv[2] * r, xv[3] * r, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xv[4] * r, xv[5] * r, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, xv[6] * r, xv[7] * r, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xv[8] * r, xv[9] * r, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xv[10] * r, xv[11] * r, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xv[12] * r, xv[13] * r, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, xv[14] * r, xv[15] * r, 1.0f, 3);
  packed = make_uint2(lo, hi);
  return sbyte;
}

__device__ __forceinline__ int shift_from_maxbits(uint32_t mbits) {
  const uint32_t e = (mbits >> 23) & 0xFFu;
  if (mbits == 0u || e == 0xFFu) return 0;
  if (e == 0u) return 140;
  return 141 - (int)e;
}

// fp16 activation copies are stored step-major inside every 256-element K
// chunk: element k = 64*g + 8*q + e of a chunk (g = MFMA lane group, q = MFMA
// step) sits at position (4*q + g)*8 + e, so at each MFMA step the four lane
// groups of a row read 64 contiguous bytes.  `c` is a multiple of 8.
__device__ __forceinline__ int step_major_pos(int c) {
  const int kk = c & 255;
  return (c & ~255) + (((kk & 63) >> 3) * 4 + (kk >> 6)) * 8;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// bf16 round-to-nearest-even of a float (hardware conversion, NaN preserving).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float v) {
  __bf16 b = (__bf16)v;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}



}  // namespace nvfp4
