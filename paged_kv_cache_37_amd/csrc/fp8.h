// E4M3 codes of an FP8 pool on gfx950: a stored code c stands for c * scale
// (one K and one V scale per layer).  Writes round x * (1 / scale) (float32
// product) to the nearest code, ties to the even mantissa, and saturate at
// +-448: the hardware conversion rounds that way but gives NaN past the
// largest code, so values are clamped first.  Reads widen codes to bf16,
// which holds every E4M3 value exactly; the scales are applied to the fp32
// scores and outputs instead.
#pragma once

#include "internal.h"

namespace kvp {

typedef __attribute__((ext_vector_type(2))) __bf16 fp8_bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned fp8_u4;
typedef __attribute__((ext_vector_type(2))) unsigned fp8_u2;

constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_f32(unsigned b) { return __uint_as_float(b << 16); }

// Clamp to the largest code's magnitude; a NaN stays NaN (a NaN code).
__device__ __forceinline__ float fp8_clamp(float x) { return x > kFp8Max ? kFp8Max : (x < -kFp8Max ? -kFp8Max : x); }

// Two values (already multiplied by 1 / scale) as two codes: bits 0..7 and 8..15.
__device__ __forceinline__ unsigned fp8_pack2(float a, float b) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false) & 0xffffu;
}

// A 32-bit word of two bf16 values -> their two codes (bits 0..15).
__device__ __forceinline__ unsigned fp8_quant2(unsigned bf2, float inv) {
  return fp8_pack2(bf16_bits_to_f32(bf2 & 0xffffu) * inv, bf16_bits_to_f32(bf2 >> 16) * inv);
}

// Eight bf16 values (16 bytes) -> eight codes (8 bytes), in order.
__device__ __forceinline__ fp8_u2 fp8_quant8(fp8_u4 x, float inv) {
  return fp8_u2{fp8_quant2(x.x, inv) | (fp8_quant2(x.y, inv) << 16), fp8_quant2(x.z, inv) | (fp8_quant2(x.w, inv) << 16)};
}

// Four codes (one word, in byte order) -> four bf16 values (two words, in order), exact.
__device__ __forceinline__ fp8_u2 fp8_widen4(unsigned w) {
  const fp8_bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const fp8_bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return fp8_u2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Eight codes -> eight bf16 values (the 16-byte MFMA operand of the bf16 path).
__device__ __forceinline__ fp8_u4 fp8_widen8(fp8_u2 c) {
  const fp8_u2 a = fp8_widen4(c.x), b = fp8_widen4(c.y);
  return fp8_u4{a.x, a.y, b.x, b.y};
}

}  // namespace kvp
