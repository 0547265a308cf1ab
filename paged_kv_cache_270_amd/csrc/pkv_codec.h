// pkv_codec.h — the FP8 E4M3 encoder shared by libpkv's kernels that write
// the cache: the cache writes in pkv_write.hip and the decode kernel's write
// of each sequence's newest token.  Included by the .hip sources only.
//
// Format: OCP 8-bit floating point, E4M3FN variant, as used by "Optimización
// de KV Cache con PagedAttention y Cuantización FP8 para Contextos Largos
// (128K)" §4.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv_dev {

// fp32 -> OCP E4M3FN code: round to nearest, ties to even, finite values
// at or above 448 (and infinities) saturate to +-448, NaN -> 0x7F | sign.
// Written from the format definition: below 2^-6 the codes are a uniform
// grid of 2^-9 (subnormals), above it 3 mantissa bits are kept.
// Every case is computed and the right one selected, so a wave never splits.
__device__ __forceinline__ uint32_t e4m3_from_f32(float u) {
  const uint32_t bits = __float_as_uint(u);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  const float a = __uint_as_float(abits);
  // below 2^-6: 0..8, exact scaling
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  // from 2^-6: keep the top 3 mantissa bits, round the 20 dropped bits
  // half-to-even; a carry moves into the exponent, which is what the code
  // needs (rebias 127 -> 7)
  const uint32_t nrm = ((abits + 0x7FFFFu + ((abits >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t code = a < 0.015625f ? sub : nrm;
  code = a >= 448.0f ? 0x7Eu : code;                         // saturate (and infinities)
  code = abits > 0x7F800000u ? 0x7Fu : code;                 // NaN
  return sign | code;
}

// Division of many values by one positive finite scale s, rounded as IEEE
// fp32 division rounds x / s, with no division per value.  With s = m * 2^e,
// m in [1, 2), and y = fp32(1 / m) correctly rounded, for each x:
//   q0 = x * y                 (within one ulp of x / m)
//   r  = x - q0 * m            (one fused multiply-add; exact)
//   q  = q0 + r * y            (one fused multiply-add)
// q is x / m correctly rounded (Markstein's theorem: y within half an ulp of
// 1 / m and q0 within one ulp of the quotient suffice); for x of at most 11
// significant bits -- every fp16 value -- this was also checked against
// double-precision division for every pair of significands.  Then x / s =
// q * 2^-e, exact while the quotient is a normal fp32 number; below 2^-126
// (where ldexp may round once more) every quotient encodes to a signed zero
// E4M3 code all the same.
struct ScaleDiv {
  float m, y;
  int e;
};

__device__ __forceinline__ ScaleDiv scale_div(float s) {
  int e = 0;
  const float m = 2.0f * __builtin_frexpf(s, &e);  // s = (m / 2) * 2^e, m / 2 in [0.5, 1)
  return ScaleDiv{m, 1.0f / m, e - 1};
}

__device__ __forceinline__ float div_by(float x, const ScaleDiv& d) {
  const float q0 = x * d.y;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, d.m, x), d.y, q0);
  // +-0 keeps its sign; an infinite x gives its infinity (q1 is NaN there)
  const float q = __builtin_isfinite(q1) ? __builtin_copysignf(q1, x) : q0;
  return __builtin_ldexpf(q, -d.e);
}

// Four E4M3 codes at once, through the hardware conversion: the encoder for
// bulk writes.  gfx950's fp32 -> E4M3 conversion rounds to nearest even,
// subnormal codes included, exactly as e4m3_from_f32 does below 448; it does
// not saturate (larger values become NaN) and writes every NaN as 0xFF.  So
// each quotient goes in as its magnitude, clamped to 448 when it is at or
// above 448, and the sign bit of each code is then taken from the input (a
// NaN input keeps the code 0x7F and gets its own sign).
//
// The quotient x / s is computed as div_by does, without the exponent
// split: y = fp32(1 / s) (correctly rounded; FLT_MAX where 1 / s overflows),
// q0 = x * y, q1 = q0 + (x - q0 * s) * y by two fused multiply-adds.  q1 is
// the correctly rounded quotient wherever it matters: the remainder is
// exact for every fp16 x and any positive finite s (it is about |x| * 2^-23,
// far from underflow), and where q0 or y leave the normal range the quotient
// is either >= 448 (q0 shows it, including x = +-inf) or encodes to a signed
// zero.  This was checked, code for code, for every fp16 x against the
// correctly rounded division over scales from the smallest subnormal to
// FLT_MAX.
struct Fp8Enc {
  float s, y;
};

__device__ __forceinline__ Fp8Enc fp8_enc(float s) {
  const float y = 1.0f / s;
  return Fp8Enc{s, y > 3.40282347e38f ? 3.40282347e38f : y};
}

__device__ __forceinline__ float fp8_enc_magnitude(float x, const Fp8Enc& e) {
  const float q0 = x * e.y;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, e.s, x), e.y, q0);
  return __builtin_fabsf(q0) >= 448.0f ? 448.0f : __builtin_fabsf(q1);
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Codes of the fp16 values 0, 1 (lo) and 2, 3 (hi) divided by the scale:
// byte i of the result is the code of value i.
__device__ __forceinline__ uint32_t e4m3x4_from_f16x4(uint32_t lo, uint32_t hi,
                                                      const Fp8Enc& e) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_enc_magnitude(f16_lo(lo), e),
                                          fp8_enc_magnitude(f16_hi(lo), e), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_enc_magnitude(f16_lo(hi), e),
                                      fp8_enc_magnitude(f16_hi(hi), e), w, true);
  // the byte holding each input's sign bit: bytes 1 and 3 of lo, then of hi
  const uint32_t signs = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
  return (signs & 0x80808080u) | ((uint32_t)w & 0x7F7F7F7Fu);
}

}  // namespace pkv_dev
