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
__device__ __forceinline__ uint32_t e4m3_from_f32(float u) {
  const uint32_t bits = __float_as_uint(u);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  if (abits > 0x7F800000u) return sign | 0x7Fu;              // NaN
  const float a = __uint_as_float(abits);
  if (a >= 448.0f) return sign | 0x7Eu;                      // saturate
  if (a < 0.015625f)                                         // < 2^-6
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);     // 0..8, exact scaling
  // keep the top 3 mantissa bits, round the 20 dropped bits half-to-even;
  // a carry moves into the exponent, which is what the code needs
  const uint32_t r = abits + 0x7FFFFu + ((abits >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));                   // rebias 127 -> 7
}

}  // namespace pkv_dev
