// e4m3 helpers shared by the FP8 kernels (gfx950): the encoder, the two
// tile-scale rules of the 1x128 quantiser and the MFMA operand packing.
//
// Quantiser ("深入理解 DeepSeek-V3：大规模缩放挑战与对 AI 架构硬件的反思（中文精读）",
// section 3.2: activations per 1x128 tile): scale = a / 448 with a = max |v|
// of the tile (or, for power-of-two scales, the smallest 2^e >= a / 448);
// code = OCP e4m3fn nearest to v * (1 / scale), ties to even, saturated.
#pragma once

#include "moe_internal.hpp"

namespace moe {

// fp32 -> e4m3fn bits: round to nearest even, saturate at 448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;            // |v| >= 448 (or inf/nan)
  if (a >= 0x3C800000u) {                               // |v| >= 2^-6: normal
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t code = (((a >> 23) - 120u) << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | (code > 0x7Eu ? 0x7Eu : code);
  }
  // subnormal: count of 2^-9 steps, round half to even
  const float sc = __uint_as_float(a) * 512.0f;
  return sign | (uint32_t)__builtin_rintf(sc);
}

__device__ __forceinline__ void tile_scale(float amax, float& scale, float& inv) {
  if (amax > 0.0f) {
    scale = (float)((double)amax / 448.0);
    inv = (float)(448.0 / (double)amax);
  } else {
    scale = 1.0f;
    inv = 0.0f;
  }
}

// Power-of-two scale of a tile with maximum amax > 0: the smallest 2^e >=
// amax / 448 (e in [-126, 127]); amax / 448 in double is a power of two only
// when it is computed exactly, so its mantissa bits decide.
__device__ __forceinline__ void tile_scale_pow2(float amax, float& scale, float& inv) {
  if (amax > 0.0f) {
    const uint64_t b = (uint64_t)__double_as_longlong((double)amax / 448.0);
    int e = (int)((b >> 52) & 0x7FF) - 1023;
    if (b & 0xFFFFFFFFFFFFFull) ++e;
    e = min(max(e, -126), 127);
    scale = __uint_as_float((uint32_t)(e + 127) << 23);
    inv = __uint_as_float((uint32_t)(127 - e) << 23);
  } else {
    scale = 1.0f;
    inv = 0.0f;
  }
}

__device__ __forceinline__ i32x8 as_i32x8(uint4 p, uint4 q) {
  i32x8 r;
  r[0] = p.x; r[1] = p.y; r[2] = p.z; r[3] = p.w;
  r[4] = q.x; r[5] = q.y; r[6] = q.z; r[7] = q.w;
  return r;
}

}  // namespace moe
