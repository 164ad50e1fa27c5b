// FP8 (OCP E4M3) cache rows for gfx950: decode to bf16 for the MFMA
// operands, and the encoder of the row quantizer.
//
// models.inteligile.com "GLM-5.2 / Model techniques map", "inference
// quantization" (FP8 inference); llm-atlas "GLM-5.2", "Faits clés"
// (precision fp8).  The pages name FP8 only; the format taken is OCP E4M3
// (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals m * 2^-9,
// largest finite magnitude 448 = code 0x7E), one fp32 scale per row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_common.h"

namespace sa {

// Every E4M3 value has at most 4 significant bits and an exponent in
// [-9, 8], so it is exact in bf16 and in fp32; the hardware conversion gives
// fp32 and the bf16 value is its upper half.
// Four codes (one 32-bit word) -> four bf16 values (two 32-bit words).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);   // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);    // bytes 2, 3
  return u32x2{__builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u)};
}

// 16 codes -> 16 bf16 values (two 16-byte MFMA operand chunks).
__device__ __forceinline__ void e4m3x16_to_bf16x16(u32x4 c, u32x4& lo, u32x4& hi) {
  const u32x2 a = e4m3x4_to_bf16x4(c[0]), b = e4m3x4_to_bf16x4(c[1]);
  const u32x2 d = e4m3x4_to_bf16x4(c[2]), e = e4m3x4_to_bf16x4(c[3]);
  lo = u32x4{a[0], a[1], b[0], b[1]};
  hi = u32x4{d[0], d[1], e[0], e[1]};
}

// fp32 -> E4M3 code: the nearest value, ties to the even code, magnitudes
// above 448 saturating to 448; a result of zero carries no sign (input
// finite).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                       // >= 448
    code = 0x7eu;
  } else if (a >= 0x3c800000u) {                // >= 2^-6: normal codes
    const uint32_t m = a & 0x7fffffu;
    code = (((a >> 23) - 120u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xfffffu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;   // a carry moves to the next binade
    code = code < 0x7eu ? code : 0x7eu;
  } else {                                      // subnormal codes: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, then ties to even
  }
  return code ? (code | ((u >> 24) & 0x80u)) : 0u;
}

}  // namespace sa
