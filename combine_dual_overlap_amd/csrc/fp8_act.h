// fp8 activations for gfx950: per-row quantisation in groups of 128 columns
// with power-of-two (E8M0) scales.
//
// The pages name a fused SiLU-mul + fp8 quantisation op that feeds an fp8 GEMM
// ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM", CI discussion)
// but give no rule.  Reading: a group of 128 consecutive columns of a row is
// stored as OCP E4M3 (fn) codes plus one byte b, the scale being 2^(b - 127);
// b - 127 is the smallest exponent e >= -127 with amax(|group|) <= 448 * 2^e,
// and code = round-to-nearest-even(value * 2^-e).  Scaling by a power of two is
// exact in fp32, so the codes do not depend on how the value was scaled, and
// the gfx950 scaled MFMA applies an E8M0 byte to its operand rows itself.
// Inputs must be finite.
#pragma once

#include "common.h"

namespace dbomoe {

constexpr int kQGroup = 128;   // columns per scale group

// E8M0 byte of the group scale for a group whose largest magnitude is amax.
// amax = m * 2^E (m in [1, 2)) and 448 = 1.75 * 2^8, so amax <= 448 * 2^e holds
// first at e = E - 8 when m <= 1.75 and at e = E - 7 otherwise.
__device__ __forceinline__ uint32_t e8m0_for_amax(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int be = static_cast<int>(u >> 23);              // biased exponent; 0: zero or subnormal
  if (be == 0) return 0;                                 // amax < 2^-126: e = -127
  const int e = be - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return static_cast<uint32_t>(max(e, -127) + 127);
}

// 2^-e for the E8M0 byte b = e + 127 (b in [0, 254]: 2^-e in [2^-127, 2^127]).
__device__ __forceinline__ float e8m0_inv_scale(uint32_t b) {
  return __uint_as_float((254u - b) << 23);
}

// Four values (already multiplied by 2^-e, |v| <= 448) -> four E4M3 codes,
// round to nearest even, packed little-endian into one word.
__device__ __forceinline__ uint32_t fp8x4_rne(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__device__ __forceinline__ uint8_t fp8_rne1(float a) {
  return static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.f, 0, false) & 0xff);
}

}  // namespace dbomoe
