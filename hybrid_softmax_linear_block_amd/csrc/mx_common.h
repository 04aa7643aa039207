// MX (OCP microscaling) e4m3 helpers for gfx950: the scaled f8f6f4 MFMA and
// the per-block exponent and element conversion of the quantisers.
#pragma once
#include "mfma_common.h"

namespace hyb {

typedef __attribute__((ext_vector_type(8))) int i32x8;

// v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 operands (lane layout measured on
// gfx950): lane l holds row l % 32; its bytes 0-15 are k = 16 (l / 32) + b and
// bytes 16-31 are k = 32 + 16 (l / 32) + (b - 16).  Byte 0 of ea / eb is an
// E8M0 exponent (2^(e-127)): lanes 0-31 give the scale of k 0-31 of their
// row, lanes 32-63 that of k 32-63.
__device__ __forceinline__ floatx16 mfma32_f8_mx(const i32x8& a, const i32x8& b, const floatx16& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// MX block exponent for e4m3 elements: the smallest s >= -127 with
// amax <= 448 * 2^s, so that no element of the block saturates.  amax is
// finite and >= 0; amax = m 2^e with m in [1, 2) needs s = e - 8, or e - 7
// when m > 1.75 (448 = 1.75 * 2^8).
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int be = (int)(b >> 23);
  if (be == 0) return -127;  // zero or subnormal
  const int s = be - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return s < -127 ? -127 : s;
}
// 2^-s as a float (exact: -127 <= s <= 120)
__device__ __forceinline__ float mx_inverse_scale(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }

// Four floats -> four e4m3 bytes (round to nearest even, saturated to +-448),
// first argument in the lowest byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

}  // namespace hyb
