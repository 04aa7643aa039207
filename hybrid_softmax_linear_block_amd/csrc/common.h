// Shared device helpers: storage types, conversions, MFMA fragment types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace hyb {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(16))) float floatx16;
typedef __attribute__((ext_vector_type(8))) int intx8;
typedef __attribute__((ext_vector_type(4))) int intx4;
typedef __attribute__((ext_vector_type(2))) int intx2;

// Problem geometry shared by all kernels.
struct Dims {
  int B, T, n, L, H, D;
  long long N;  // T * n video tokens per batch
  int hid;      // H * D
  FrameGeom g;
};

// [B, tokens, H, D] view with element strides; D contiguous.
struct Tensor4 {
  const void* p;
  long long sb, st, sh;
};

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // one packed round-to-nearest-even conversion
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, long long i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, long long i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p, long long i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, long long i, float v) { p[i] = f32_to_bf16(v); }
};

// phi(u) = elu(u) + 1
__device__ __forceinline__ float phi_f(float u) { return u > 0.f ? u + 1.f : __expf(u); }

__device__ __forceinline__ float sigmoid_f(float u) { return 1.f / (1.f + __expf(-u)); }
// The same with the hardware reciprocal (v_rcp_f32, within 1 ulp) in place of
// the IEEE division: 4 vector instructions instead of about 14.  Exact at
// u = 0 (1/2), 0 for u -> -inf, 1 for u -> +inf.
__device__ __forceinline__ float sigmoid_rcp(float u) { return __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

__device__ __forceinline__ long long tok_off(const Tensor4& t, int b, long long tok, int h) {
  return (long long)b * t.sb + tok * t.st + (long long)h * t.sh;
}

}  // namespace hyb
