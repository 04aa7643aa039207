// MFMA / LDS building blocks for gfx950 (CDNA4, wave64).
//
// Lane layouts used throughout (verified on gfx950):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row (l % 32), k = 8*(l/32) + e, e = 0..7
//                             B: lane l holds col (l % 32), k = 8*(l/32) + e
//                             C: lane l, element r: row 8*(r/4) + 4*(l/32) + r%4, col l % 32
//   ds_read_b64_tr_b16        within each group of 16 lanes, result lane j element r
//                             is element (j % 4) of the 8-byte row addressed by lane
//                             (j/4 + 4r) of the group.
// Because the contraction index of an MFMA may be permuted freely as long as A
// and B agree, the kernels pick the key/token order inside each 16-wide k-step
// to match the register layout the previous MFMA produced.
#pragma once
#include <type_traits>
#include "common.h"

namespace hyb {

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(8))) _Float16 halfx8;

// Same lane layout as the bf16 variant.
__device__ __forceinline__ floatx16 mfma32_f16(const halfx8& a, const halfx8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// float -> fp16 bits, round to nearest even, saturated to the finite range.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  f = fminf(fmaxf(f, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  // clamp to +-65504, then one packed round-to-nearest-even conversion
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  const f32x2_t v = {fminf(fmaxf(lo, -65504.f), 65504.f), fminf(fmaxf(hi, -65504.f), 65504.f)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// The same without the clamp, for values known to lie inside fp16's range.
__device__ __forceinline__ uint32_t pack_f16x2_unsat(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// Four floats -> four saturated fp16 in one 8-byte store, and back.
__device__ __forceinline__ void store_f16x4(uint16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
}
__device__ __forceinline__ float4 unpack_f16x4(uint2 u) {
  typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
  const half2_t lo = __builtin_bit_cast(half2_t, u.x), hi = __builtin_bit_cast(half2_t, u.y);
  return make_float4((float)lo[0], (float)lo[1], (float)hi[0], (float)hi[1]);
}
__device__ __forceinline__ float4 load_f16x4(const uint16_t* p) { return unpack_f16x4(*(const uint2*)p); }

typedef __attribute__((address_space(3))) short4_t lds_short4;

// Two transposing 8-byte LDS reads -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 tr_pair(const bf16_t* p0, const bf16_t* p1) {
  short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
  short4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1));
  typedef __attribute__((ext_vector_type(8))) short short8_t;
  short8_t c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Row-major bf16 tile in LDS, COLS elements per row, with the 16-byte granule
// index XOR-swizzled by row so that (a) 16 consecutive rows read at one
// granule and (b) 4 consecutive rows read across 4 consecutive granules both
// touch distinct banks.
template <int COLS>
struct Swz {
  static constexpr int G = COLS / 8;
  static_assert(G == 4 || G == 8 || G == 16, "tile width must be 32, 64 or 128 16-bit elements");
  __device__ static __forceinline__ int key(int row) {
    if constexpr (G == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (G == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else return (row >> 2) & 3;
  }
  // element offset of (row, col); col may be any value, its granule is swizzled
  __device__ static __forceinline__ int off(int row, int col) {
    return row * COLS + ((((col >> 3) ^ key(row))) << 3) + (col & 7);
  }
};

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *(const uint4*)p; }

// s_waitcnt with only vmcnt = N (expcnt / lgkmcnt left at "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS byte address of a __shared__ object (the generic-to-LDS cast done once,
// outside any loop).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// Direct-to-LDS 16-byte-per-lane load (global_load_lds_dwordx4): lane l's
// 16 bytes from gbase + voff land at LDS byte address lds + 16 * l; gbase and
// lds are wave-uniform.  Issued from inline asm so that the compiler does not
// order it against unrelated LDS reads (it cannot tell which LDS buffer the
// load targets and would otherwise wait for it before every LDS read).  The
// instruction has no register results; completion is tracked by vmcnt, which
// callers wait on explicitly (wait_vmcnt) before the tile_barrier that
// publishes the tile.
__device__ __forceinline__ void dma16(const void* gbase, unsigned voff, unsigned lds) {
  // gbase must be wave-uniform; readfirstlane moves it to scalar registers
  // where the compiler cannot prove it uniform by itself.  readfirstlane
  // returns a signed int: each half goes through unsigned before widening so
  // that the low half is not sign-extended into the high one.
  const unsigned long long g = (unsigned long long)(uintptr_t)gbase;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)g);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(g >> 32));
  const unsigned long long gs = (unsigned long long)lo | ((unsigned long long)hi << 32);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gs),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}

// Workgroup barrier for LDS tiles filled by dma16: waits for this wave's LDS
// reads (lgkmcnt) and synchronises, without the full fence of __syncthreads
// (which would also drain every prefetch still in flight).  The caller waits
// (wait_vmcnt) for its own loads of the tile the next step reads.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// XCD-aware remap: hardware dispatches workgroup i to XCD i % 8.  Return the
// logical index so that each XCD runs a contiguous range of logical work.
__device__ __forceinline__ unsigned xcd_remap(unsigned i, unsigned total) {
  const unsigned xcd = i & 7u, local = i >> 3;
  const unsigned q = total >> 3, r = total & 7u;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

}  // namespace hyb
