// Work-item decoding and cross-half lane reductions shared by the softmax
// kernels (bf16 and fp8).
#pragma once
#include "common.h"

namespace hyb {

// Work item of workgroup blockIdx.x.  A group = all query tiles of one
// (frame, b, h).  Groups are ordered longest first (anchor frames) and dealt
// to the 8 XCDs round-robin; within an XCD a group's tiles run back to back.
// (Workgroup i is dispatched to XCD i % 8.)
struct Item {
  int qt, h, b, f;
};

__device__ __forceinline__ Item decode_item(const Dims& d, int qtiles) {
  const unsigned ngroups = (unsigned)d.T * d.B * d.H;
  const unsigned nfull = (ngroups / 8u) * 8u * (unsigned)qtiles;
  unsigned grp, qtu;
  if (blockIdx.x < nfull) {
    const unsigned local = blockIdx.x >> 3;
    grp = (local / qtiles) * 8u + (blockIdx.x & 7u);
    qtu = local % qtiles;
  } else {
    grp = blockIdx.x / qtiles;
    qtu = blockIdx.x % qtiles;
  }
  Item it;
  it.qt = (int)qtu;
  it.h = grp % d.H;
  it.b = (grp / d.H) % d.B;
  it.f = frame_by_cost(d.g, (int)(grp / ((unsigned)d.H * d.B)));
  return it;
}

// Combine a per-lane value with that of lane l ^ 32 (the other half of the
// query row's keys) with one cross-half lane swap.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace hyb
