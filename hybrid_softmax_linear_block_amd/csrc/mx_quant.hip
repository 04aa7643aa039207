// MX (microscaling) e4m3 quantisers for the fp8 GEMMs.
//
// The VDN-H3 article's performance section reports an fp8 version of the
// model without saying which products run in fp8.  With the fp8 GEMM option
// the Q/K/V projection, the gate GEMM, the output GEMM and the DiT block's
// feed-forward GEMMs take e4m3 operands with one power-of-two (E8M0) scale
// per 32 consecutive contraction elements (the OCP microscaling block
// format), which gfx950's scaled MFMA applies in hardware.  The block
// exponent is the smallest one that keeps the block's largest magnitude
// within e4m3's 448 (mx_exponent), so no element saturates; elements are
// rounded to nearest even.
//
// Layouts (bytes):
//   codes      [rows][K]            row-major, contraction contiguous
//   exponents  [K / 128][rows][4]   byte j of word (g, r) = block 4 g + j of row r
// Activation exponent arrays have mpad rows (tokens rounded up to 256), so
// that a GEMM's last token tile loads whole exponent chunks.  k_mx_rows fills
// the rows past the last token with exponent 0 (scale 1); the GEMM epilogues
// that quantise A' and the GELU output leave them unset.  Either way they
// only feed output rows that are never stored.
#include "kernels_bf16.h"
#include "mx_common.h"

namespace hyb {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One thread per (row, 32-element block); blocks of a row are adjacent
// threads, so the 64-byte reads and 32-byte writes of a wave are contiguous.
__global__ __launch_bounds__(256) void k_mx_rows(const bf16_t* __restrict__ x, long long M, int K, long long mpad,
                                                 uint8_t* __restrict__ codes, uint8_t* __restrict__ ex) {
  const int nb = K / 32;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= mpad * nb) return;
  const long long m = t / nb;
  const int kb = (int)(t - m * nb);
  uint8_t* ep = ex + ((long long)(kb >> 2) * mpad + m) * 4 + (kb & 3);
  if (m >= M) {
    *ep = 127;
    return;
  }
  const uint4* src = (const uint4*)(x + m * K + kb * 32);
  uint4 u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = src[i];
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[8 * i + 0] = bf_lo(u[i].x); v[8 * i + 1] = bf_hi(u[i].x);
    v[8 * i + 2] = bf_lo(u[i].y); v[8 * i + 3] = bf_hi(u[i].y);
    v[8 * i + 4] = bf_lo(u[i].z); v[8 * i + 5] = bf_hi(u[i].z);
    v[8 * i + 6] = bf_lo(u[i].w); v[8 * i + 7] = bf_hi(u[i].w);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int se = mx_exponent(amax);
  const float inv = mx_inverse_scale(se);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
  uint4* dst = (uint4*)(codes + m * K + kb * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  *ep = (uint8_t)(se + 127);
}

// Weights [in][out] (y = x W) -> the GEMM's [N][K] operand, blocks along the
// input dimension of each output column.
//   mode 0 (gate):  N = 2 hid, K = hid:   W(k, n) = n < hid ? W_gs[k][n] : W_gl[k][n - hid]
//   mode 1 (out):   N = hid,   K = 2 hid: W(k, n) = k < hid ? W_os[k][n] : W_ol[k - hid][n]
//   mode 2 (qkv):   N = 3 hid, K = hid:   W(k, n) = W_{q,k,v}[k][n mod hid], tensor n / hid
// One thread per (column, block); adjacent threads take adjacent columns so
// that each of the 32 row reads is coalesced.
__global__ __launch_bounds__(256) void k_mx_weights(const bf16_t* __restrict__ w0, const bf16_t* __restrict__ w1,
                                                    const bf16_t* __restrict__ w2, int hid, int mode,
                                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ ex) {
  const int N = mode == 0 ? 2 * hid : (mode == 1 ? hid : 3 * hid);
  const int K = mode == 1 ? 2 * hid : hid;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)N * (K / 32)) return;
  const int n = (int)(t % N), kb = (int)(t / N);
  const bf16_t* src;
  int col = n, k0 = kb * 32;
  if (mode == 0) {
    src = n < hid ? w0 : w1;
    col = n < hid ? n : n - hid;
  } else if (mode == 1) {
    src = k0 < hid ? w0 : w1;  // a 32-row block never straddles (hid % 32 == 0)
    k0 = k0 < hid ? k0 : k0 - hid;
  } else {
    const int tt = n / hid;
    src = tt == 0 ? w0 : (tt == 1 ? w1 : w2);
    col = n - tt * hid;
  }
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    v[j] = bf16_to_f32(src[(long long)(k0 + j) * hid + col]);
    amax = fmaxf(amax, fabsf(v[j]));
  }
  const int se = mx_exponent(amax);
  const float inv = mx_inverse_scale(se);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
  uint4* dst = (uint4*)(codes + (long long)n * K + kb * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  ex[((long long)(kb >> 2) * N + n) * 4 + (kb & 3)] = (uint8_t)(se + 127);
}

// Any [K][N] row-major weight ([in][out]) -> codes [N][K], exponents
// [K/128][N][4] (the feed-forward weights).
__global__ __launch_bounds__(256) void k_mx_weights_kn(const bf16_t* __restrict__ w, int K, int N,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ ex) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)N * (K / 32)) return;
  const int n = (int)(t % N), kb = (int)(t / N);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    v[j] = bf16_to_f32(w[(long long)(kb * 32 + j) * N + n]);
    amax = fmaxf(amax, fabsf(v[j]));
  }
  const int se = mx_exponent(amax);
  const float inv = mx_inverse_scale(se);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = e4m3x4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
  uint4* dst = (uint4*)(codes + (long long)n * K + kb * 32);
  dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
  dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
  ex[((long long)(kb >> 2) * N + n) * 4 + (kb & 3)] = (uint8_t)(se + 127);
}

hipError_t launch_mx_weights_kn(const bf16_t* w, int K, int N, uint8_t* codes, uint8_t* ex, hipStream_t s) {
  if (K % 128 != 0 || N <= 0) return hipErrorInvalidValue;
  const long long blocks = ((long long)N * (K / 32) + 255) / 256;
  hipLaunchKernelGGL(k_mx_weights_kn, dim3((unsigned)blocks), dim3(256), 0, s, w, K, N, codes, ex);
  return hipGetLastError();
}

hipError_t launch_mx_rows(const bf16_t* x, long long M, int K, long long mpad, uint8_t* codes, uint8_t* ex,
                          hipStream_t s) {
  if (K % 128 != 0 || mpad < M || mpad % 256 != 0) return hipErrorInvalidValue;
  const long long threads = mpad * (K / 32);
  const long long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mx_rows, dim3((unsigned)blocks), dim3(256), 0, s, x, M, K, mpad, codes, ex);
  return hipGetLastError();
}

hipError_t launch_mx_weights(int mode, const bf16_t* w0, const bf16_t* w1, const bf16_t* w2, int hid,
                             uint8_t* codes, uint8_t* ex, hipStream_t s) {
  if (hid % 128 != 0 || mode < 0 || mode > 2) return hipErrorInvalidValue;
  const long long N = mode == 0 ? 2LL * hid : (mode == 1 ? hid : 3LL * hid);
  const long long K = mode == 1 ? 2LL * hid : hid;
  const long long blocks = (N * (K / 32) + 255) / 256;
  hipLaunchKernelGGL(k_mx_weights, dim3((unsigned)blocks), dim3(256), 0, s, w0, w1, w2, hid, mode, codes, ex);
  return hipGetLastError();
}

}  // namespace hyb
