// Feed-forward half of a DiT block around the hybrid layer.
//
// VDN-H3 article (tahou.com), section "分阶段适配预训练模型": every block of
// the denoiser has Q/K/V/O projections and a feed-forward network (frozen in
// stages A1/A2).  The article does not describe the feed-forward network;
// the library takes z = y + GELU_tanh(RMSNorm(y) W_1) W_2 on the layer output
// y (RMSNorm is the article's normalisation; the tanh GELU and no biases are
// the library's reading).  Two MFMA GEMMs from the layer's GEMM kernel: the
// first with a GELU epilogue, the second with the residual epilogue.
#include "kernels_bf16.h"
#include "mx_common.h"

namespace hyb {

// h = y w / sqrt(mean(y^2) + eps) per row, bf16 in and out; one wave per row.
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const bf16_t* __restrict__ y, const bf16_t* __restrict__ w,
                                                      long long M, int hid, float eps, bf16_t* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const long long m = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave
  const bf16_t* yr = y + m * hid;
  float ss = 0.f;
  for (int c = 4 * lane; c < hid; c += 256) {
    const uint2 u = *(const uint2*)(yr + c);
    const float a = __uint_as_float(u.x << 16), b = __uint_as_float(u.x & 0xffff0000u);
    const float e = __uint_as_float(u.y << 16), f = __uint_as_float(u.y & 0xffff0000u);
    ss = fmaf(a, a, fmaf(b, b, fmaf(e, e, fmaf(f, f, ss))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = rsqrtf(ss / (float)hid + eps);
  for (int c = 4 * lane; c < hid; c += 256) {
    const uint2 u = *(const uint2*)(yr + c);
    const uint2 wv = *(const uint2*)(w + c);
    const float a = __uint_as_float(u.x << 16) * r * __uint_as_float(wv.x << 16);
    const float b = __uint_as_float(u.x & 0xffff0000u) * r * __uint_as_float(wv.x & 0xffff0000u);
    const float e = __uint_as_float(u.y << 16) * r * __uint_as_float(wv.y << 16);
    const float f = __uint_as_float(u.y & 0xffff0000u) * r * __uint_as_float(wv.y & 0xffff0000u);
    *(uint2*)(h + m * hid + c) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(e, f));
  }
}

// The fp8 version: the normalised input (stored in bf16) and the weights as
// MX e4m3 operands, the GELU output quantised in the first GEMM's epilogue.
static hipError_t run_ffn_mx(const FfnArgs& a, hipStream_t s) {
  hipError_t e = launch_mx_weights_kn(a.w1, a.hid, a.F, (uint8_t*)a.w1t, a.w1s, s);  // [hid][F] -> codes [F][hid]
  if (e != hipSuccess) return e;
  e = launch_mx_weights_kn(a.w2, a.F, a.hid, (uint8_t*)a.w2t, a.w2s, s);            // [F][hid] -> codes [hid][F]
  if (e != hipSuccess) return e;
  const long long blocks = (a.M + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3((unsigned)blocks), dim3(256), 0, s, a.y, a.wn, a.M, a.hid, a.eps, a.h);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_mx_rows(a.h, a.M, a.hid, a.mpad, a.h8, a.hs, s);
  if (e != hipSuccess) return e;
  e = launch_gelu_gemm_mx(a.M, a.hid, a.F, a.h8, a.hs, a.mpad, (const uint8_t*)a.w1t, a.w1s, (uint8_t*)a.u, a.us, s);
  if (e != hipSuccess) return e;
  return launch_resid_gemm_mx(a.M, a.hid, a.F, (const uint8_t*)a.u, a.us, a.mpad, (const uint8_t*)a.w2t, a.w2s, a.y,
                              a.z, s);
}

hipError_t run_ffn_bf16(const FfnArgs& a, hipStream_t s) {
  if (a.mx) return run_ffn_mx(a, s);
  // weights into the GEMMs' [N][K] operand layout
  hipError_t e = transpose_tok(a.w1, false, a.hid, a.F, a.hid, a.w1t, s);  // [hid][F] -> [F][hid]
  if (e != hipSuccess) return e;
  e = transpose_tok(a.w2, false, a.F, a.hid, a.F, a.w2t, s);                // [F][hid] -> [hid][F]
  if (e != hipSuccess) return e;
  const long long blocks = (a.M + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3((unsigned)blocks), dim3(256), 0, s, a.y, a.wn, a.M, a.hid, a.eps, a.h);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gelu_gemm(a.M, a.hid, a.F, a.h, a.w1t, a.u, s);
  if (e != hipSuccess) return e;
  return launch_resid_gemm(a.M, a.hid, a.F, a.u, a.w2t, a.y, a.z, s);
}

}  // namespace hyb
