// Launch sequence of the bf16 (optionally fp8-softmax) forward pass.
// Everything is enqueued on the caller's stream; nothing synchronises.
#include "kernels_bf16.h"

namespace hyb {

#define HYB_TRY(x)                 \
  do {                             \
    hipError_t e_ = (x);           \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// Stage indices match HYB_STAGE_* of the public header.
enum { ST_WEIGHTS, ST_QUANT, ST_SOFTMAX, ST_STATES, ST_SCAN, ST_READOUT, ST_GATE, ST_OUT };

#define HYB_STAGE(st, call)                                        \
  do {                                                             \
    if (a.ev) HYB_TRY(hipEventRecord(a.ev[2 * (st)], s));          \
    HYB_TRY(call);                                                 \
    if (a.ev) HYB_TRY(hipEventRecord(a.ev[2 * (st) + 1], s));      \
  } while (0)

static hipError_t nothing() { return hipSuccess; }

__global__ __launch_bounds__(256) void k_f16_to_f32(const uint16_t* __restrict__ src, float* __restrict__ dst,
                                                    long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = (float)__builtin_bit_cast(_Float16, src[i]);
}

hipError_t launch_f16_to_f32(const uint16_t* src, float* dst, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_f16_to_f32, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

// MX operands of the gate and output GEMMs: weights, and x unless the
// projection already quantised it.
static hipError_t quantise_mx(const Dims& d, const Bf16Args& a, hipStream_t s) {
  HYB_TRY(launch_mx_weights(0, a.wgs, a.wgl, nullptr, d.hid, (uint8_t*)a.wg_t, a.wgs8, s));
  HYB_TRY(launch_mx_weights(1, a.wos, a.wol, nullptr, d.hid, (uint8_t*)a.wo_t, a.wos8, s));
  if (!a.mx_x_ready) HYB_TRY(launch_mx_rows(a.x, (long long)d.B * d.N, d.hid, a.mpad, a.x8, a.xs, s));
  return hipSuccess;
}

hipError_t run_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  HYB_STAGE(ST_WEIGHTS, a.mx ? quantise_mx(d, a, s) : launch_weights_bf16(d, a, s));
  if (a.fp8) {
    HYB_STAGE(ST_QUANT, launch_quant_fp8(d, a, s));
    HYB_STAGE(ST_SOFTMAX, launch_softmax_fp8(d, a, s));
  } else {
    HYB_STAGE(ST_QUANT, nothing());
    HYB_STAGE(ST_SOFTMAX, launch_softmax_bf16(d, a, s));
  }
  HYB_STAGE(ST_STATES, launch_states_bf16(d, a, s));
  HYB_STAGE(ST_SCAN, launch_scan_bf16(d, a, s));
  HYB_STAGE(ST_READOUT, launch_readout_bf16(d, a, s));
  HYB_STAGE(ST_GATE, a.mx ? launch_gate_gemm_mx(d, a, s) : launch_gate_gemm_bf16(d, a, s));
  HYB_STAGE(ST_OUT, a.mx ? launch_out_gemm_mx(d, a, s) : launch_out_gemm_bf16(d, a, s));
  return hipSuccess;
}

}  // namespace hyb
