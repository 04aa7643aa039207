// Launchers of the bf16 / fp8 MFMA kernels (internal).
#pragma once
#include "kernels.h"
#include "mfma_common.h"

namespace hyb {

hipError_t launch_softmax_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_softmax_fp8(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_quant_fp8(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_states_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_scan_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_readout_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_weights_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_gate_gemm_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_out_gemm_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);
// backward pass
hipError_t launch_da_gemm(const Dims& d, const bf16_t* dy, const bf16_t* wo_cat, const uint16_t* gsv,
                          const uint16_t* os, const uint16_t* ol, const float* rinv, const bf16_t* rmsw,
                          bf16_t* dos, bf16_t* dz, bf16_t* dr, hipStream_t s);
hipError_t launch_res_gemm(const Dims& d, const bf16_t* dz, const bf16_t* wg_cat, const bf16_t* dy, bf16_t* dx,
                           hipStream_t s);
hipError_t launch_wgrad_gemm(const bf16_t* aT, const bf16_t* bT, int Mop, int Nop, long long kpad, int ksplit,
                             float* part, hipStream_t s);
hipError_t launch_states_weighted(const Dims& d, Tensor4 q, const bf16_t* dnum, const float* dden, int split,
                                  float* part, hipStream_t s);
hipError_t launch_softmax_backward(const Dims& d, const BwdArgs& a, hipStream_t s);
hipError_t launch_linear_backward(const Dims& d, const BwdArgs& a, hipStream_t s);

}  // namespace hyb
