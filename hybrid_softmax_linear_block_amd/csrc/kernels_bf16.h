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

}  // namespace hyb
