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
// MX fp8 GEMMs (gemm_epilogue.hip) and their quantisers (mx_quant.hip)
hipError_t launch_gate_gemm_mx(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_out_gemm_mx(const Dims& d, const Bf16Args& a, hipStream_t s);
hipError_t launch_gelu_gemm_mx(long long M, int hid, int F, const uint8_t* h8, const uint8_t* hs, long long mpad,
                               const uint8_t* w1c, const uint8_t* w1s, uint8_t* u8, uint8_t* us, hipStream_t s);
hipError_t launch_resid_gemm_mx(long long M, int N, int K, const uint8_t* a8, const uint8_t* as, long long mpad,
                                const uint8_t* bc, const uint8_t* bs, const bf16_t* resid, bf16_t* out,
                                hipStream_t s);
hipError_t launch_mx_weights_kn(const bf16_t* w, int K, int N, uint8_t* codes, uint8_t* ex, hipStream_t s);

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
// src [M][C] (bf16, or fp16 when f16) -> dst [C][mpad] bf16, zero past M; mpad % 64 == 0
hipError_t transpose_tok(const uint16_t* src, bool f16, long long M, int C, long long mpad, bf16_t* dst,
                         hipStream_t s);
// feed-forward of the block
hipError_t launch_gelu_gemm(long long M, int hid, int F, const bf16_t* h, const bf16_t* w1t, bf16_t* out,
                            hipStream_t s);
hipError_t launch_resid_gemm(long long M, int N, int K, const bf16_t* a, const bf16_t* bt, const bf16_t* resid,
                             bf16_t* out, hipStream_t s);

}  // namespace hyb
