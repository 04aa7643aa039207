// Internal launch interface between the C-ABI layer (api.hip) and the
// kernel files.  Not part of the public ABI.
#pragma once
#include "common.h"

namespace hyb {

// ---- float32 activations: vector-ALU kernels (valu_f32.hip) ----
struct F32Args {
  Tensor4 q, k, v, tk, tv;
  const float *x, *wgs, *wgl, *wos, *wol, *rmsw;
  float scale_log2, eps;
  float *os, *ol, *ss, *states, *comb, *ap, *y;
  float *gates_dbg, *delta_dbg;
};
hipError_t run_f32(const Dims& d, const F32Args& a, hipStream_t s);

// ---- bf16 activations (optionally fp8 softmax branch): MFMA kernels ----
struct Bf16Args {
  Tensor4 q, k, v, tk, tv;
  const bf16_t *x, *wgs, *wgl, *wos, *wol, *rmsw;
  float scale_log2, eps;
  bool fp8;
  // workspace
  uint16_t* os;           // [B*N][hid] fp16 softmax-branch output
  uint16_t* ol;           // [B*N][hid] fp16 linear-branch output
  float* ss;              // [B*N][H]   sum of squares of O_l per head
  float* rinv;            // [B*N]      1 / sqrt(mean over hid of O_l^2 + eps)
  float* part;            // [B*H][slots][D*D+D] partial frame states: S^T [e][d], then z[d]
  bf16_t* comb_hi;        // [B*H][T][D][D] combined state, transposed [e][d], hi part
  bf16_t* comb_lo;        // same, residual part
  float* comb_z;          // [B*H][T][D] combined normaliser vector
  float* pre;             // [B*H][T][D*D+D] forward prefix scratch of the scan
  uint16_t* ap;           // [B*N][2*hid] gated branch outputs, fp16 (output GEMM operand)
  bf16_t* wg_t;           // [2*hid][hid]  [W_gs | W_gl] transposed, bf16
  uint16_t* wo_t;         // [hid][2*hid]  [W_os ; W_ol] transposed, fp16
  // fp8 softmax branch
  uint8_t *q8, *k8, *v8t, *tk8, *tv8t;  // e4m3 copies (v transposed per 64-key tile)
  float* scales;          // [5][B][H] dequantisation scales
  uint32_t* absmax;       // [5][B][H] absmax bit patterns
  bool qkv_absmax_ready;  // absmax[0 .. 3*B*H) already holds q, k, v (from the projection)
  bf16_t* y;
  float *gates_dbg, *delta_dbg;
  hipEvent_t* ev;         // NULL or 2 events per stage (timing hook)
  int state_split;        // token splits per frame in the state build
  int state_slots;        // T*state_split + text splits
  int text_split;
};

hipError_t run_bf16(const Dims& d, const Bf16Args& a, hipStream_t s);
// Q/K/V input projection (gemm_epilogue.hip): weights [W_q | W_k | W_v]
// transposed to [3*hid][hid], then q, k, v = x W (bf16, [B*N][hid] each) with
// the per-(tensor, batch, head) absmax of the stored values (nullable).
hipError_t launch_qkv_weights(const bf16_t* wq, const bf16_t* wk, const bf16_t* wv, int hid, bf16_t* out,
                              hipStream_t s);
hipError_t launch_qkv_gemm(const Dims& d, const bf16_t* x, const bf16_t* wt, bf16_t* q, bf16_t* k, bf16_t* v,
                           uint32_t* absmax, hipStream_t s);
// fp16 bits -> float32 (debug copies of the fp16 branch outputs)
hipError_t launch_f16_to_f32(const uint16_t* src, float* dst, long long n, hipStream_t s);

// Workspace sizes (bytes) of each buffer in the plans above.
struct WsPlan {
  size_t off[24];
  size_t size[24];
  int count;
  size_t total;
};

}  // namespace hyb
