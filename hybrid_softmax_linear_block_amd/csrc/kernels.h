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
  float* lse;             // nullable: [B][H][N] log2-sum-exp2 of the softmax rows (for the backward)
  uint16_t* gates16;      // nullable: [B*N][2*hid] fp16 gates (for the backward)
  bf16_t* wg_t;           // [2*hid][hid]  [W_gs | W_gl] transposed, bf16
  uint16_t* wo_t;         // [hid][2*hid]  [W_os ; W_ol] transposed, fp16
  // fp8 softmax branch
  uint8_t *q8, *k8, *v8t, *tk8, *tv8t;  // e4m3 copies (v transposed per 64-key tile)
  float* scales;          // [5][B][H] dequantisation scales
  uint32_t* absmax;       // [5][B][H] absmax bit patterns
  bool qkv_absmax_ready;  // absmax[0 .. 3*B*H) already holds q, k, v (from the projection)
  // MX fp8 GEMMs (gate and output): e4m3 codes with E8M0 exponents per 32
  // contraction elements; wg_t / wo_t / ap then hold codes, and
  bool mx;
  bool mx_x_ready;        // x8 / xs already written (by the projection)
  uint8_t *x8, *xs;       // x codes [B*N][hid], exponents [hid/128][mpad][4]
  uint8_t* aps;           // A' exponents [2 hid/128][mpad][4]
  uint8_t *wgs8, *wos8;   // weight exponents [hid/128][2 hid][4], [2 hid/128][hid][4]
  long long mpad;         // B*N rounded up to 256
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
// MX fp8 operands (mx_quant.hip): x [M][K] bf16 -> e4m3 codes [M][K] and
// E8M0 exponents [K/128][mpad][4]; weights (mode 0 gate, 1 out, 2 q/k/v) ->
// codes [N][K] and exponents [K/128][N][4].  The projection GEMM on them
// (gemm_epilogue.hip), with the outputs and absmax of launch_qkv_gemm.
hipError_t launch_mx_rows(const bf16_t* x, long long M, int K, long long mpad, uint8_t* codes, uint8_t* ex,
                          hipStream_t s);
hipError_t launch_mx_weights(int mode, const bf16_t* w0, const bf16_t* w1, const bf16_t* w2, int hid,
                             uint8_t* codes, uint8_t* ex, hipStream_t s);
hipError_t launch_qkv_gemm_mx(const Dims& d, const uint8_t* x8, const uint8_t* xs, long long mpad,
                              const uint8_t* wt8, const uint8_t* wts, bf16_t* q, bf16_t* k, bf16_t* v,
                              uint32_t* absmax, hipStream_t s);
// fp16 bits -> float32 (debug copies of the fp16 branch outputs)
hipError_t launch_f16_to_f32(const uint16_t* src, float* dst, long long n, hipStream_t s);

// ---- backward pass (bf16 activations) ----
// Forward values it reads are recomputed into the forward workspace by the
// same kernels (softmax also saving its row log2-sum-exp2, the gate GEMM its
// gates); the fields below point into that workspace and the backward's own.
struct BwdArgs {
  Tensor4 q, k, v, tk, tv;
  const bf16_t *x, *wgs, *wgl, *wos, *wol, *rmsw, *dy;
  float scale_log2, tau, eps;
  // saved forward values
  const uint16_t *os, *ol, *ap, *gates16;  // fp16 [M][hid], [M][hid], [M][2hid], [M][2hid]
  const float *rinv, *lse;                 // [M], [B][H][N] (+ padding)
  const bf16_t *comb_hi, *comb_lo;         // [B*H][T][e][d]
  const float* comb_z;                     // [B*H][T][D]
  // outputs (contiguous [B][tokens][H][D] / [B][N][hid]); weight gradients nullable
  bf16_t *dx, *dq, *dk, *dv, *dtk, *dtv;
  int ld_qkv;                              // row stride of dq, dk, dv in elements (hid, or 3 hid when interleaved)
  float *dwgs, *dwgl, *dwos, *dwol, *drmsw;
  // scratch
  bf16_t *wo_cat, *wg_cat;                 // [2hid][hid] = [W_os; W_ol], [hid][2hid] rows (W_gs[i], W_gl[i])
  bf16_t *dyT, *xT, *apT, *dzT;            // token-transposed operands [C][mpad] (zero past M)
  long long mpad;
  int ksplit;
  float* wpart;                            // weight-gradient partials [ksplit][rows][cols]
  bf16_t *dos, *dz, *dr;                   // [M][hid] dO_s, [M][2hid] dZ, [M][hid] dR (bf16)
  float *tcoef, *dol;                      // [M] rinv^3 sum(dR w O_l) / hid, [M][hid] dO_l
  float* rms_part;                         // [rms_blocks][hid]
  int rms_blocks;
  float* dvr;                              // [B][H][N] (+ padding) rowsum(dO_s * O_s)
  float *dq_s, *dk_s, *dv_s, *dtk_s, *dtv_s;  // softmax-branch gradients fp32 [tokens][hid]
  bf16_t* dnum;                            // [M][hid]
  float* dden;                             // [M][H]
  float* lpart;                            // [B*H][T*lin_split][D*D+D]
  int lin_split;
  float* dcf;                              // [B*H][T][D*D+D]
  bf16_t *dsh, *dsl;                       // [B*H][T+1][d][e]
  float* dsz;                              // [B*H][T+1][D]
  hipEvent_t* ev;                          // NULL or 2 events per backward stage
  bool recompute;                          // false: the saved forward values come from a training forward
};
hipError_t run_bwd_bf16(const Dims& d, const Bf16Args& fwd, const BwdArgs& a, hipStream_t s);
hipError_t launch_bf16_to_f32(const bf16_t* src, float* dst, long long n, hipStream_t s);

// Backward through the Q/K/V projection (backward_bf16.hip).
struct QkvBwdArgs {
  long long M, mpad;
  int hid, ksplit;
  const bf16_t *x, *wq, *wk, *wv;
  const bf16_t *dxl, *dqkv;     // the layer's dx [M][hid]; [dq | dk | dv] rows [M][3 hid]
  bf16_t* dx;                   // output [M][hid]
  float *dwq, *dwk, *dwv;       // nullable [hid][hid]
  bf16_t *wcat, *xT, *dqkvT;    // scratch [hid][3 hid], [hid][mpad], [3 hid][mpad]
  float* wpart;                 // [ksplit][hid][3 hid]
};
hipError_t run_qkv_backward(const QkvBwdArgs& a, hipStream_t s);

// ---- feed-forward of the block (dit_block.hip) ----
// z = y + GELU_tanh(RMSNorm(y) W_1) W_2 for y [M][hid] bf16; weights [in][out]
// bf16 (w_1 [hid][F], w_2 [F][hid]), w_n [hid]; scratch: h [M][hid],
// u [M][F], w1t [F][hid], w2t [hid][F] (bf16).
struct FfnArgs {
  long long M;
  int hid, F;
  float eps;
  const bf16_t *y, *wn, *w1, *w2;
  bf16_t *h, *u, *w1t, *w2t, *z;
  // MX fp8 GEMMs: u, w1t and w2t then hold e4m3 codes, with
  bool mx;
  uint8_t *h8, *hs, *us, *w1s, *w2s;  // h codes [M][hid]; exponents [hid/128][mpad][4], [F/128][mpad][4],
                                      // [hid/128][F][4], [F/128][hid][4]
  long long mpad;                     // M rounded up to 256
};
hipError_t run_ffn_bf16(const FfnArgs& a, hipStream_t s);

// Workspace sizes (bytes) of each buffer in the plans above.
struct WsPlan {
  size_t off[24];
  size_t size[24];
  int count;
  size_t total;
};

}  // namespace hyb
