/*
 * hyb_attn.h -- C ABI of the MI355X (gfx950) VDN-H3 dual-branch hybrid
 * attention layer (forward and backward passes).
 *
 * The layer is defined in the VDN-H3 open-source article (tahou.com, article
 * 216474224916730885):
 *   - section "双分支混合注意力机制" (dual-branch hybrid attention):
 *       softmax branch: exact softmax attention of each video token over the
 *       key frames of its local window (chunks of consecutive latent frames,
 *       a chunk seeing itself and its neighbouring chunks), the first and last
 *       frames as boundary anchors, and all text tokens;
 *       linear branch: a forward state summing phi(K)^T V over the frames
 *       before the window and a backward state over the frames after it, both
 *       leaving out window and anchor frames, each holding half of the text;
 *       the two reads are merged so that text counts once;
 *       worked example: frame 7 of 0..14 keeps 6, 7, 8, 0, 14 in softmax,
 *       forward state 1-5, backward state 9-13;
 *   - section "自适应门控融合双分支输出" (adaptive gated fusion): one
 *       content-dependent sigmoid gate per branch, RMSNorm before the linear
 *       branch's element-wise gate, a separate output projection per branch,
 *       summed into the residual stream.
 *
 * Readings fixed by this library where the article is silent:
 *   tau = 1/sqrt(D) unless softmax_scale > 0;  phi(u) = elu(u) + 1;
 *   O_l = phi(q)^T (S+ + S-) / (phi(q)^T (z+ + z-) + eps);
 *   g_s = sigmoid(x W_gs), g_l = sigmoid(x W_gl), element-wise over hidden;
 *   r = O_l * w / sqrt(mean_hidden(O_l^2) + eps)  (per token, full hidden);
 *   y = x + (g_s * O_s) W_os + (g_l * r) W_ol,  weights [in][out] row-major;
 *   an anchor frame used as a query attends to every frame and its linear
 *   states hold text only; chunks are formed over the non-anchor frames in
 *   order (the last one may be short).
 *
 * Conventions for every call:
 *   - All tensor pointers are device memory owned by the caller.  The library
 *     never allocates or frees memory; scratch space is the caller's
 *     workspace, sized with hyb_workspace_size() (hyb_attn_forward_noalloc:
 *     a device array built into the library).
 *   - hyb_attn_forward() only enqueues work on `stream` and returns; it never
 *     synchronises.  Device faults surface at the caller's next sync.
 *   - Every argument is validated before the first launch; on failure nothing
 *     is launched, the status is returned and hyb_last_error() (thread-local)
 *     describes it.  A failed launch returns HYB_ERR_HIP.
 *   - The library keeps no mutable global state besides the thread-local
 *     error message and the built-in scratch of hyb_attn_forward_noalloc
 *     (with its per-device address table); concurrent calls on different
 *     streams with distinct workspaces are independent.
 */
#ifndef HYB_ATTN_H
#define HYB_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HYB_OK = 0,
  HYB_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size, bad stride */
  HYB_ERR_UNSUPPORTED = 2,        /* valid but not implemented (head_dim, dtype combination) */
  HYB_ERR_WORKSPACE_TOO_SMALL = 3,
  HYB_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} hyb_status;

/* HYB_FP8_MX (as `soft`, with bf16 activations) is the whole fp8 version:
 * the softmax branch as with HYB_FP8_E4M3, and the gate GEMM, the output
 * GEMM and (hyb_block_forward) the Q/K/V projection on OCP microscaling
 * e4m3 operands -- one power-of-two (E8M0) scale per 32 consecutive
 * contraction elements, the smallest that keeps the block's largest
 * magnitude within 448 (no saturation), elements rounded to nearest even,
 * products accumulated in fp32.  Activations (x, A') are blocked along the
 * feature axis of each token, weights along the input axis of each output
 * column; A' is quantised in the gate GEMM's epilogue.  The article's
 * performance section names an fp8 version without saying which products
 * it quantises; this is the library's reading.  Needs hid % 256 == 0. */
typedef enum { HYB_F32 = 0, HYB_BF16 = 1, HYB_FP8_E4M3 = 2, HYB_FP8_MX = 3 } hyb_dtype;

/* Shape and window of one call.
 *   video tokens N = frames * tokens_per_frame, token index = f * n + p
 *   (frame major).  Supported: batch, frames, tokens_per_frame, heads >= 1;
 *   text_tokens >= 0; head_dim in {32, 64, 128} (bf16 and fp8 softmax:
 *   {64, 128}); chunk_frames >= 1 (1 = per-frame window; 5 = the article's
 *   chunking); chunk_radius >= 0 (1 = self + adjacent chunks);
 *   anchor_first / anchor_last are 0 or 1. */
typedef struct {
  int32_t batch, frames, tokens_per_frame, text_tokens, heads, head_dim;
  int32_t chunk_frames;
  int32_t chunk_radius;
  int32_t anchor_first, anchor_last;
} hyb_layout;

/* A [B, tokens, H, D] activation in the activation dtype; strides in
 * elements; the D dimension is contiguous.  ptr must be 16-byte aligned and
 * every stride a multiple of 16 bytes' worth of elements. */
typedef struct {
  const void* ptr;
  int64_t stride_b, stride_tok, stride_head;
} hyb_tensor;

/* Stages of one forward call, in launch order (see hyb_debug.stage_events). */
enum {
  HYB_STAGE_WEIGHTS = 0,   /* weight transposes into the GEMM operand layout */
  HYB_STAGE_QUANT = 1,     /* fp8 absmax + quantisation (fp8 softmax only) */
  HYB_STAGE_SOFTMAX = 2,   /* block-sparse softmax branch */
  HYB_STAGE_STATES = 3,    /* per-frame linear states */
  HYB_STAGE_SCAN = 4,      /* prefix/suffix scan across frames */
  HYB_STAGE_READOUT = 5,   /* phi(Q) readout */
  HYB_STAGE_GATE = 6,      /* gate GEMM + RMSNorm/gating epilogue */
  HYB_STAGE_OUT = 7,       /* output GEMM + residual */
  HYB_STAGE_QKV = 8,       /* Q/K/V projection (hyb_block_forward only; recorded first) */
  HYB_STAGE_FFN = 9,       /* feed-forward of the block (hyb_dit_block_forward only; recorded last) */
  HYB_STAGE_COUNT = 10
};

/* Optional float32 copies of intermediate results (each pointer may be NULL):
 *   o_soft    [B, N, H, D]   softmax-branch output
 *   o_lin     [B, N, H, D]   linear-branch output (before RMSNorm)
 *   delta_f32 [B, N, hid]    y - x before rounding to the activation dtype
 *   gates     [B, N, 2*hid]  [g_s | g_l]
 *   scales    [5, B, H]      fp8 dequantisation scales of q, k, v, text_k,
 *                            text_v (only written when soft is HYB_FP8_E4M3
 *                            or HYB_FP8_MX)
 *   stage_events  NULL or an array of 2*HYB_STAGE_COUNT hipEvent_t created by
 *                 the caller; events 2s and 2s+1 are recorded on `stream`
 *                 right before and after stage s (for timing; a stage that
 *                 does not run records both back to back).
 * With fp8 softmax the dequantisation scales are absmax / 448 (1 for an
 * all-zero tensor). */
typedef struct {
  void *o_soft, *o_lin, *delta_f32, *gates, *scales;
  void* stage_events;
} hyb_debug;

/* Host-only: the integer frame tables of the layout (frames and window
 * fields of *layout are used; the rest is ignored).  T = frames.
 *   soft_frames [T*T]  row f: the softmax key frames of query frame f in
 *                      ascending order, padded with -1
 *   soft_count  [T]    number of softmax key frames of frame f
 *   fwd, bwd    [T*2]  half-open frame ranges [lo, hi) summed into the
 *                      forward / backward linear state; {0, 0} when empty
 * All four are caller-owned host arrays. */
hyb_status hyb_layout_tables(const hyb_layout* layout, int32_t* soft_frames, int32_t* soft_count,
                             int32_t* fwd, int32_t* bwd);

/* Bytes of device workspace hyb_attn_forward() needs for this layout and
 * dtype combination (act: HYB_F32 or HYB_BF16; soft: act, or HYB_FP8_E4M3 or
 * HYB_FP8_MX with act == HYB_BF16). */
hyb_status hyb_workspace_size(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft, size_t* bytes);

/* The hybrid attention layer, y = x + delta.
 *   x, y          [B, N, hid] contiguous, activation dtype; y may alias x
 *                 (in-place residual) but must not overlap q, k, v
 *   q, k, v       [B, N, H, D]; text_k, text_v [B, L, H, D]
 *   w_gate_soft, w_gate_lin, w_out_soft, w_out_lin  [hid][hid] row-major
 *                 ([in][out], y = x W), activation dtype
 *   rms_weight    [hid], activation dtype
 *   softmax_scale 0 selects 1/sqrt(D); eps > 0 (1e-6 in the article's setup)
 *   workspace     device memory of at least hyb_workspace_size() bytes,
 *                 256-byte aligned; its contents on entry are ignored
 *   dbg           NULL or a hyb_debug whose non-null members receive float32
 *                 intermediates
 * Enqueued on `stream` (a hipStream_t; NULL = default stream). */
hyb_status hyb_attn_forward(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft,
                            const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                            hyb_tensor text_k, hyb_tensor text_v,
                            const void* w_gate_soft, const void* w_gate_lin,
                            const void* w_out_soft, const void* w_out_lin,
                            const void* rms_weight, float softmax_scale, float eps,
                            void* y, void* workspace, size_t workspace_bytes,
                            void* stream, const hyb_debug* dbg);

/*
 * hyb_attn_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, layer and results as
 * hyb_attn_forward (the same kernels run), but its scratch is a device array
 * built into the library:
 *   - HYB_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU, reserved on each GPU the
 *     library runs this call on, from its first call there until the
 *     process ends; the calling thread's current device is the one used and
 *     `stream` must belong to it;
 *   - a call whose hyb_workspace_size() exceeds it returns
 *     HYB_ERR_WORKSPACE_TOO_SMALL before touching the GPU (it holds, e.g.,
 *     every precision of a 2 x 15 x 1024-token, 512-hidden layer, 146 to
 *     208 MiB; not the 768p-shaped layer, 1.6 GB and more);
 *   - every call on one GPU shares that GPU's array and leaves its contents
 *     behind (nothing in it is read before the call writes it): calls that
 *     overlap on one GPU, on any streams, race -- serialise them;
 *   - it calls no allocating routine (no hipMalloc, hipFree or library
 *     allocator); the first call on a device looks the array's address up
 *     with hipGetSymbolAddress.
 */
#define HYB_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)
hyb_status hyb_attn_forward_noalloc(const hyb_layout* layout, hyb_dtype act, hyb_dtype soft,
                                    const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                                    hyb_tensor text_k, hyb_tensor text_v,
                                    const void* w_gate_soft, const void* w_gate_lin,
                                    const void* w_out_soft, const void* w_out_lin,
                                    const void* rms_weight, float softmax_scale, float eps,
                                    void* y, void* stream, const hyb_debug* dbg);

/*
 * Q/K/V input projection -- the step before the layer.  Article section
 * "分阶段适配预训练模型" (staged adaptation): both attention branches read one
 * set of Q/K/V projections of the block input (stages A2 and B).  The
 * performance section's fp8 version quantises the softmax branch's Q/K/V;
 * the per-(tensor, batch, head) absmax that sets those scales is taken here,
 * in the projection GEMM's epilogue, instead of by a separate pass.
 *
 *   q = x W_q, k = x W_k, v = x W_v   (bf16 operands, fp32 accumulation,
 *                                      outputs rounded to bf16, no bias)
 *   x            [B, N, hid] bf16 contiguous
 *   w_q, w_k, w_v [hid][hid] bf16 row-major ([in][out]); feature h*D + d of
 *                an output is head h, dim d
 *   q, k, v      [B, N, H, D] bf16 contiguous outputs; must not overlap x or
 *                each other
 *   absmax       NULL or uint32 [3][B][H]: the float32 bit pattern of the
 *                largest |value| of the stored q (index 0), k (1), v (2) per
 *                (batch, head); NaN inputs propagate into it
 *   workspace    at least hyb_qkv_workspace_size() bytes, 256-byte aligned
 *                (the transposed weights)
 * head_dim 64 or 128; enqueued on `stream`, no synchronisation; same error
 * behaviour as hyb_attn_forward().
 */
hyb_status hyb_qkv_workspace_size(const hyb_layout* layout, size_t* bytes);
hyb_status hyb_qkv_project(const hyb_layout* layout, const void* x, const void* w_q, const void* w_k,
                           const void* w_v, void* q, void* k, void* v, uint32_t* absmax, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * The layer with its input projection: q, k, v = hyb_qkv_project(x) into the
 * workspace, then hyb_attn_forward() on them (activations bf16; soft is
 * HYB_BF16, HYB_FP8_E4M3 or HYB_FP8_MX; with HYB_FP8_MX the projection runs
 * on MX e4m3 operands too, sharing x's codes with the gate GEMM).  With fp8
 * the projection's absmax is the one
 * the softmax branch's quantisation uses, so the layer scans only the text
 * tensors for theirs.  Arguments as in hyb_attn_forward(); the workspace
 * (hyb_block_workspace_size(), 256-byte aligned) also holds q, k, v; dbg's
 * stage_events include HYB_STAGE_QKV.
 */
hyb_status hyb_block_workspace_size(const hyb_layout* layout, hyb_dtype soft, size_t* bytes);
hyb_status hyb_block_forward(const hyb_layout* layout, hyb_dtype soft, const void* x, const void* w_q,
                             const void* w_k, const void* w_v, hyb_tensor text_k, hyb_tensor text_v,
                             const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                             const void* w_out_lin, const void* rms_weight, float softmax_scale, float eps,
                             void* y, void* workspace, size_t workspace_bytes, void* stream,
                             const hyb_debug* dbg);

/*
 * Backward pass of the layer -- article section "分阶段适配预训练模型" (staged
 * adaptation): stages A1 and A2 train the new linear branch inside the frozen
 * denoiser, stage B adds LoRA adapters on the Q/K/V and output projections
 * and unfreezes the softmax gate; all of them run this pass.  It returns the
 * chain-rule gradients of L = sum(dy * y) for the forward of
 * hyb_attn_forward() (bf16 activations, bf16 softmax branch, same readings).
 *
 * Stages of one call (see hyb_bwd_debug.stage_events): */
enum {
  HYB_BSTAGE_FORWARD = 0,   /* forward recompute: O_s with softmax row statistics, states, O_l, gates, A' */
  HYB_BSTAGE_EPILOGUE = 1,  /* dA' = dy W_o^T with the gate/RMSNorm-input gradients; dx = dy + dZ W_g^T */
  HYB_BSTAGE_WGRAD = 2,     /* weight gradients of W_gs, W_gl, W_os, W_ol (those requested) */
  HYB_BSTAGE_RMS = 3,       /* RMSNorm backward: dO_l and drms_weight */
  HYB_BSTAGE_SOFTMAX = 4,   /* softmax-branch backward: dq, dk, dv, dtext_k, dtext_v parts */
  HYB_BSTAGE_LINEAR = 5,    /* linear-branch backward, adds the softmax parts, writes dq, dk, dv, dtext_* */
  HYB_BSTAGE_COUNT = 6
};

/* Optional outputs for checking intermediates (each may be NULL):
 *   d_os  float32 [B, N, H, D]  dL/dO_s (the softmax-branch output)
 *   d_ol  float32 [B, N, H, D]  dL/dO_l (the linear-branch output, before RMSNorm)
 *   lse2  float32 [B, H, N]     log2 sum_j exp(tau q_i . k_j) over each query's key set
 *   stage_events  NULL or 2*HYB_BSTAGE_COUNT hipEvent_t, recorded around each stage */
typedef struct {
  void *d_os, *d_ol, *lse2;
  void* stage_events;
} hyb_bwd_debug;

/* Bytes of device workspace hyb_attn_backward() needs (bf16 activations). */
hyb_status hyb_backward_workspace_size(const hyb_layout* layout, size_t* bytes);

/*
 * Backward of the layer with its Q/K/V projection (hyb_block_forward): stage
 * B's LoRA adapters on the Q/K/V projections need the gradients through it.
 * Recomputes q, k, v = x W_q, x W_k, x W_v (bf16) and the layer, runs the
 * layer's backward, then
 *   dx = dx_layer + dq W_q^T + dk W_k^T + dv W_v^T   (one GEMM over [dq|dk|dv])
 *   dW_q = x^T dq, dW_k = x^T dk, dW_v = x^T dv       (float32, each NULL when frozen)
 * Other gradients and arguments as in hyb_attn_backward() (without `saved`);
 * workspace of hyb_block_backward_workspace_size() bytes.  dx, dw_q, dw_k,
 * dw_v must not overlap each other, x, dy or the workspace.
 */
hyb_status hyb_block_backward_workspace_size(const hyb_layout* layout, size_t* bytes);
hyb_status hyb_block_backward(const hyb_layout* layout, const void* x, const void* w_q, const void* w_k,
                              const void* w_v, hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft,
                              const void* w_gate_lin, const void* w_out_soft, const void* w_out_lin,
                              const void* rms_weight, float softmax_scale, float eps, const void* dy, void* dx,
                              void* dtext_k, void* dtext_v, float* dw_q, float* dw_k, float* dw_v,
                              float* dw_gate_soft, float* dw_gate_lin, float* dw_out_soft, float* dw_out_lin,
                              float* drms_weight, void* workspace, size_t workspace_bytes, void* stream,
                              const hyb_bwd_debug* dbg);

/* Bytes of the `saved` buffer of hyb_attn_forward_train(). */
hyb_status hyb_saved_size(const hyb_layout* layout, size_t* bytes);

/*
 * Training forward: hyb_attn_forward() (act = soft = HYB_BF16) that also
 * keeps, in `saved` (at least hyb_saved_size() bytes, 256-byte aligned,
 * caller-owned, not overlapping y or the workspace), every forward value the
 * backward reads: O_s and O_l (fp16), each softmax row's log-sum-exp, the
 * combined linear states, the RMS factors, the gates and A'.  Passing that
 * buffer to hyb_attn_backward() skips the backward's forward recompute.  The
 * buffer is only meaningful for the layout, inputs and weights of the call
 * that filled it; the backward does not check that.  Other arguments and
 * errors as in hyb_attn_forward(); the workspace is hyb_workspace_size().
 */
hyb_status hyb_attn_forward_train(const hyb_layout* layout, const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                                  hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft,
                                  const void* w_gate_lin, const void* w_out_soft, const void* w_out_lin,
                                  const void* rms_weight, float softmax_scale, float eps, void* y, void* saved,
                                  size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                                  const hyb_debug* dbg);

/*
 *   inputs        as hyb_attn_forward() with act = soft = HYB_BF16 (q, k, v,
 *                 text_k, text_v may be strided views); dy [B, N, hid] bf16
 *                 contiguous, the gradient of y
 *   dx            [B, N, hid] bf16: dL/dx (residual + both gate projections)
 *   dq, dk, dv    [B, N, H, D] bf16 contiguous
 *   dtext_k, dtext_v [B, L, H, D] bf16 contiguous (may be NULL when L == 0)
 *   dw_gate_soft, dw_gate_lin, dw_out_soft, dw_out_lin  float32 [hid][hid]
 *                 ([in][out], like the weights), each NULL when that weight
 *                 is frozen (its gradient is then not computed)
 *   drms_weight   float32 [hid] or NULL
 *   saved         NULL (the call recomputes the forward first) or the buffer
 *                 a hyb_attn_forward_train() call on the same inputs filled
 *                 (saved_bytes >= hyb_saved_size()); then no recompute runs
 *                 and HYB_BSTAGE_FORWARD records an empty interval
 *   workspace     at least hyb_backward_workspace_size() bytes, 256-byte
 *                 aligned; contents on entry ignored
 * All outputs must be 16-byte aligned and must not overlap any input or each
 * other.  head_dim 64 or 128, hidden size at most 16384.  Enqueued on
 * `stream`; no synchronisation; same error behaviour as hyb_attn_forward().
 */
hyb_status hyb_attn_backward(const hyb_layout* layout, const void* x, hyb_tensor q, hyb_tensor k, hyb_tensor v,
                             hyb_tensor text_k, hyb_tensor text_v, const void* w_gate_soft, const void* w_gate_lin,
                             const void* w_out_soft, const void* w_out_lin, const void* rms_weight,
                             float softmax_scale, float eps, const void* dy, void* dx, void* dq, void* dk, void* dv,
                             void* dtext_k, void* dtext_v, float* dw_gate_soft, float* dw_gate_lin,
                             float* dw_out_soft, float* dw_out_lin, float* drms_weight, const void* saved,
                             size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream,
                             const hyb_bwd_debug* dbg);

/*
 * One DiT block around the layer -- article section "分阶段适配预训练模型": a
 * block of the denoiser has Q/K/V/O projections and a feed-forward network.
 * The article describes no more of the block; this library's reading:
 *   y = hyb_block_forward(x)                      (projection + layer, bf16)
 *   z = y + GELU_tanh(RMSNorm(y) W_1) W_2         (RMSNorm over hid with
 *                                                  ffn_norm_weight and eps;
 *                                                  no biases)
 *   ffn_norm_weight [hid]; w_ff1 [hid][ffn_hidden]; w_ff2 [ffn_hidden][hid]
 *   (bf16, [in][out]); ffn_hidden a positive multiple of 64 (4 * hid in the
 *   usual block; a multiple of 256 with soft == HYB_FP8_MX, where both
 *   feed-forward GEMMs also take MX e4m3 operands: the normalised y from its
 *   bf16 value, the GELU output from its fp32 value).  z [B, N, hid] bf16
 *   may alias x.  Other arguments as in
 *   hyb_block_forward(); the workspace (hyb_dit_block_workspace_size())
 *   also holds y, the normalised y, the GELU output and the transposed
 *   feed-forward weights; dbg's stage_events include HYB_STAGE_FFN.
 * Timestep modulation and cross-attention are not in the article and are not
 * part of the block.
 */
hyb_status hyb_dit_block_workspace_size(const hyb_layout* layout, hyb_dtype soft, int32_t ffn_hidden,
                                        size_t* bytes);
hyb_status hyb_dit_block_forward(const hyb_layout* layout, hyb_dtype soft, const void* x, const void* w_q,
                                 const void* w_k, const void* w_v, hyb_tensor text_k, hyb_tensor text_v,
                                 const void* w_gate_soft, const void* w_gate_lin, const void* w_out_soft,
                                 const void* w_out_lin, const void* rms_weight, const void* ffn_norm_weight,
                                 const void* w_ff1, const void* w_ff2, int32_t ffn_hidden, float softmax_scale,
                                 float eps, void* z, void* workspace, size_t workspace_bytes, void* stream,
                                 const hyb_debug* dbg);

/* Static description of a status code. */
const char* hyb_status_string(hyb_status status);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* hyb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HYB_ATTN_H */
