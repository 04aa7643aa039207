// Launch sequence of the backward pass (bf16 activations), and its
// memory-bound helper kernels: token transposes for the weight-gradient GEMMs,
// the RMSNorm backward and the partial-sum reductions.
//
// VDN-H3 article (tahou.com), section "分阶段适配预训练模型": stages A1/A2
// train the linear branch (its gate, RMSNorm and output projection) with the
// softmax branch and the Q/K/V/O projections frozen; stage B adds LoRA on the
// Q/K/V and output projections and unfreezes the softmax gate.  The pass
// therefore produces the activation gradients (dx, dq, dk, dv, dtext_k,
// dtext_v) and, for each weight the caller asks for, its gradient.
//
// The forward values the pass needs are recomputed first by the forward
// kernels (the output projection excepted): O_s (fp16) with each softmax
// row's log2-sum-exp2, the linear states, O_l (fp16), the RMS factors, and
// the gates (fp16) with A' = [G_s O_s | G_l R] (fp16).
#include "kernels_bf16.h"

namespace hyb {

#define HYB_TRY(x)                   \
  do {                               \
    hipError_t e_ = (x);             \
    if (e_ != hipSuccess) return e_; \
  } while (0)

// Backward stage indices match HYB_BSTAGE_* of the public header.
enum { BST_FORWARD, BST_EPILOGUE, BST_WGRAD, BST_RMS, BST_SOFTMAX, BST_LINEAR };

#define HYB_BSTAGE(st, ...)                                     \
  do {                                                          \
    if (a.ev) HYB_TRY(hipEventRecord(a.ev[2 * (st)], s));       \
    __VA_ARGS__;                                                \
    if (a.ev) HYB_TRY(hipEventRecord(a.ev[2 * (st) + 1], s));   \
  } while (0)

// src [M][C] (bf16, or fp16 converted to bf16) -> dst [C][mpad] bf16, zero for
// tokens >= M.  64 x 64 tiles through LDS.
template <bool F16>
__global__ __launch_bounds__(256) void k_transpose_tok(const uint16_t* __restrict__ src, long long M, int C,
                                                       long long mpad, bf16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][65];
  const int ctiles = (C + 63) / 64;
  const long long m0 = (long long)(blockIdx.x / ctiles) * 64;
  const int c0 = (int)(blockIdx.x % ctiles) * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = tid + 256 * i, r = idx >> 6, cc = idx & 63;
    const long long m = m0 + r;
    const int c = c0 + cc;
    uint16_t val = 0;
    if (m < M && c < C) {
      const uint16_t raw = src[m * C + c];
      val = F16 ? f32_to_bf16((float)__builtin_bit_cast(_Float16, raw)) : raw;
    }
    tile[r][cc] = val;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int idx = tid + 256 * i, cr = idx >> 6, mm = idx & 63;
    const int c = c0 + cr;
    const long long m = m0 + mm;
    if (c < C && m < mpad) dst[(long long)c * mpad + m] = tile[mm][cr];
  }
}

hipError_t transpose_tok(const uint16_t* src, bool f16, long long M, int C, long long mpad, bf16_t* dst,
                         hipStream_t s) {
  const long long blocks = (mpad / 64) * ((C + 63) / 64);
  if (blocks > 0x7fffffffLL || mpad % 64) return hipErrorInvalidValue;
  if (f16)
    hipLaunchKernelGGL(k_transpose_tok<true>, dim3((unsigned)blocks), dim3(256), 0, s, src, M, C, mpad, dst);
  else
    hipLaunchKernelGGL(k_transpose_tok<false>, dim3((unsigned)blocks), dim3(256), 0, s, src, M, C, mpad, dst);
  return hipGetLastError();
}

// out = sum over ksplit partials [ksplit][R][C], split into [hid]-sized
// chunks along the rows (split_rows: chunk t = r / hid -> out_t[r - t hid][c],
// C = hid) or along the columns (chunk t = c / hid -> out_t[r][c - t hid],
// R = hid).  Null outputs are skipped.
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int ksplit, int R, int C,
                                                      int hid, bool split_rows, float* __restrict__ out0,
                                                      float* __restrict__ out1, float* __restrict__ out2) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = (long long)R * C;
  if (idx >= n) return;
  const int r = (int)(idx / C), c = (int)(idx % C);
  const int t = (split_rows ? r : c) / hid;
  float* o = t == 0 ? out0 : (t == 1 ? out1 : out2);
  if (!o) return;
  float* dst = split_rows ? o + (long long)(r - t * hid) * C + c : o + (long long)r * hid + (c - t * hid);
  float v = 0.f;
  for (int z = 0; z < ksplit; ++z) v += part[z * n + idx];
  *dst = v;
}

// RMSNorm backward, part 1: per token t = rinv^3 sum_c dR_c w_c O_l,c / hid.
__global__ __launch_bounds__(256) void k_rms_t(const bf16_t* __restrict__ dr, const uint16_t* __restrict__ ol,
                                               const bf16_t* __restrict__ rmsw, const float* __restrict__ rinv,
                                               long long M, int hid, float* __restrict__ tcoef) {
  const int lane = threadIdx.x & 63;
  const long long m = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave
  float t = 0.f;
  for (int c = 4 * lane; c < hid; c += 256) {
    const uint2 g = *(const uint2*)(dr + m * hid + c);
    const uint2 w = *(const uint2*)(rmsw + c);
    const float4 o = load_f16x4(ol + m * hid + c);
    t = fmaf(__uint_as_float(g.x << 16) * __uint_as_float(w.x << 16), o.x, t);
    t = fmaf(__uint_as_float(g.x & 0xffff0000u) * __uint_as_float(w.x & 0xffff0000u), o.y, t);
    t = fmaf(__uint_as_float(g.y << 16) * __uint_as_float(w.y << 16), o.z, t);
    t = fmaf(__uint_as_float(g.y & 0xffff0000u) * __uint_as_float(w.y & 0xffff0000u), o.w, t);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
  if (lane == 0) {
    const float r = rinv[m];
    tcoef[m] = t * r * r * r / (float)hid;
  }
}

// RMSNorm backward, part 2: dO_l = rinv w dR - O_l t (fp32), and per-block
// column partials of drms_w = sum_tokens dR O_l rinv.  Each wave walks a
// strided set of tokens; columns in chunks of 256 (4 per lane).
__global__ __launch_bounds__(256) void k_rms_back(const bf16_t* __restrict__ dr, const uint16_t* __restrict__ ol,
                                                  const bf16_t* __restrict__ rmsw, const float* __restrict__ rinv,
                                                  const float* __restrict__ tcoef, long long M, int hid,
                                                  float* __restrict__ dol, float* __restrict__ part) {
  __shared__ float red[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long mstep = (long long)gridDim.x * 4;
  for (int c0 = 0; c0 < hid; c0 += 256) {
    const int c = c0 + 4 * lane;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    if (c < hid) {
      const uint2 w = *(const uint2*)(rmsw + c);
      const float w0 = __uint_as_float(w.x << 16), w1 = __uint_as_float(w.x & 0xffff0000u);
      const float w2 = __uint_as_float(w.y << 16), w3 = __uint_as_float(w.y & 0xffff0000u);
      for (long long m = (long long)blockIdx.x * 4 + wave; m < M; m += mstep) {
        const float r = rinv[m], tc = tcoef[m];
        const uint2 g = *(const uint2*)(dr + m * hid + c);
        const float4 o = load_f16x4(ol + m * hid + c);
        const float g0 = __uint_as_float(g.x << 16), g1 = __uint_as_float(g.x & 0xffff0000u);
        const float g2 = __uint_as_float(g.y << 16), g3 = __uint_as_float(g.y & 0xffff0000u);
        *(float4*)(dol + m * hid + c) =
            make_float4(r * w0 * g0 - o.x * tc, r * w1 * g1 - o.y * tc, r * w2 * g2 - o.z * tc, r * w3 * g3 - o.w * tc);
        a0 = fmaf(g0 * o.x, r, a0);
        a1 = fmaf(g1 * o.y, r, a1);
        a2 = fmaf(g2 * o.z, r, a2);
        a3 = fmaf(g3 * o.w, r, a3);
      }
    }
    red[wave][4 * lane] = a0;
    red[wave][4 * lane + 1] = a1;
    red[wave][4 * lane + 2] = a2;
    red[wave][4 * lane + 3] = a3;
    __syncthreads();
    if (threadIdx.x < 256 && c0 + (int)threadIdx.x < hid) {
      const int j = threadIdx.x;
      part[(long long)blockIdx.x * hid + c0 + j] = red[0][j] + red[1][j] + red[2][j] + red[3][j];
    }
    __syncthreads();
  }
}

// out[c] = sum_r part[r][c]: 64 columns per workgroup, its four waves sum
// interleaved rows, then one LDS combine (fixed order).
__global__ __launch_bounds__(256) void k_colsum(const float* __restrict__ part, int rows, int cols,
                                                float* __restrict__ out) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float v = 0.f;
  if (c < cols)
    for (int r = wave; r < rows; r += 4) v += part[(long long)r * cols + c];
  red[wave][lane] = v;
  __syncthreads();
  if (wave == 0 && c < cols) out[c] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

__global__ __launch_bounds__(256) void k_bf16_to_f32(const bf16_t* __restrict__ src, float* __restrict__ dst,
                                                     long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf16_to_f32(src[i]);
}

hipError_t launch_bf16_to_f32(const bf16_t* src, float* dst, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bf16_to_f32, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t run_bwd_bf16(const Dims& d, const Bf16Args& f, const BwdArgs& a, hipStream_t s) {
  const long long M = (long long)d.B * d.N;
  const int hid = d.hid;
  HYB_BSTAGE(BST_FORWARD, if (a.recompute) {
    HYB_TRY(launch_weights_bf16(d, f, s));
    HYB_TRY(launch_softmax_bf16(d, f, s));
    HYB_TRY(launch_states_bf16(d, f, s));
    HYB_TRY(launch_scan_bf16(d, f, s));
    HYB_TRY(launch_readout_bf16(d, f, s));
    HYB_TRY(launch_gate_gemm_bf16(d, f, s));
  });
  HYB_BSTAGE(BST_EPILOGUE, {
    const size_t wb = (size_t)hid * hid * 2;
    HYB_TRY(hipMemcpyAsync(a.wo_cat, a.wos, wb, hipMemcpyDeviceToDevice, s));
    HYB_TRY(hipMemcpyAsync(a.wo_cat + (size_t)hid * hid, a.wol, wb, hipMemcpyDeviceToDevice, s));
    HYB_TRY(hipMemcpy2DAsync(a.wg_cat, (size_t)2 * hid * 2, a.wgs, (size_t)hid * 2, (size_t)hid * 2, hid,
                             hipMemcpyDeviceToDevice, s));
    HYB_TRY(hipMemcpy2DAsync(a.wg_cat + hid, (size_t)2 * hid * 2, a.wgl, (size_t)hid * 2, (size_t)hid * 2, hid,
                             hipMemcpyDeviceToDevice, s));
    HYB_TRY(launch_da_gemm(d, a.dy, a.wo_cat, a.gates16, a.os, a.ol, a.rinv, a.rmsw, a.dos, a.dz, a.dr, s));
    HYB_TRY(launch_res_gemm(d, a.dz, a.wg_cat, a.dy, a.dx, s));
  });
  HYB_BSTAGE(BST_WGRAD, {
    const int rblocks = 256;
    if (a.dwos || a.dwol) {
      HYB_TRY(transpose_tok(a.dy, false, M, hid, a.mpad, a.dyT, s));
      HYB_TRY(transpose_tok(a.ap, true, M, 2 * hid, a.mpad, a.apT, s));
      HYB_TRY(launch_wgrad_gemm(a.apT, a.dyT, 2 * hid, hid, a.mpad, a.ksplit, a.wpart, s));
      const long long n = 2LL * hid * hid;
      hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((n + rblocks - 1) / rblocks)), dim3(256), 0, s, a.wpart,
                         a.ksplit, 2 * hid, hid, hid, true, a.dwos, a.dwol, nullptr);
      HYB_TRY(hipGetLastError());
    }
    if (a.dwgs || a.dwgl) {
      HYB_TRY(transpose_tok(a.x, false, M, hid, a.mpad, a.xT, s));
      HYB_TRY(transpose_tok(a.dz, false, M, 2 * hid, a.mpad, a.dzT, s));
      HYB_TRY(launch_wgrad_gemm(a.xT, a.dzT, hid, 2 * hid, a.mpad, a.ksplit, a.wpart, s));
      const long long n = 2LL * hid * hid;
      hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((n + rblocks - 1) / rblocks)), dim3(256), 0, s, a.wpart,
                         a.ksplit, hid, 2 * hid, hid, false, a.dwgs, a.dwgl, nullptr);
      HYB_TRY(hipGetLastError());
    }
  });
  HYB_BSTAGE(BST_RMS, {
    hipLaunchKernelGGL(k_rms_t, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, a.dr, a.ol, a.rmsw, a.rinv, M, hid,
                       a.tcoef);
    HYB_TRY(hipGetLastError());
    hipLaunchKernelGGL(k_rms_back, dim3((unsigned)a.rms_blocks), dim3(256), 0, s, a.dr, a.ol, a.rmsw, a.rinv,
                       a.tcoef, M, hid, a.dol, a.rms_part);
    HYB_TRY(hipGetLastError());
    if (a.drmsw) {
      hipLaunchKernelGGL(k_colsum, dim3((unsigned)((hid + 63) / 64)), dim3(256), 0, s, a.rms_part, a.rms_blocks,
                         hid, a.drmsw);
      HYB_TRY(hipGetLastError());
    }
  });
  HYB_BSTAGE(BST_SOFTMAX, HYB_TRY(launch_softmax_backward(d, a, s)));
  HYB_BSTAGE(BST_LINEAR, HYB_TRY(launch_linear_backward(d, a, s)));
  return hipSuccess;
}

// Through the Q/K/V projection: dx = dx_layer + [dq | dk | dv] [W_q | W_k | W_v]^T
// (one GEMM, K = 3 hid) and, when requested, dW_t = x^T d(q, k, v)_t (one
// token-contraction GEMM into [hid][3 hid], split into the three weights).
hipError_t run_qkv_backward(const QkvBwdArgs& a, hipStream_t s) {
  const int hid = a.hid;
  const size_t row = (size_t)hid * 2;
  const bf16_t* w[3] = {a.wq, a.wk, a.wv};
  for (int t = 0; t < 3; ++t)  // wcat row i = (W_q[i], W_k[i], W_v[i])
    HYB_TRY(hipMemcpy2DAsync(a.wcat + (size_t)t * hid, 3 * row, w[t], row, row, hid, hipMemcpyDeviceToDevice, s));
  HYB_TRY(launch_resid_gemm(a.M, hid, 3 * hid, a.dqkv, a.wcat, a.dxl, a.dx, s));
  if (a.dwq || a.dwk || a.dwv) {
    HYB_TRY(transpose_tok(a.x, false, a.M, hid, a.mpad, a.xT, s));
    HYB_TRY(transpose_tok(a.dqkv, false, a.M, 3 * hid, a.mpad, a.dqkvT, s));
    HYB_TRY(launch_wgrad_gemm(a.xT, a.dqkvT, hid, 3 * hid, a.mpad, a.ksplit, a.wpart, s));
    const long long n = 3LL * hid * hid;
    hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.wpart, a.ksplit, hid,
                       3 * hid, hid, false, a.dwq, a.dwk, a.dwv);
    HYB_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace hyb
