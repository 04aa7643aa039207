// float32 path of the hybrid layer on the vector ALUs.
//
// Used for float32 activations (the float32 workload is a correctness-size
// case: 15 frames x 64 tokens, 2 heads x 32).  Every step computes in fp32;
// the bf16 / fp8 path uses the MFMA kernels instead.  Steps follow the layer
// definition of the VDN-H3 article, section "双分支混合注意力机制" (softmax
// over window + anchors + text; forward/backward linear states with half the
// text each, read with one shared normaliser) and section
// "自适应门控融合双分支输出" (sigmoid gates, RMSNorm, per-branch projections).
#include "kernels.h"

namespace hyb {

// --- softmax branch: one thread per query row, online softmax over S(f) + text.
template <int D>
__global__ __launch_bounds__(64) void k_softmax_f32(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk,
                                                    Tensor4 tv, float scale_log2, float* __restrict__ os) {
  const int tiles = (d.n + 63) / 64;
  int w = blockIdx.x;
  const int tile = w % tiles; w /= tiles;
  const int f = w % d.T; w /= d.T;
  const int h = w % d.H;
  const int b = w / d.H;
  const int p = tile * 64 + threadIdx.x;
  if (p >= d.n) return;
  const long long tok = (long long)f * d.n + p;
  const float* qp = (const float*)q.p + tok_off(q, b, tok, h);
  float qr[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) { qr[i] = qp[i] * scale_log2; o[i] = 0.f; }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const float* kp, const float* vp) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) s += qr[i] * kp[i];
    if (s > m) {
      const float a = exp2f(m - s);
      l *= a;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] *= a;
      m = s;
    }
    const float e = exp2f(s - m);
    l += e;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] += e * vp[i];
  };
  const SoftRanges sr = soft_ranges(d.g, f);
  for (int r = 0; r < sr.n; ++r)
    for (long long j = (long long)sr.lo[r] * d.n; j < (long long)sr.hi[r] * d.n; ++j)
      visit((const float*)k.p + tok_off(k, b, j, h), (const float*)v.p + tok_off(v, b, j, h));
  for (int j = 0; j < d.L; ++j)
    visit((const float*)tk.p + tok_off(tk, b, j, h), (const float*)tv.p + tok_off(tv, b, j, h));
  float* op = os + (((long long)b * d.N + tok) * d.H + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < D; ++i) op[i] = o[i] * inv;
}

// --- per-frame states: S_g[d][e] = sum phi(k)[d] v[e], z_g[d] = sum phi(k)[d];
// slot T is the text state.  Block = (b, h, slot, row d); thread = column e
// (e == D is the z column).  Output layout [B*H][T+1][D][D+1].
template <int D>
__global__ __launch_bounds__(256) void k_states_f32(Dims d, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv,
                                                    float* __restrict__ st) {
  int w = blockIdx.x;
  const int row = w % D; w /= D;
  const int slot = w % (d.T + 1); w /= (d.T + 1);
  const int h = w % d.H;
  const int b = w / d.H;
  const int e = threadIdx.x;
  if (e > D) return;
  const bool text = slot == d.T;
  const Tensor4& kk = text ? tk : k;
  const Tensor4& vv = text ? tv : v;
  const long long t0 = text ? 0 : (long long)slot * d.n;
  const long long cnt = text ? d.L : d.n;
  float acc = 0.f;
  for (long long t = t0; t < t0 + cnt; ++t) {
    const float pk = phi_f(((const float*)kk.p)[tok_off(kk, b, t, h) + row]);
    const float ve = e < D ? ((const float*)vv.p)[tok_off(vv, b, t, h) + e] : 1.f;
    acc += pk * ve;
  }
  st[((((long long)b * d.H + h) * (d.T + 1) + slot) * D + row) * (D + 1) + e] = acc;
}

// --- combined state per query frame:
// comb(f) = 1/2 text + sum_{g in F(f)} S_g + 1/2 text + sum_{g in B(f)} S_g.
// One thread per state element, direct range sums (the float32 workload has
// few frames; the MFMA path uses a prefix/suffix scan instead).
__global__ __launch_bounds__(256) void k_combine_f32(Dims d, const float* __restrict__ st, float* __restrict__ comb) {
  const int D = d.D, E = D * (D + 1);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.H * E) return;
  const int el = (int)(gid % E);
  const long long bh = gid / E;
  const float* s = st + bh * (long long)(d.T + 1) * E + el;
  float* c = comb + bh * (long long)d.T * E + el;
  const float text = s[(long long)d.T * E];
  for (int f = 0; f < d.T; ++f) {
    int flo, fhi, blo, bhi;
    linear_ranges(d.g, f, &flo, &fhi, &blo, &bhi);
    float fw = 0.5f * text, bw = 0.5f * text;
    for (int g = flo; g < fhi; ++g) fw += s[(long long)g * E];
    for (int g = blo; g < bhi; ++g) bw += s[(long long)g * E];
    c[(long long)f * E] = fw + bw;
  }
}

// --- readout: one thread per (b, token, h):
// O_l = phi(q)^T comb[:, :D] / (phi(q)^T comb[:, D] + eps); ss = sum O_l^2.
template <int D>
__global__ __launch_bounds__(64) void k_readout_f32(Dims d, Tensor4 q, const float* __restrict__ comb, float eps,
                                                    float* __restrict__ ol, float* __restrict__ ss) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.N * d.H) return;
  const int h = (int)(gid % d.H);
  const long long bt = gid / d.H;
  const long long tok = bt % d.N;
  const int b = (int)(bt / d.N);
  const int f = (int)(tok / d.n);
  const float* qp = (const float*)q.p + tok_off(q, b, tok, h);
  float pq[D];
#pragma unroll
  for (int i = 0; i < D; ++i) pq[i] = phi_f(qp[i]);
  const float* c = comb + (((long long)b * d.H + h) * d.T + f) * (long long)D * (D + 1);
  float den = eps;
  for (int i = 0; i < D; ++i) den += pq[i] * c[i * (D + 1) + D];
  const float inv = 1.f / den;
  float* op = ol + gid * D;
  float sq = 0.f;
  for (int e = 0; e < D; ++e) {
    float num = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) num += pq[i] * c[i * (D + 1) + e];
    const float o = num * inv;
    op[e] = o;
    sq += o * o;
  }
  ss[gid] = sq;
}

// --- gates + gated branch outputs: one thread per (token, feature in 2*hid).
__global__ __launch_bounds__(256) void k_gate_f32(Dims d, const float* __restrict__ x, const float* __restrict__ wgs,
                                                  const float* __restrict__ wgl, const float* __restrict__ os,
                                                  const float* __restrict__ ol, const float* __restrict__ ss,
                                                  const float* __restrict__ rmsw, float eps, float* __restrict__ ap,
                                                  float* __restrict__ gates_dbg) {
  const int hid = d.hid, n2 = 2 * hid;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.N * n2) return;
  const int n = (int)(gid % n2);
  const long long m = gid / n2;
  const bool lin = n >= hid;
  const int c = lin ? n - hid : n;
  const float* W = lin ? wgl : wgs;
  const float* xr = x + m * hid;
  float acc = 0.f;
  for (int kk = 0; kk < hid; ++kk) acc += xr[kk] * W[(long long)kk * hid + c];
  const float g = sigmoid_f(acc);
  float val;
  if (!lin) {
    val = os[m * hid + c];
  } else {
    float tot = 0.f;
    for (int hh = 0; hh < d.H; ++hh) tot += ss[m * d.H + hh];
    val = ol[m * hid + c] * rmsw[c] * rsqrtf(tot / hid + eps);
  }
  ap[gid] = g * val;
  if (gates_dbg) gates_dbg[gid] = g;
}

// --- output projections + residual: one thread per (token, feature).
__global__ __launch_bounds__(256) void k_out_f32(Dims d, const float* __restrict__ x, const float* __restrict__ ap,
                                                 const float* __restrict__ wos, const float* __restrict__ wol,
                                                 float* __restrict__ y, float* __restrict__ delta_dbg) {
  const int hid = d.hid;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.N * hid) return;
  const int n = (int)(gid % hid);
  const long long m = gid / hid;
  const float* a = ap + m * 2 * hid;
  float acc = 0.f;
  for (int kk = 0; kk < hid; ++kk) acc += a[kk] * wos[(long long)kk * hid + n];
  for (int kk = 0; kk < hid; ++kk) acc += a[hid + kk] * wol[(long long)kk * hid + n];
  if (delta_dbg) delta_dbg[gid] = acc;
  y[gid] = x[gid] + acc;
}

#define HYB_LAUNCH(kern, grid, block, ...)                              \
  do {                                                                  \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, s, __VA_ARGS__); \
    hipError_t e_ = hipGetLastError();                                  \
    if (e_ != hipSuccess) return e_;                                    \
  } while (0)

template <int D>
static hipError_t run_f32_d(const Dims& d, const F32Args& a, hipStream_t s) {
  const long long tiles = (d.n + 63) / 64;
  HYB_LAUNCH(k_softmax_f32<D>, (unsigned)(d.B * d.H * d.T * tiles), 64, d, a.q, a.k, a.v, a.tk, a.tv,
             a.scale_log2, a.os);
  HYB_LAUNCH(k_states_f32<D>, (unsigned)(d.B * d.H * (d.T + 1) * D), 256, d, a.k, a.v, a.tk, a.tv, a.states);
  const long long ne = (long long)d.B * d.H * D * (D + 1);
  HYB_LAUNCH(k_combine_f32, (unsigned)((ne + 255) / 256), 256, d, a.states, a.comb);
  const long long nr = (long long)d.B * d.N * d.H;
  HYB_LAUNCH(k_readout_f32<D>, (unsigned)((nr + 63) / 64), 64, d, a.q, a.comb, a.eps, a.ol, a.ss);
  const long long ng = (long long)d.B * d.N * 2 * d.hid;
  HYB_LAUNCH(k_gate_f32, (unsigned)((ng + 255) / 256), 256, d, a.x, a.wgs, a.wgl, a.os, a.ol, a.ss, a.rmsw,
             a.eps, a.ap, a.gates_dbg);
  const long long no = (long long)d.B * d.N * d.hid;
  HYB_LAUNCH(k_out_f32, (unsigned)((no + 255) / 256), 256, d, a.x, a.ap, a.wos, a.wol, a.y, a.delta_dbg);
  return hipSuccess;
}

hipError_t run_f32(const Dims& d, const F32Args& a, hipStream_t s) {
  switch (d.D) {
    case 32: return run_f32_d<32>(d, a, s);
    case 64: return run_f32_d<64>(d, a, s);
    case 128: return run_f32_d<128>(d, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hyb
