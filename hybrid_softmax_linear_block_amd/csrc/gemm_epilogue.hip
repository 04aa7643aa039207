// Gated fusion of the two branches into the residual stream, as two MFMA
// GEMMs with fused epilogues.
//
// VDN-H3 article (tahou.com), section "自适应门控融合双分支输出": the two branch
// outputs differ in scale, so each gets its own content-dependent sigmoid gate
// and its own output projection, and the result is added to the residual
// stream; the linear branch is RMS-normalised before its element-wise gate.
//   gate GEMM:   G = sigmoid(x [W_gs | W_gl])             (bf16 operands, exact inputs)
//                A' = [G_s * O_s | G_l * (O_l * w / sqrt(mean(O_l^2) + eps))]
//   output GEMM: y = x + A' [W_os ; W_ol]                 (fp16 operands)
// A' is a computed intermediate, so it is rounded once, to fp16 (11-bit
// significand, 8x finer than bf16); W_os / W_ol convert to fp16 exactly
// within its range.  Values beyond +-65504 saturate.
// Both GEMMs compute C^T = W^T X^T so that a lane owns one token (the RMS
// factor is a per-lane scalar) and four consecutive features (vector stores).
#include "kernels_bf16.h"

namespace hyb {

enum { EPI_GATE = 0, EPI_OUT = 1 };

struct GemmArgs {
  const uint16_t* A;   // [M][K] token rows (bf16 or fp16 bits)
  const uint16_t* Bt;  // [N][K] feature rows (weights transposed, same type)
  long long M;
  int N, K;
  int hid, H;
  float eps;
  // gate epilogue
  const float *os, *ol, *ss;
  const bf16_t* rmsw;
  uint16_t* ap;
  float* gates_dbg;
  // output epilogue
  const bf16_t* x;
  bf16_t* y;
  float* delta_dbg;
};

typedef __attribute__((address_space(3))) void lds_void_g;

// WG = 4 waves in a 2 (tokens) x 2 (features) grid; each wave computes
// WTM x WFN blocks of 32 x 32.  BK-deep k-tiles live in a 3-stage LDS ring
// filled by wave-wide direct-to-LDS loads (1 KB per wave instruction, 16-byte
// granules XOR-swizzled by row); loads for k-tile t + 2 are in flight while
// k-tile t is multiplied.  Each stage is its own LDS object and the loop is
// unrolled by three, so the compiler sees that the loads in flight never
// alias the tile being read and does not wait for them.
template <int WTM, int WFN, int BK, int WPE, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WPE, WPE)))
void k_gemm_bf16(GemmArgs g) {
  constexpr int BM = 2 * WTM * 32, BN = 2 * WFN * 32;
  constexpr int G = BK / 8, RPC = 64 / G;           // granules per row, rows per 1 KB chunk
  constexpr int CA = BM / RPC / 4, CB = BN / RPC / 4;  // chunks per wave
  constexpr int LPT = CA + CB;                       // loads per k-tile per wave
  static_assert(CA >= 1 && CB >= 1 && (BM / RPC) % 4 == 0 && (BN / RPC) % 4 == 0, "tile/chunk mismatch");
  static_assert(LPT < 64, "vmcnt range");
  using SW = Swz<BK>;
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As2[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs2[BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int ntn = g.N / BN;
  const unsigned wid = xcd_remap(blockIdx.x, gridDim.x);
  const long long m0 = (long long)(wid / ntn) * BM;
  const int n0 = (int)(wid % ntn) * BN;

  floatx16 acc[WFN][WTM];
#pragma unroll
  for (int i = 0; i < WFN; ++i)
#pragma unroll
    for (int j = 0; j < WTM; ++j) acc[i][j] = zero16();

  // per-lane source pointers of the first k-tile; later tiles add k0 elements
  const uint16_t* asrc[CA];
  const uint16_t* bsrc[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int row = (wave * CA + i) * RPC + lane / G;
    long long m = m0 + row;
    if (m >= g.M) m = g.M - 1;  // rows past the end repeat the last row; never stored
    asrc[i] = g.A + m * g.K + ((lane % G) ^ SW::key(row)) * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int row = (wave * CB + i) * RPC + lane / G;
    bsrc[i] = g.Bt + (long long)(n0 + row) * g.K + ((lane % G) ^ SW::key(row)) * 8;
  }
  auto issue = [&](int kt, uint16_t* adst, uint16_t* bdst) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < CA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + k0),
                                       (lds_void_g*)(adst + (wave * CA + i) * RPC * BK), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < CB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + k0),
                                       (lds_void_g*)(bdst + (wave * CB + i) * RPC * BK), 16, 0, 0);
  };
  // (separate LDS objects per stage let the compiler keep these loads in
  // flight across the LDS reads of other stages)
  auto mma = [&](const uint16_t* at, const uint16_t* bt_) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      uint4 bt[WTM];
#pragma unroll
      for (int tb = 0; tb < WTM; ++tb)
        bt[tb] = *(const uint4*)&at[SW::off(wm * WTM * 32 + tb * 32 + l32, 16 * ks + 8 * half)];
#pragma unroll
      for (int fb = 0; fb < WFN; ++fb) {
        const uint4 a = *(const uint4*)&bt_[SW::off(wn * WFN * 32 + fb * 32 + l32, 16 * ks + 8 * half)];
#pragma unroll
        for (int tb = 0; tb < WTM; ++tb) {
          if constexpr (EPI == EPI_GATE)
            acc[fb][tb] = mfma32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bt[tb]), acc[fb][tb]);
          else
            acc[fb][tb] = mfma32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, bt[tb]), acc[fb][tb]);
        }
      }
    }
  };

  const int nk = g.K / BK;
  // step kt: multiply the tile in (ac, bc) while k-tile kt+2 loads into (an, bn)
  auto step = [&](int kt, const uint16_t* ac, const uint16_t* bc, uint16_t* an, uint16_t* bn) {
    const bool more = kt + 2 < nk;
    if (more) issue(kt + 2, an, bn);
    mma(ac, bc);
    if (more) wait_vmcnt<LPT>();  // k-tile kt+1 landed; kt+2 may stay in flight
    else wait_vmcnt<0>();
    tile_barrier();
  };
  issue(0, As0, Bs0);
  if (nk > 1) issue(1, As1, Bs1);
  if (nk > 1) wait_vmcnt<LPT>();
  else wait_vmcnt<0>();
  tile_barrier();
  for (int kt = 0; kt < nk; kt += 3) {
    step(kt, As0, Bs0, As2, Bs2);
    if (kt + 1 < nk) step(kt + 1, As1, Bs1, As0, Bs0);
    if (kt + 2 < nk) step(kt + 2, As2, Bs2, As1, Bs1);
  }

  // ---- epilogue: lane owns token m, features n0' + 8*jg + 4*half + 0..3
#pragma unroll
  for (int tb = 0; tb < WTM; ++tb) {
    const long long m = m0 + wm * WTM * 32 + tb * 32 + l32;
    if (m >= g.M) continue;
    float rinv = 0.f;
    if constexpr (EPI == EPI_GATE) {
      float tot = 0.f;
      for (int hh = 0; hh < g.H; ++hh) tot += g.ss[m * g.H + hh];
      rinv = rsqrtf(tot / (float)g.hid + g.eps);
    }
#pragma unroll
    for (int fb = 0; fb < WFN; ++fb)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int n = n0 + wn * WFN * 32 + fb * 32 + 8 * jg + 4 * half;
        const float c0 = acc[fb][tb][4 * jg], c1 = acc[fb][tb][4 * jg + 1];
        const float c2 = acc[fb][tb][4 * jg + 2], c3 = acc[fb][tb][4 * jg + 3];
        if constexpr (EPI == EPI_GATE) {
          const float g0 = sigmoid_f(c0), g1 = sigmoid_f(c1), g2 = sigmoid_f(c2), g3 = sigmoid_f(c3);
          float4 val;
          if (n < g.hid) {
            val = *(const float4*)(g.os + m * g.hid + n);
          } else {
            const int c = n - g.hid;
            const float4 o = *(const float4*)(g.ol + m * g.hid + c);
            const uint2 wv = *(const uint2*)(g.rmsw + c);
            val.x = o.x * __uint_as_float(wv.x << 16) * rinv;
            val.y = o.y * __uint_as_float(wv.x & 0xffff0000u) * rinv;
            val.z = o.z * __uint_as_float(wv.y << 16) * rinv;
            val.w = o.w * __uint_as_float(wv.y & 0xffff0000u) * rinv;
          }
          uint2 st;
          st.x = pack_f16x2(g0 * val.x, g1 * val.y);
          st.y = pack_f16x2(g2 * val.z, g3 * val.w);
          *(uint2*)(g.ap + m * (2LL * g.hid) + n) = st;
          if (g.gates_dbg) *(float4*)(g.gates_dbg + m * (2LL * g.hid) + n) = make_float4(g0, g1, g2, g3);
        } else {
          const uint2 xv = *(const uint2*)(g.x + m * g.hid + n);
          uint2 st;
          st.x = pack_bf16x2(__uint_as_float(xv.x << 16) + c0, __uint_as_float(xv.x & 0xffff0000u) + c1);
          st.y = pack_bf16x2(__uint_as_float(xv.y << 16) + c2, __uint_as_float(xv.y & 0xffff0000u) + c3);
          *(uint2*)(g.y + m * g.hid + n) = st;
          if (g.delta_dbg) *(float4*)(g.delta_dbg + m * g.hid + n) = make_float4(c0, c1, c2, c3);
        }
      }
  }
}

// Weight transposes into the GEMMs' [N][K] operand layout.
//   mode 0: out[2*hid][hid] bf16,  out[c][r] = c < hid ? W_gs[r][c] : W_gl[r][c - hid]
//   mode 1: out[hid][2*hid] fp16,  out[c][r] = r < hid ? W_os[r][c] : W_ol[r - hid][c]
__global__ __launch_bounds__(256) void k_weight_transpose(const bf16_t* __restrict__ s0,
                                                          const bf16_t* __restrict__ s1, int hid, int mode,
                                                          uint16_t* __restrict__ out) {
  __shared__ uint16_t t[64][66];
  const int R = mode == 0 ? hid : 2 * hid;  // source rows
  const int C = mode == 0 ? 2 * hid : hid;  // source cols
  const int tc = blockIdx.x % (C / 64), tr = blockIdx.x / (C / 64);
  const int r0 = tr * 64, c0 = tc * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    const int r = r0 + rr, c = c0 + cc;
    bf16_t val;
    if (mode == 0) val = c < hid ? s0[(long long)r * hid + c] : s1[(long long)r * hid + c - hid];
    else val = r < hid ? s0[(long long)r * hid + c] : s1[(long long)(r - hid) * hid + c];
    t[rr][cc] = mode == 0 ? val : f32_to_f16_sat(bf16_to_f32(val));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    out[(long long)(c0 + cc) * R + r0 + rr] = t[rr][cc];
  }
}

hipError_t launch_weights_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const int hid = d.hid;
  const unsigned grid = (unsigned)((hid / 64) * (2 * hid / 64));
  hipLaunchKernelGGL(k_weight_transpose, dim3(grid), dim3(256), 0, s, a.wgs, a.wgl, hid, 0, (uint16_t*)a.wg_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_weight_transpose, dim3(grid), dim3(256), 0, s, a.wos, a.wol, hid, 1, a.wo_t);
  return hipGetLastError();
}

template <int WTM, int WFN, int BK, int WPE, int EPI>
static hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  constexpr int BM = 2 * WTM * 32, BN = 2 * WFN * 32;
  if (g.N % BN != 0 || g.K % BK != 0) return hipErrorInvalidValue;
  const long long grid = ((g.M + BM - 1) / BM) * (g.N / BN);
  hipLaunchKernelGGL((k_gemm_bf16<WTM, WFN, BK, WPE, EPI>), dim3((unsigned)grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

static GemmArgs base_args(const Dims& d, const Bf16Args& a) {
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
  g.eps = a.eps;
  return g;
}

hipError_t launch_gate_gemm_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  GemmArgs g = base_args(d, a);
  g.A = a.x;
  g.Bt = a.wg_t;
  g.N = 2 * d.hid;
  g.K = d.hid;
  g.os = a.os;
  g.ol = a.ol;
  g.ss = a.ss;
  g.rmsw = a.rmsw;
  g.ap = a.ap;
  g.gates_dbg = a.gates_dbg;
  if (g.N % 128 == 0) return launch_gemm<4, 2, 32, 2, EPI_GATE>(g, s);
  return launch_gemm<4, 1, 32, 2, EPI_GATE>(g, s);  // hid multiple of 64 only
}

hipError_t launch_out_gemm_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  GemmArgs g = base_args(d, a);
  g.A = a.ap;
  g.Bt = a.wo_t;
  g.N = d.hid;
  g.K = 2 * d.hid;
  g.x = a.x;
  g.y = a.y;
  g.delta_dbg = a.delta_dbg;
  if (g.N % 128 == 0) return launch_gemm<4, 2, 32, 2, EPI_OUT>(g, s);
  return launch_gemm<4, 1, 32, 2, EPI_OUT>(g, s);
}

}  // namespace hyb
