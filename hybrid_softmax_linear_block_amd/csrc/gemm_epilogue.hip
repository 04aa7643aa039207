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
#include <type_traits>

#include "kernels_bf16.h"
#include "mx_common.h"

namespace hyb {

enum { EPI_GATE = 0, EPI_OUT = 1, EPI_QKV = 2, EPI_DA = 3, EPI_RES = 4, EPI_WGRAD = 5, EPI_GELU = 6 };

struct GemmArgs {
  const uint16_t* A;   // [M][ldk] token rows (bf16 or fp16 bits)
  const uint16_t* Bt;  // [N][ldk] feature rows (weights transposed, same type)
  long long M;
  int N, K;            // K: contraction length of one split
  int ldk;             // row stride of A and Bt in elements (0: K)
  int ksplit;          // contraction splits (EPI_WGRAD; 1 otherwise): split z covers [z K, (z+1) K)
  int hid, H;
  // gate epilogue
  const uint16_t *os, *ol;  // fp16 branch outputs [M][hid]
  const float* rinv;
  const bf16_t* rmsw;
  uint16_t* ap;
  float* gates_dbg;
  uint16_t* gates16;  // nullable: [M][2 hid] fp16 copy of the gates (saved for the backward pass)
  // output epilogue
  const bf16_t* x;
  bf16_t* y;
  float* delta_dbg;
  // projection epilogue: q, k, v [M][hid] and absmax [3][B][H] (nullable)
  bf16_t *qo, *ko, *vo;
  uint32_t* absmax;
  int B, n_video, D;
  // backward of the output GEMM (EPI_DA): dA' = dy [W_os; W_ol]^T, then
  //   c <  hid: dO_s = dA'_s G_s,            dZ_s = dA'_s O_s G_s (1 - G_s)
  //   c >= hid: dR   = dA'_l G_l,            dZ_l = dA'_l R G_l (1 - G_l),  R = O_l w rinv
  const uint16_t* gsv;  // [M][2 hid] fp16 saved gates
  bf16_t *dos, *dz, *dr;  // [M][hid], [M][2 hid], [M][hid] bf16
  // weight gradients (EPI_WGRAD): fp32 partial sums [ksplit][M][N]
  float* part;
  // feed-forward (EPI_GELU): out[M][N] = bf16(GELU_tanh(acc))
  bf16_t* out;
  // MX operands (MX = true): A and Bt hold e4m3 codes ([M][ldk], [N][ldk]
  // bytes); sa [K/128][mpad][4] and sb [K/128][N][4] hold one E8M0 exponent
  // per 32 contraction elements of each row (mpad: M rounded up to 256)
  const uint8_t *sa, *sb;
  long long mpad;
  // gate epilogue with MX output: A' codes [M][2 hid] and exponents [2 hid / 128][mpad][4]
  uint8_t *ap8, *aps;
};

// GELU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))), with
// tanh(a) = 1 - 2 / (exp(2a) + 1) (saturates correctly for large |a|).
__device__ __forceinline__ float gelu_tanh_f(float u) {
  const float a = 0.7978845608028654f * fmaf(0.044715f * u, u * u, u);
  const float t = 1.f - 2.f / (__expf(2.f * a) + 1.f);
  return 0.5f * u * (1.f + t);
}

// Row-layout epilogue of the gate GEMM (EPI_GATE, bf16 operands) and of the
// output / residual GEMMs (EPI_OUT, EPI_RES).  In the MFMA layout a lane owns
// one token and 16 features in four 16-byte pieces, so every global access
// of the epilogue would touch 32 rows (32 cache lines, 16 bytes of each).
// Instead each wave passes its accumulators (gates for EPI_GATE) through a
// private LDS region, one group of 32 tokens at a time, and reads them back
// so that 32 lanes cover one token's 128 features: every global load and
// store then covers two whole rows of 256 bytes.  All loads of a group are
// issued before its stores.  Region: 32 rows of 128
// floats plus 4 of padding (conflict-free writes of 16 lanes at one column
// and reads of 16 lanes along one row).  The operand stages are free here:
// the main loop ended on a barrier after every wave's last LDS read.
constexpr int EPI_ROW = 132;                       // floats per LDS row
constexpr int EPI_WAVE_BYTES = 32 * EPI_ROW * 4;  // LDS bytes per wave (32-row groups)

// RG: rows per pass through the LDS region (32, or 16 in half the LDS: each
// 32-token block then takes two passes, lanes 0-15 / 16-31 of a half-wave
// writing their tokens in turn).
template <int WTM, int WFN, int EPI, int RG = 32>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& g, floatx16 (&acc)[WFN][WTM], long long mw, int nwave,
                                              int lane, float* ldsw) {
  static_assert(WFN == 4, "row epilogue: 128 features per wave");
  static_assert(RG == 16 || RG == 32, "rows per pass");
  constexpr int NP = 32 / RG, KR = RG / 2;  // passes per 32-token block, row pairs per pass
  const int l32 = lane & 31, half = lane >> 5;
  const int lc = l32, lr = half;  // row layout: features 4 lc .. 4 lc + 3 of row 2 k + lr
  const bool lin = EPI == EPI_GATE && nwave >= g.hid;  // a wave's features are all in one half (hid % BN == 0)
  // Source rows (branch output or residual) and destination rows: a
  // wave-uniform row base (mw + 2 k + 32 i) plus a fixed 32-bit lane offset
  const uint16_t* src;
  long long lds_, ldd;  // row strides of source and destination (elements)
  int scol;             // this lane's first source column
  if constexpr (EPI == EPI_GATE) {
    src = lin ? g.ol : g.os;
    lds_ = g.hid;
    ldd = 2LL * g.hid;
    scol = (lin ? nwave - g.hid : nwave) + 4 * lc;
  } else {
    src = (const uint16_t*)g.x;
    lds_ = ldd = g.N;
    scol = nwave + 4 * lc;
  }
  const int dcol = nwave + 4 * lc;
  const unsigned soff = (unsigned)((lr * lds_ + scol) * 2), doff = (unsigned)((lr * ldd + dcol) * 2);
  float4 wf = make_float4(0.f, 0.f, 0.f, 0.f);
  float rv = 0.f;
  if (lin) {
    const uint2 w = *(const uint2*)(g.rmsw + scol);
    wf = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u));
    rv = g.rinv[min(mw + lane, g.M - 1)];  // token mw + lane; row r's factor sits in lane r
  }
  // FULL: every row of the wave is below M (all tiles but the last row of
  // tiles); otherwise rows past M load row M - 1 and are not stored.
  auto run = [&](auto full_c, auto extra_c) {
    constexpr bool FULL = decltype(full_c)::value, EXTRA = decltype(extra_c)::value;
    auto saddr = [&](int i, int k) -> const char* {
      if constexpr (FULL) return (const char*)src + (mw + 32 * i + 2 * k) * lds_ * 2 + soff;
      else return (const char*)src + (min(mw + 32 * i + 2 * k + lr, g.M - 1) * lds_ + scol) * 2;
    };
    uint2 in[WTM][16];
    auto load_in = [&](int i) {
#pragma unroll
      for (int k = 0; k < 16; ++k) in[i][k] = *(const uint2*)saddr(i, k);
    };
    load_in(0);
#pragma unroll
    for (int ip = 0; ip < WTM * NP; ++ip) {
      const int i = ip / NP, pp = ip % NP;  // token block, pass
      // MFMA layout -> LDS: token l32 (those of this pass), features 32 f + 8 jg + 4 half
      if (NP == 1 || l32 / RG == pp) {
#pragma unroll
        for (int f = 0; f < WFN; ++f)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            float4 v = make_float4(acc[f][i][4 * jg], acc[f][i][4 * jg + 1], acc[f][i][4 * jg + 2], acc[f][i][4 * jg + 3]);
            if constexpr (EPI == EPI_GATE) v = make_float4(sigmoid_rcp(v.x), sigmoid_rcp(v.y), sigmoid_rcp(v.z), sigmoid_rcp(v.w));
            *(float4*)&ldsw[(l32 % RG) * EPI_ROW + 32 * f + 8 * jg + 4 * half] = v;
          }
      }
      if (pp == 0 && i + 1 < WTM) load_in(i + 1);
      // LDS -> row layout.  A wave's LDS operations execute in issue order, so
      // these reads see the writes above and the next pass's writes follow
      // them; the empty asm keeps the compiler from reordering across lanes.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int kr = 0; kr < KR; ++kr) {
        const int k = pp * KR + kr;  // row pair inside the block: rows 2 k + lr
        const int r = 2 * k + lr;
        const float4 a = *(const float4*)&ldsw[(2 * kr + lr) * EPI_ROW + 4 * lc];
        float rk = 0.f;
        if (lin) rk = __shfl(rv, 32 * i + r);
        const long long m = mw + 32 * i + r;
        if constexpr (!FULL) {
          if (m >= g.M) continue;
        }
        char* drow = nullptr;
        if constexpr (EPI == EPI_GATE) drow = (char*)g.ap;
        else drow = (char*)g.y;
        drow += (mw + 32 * i + 2 * k) * ldd * 2 + doff;
        if constexpr (EPI == EPI_GATE) {
          // fp16 operands enter the products directly (fma with a zero addend:
          // one rounding, as product of the widened value)
          typedef __attribute__((ext_vector_type(2))) _Float16 h2_t;
          const h2_t o01 = __builtin_bit_cast(h2_t, in[i][k].x), o23 = __builtin_bit_cast(h2_t, in[i][k].y);
          if (lin) {  // A'_l = G_l RMSNorm(O_l), RMSNorm(O_l) = O_l w / rms; saturated to fp16
            const float v0 = __builtin_fmaf((float)o01[0], wf.x, 0.f) * rk, v1 = __builtin_fmaf((float)o01[1], wf.y, 0.f) * rk;
            const float v2 = __builtin_fmaf((float)o23[0], wf.z, 0.f) * rk, v3 = __builtin_fmaf((float)o23[1], wf.w, 0.f) * rk;
            *(uint2*)drow = make_uint2(pack_f16x2(a.x * v0, a.y * v1), pack_f16x2(a.z * v2, a.w * v3));
          } else {  // A'_s = G_s O_s: |G_s O_s| <= |O_s|, inside fp16's range
            *(uint2*)drow = make_uint2(pack_f16x2_unsat(__builtin_fmaf((float)o01[0], a.x, 0.f), __builtin_fmaf((float)o01[1], a.y, 0.f)),
                                       pack_f16x2_unsat(__builtin_fmaf((float)o23[0], a.z, 0.f), __builtin_fmaf((float)o23[1], a.w, 0.f)));
          }
          if constexpr (EXTRA) {
            const long long n = m * ldd + dcol;
            if (g.gates_dbg) *(float4*)(g.gates_dbg + n) = a;
            if (g.gates16) store_f16x4(g.gates16 + n, a.x, a.y, a.z, a.w);
          }
        } else {
          const uint2 x = in[i][k];
          *(uint2*)drow = make_uint2(pack_bf16x2(__uint_as_float(x.x << 16) + a.x, __uint_as_float(x.x & 0xffff0000u) + a.y),
                                     pack_bf16x2(__uint_as_float(x.y << 16) + a.z, __uint_as_float(x.y & 0xffff0000u) + a.w));
          if constexpr (EXTRA) *(float4*)(g.delta_dbg + m * ldd + dcol) = a;
        }
      }
      asm volatile("" ::: "memory");
    }
  };
  const bool full = mw + 32 * WTM <= g.M;
  const bool extra = EPI == EPI_GATE ? (g.gates_dbg || g.gates16) : g.delta_dbg != nullptr;
  if (full && !extra) run(std::true_type{}, std::false_type{});
  else if (full) run(std::true_type{}, std::true_type{});
  else if (!extra) run(std::false_type{}, std::false_type{});
  else run(std::false_type{}, std::true_type{});
}

// Epilogue of the gate GEMM (EPI_GATE) and of the output / residual GEMMs
// (EPI_OUT, EPI_RES).  Lane owns tokens mb + 32 i (i < WTM) and features
// nw + 32 f + 8 jg + 0..3 (f < WFN, jg < 4); nwave is the wave's first
// feature (wave-uniform).  Every global load of the tile (branch outputs or
// residual rows, RMS weights and factors) is issued before the first store,
// so the epilogue costs one memory round trip (the MX gate, short of
// registers, does so per token group i); rows past M load the last row and
// are not stored.
template <int WTM, int WFN, int EPI, bool MX>
__device__ __forceinline__ void epilogue_gate_out(const GemmArgs& g, floatx16 (&acc)[WFN][WTM], long long mb, int nwave,
                                                  int half) {
  const int nw = nwave + 4 * half;
  long long mc[WTM];
#pragma unroll
  for (int i = 0; i < WTM; ++i) mc[i] = min(mb + 32 * i, g.M - 1);
  if constexpr (EPI == EPI_GATE) {
    const bool lin = nwave >= g.hid;  // a wave's features are all in one half (hid % BN == 0)
    const uint16_t* src = lin ? g.ol : g.os;
    const int cw = (lin ? nwave - g.hid : nwave) + 4 * half;  // this lane's first column in [0, hid)
    uint2 ov[WTM][WFN][4];  // fp16 branch outputs
    uint2 wv[WFN][4];       // bf16 RMS weights (linear half)
    float rinv[WTM];
    auto load_w = [&]() {
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) wv[f][jg] = *(const uint2*)(g.rmsw + cw + 32 * f + 8 * jg);
    };
    auto load_i = [&](int i) {
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) ov[i][f][jg] = *(const uint2*)(src + mc[i] * g.hid + cw + 32 * f + 8 * jg);
      if (lin) {
        rinv[i] = g.rinv[mc[i]];
        if constexpr (MX) load_w();
      }
    };
    if constexpr (!MX) {
      if (lin) load_w();
#pragma unroll
      for (int i = 0; i < WTM; ++i) load_i(i);
    }
    // the debug / saved-gate stores only in a separate copy of the loop (the
    // MX gate keeps one copy: two spill its registers)
    auto gate_out = [&](auto extra_c) {
      constexpr bool EXTRA = decltype(extra_c)::value;
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        if constexpr (MX) load_i(i);
        const long long m = mb + 32 * i;
        if (m >= g.M) continue;
#pragma unroll
        for (int f = 0; f < WFN; ++f) {
          float4 av[4];
          float amax = 0.f;
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int n = nw + 32 * f + 8 * jg;
            float4 o = unpack_f16x4(ov[i][f][jg]);
            if (lin) {  // RMSNorm(O_l) = O_l w / rms
              const uint2 w = wv[f][jg];
              o.x = o.x * __uint_as_float(w.x << 16) * rinv[i];
              o.y = o.y * __uint_as_float(w.x & 0xffff0000u) * rinv[i];
              o.z = o.z * __uint_as_float(w.y << 16) * rinv[i];
              o.w = o.w * __uint_as_float(w.y & 0xffff0000u) * rinv[i];
            }
            const float g0 = sigmoid_rcp(acc[f][i][4 * jg]), g1 = sigmoid_rcp(acc[f][i][4 * jg + 1]);
            const float g2 = sigmoid_rcp(acc[f][i][4 * jg + 2]), g3 = sigmoid_rcp(acc[f][i][4 * jg + 3]);
            av[jg] = make_float4(g0 * o.x, g1 * o.y, g2 * o.z, g3 * o.w);
            if constexpr (MX) {
              amax = fmaxf(amax, fmaxf(fmaxf(fabsf(av[jg].x), fabsf(av[jg].y)), fmaxf(fabsf(av[jg].z), fabsf(av[jg].w))));
            } else {
              *(uint2*)(g.ap + m * (2LL * g.hid) + n) = make_uint2(pack_f16x2(av[jg].x, av[jg].y),
                                                                   pack_f16x2(av[jg].z, av[jg].w));
            }
            if constexpr (EXTRA) {
              if (g.gates_dbg) *(float4*)(g.gates_dbg + m * (2LL * g.hid) + n) = make_float4(g0, g1, g2, g3);
              if (g.gates16) store_f16x4(g.gates16 + m * (2LL * g.hid) + n, g0, g1, g2, g3);
            }
          }
          if constexpr (MX) {
            // A' as MX e4m3: the 32 features of block f of this token sit in
            // lanes l and l ^ 32 (4 groups of 4 each)
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int se = mx_exponent(amax);
            const float inv = mx_inverse_scale(se);
            const int nb = nwave + 32 * f;  // first feature of the block
            uint8_t* cp = g.ap8 + m * (2LL * g.hid) + nw + 32 * f;
#pragma unroll
            for (int jg = 0; jg < 4; ++jg)
              *(uint32_t*)(cp + 8 * jg) = e4m3x4(av[jg].x * inv, av[jg].y * inv, av[jg].z * inv, av[jg].w * inv);
            if (half == 0) g.aps[((long long)(nb >> 7) * g.mpad + m) * 4 + ((nb >> 5) & 3)] = (uint8_t)(se + 127);
          }
        }
      }
    };
    if (MX || g.gates_dbg || g.gates16) gate_out(std::true_type{});
    else if constexpr (!MX) gate_out(std::false_type{});
  } else {
    // y = x + acc (bf16), x the residual rows
    uint2 xv[WTM][WFN][4];
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) xv[i][f][jg] = *(const uint2*)(g.x + mc[i] * g.N + nw + 32 * f + 8 * jg);
    auto out = [&](auto dbg_c) {
      constexpr bool DBG = decltype(dbg_c)::value;
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const long long m = mb + 32 * i;
        if (m >= g.M) continue;
#pragma unroll
        for (int f = 0; f < WFN; ++f)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int n = nw + 32 * f + 8 * jg;
            const float c0 = acc[f][i][4 * jg], c1 = acc[f][i][4 * jg + 1];
            const float c2 = acc[f][i][4 * jg + 2], c3 = acc[f][i][4 * jg + 3];
            const uint2 x = xv[i][f][jg];
            *(uint2*)(g.y + m * g.N + n) =
                make_uint2(pack_bf16x2(__uint_as_float(x.x << 16) + c0, __uint_as_float(x.x & 0xffff0000u) + c1),
                           pack_bf16x2(__uint_as_float(x.y << 16) + c2, __uint_as_float(x.y & 0xffff0000u) + c3));
            if constexpr (DBG) *(float4*)(g.delta_dbg + m * g.N + n) = make_float4(c0, c1, c2, c3);
          }
      }
    };
    if (g.delta_dbg) out(std::true_type{});
    else out(std::false_type{});
  }
}

// WG = WM x WN waves; each wave computes WTM x WFN blocks of 32 x 32 (tokens x
// features).  BK-deep k-tiles live in an ST-stage LDS ring filled by
// wave-wide direct-to-LDS loads (1 KB per wave instruction, 16-byte granules
// XOR-swizzled by row); loads for k-tile t + ST - 1 are in flight while
// k-tile t is multiplied.  The k loop is unrolled by ST so that every LDS
// address is a per-lane base plus an immediate, and the DMA source is a
// scalar base (bumped per k-tile) plus a fixed per-lane offset.
//
// MX = true: e4m3 operands with E8M0 block exponents (OCP microscaling), on
// the 32x32x64 scaled f8f6f4 MFMA, which applies both operands' exponents in
// hardware.  A k-tile then holds 2 BK fp8 elements in the same 2 BK-byte rows,
// and one more 1 KB chunk per k-tile and operand carries the exponents of
// its rows (4 bytes per row: the tile's four 32-element blocks), loaded by
// 16 lanes of every wave.
template <int WM, int WN, int WTM, int WFN, int BK, int ST, int WPE, int EPI, int GM = 1, bool MX = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WM * WN, 64 * WM * WN),
                          amdgpu_waves_per_eu(WPE, WPE)))
void k_gemm_bf16(GemmArgs g) {
  constexpr int NWV = WM * WN;
  constexpr int BM = WM * WTM * 32, BN = WN * WFN * 32;
  constexpr int ESZ = MX ? 1 : 2;                           // operand element bytes
  constexpr int KT = MX ? 2 * BK : BK;                      // contraction elements per k-tile
  constexpr int G = BK / 8, RPC = 64 / G;                   // granules per row, rows per 1 KB chunk
  constexpr int CA = BM / RPC / NWV, CB = BN / RPC / NWV;   // chunks per wave
  constexpr int LPT = CA + CB + (MX ? 1 : 0);               // loads per k-tile per wave
  static_assert(CA >= 1 && CB >= 1 && (BM / RPC) % NWV == 0 && (BN / RPC) % NWV == 0, "tile/chunk mismatch");
  static_assert(LPT * ST < 64, "vmcnt range");
  static_assert(!MX || (BM == 256 && BN == 256 && NWV == 8 && BK == 64), "MX tiles: 256 x 256, 8 waves, 128-deep");
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int XBYTES = MX ? (BM + BN) * 4 : 0;            // block exponents of the k-tile's rows
  constexpr int SBYTES = ABYTES + BBYTES + XBYTES;
  using SW = Swz<BK>;
  // the row epilogue reuses the operand stages as 8 wave regions
  constexpr bool ROWEPI = (EPI == EPI_GATE && !MX) || EPI == EPI_OUT || EPI == EPI_RES;
  constexpr bool USE_ROWEPI = ROWEPI && NWV == 8 && WTM == 2 && WFN == 4;
  constexpr int LDSB = USE_ROWEPI && 8 * EPI_WAVE_BYTES > ST * SBYTES ? 8 * EPI_WAVE_BYTES : ST * SBYTES;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDSB / 2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = wave % WM, wn = wave / WM;
  const int ntn = g.N / BN;
  // Each XCD takes a contiguous range of tiles (xcd_remap), walked in groups
  // of GM token tiles: the workgroups running together on an XCD share GM
  // rows of A and a run of weight tiles, so both stay in its L2.
  unsigned wid = xcd_remap(blockIdx.x, gridDim.x);
  const unsigned ntm = (unsigned)((g.M + BM - 1) / BM);
  const int ldk = g.ldk;
  unsigned kz = 0;
  if constexpr (EPI == EPI_WGRAD) {
    const unsigned tiles = ntm * (unsigned)ntn;
    kz = wid / tiles;
    wid -= kz * tiles;
  }
  const unsigned per_group = (unsigned)GM * (unsigned)ntn;
  const unsigned grp = wid / per_group, in = wid % per_group;
  const unsigned gm0 = grp * GM, gsz = min((unsigned)GM, ntm - gm0);
  const long long m0 = (long long)(gm0 + in % gsz) * BM;
  const int n0 = (int)(in / gsz) * BN;

  floatx16 acc[WFN][WTM];
#pragma unroll
  for (int i = 0; i < WFN; ++i)
#pragma unroll
    for (int j = 0; j < WTM; ++j) acc[i][j] = zero16();

  // DMA sources: scalar bases at k = 0, per-lane byte offsets (rows past M
  // repeat the last row; never stored)
  const long long mlast = g.M - 1 - m0;
  const char* abase = (const char*)g.A + (m0 * ldk + (long long)kz * g.K) * ESZ;
  const char* bbase = (const char*)g.Bt + ((long long)n0 * ldk + (long long)kz * g.K) * ESZ;
  unsigned aoff[CA], boff[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int row = (wave * CA + i) * RPC + lane / G;
    const long long r = row < mlast ? row : mlast;
    aoff[i] = (unsigned)(r * ldk * ESZ) + ((lane % G) ^ SW::key(row)) * 16;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int row = (wave * CB + i) * RPC + lane / G;
    boff[i] = (unsigned)((long long)row * ldk * ESZ) + ((lane % G) ^ SW::key(row)) * 16;
  }
  // MX: waves 0-3 load the exponents of the tile's 256 A rows, waves 4-7
  // those of its 256 B rows, 256 bytes (16 lanes) each.  The exponent rows of
  // A are padded to mpad, so the chunk of the last token tile is in bounds.
  const uint8_t* xbase = nullptr;
  long long xstride = 0;
  if constexpr (MX) {
    xbase = wave < 4 ? g.sa + (m0 + 64 * wave) * 4 : g.sb + ((long long)n0 + 64 * (wave - 4)) * 4;
    xstride = (wave < 4 ? g.mpad : (long long)g.N) * 4;  // bytes per 128-deep exponent group
  }
  const unsigned lds0 = lds_addr(lds);
  auto issue = [&](int kt, int stage) {
    const char* ab = abase + (long long)kt * BK * 2;
    const char* bb = bbase + (long long)kt * BK * 2;
    const unsigned la = lds0 + stage * SBYTES, lb = la + ABYTES;
#pragma unroll
    for (int i = 0; i < CA; ++i) dma16(ab, aoff[i], la + (wave * CA + i) * 1024);
#pragma unroll
    for (int i = 0; i < CB; ++i) dma16(bb, boff[i], lb + (wave * CB + i) * 1024);
    if constexpr (MX) {
      if (lane < 16) dma16(xbase + (long long)(kz * (g.K / KT) + kt) * xstride, lane * 16, lb + BBYTES + wave * 256);
    }
  };
  // MX: one k-tile, all operand reads first, then the MFMAs
  auto mma = [&](auto stc) {
    constexpr int STG = decltype(stc)::value;
    const uint16_t* at = lds + STG * SBYTES / 2;
    const uint16_t* bt_ = at + ABYTES / 2;
    if constexpr (MX) {
      // k-step ks (64 fp8): lane half h feeds bytes [64 ks + 16 h, +16) and
      // [64 ks + 32 + 16 h, +16) of its row (the MFMA's k order), and the
      // exponent of block 2 ks + h (the scale register of lane half h covers
      // the step's block h)
      const uint32_t* xa = (const uint32_t*)(bt_ + BBYTES / 2);
      const uint32_t* xb = xa + BM;
      i32x8 fa[2][WTM], fb[2][WFN];
      uint32_t ea[WTM], eb[WFN];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
          const int row = wm * WTM * 32 + i * 32 + l32;
          const uint4 u0 = *(const uint4*)&at[SW::off(row, 32 * ks + 8 * half)];
          const uint4 u1 = *(const uint4*)&at[SW::off(row, 32 * ks + 16 + 8 * half)];
          fa[ks][i] = i32x8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        }
#pragma unroll
        for (int f = 0; f < WFN; ++f) {
          const int row = wn * WFN * 32 + f * 32 + l32;
          const uint4 u0 = *(const uint4*)&bt_[SW::off(row, 32 * ks + 8 * half)];
          const uint4 u1 = *(const uint4*)&bt_[SW::off(row, 32 * ks + 16 + 8 * half)];
          fb[ks][f] = i32x8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        }
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i) ea[i] = xa[wm * WTM * 32 + i * 32 + l32] >> (8 * half);
#pragma unroll
      for (int f = 0; f < WFN; ++f) eb[f] = xb[wn * WFN * 32 + f * 32 + l32] >> (8 * half);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int f = 0; f < WFN; ++f)
#pragma unroll
          for (int i = 0; i < WTM; ++i)
            acc[f][i] = mfma32_f8_mx(fb[ks][f], fa[ks][i], acc[f][i], (int)(eb[f] >> (16 * ks)),
                                     (int)(ea[i] >> (16 * ks)));
      return;
    }
  };

  const int nk = g.K / KT;
  // bf16 / fp16 operands: the k-steps of a k-tile read their operands into
  // registers that persist across k-tiles, so that the last k-step's MFMAs
  // run after the barrier, while the first k-step of the next k-tile is read.
  // Each k-step's WTM x WFN MFMAs are interleaved with the memory operations
  // (one DMA chunk and one operand read after each MFMA, round robin): the
  // matrix pipe keeps busy while they issue.
  constexpr int KS = BK / 16, NSL = WTM * WFN, NR = WTM + WFN;
  uint4 ra[KS][WTM], rb[KS][WFN];
  auto rd1 = [&](int stage, auto ksc, int j) {  // operand row block j (A: j < WTM, B: j >= WTM)
    constexpr int ks = decltype(ksc)::value;
    const uint16_t* at = lds + stage * (SBYTES / 2);
    if (j < WTM) ra[ks][j] = *(const uint4*)&at[SW::off(wm * WTM * 32 + j * 32 + l32, 16 * ks + 8 * half)];
    else rb[ks][j - WTM] = *(const uint4*)&at[ABYTES / 2 + SW::off(wn * WFN * 32 + (j - WTM) * 32 + l32, 16 * ks + 8 * half)];
  };
  auto dma1 = [&](int kt2, int stage, int j) {  // 1 KB chunk j of k-tile kt2 (A: j < CA, B: j >= CA)
    const unsigned la = lds0 + stage * SBYTES;
    if (j < CA) dma16(abase + (long long)kt2 * BK * 2, aoff[j], la + (wave * CA + j) * 1024);
    else dma16(bbase + (long long)kt2 * BK * 2, boff[j - CA], la + ABYTES + (wave * CB + j - CA) * 1024);
  };
  // k-step ks: MFMA s (s = f * WTM + i) is followed by ops(s)
  auto phase = [&](auto ksc, auto&& ops) {
    constexpr int ks = decltype(ksc)::value;
#pragma unroll
    for (int f = 0; f < WFN; ++f)
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        if constexpr (EPI == EPI_OUT)  // fp16 operands (A' and W_o)
          acc[f][i] = mfma32_f16(__builtin_bit_cast(halfx8, rb[ks][f]), __builtin_bit_cast(halfx8, ra[ks][i]), acc[f][i]);
        else
          acc[f][i] = mfma32(__builtin_bit_cast(bf16x8, rb[ks][f]), __builtin_bit_cast(bf16x8, ra[ks][i]), acc[f][i]);
        __builtin_amdgcn_sched_barrier(0);
        ops(f * WTM + i);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // k-tile kt in stage STG: issue k-tile kt + ST - 1 into the stage read at
  // kt - 1 (free after the previous barrier), multiply, wait for kt + 1.
  auto step = [&](int kt, auto stc) {
    constexpr int STG = decltype(stc)::value;
    const bool more = kt + ST - 1 < nk;
    if constexpr (MX) {
      if (more) issue(kt + ST - 1, (STG + ST - 1) % ST);
      mma(stc);
    } else {
      // k-steps 0 .. KS-2 before the barrier, reading k-steps 1 .. KS-1
      // (k-step 0 was read after the previous barrier); the DMA of k-tile
      // kt + ST - 1 goes with k-step 0
      static_for<0, KS - 1>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        phase(ksc, [&](int sl) {
          if constexpr (ks == 0) {
#pragma unroll
            for (int j = sl; j < CA + CB; j += NSL)
              if (more) dma1(kt + ST - 1, (STG + ST - 1) % ST, j);
          }
#pragma unroll
          for (int j = sl; j < NR; j += NSL) rd1(STG, std::integral_constant<int, ks + 1>{}, j);
        });
      });
    }
    if (more) wait_vmcnt<(ST - 2) * LPT>();  // k-tile kt+1 landed; later ones may stay in flight
    else wait_vmcnt<0>();
    tile_barrier();  // every wave's reads of this stage are done, k-tile kt+1 is visible
    if constexpr (!MX) {
      const bool nxt = kt + 1 < nk;
      phase(std::integral_constant<int, KS - 1>{}, [&](int sl) {
#pragma unroll
        for (int j = sl; j < NR; j += NSL)
          if (nxt) rd1((STG + 1) % ST, std::integral_constant<int, 0>{}, j);
      });
    }
  };
#pragma unroll
  for (int s0 = 0; s0 < ST - 1; ++s0)
    if (s0 < nk) issue(s0, s0);
  if (nk >= ST - 1) wait_vmcnt<(ST - 2) * LPT>();
  else wait_vmcnt<0>();
  tile_barrier();
  if constexpr (!MX) {
#pragma unroll
    for (int j = 0; j < NR; ++j) rd1(0, std::integral_constant<int, 0>{}, j);
  }
  for (int kt = 0; kt < nk; kt += ST) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1 % ST>{});
    if constexpr (ST > 2)
      if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2 % ST>{});
    if constexpr (ST > 3)
      if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 3 % ST>{});
  }

  if constexpr (EPI == EPI_WGRAD) {
    // fp32 partial of split kz: lane owns row m, columns n .. n+3
    float* outp = g.part + (long long)kz * g.M * g.N;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const long long m = m0 + wm * WTM * 32 + i * 32 + l32;
      if (m >= g.M) continue;
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int n = n0 + wn * WFN * 32 + 32 * f + 8 * jg + 4 * half;
          *(float4*)(outp + m * g.N + n) =
              make_float4(acc[f][i][4 * jg], acc[f][i][4 * jg + 1], acc[f][i][4 * jg + 2], acc[f][i][4 * jg + 3]);
        }
    }
    return;
  }
  if constexpr (EPI == EPI_GELU) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const long long m = m0 + wm * WTM * 32 + i * 32 + l32;
      if (m >= g.M) continue;
#pragma unroll
      for (int f = 0; f < WFN; ++f) {
        if constexpr (MX) {
          // GELU output as MX e4m3 (block f of the token: lanes l and l ^ 32)
          float4 uv[4];
          float amax = 0.f;
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            uv[jg] = make_float4(gelu_tanh_f(acc[f][i][4 * jg]), gelu_tanh_f(acc[f][i][4 * jg + 1]),
                                 gelu_tanh_f(acc[f][i][4 * jg + 2]), gelu_tanh_f(acc[f][i][4 * jg + 3]));
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(uv[jg].x), fabsf(uv[jg].y)), fmaxf(fabsf(uv[jg].z), fabsf(uv[jg].w))));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const int se = mx_exponent(amax);
          const float inv = mx_inverse_scale(se);
          const int nb = n0 + wn * WFN * 32 + 32 * f;  // first feature of the block
          uint8_t* cp = g.ap8 + m * g.N + nb + 4 * half;
#pragma unroll
          for (int jg = 0; jg < 4; ++jg)
            *(uint32_t*)(cp + 8 * jg) = e4m3x4(uv[jg].x * inv, uv[jg].y * inv, uv[jg].z * inv, uv[jg].w * inv);
          if (half == 0) g.aps[((long long)(nb >> 7) * g.mpad + m) * 4 + ((nb >> 5) & 3)] = (uint8_t)(se + 127);
        } else {
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            const int n = n0 + wn * WFN * 32 + 32 * f + 8 * jg + 4 * half;
            *(uint2*)(g.out + m * g.N + n) =
                make_uint2(pack_bf16x2(gelu_tanh_f(acc[f][i][4 * jg]), gelu_tanh_f(acc[f][i][4 * jg + 1])),
                           pack_bf16x2(gelu_tanh_f(acc[f][i][4 * jg + 2]), gelu_tanh_f(acc[f][i][4 * jg + 3])));
          }
        }
      }
    }
    return;
  }
  if constexpr (EPI == EPI_DA) {
    // a tile lies in one half of [0, 2 hid) (hid % BN == 0)
    const bool lin = n0 >= g.hid;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const long long m = m0 + wm * WTM * 32 + i * 32 + l32;
      if (m >= g.M) continue;
      const float rinv = lin ? g.rinv[m] : 0.f;
      float4 ov[WFN][4], gv[WFN][4];
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int n = n0 + wn * WFN * 32 + 32 * f + 8 * jg + 4 * half;
          gv[f][jg] = load_f16x4(g.gsv + m * (2LL * g.hid) + n);
          if (!lin) {
            ov[f][jg] = load_f16x4(g.os + m * g.hid + n);
          } else {
            const int c = n - g.hid;
            const float4 o = load_f16x4(g.ol + m * g.hid + c);
            const uint2 wv = *(const uint2*)(g.rmsw + c);
            ov[f][jg] = make_float4(o.x * __uint_as_float(wv.x << 16) * rinv,
                                    o.y * __uint_as_float(wv.x & 0xffff0000u) * rinv,
                                    o.z * __uint_as_float(wv.y << 16) * rinv,
                                    o.w * __uint_as_float(wv.y & 0xffff0000u) * rinv);
          }
        }
#pragma unroll
      for (int f = 0; f < WFN; ++f)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int n = n0 + wn * WFN * 32 + 32 * f + 8 * jg + 4 * half;
          const float a0 = acc[f][i][4 * jg], a1 = acc[f][i][4 * jg + 1];
          const float a2 = acc[f][i][4 * jg + 2], a3 = acc[f][i][4 * jg + 3];
          const float4 gg = gv[f][jg], o = ov[f][jg];
          // dA * gate -> dO_s (softmax half) or dR (linear half)
          const uint2 dg = make_uint2(pack_bf16x2(a0 * gg.x, a1 * gg.y), pack_bf16x2(a2 * gg.z, a3 * gg.w));
          // dA * branch value * sigmoid'(z) -> dZ
          const uint2 dzv = make_uint2(pack_bf16x2(a0 * o.x * gg.x * (1.f - gg.x), a1 * o.y * gg.y * (1.f - gg.y)),
                                       pack_bf16x2(a2 * o.z * gg.z * (1.f - gg.z), a3 * o.w * gg.w * (1.f - gg.w)));
          *(uint2*)(g.dz + m * (2LL * g.hid) + n) = dzv;
          if (!lin) *(uint2*)(g.dos + m * g.hid + n) = dg;
          else *(uint2*)(g.dr + m * g.hid + (n - g.hid)) = dg;
        }
    }
    return;
  }
  if constexpr (EPI == EPI_QKV) {
    // q / k / v column block of this tile (hid % BN == 0: one tensor per tile)
    const int t = n0 / g.hid;
    bf16_t* outp = t == 0 ? g.qo : (t == 1 ? g.ko : g.vo);
    const int cw = n0 - t * g.hid + wn * WFN * 32;  // first column of this wave
    uint32_t mx[WTM][WFN];  // largest |bf16 value| (float bits) per token group and 32-column block
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const long long m = m0 + wm * WTM * 32 + i * 32 + l32;
      const bool ok = m < g.M;
#pragma unroll
      for (int f = 0; f < WFN; ++f) {
        uint32_t a = 0;
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const uint32_t lo = pack_bf16x2(acc[f][i][4 * jg], acc[f][i][4 * jg + 1]);
          const uint32_t hi = pack_bf16x2(acc[f][i][4 * jg + 2], acc[f][i][4 * jg + 3]);
          if (ok) *(uint2*)(outp + m * g.hid + cw + 32 * f + 8 * jg + 4 * half) = make_uint2(lo, hi);
          a = max(a, max(max((lo & 0x7fffu) << 16, lo & 0x7fff0000u), max((hi & 0x7fffu) << 16, hi & 0x7fff0000u)));
        }
        mx[i][f] = ok ? a : 0u;
      }
    }
    if (g.absmax) {
      const long long mw0 = m0 + wm * WTM * 32;  // first token of this wave
      if (mw0 < g.M) {
        const long long mw1 = min(g.M - 1, mw0 + WTM * 32 - 1);
        const int b0 = (int)(mw0 / g.n_video), b1 = (int)(mw1 / g.n_video);
        if (b0 == b1) {
          // one batch: reduce over the wave, one atomic per 32-column block
#pragma unroll
          for (int f = 0; f < WFN; ++f) {
            uint32_t v = mx[0][f];
#pragma unroll
            for (int i = 1; i < WTM; ++i) v = max(v, mx[i][f]);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
            if (lane == 0) atomicMax(g.absmax + ((long long)t * g.B + b0) * g.H + (cw + 32 * f) / g.D, v);
          }
        } else {
          // the wave straddles a batch boundary: per-lane atomics
#pragma unroll
          for (int i = 0; i < WTM; ++i) {
            const long long m = mw0 + i * 32 + l32;
            if (m >= g.M) continue;
            const int b = (int)(m / g.n_video);
#pragma unroll
            for (int f = 0; f < WFN; ++f)
              atomicMax(g.absmax + ((long long)t * g.B + b) * g.H + (cw + 32 * f) / g.D, mx[i][f]);
          }
        }
      }
    }
    return;
  }
  if constexpr (USE_ROWEPI)
    epilogue_rows<WTM, WFN, EPI>(g, acc, m0 + wm * WTM * 32, n0 + wn * WFN * 32, lane,
                                 (float*)lds + wave * (EPI_WAVE_BYTES / 4));
  else
    epilogue_gate_out<WTM, WFN, EPI, MX>(g, acc, m0 + wm * WTM * 32 + l32, n0 + wn * WFN * 32, half);
}

// Weight transposes into the GEMMs' [N][K] operand layout.
//   mode 0: out[2*hid][hid] bf16,  out[c][r] = c < hid ? W_gs[r][c] : W_gl[r][c - hid]
//   mode 1: out[hid][2*hid] fp16,  out[c][r] = r < hid ? W_os[r][c] : W_ol[r - hid][c]
//   mode 2: out[hid][hid] bf16,    out[c][r] = W[r][c]  (s0 only)
__global__ __launch_bounds__(256) void k_weight_transpose(const bf16_t* __restrict__ s0,
                                                          const bf16_t* __restrict__ s1, int hid, int mode,
                                                          uint16_t* __restrict__ out) {
  __shared__ uint16_t t[64][66];
  const int R = mode == 1 ? 2 * hid : hid;  // source rows
  const int C = mode == 0 ? 2 * hid : hid;  // source cols
  const int tc = blockIdx.x % (C / 64), tr = blockIdx.x / (C / 64);
  const int r0 = tr * 64, c0 = tc * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    const int r = r0 + rr, c = c0 + cc;
    bf16_t val;
    if (mode == 0) val = c < hid ? s0[(long long)r * hid + c] : s1[(long long)r * hid + c - hid];
    else if (mode == 1) val = r < hid ? s0[(long long)r * hid + c] : s1[(long long)(r - hid) * hid + c];
    else val = s0[(long long)r * hid + c];
    t[rr][cc] = mode == 1 ? f32_to_f16_sat(bf16_to_f32(val)) : val;
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

template <int WM, int WN, int WTM, int WFN, int BK, int ST, int WPE, int EPI, int GM = 1, bool MX = false>
static hipError_t launch_gemm(GemmArgs g, hipStream_t s) {
  constexpr int BM = WM * WTM * 32, BN = WN * WFN * 32;
  constexpr int KT = MX ? 2 * BK : BK, ESZ = MX ? 1 : 2;
  if (g.ldk == 0) g.ldk = g.K;
  if (g.ksplit < 1 || EPI != EPI_WGRAD) g.ksplit = 1;
  if (g.N % BN != 0 || g.K % KT != 0 || g.K < KT ||
      ((EPI == EPI_GATE || EPI == EPI_QKV || EPI == EPI_DA) && g.hid % BN != 0) ||
      (long long)g.K * g.ksplit > g.ldk)
    return hipErrorInvalidValue;
  // MX: exponent rows of A padded to whole token tiles; no split contraction
  if (MX && (g.ksplit != 1 || g.ldk != g.K || !g.sa || !g.sb || g.mpad < (g.M + BM - 1) / BM * BM ||
             ((EPI == EPI_GATE || EPI == EPI_GELU) && (!g.ap8 || !g.aps))))
    return hipErrorInvalidValue;
  // 32-bit per-lane DMA offsets: a tile's rows span < 4 GiB
  if ((long long)BM * g.ldk * ESZ >= (1LL << 32) || (long long)BN * g.ldk * ESZ >= (1LL << 32))
    return hipErrorInvalidValue;
  const long long grid = ((g.M + BM - 1) / BM) * (g.N / BN) * g.ksplit;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_bf16<WM, WN, WTM, WFN, BK, ST, WPE, EPI, GM, MX>), dim3((unsigned)grid),
                     dim3(64 * WM * WN), 0, s, g);
  return hipGetLastError();
}

static GemmArgs base_args(const Dims& d, const Bf16Args& a) {
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
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
  g.rinv = a.rinv;
  g.rmsw = a.rmsw;
  g.ap = a.ap;
  g.gates_dbg = a.gates_dbg;
  g.gates16 = a.gates16;
  if (d.hid % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_GATE, 4>(g, s);
  if (d.hid % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_GATE>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_GATE>(g, s);  // hid multiple of 64 only
}

// [W_q | W_k | W_v] transposed into [3*hid][hid] (one mode-2 transpose each).
hipError_t launch_qkv_weights(const bf16_t* wq, const bf16_t* wk, const bf16_t* wv, int hid, bf16_t* out,
                              hipStream_t s) {
  const bf16_t* src[3] = {wq, wk, wv};
  const unsigned grid = (unsigned)((hid / 64) * (hid / 64));
  for (int t = 0; t < 3; ++t) {
    hipLaunchKernelGGL(k_weight_transpose, dim3(grid), dim3(256), 0, s, src[t], src[t], hid, 2,
                       (uint16_t*)out + (long long)t * hid * hid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// q, k, v = x [W_q | W_k | W_v]; absmax (nullable) receives the per-(tensor,
// batch, head) maximum |value| of the stored bf16 outputs (zeroed here).
hipError_t launch_qkv_gemm(const Dims& d, const bf16_t* x, const bf16_t* wt, bf16_t* q, bf16_t* k, bf16_t* v,
                           uint32_t* absmax, hipStream_t s) {
  if (absmax) {
    hipError_t e = launch_zero_u32(absmax, 3 * d.B * d.H, s);
    if (e != hipSuccess) return e;
  }
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
  g.B = d.B;
  g.n_video = d.N;
  g.D = d.D;
  g.A = x;
  g.Bt = wt;
  g.N = 3 * d.hid;
  g.K = d.hid;
  g.qo = q;
  g.ko = k;
  g.vo = v;
  g.absmax = absmax;
  if (d.hid % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_QKV, 4>(g, s);
  if (d.hid % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_QKV>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_QKV>(g, s);  // hid multiple of 64 only
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
  if (g.N % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_OUT, 2>(g, s);
  if (g.N % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_OUT>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_OUT>(g, s);
}

// ---- MX (e4m3 + E8M0 block exponents) variants --------------------------------
// Operands come from the quantisers in mx_quant.hip; hid % 256 == 0.

hipError_t launch_gate_gemm_mx(const Dims& d, const Bf16Args& a, hipStream_t s) {
  GemmArgs g = base_args(d, a);
  g.A = (const uint16_t*)a.x8;
  g.sa = a.xs;
  g.Bt = a.wg_t;
  g.sb = a.wgs8;
  g.mpad = a.mpad;
  g.N = 2 * d.hid;
  g.K = d.hid;
  g.os = a.os;
  g.ol = a.ol;
  g.rinv = a.rinv;
  g.rmsw = a.rmsw;
  g.ap8 = (uint8_t*)a.ap;
  g.aps = a.aps;
  g.gates_dbg = a.gates_dbg;
  g.gates16 = a.gates16;
  return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_GATE, 4, true>(g, s);
}

hipError_t launch_out_gemm_mx(const Dims& d, const Bf16Args& a, hipStream_t s) {
  GemmArgs g = base_args(d, a);
  g.A = a.ap;
  g.sa = a.aps;
  g.Bt = a.wo_t;
  g.sb = a.wos8;
  g.mpad = a.mpad;
  g.N = d.hid;
  g.K = 2 * d.hid;
  g.x = a.x;
  g.y = a.y;
  g.delta_dbg = a.delta_dbg;
  return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_OUT, 2, true>(g, s);
}

hipError_t launch_qkv_gemm_mx(const Dims& d, const uint8_t* x8, const uint8_t* xs, long long mpad,
                              const uint8_t* wt8, const uint8_t* wts, bf16_t* q, bf16_t* k, bf16_t* v,
                              uint32_t* absmax, hipStream_t s) {
  if (absmax) {
    hipError_t e = launch_zero_u32(absmax, 3 * d.B * d.H, s);
    if (e != hipSuccess) return e;
  }
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
  g.B = d.B;
  g.n_video = d.N;
  g.D = d.D;
  g.A = (const uint16_t*)x8;
  g.sa = xs;
  g.Bt = (const uint16_t*)wt8;
  g.sb = wts;
  g.mpad = mpad;
  g.N = 3 * d.hid;
  g.K = d.hid;
  g.qo = q;
  g.ko = k;
  g.vo = v;
  g.absmax = absmax;
  return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_QKV, 4, true>(g, s);
}

// Feed-forward GEMMs on MX operands: u = GELU(h W_1) written as MX codes
// (u8 [M][F], us [F/128][mpad][4]), then out = resid + u W_2.
hipError_t launch_gelu_gemm_mx(long long M, int hid, int F, const uint8_t* h8, const uint8_t* hs, long long mpad,
                               const uint8_t* w1c, const uint8_t* w1s, uint8_t* u8, uint8_t* us, hipStream_t s) {
  GemmArgs g = {};
  g.M = M;
  g.N = F;
  g.K = hid;
  g.hid = hid;
  g.A = (const uint16_t*)h8;
  g.sa = hs;
  g.Bt = (const uint16_t*)w1c;
  g.sb = w1s;
  g.mpad = mpad;
  g.ap8 = u8;
  g.aps = us;
  return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_GELU, 4, true>(g, s);
}

hipError_t launch_resid_gemm_mx(long long M, int N, int K, const uint8_t* a8, const uint8_t* as, long long mpad,
                                const uint8_t* bc, const uint8_t* bs, const bf16_t* resid, bf16_t* out,
                                hipStream_t s) {
  GemmArgs g = {};
  g.M = M;
  g.N = N;
  g.K = K;
  g.hid = N;
  g.A = (const uint16_t*)a8;
  g.sa = as;
  g.Bt = (const uint16_t*)bc;
  g.sb = bs;
  g.mpad = mpad;
  g.x = resid;
  g.y = out;
  return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_RES, 2, true>(g, s);
}

// ---- backward pass ---------------------------------------------------------

// dA' = dy [W_os ; W_ol]^T with the gate / RMSNorm-input gradients in the
// epilogue.  wo_cat: [2 hid][hid] bf16 = W_os rows then W_ol rows (the
// [in][out] weights are already the [N][K] operand).
hipError_t launch_da_gemm(const Dims& d, const bf16_t* dy, const bf16_t* wo_cat, const uint16_t* gsv,
                          const uint16_t* os, const uint16_t* ol, const float* rinv, const bf16_t* rmsw,
                          bf16_t* dos, bf16_t* dz, bf16_t* dr, hipStream_t s) {
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
  g.A = dy;
  g.Bt = wo_cat;
  g.N = 2 * d.hid;
  g.K = d.hid;
  g.gsv = gsv;
  g.os = os;
  g.ol = ol;
  g.rinv = rinv;
  g.rmsw = rmsw;
  g.dos = dos;
  g.dz = dz;
  g.dr = dr;
  if (d.hid % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_DA, 4>(g, s);
  if (d.hid % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_DA>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_DA>(g, s);
}

// dx = dy + dZ [W_gs | W_gl]^T.  wg_cat: [hid][2 hid] bf16, row i = (W_gs[i], W_gl[i]).
hipError_t launch_res_gemm(const Dims& d, const bf16_t* dz, const bf16_t* wg_cat, const bf16_t* dy, bf16_t* dx,
                           hipStream_t s) {
  GemmArgs g = {};
  g.M = (long long)d.B * d.N;
  g.hid = d.hid;
  g.H = d.H;
  g.A = dz;
  g.Bt = wg_cat;
  g.N = d.hid;
  g.K = 2 * d.hid;
  g.x = dy;
  g.y = dx;
  if (g.N % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_RES, 2>(g, s);
  if (g.N % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_RES>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_RES>(g, s);
}

// Weight gradient C[Mop][Nop] = sum_t A^T[.][t] B^T[.][t] over t < kpad from
// token-transposed operands aT [Mop][kpad], bT [Nop][kpad] (bf16, zero past
// the last token), as ksplit fp32 partials part[ksplit][Mop][Nop].
// kpad % (64 ksplit) == 0.
hipError_t launch_wgrad_gemm(const bf16_t* aT, const bf16_t* bT, int Mop, int Nop, long long kpad, int ksplit,
                             float* part, hipStream_t s) {
  if (ksplit < 1 || kpad % (64LL * ksplit) != 0 || kpad > 0x7fffffffLL) return hipErrorInvalidValue;
  GemmArgs g = {};
  g.M = Mop;
  g.N = Nop;
  g.K = (int)(kpad / ksplit);
  g.ldk = (int)kpad;
  g.ksplit = ksplit;
  g.A = aT;
  g.Bt = bT;
  g.part = part;
  if (Nop % 256 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_WGRAD, 4>(g, s);
  if (Nop % 128 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_WGRAD>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_WGRAD>(g, s);
}

// ---- feed-forward of the block ------------------------------------------------

// out[M][F] = GELU_tanh(h W_1): h [M][hid], w1t [F][hid] (W_1 transposed), bf16.
hipError_t launch_gelu_gemm(long long M, int hid, int F, const bf16_t* h, const bf16_t* w1t, bf16_t* out,
                            hipStream_t s) {
  GemmArgs g = {};
  g.M = M;
  g.N = F;
  g.K = hid;
  g.hid = hid;
  g.A = h;
  g.Bt = w1t;
  g.out = out;
  if (F % 256 == 0 && hid % 64 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_GELU, 4>(g, s);
  if (F % 128 == 0 && hid % 32 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_GELU>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_GELU>(g, s);
}

// out[M][N] = resid + A Bt^T: A [M][K], bt [N][K], resid / out [M][N], bf16.
hipError_t launch_resid_gemm(long long M, int N, int K, const bf16_t* a, const bf16_t* bt, const bf16_t* resid,
                             bf16_t* out, hipStream_t s) {
  GemmArgs g = {};
  g.M = M;
  g.N = N;
  g.K = K;
  g.hid = N;
  g.A = a;
  g.Bt = bt;
  g.x = resid;
  g.y = out;
  if (N % 256 == 0 && K % 64 == 0) return launch_gemm<4, 2, 2, 4, 64, 2, 2, EPI_RES, 2>(g, s);
  if (N % 128 == 0 && K % 32 == 0) return launch_gemm<2, 2, 4, 2, 32, 3, 2, EPI_RES>(g, s);
  return launch_gemm<2, 2, 4, 1, 32, 3, 2, EPI_RES>(g, s);
}

}  // namespace hyb
