// Backward pass of the softmax branch on bf16 MFMA (block-sparse flash
// attention backward over the key frames S(f) plus the text).
//
// VDN-H3 article (tahou.com), section "分阶段适配预训练模型": training stages
// A1, A2 and B run the layer's backward pass (LoRA on the Q/K/V projections in
// stage B needs the gradients of q, k and v).  The softmax branch is the
// article's "双分支混合注意力机制" local window: query frame f sees the key
// frames S(f) and all text tokens.  With P = softmax(tau Q K^T) over that key
// set, dP = dO V^T and D_i = sum_d dO[i][d] O[i][d]:
//   dS = P * (dP - D),  dQ = tau dS K,  dK = tau dS^T Q,  dV = P^T dO.
// P is recomputed from the scores and the row's log2-sum-exp2 saved by the
// forward kernel, so no probability matrix is stored.
//
// Two kernels, neither with atomics:
//   k_attn_bwd_dq   query-centric, the forward's work items and key walk:
//                   S^T = K Q^T and dP^T = V dO^T per key tile, dQ^T += K^T dS^T;
//   k_attn_bwd_dkv  key-centric: a workgroup owns 32 keys per wave of one key
//                   frame (or of the text) and walks the query tiles of every
//                   frame that sees them.  The window relation is symmetric in
//                   chunk distance and anchor frames see every frame, so the
//                   query frames of key frame g are exactly S(g); text keys
//                   are seen by every frame.  Per 32-query tile:
//                   S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
// Both reuse the forward's MFMA tile products; every operand order is the one
// the previous MFMA's register layout gives (no transposes in registers).
#include <type_traits>

#include "attn_tiles.h"
#include "work_items.h"

namespace hyb {

// D_i = sum_d dO[i][d] O[i][d] for every (token, head): dO bf16 [M][hid],
// O fp16 [M][hid]; written as [B][H][N] (the order the softmax kernels read).
template <int D>
__global__ __launch_bounds__(256) void k_bwd_rowdot(const bf16_t* __restrict__ dos, const uint16_t* __restrict__ os,
                                                    long long M, int H, long long N, float* __restrict__ dvr) {
  constexpr int G = D / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / G;  // m * H + h
  if (row >= M * H) return;       // whole G-lane groups leave together
  const int part = (int)(gid % G);
  const long long off = row * D + part * 8;  // [M][hid] with hid = H * D
  const uint4 a = ldg16(dos + off);
  const uint32_t* au = (const uint32_t*)&a;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float4 of = load_f16x4(os + off + 4 * i);
    s = fmaf(__uint_as_float(au[2 * i] << 16), of.x, s);
    s = fmaf(__uint_as_float(au[2 * i] & 0xffff0000u), of.y, s);
    s = fmaf(__uint_as_float(au[2 * i + 1] << 16), of.z, s);
    s = fmaf(__uint_as_float(au[2 * i + 1] & 0xffff0000u), of.w, s);
  }
#pragma unroll
  for (int w = G / 2; w > 0; w >>= 1) s += __shfl_xor(s, w);
  if (part == 0) {
    const long long m = row / H, b = m / N, tok = m % N;
    const int h = (int)(row % H);
    dvr[(b * H + h) * N + tok] = s;
  }
}

// ---------------------------------------------------------------------------
// dQ.  Work item = (query frame, batch, head, query tile) as in the forward;
// 32 query rows per wave; K and V tiles (KB blocks of 32 keys) double
// buffered in LDS by direct-to-LDS loads.
template <int D, int KB, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void k_attn_bwd_dq(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, const bf16_t* __restrict__ dos,
                   const float* __restrict__ lse, const float* __restrict__ dvr, float sl2, float tau,
                   float* __restrict__ dq) {
  constexpr int BM = 32 * NW, KS = D / 16, DB = D / 32, BN = 32 * KB;
  using Ldr = TileLoader<D, NW, KB>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ldr::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][Ldr::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const Item it = decode_item(d, (d.n + BM - 1) / BM);

  KeyWalk<BN> kw;
  kw.init(d, it.f, it.b, it.h, k, v, tk, tv);
  Ldr ldr;
  ldr.init(wave, lane);
  ldr.set_k(kw.ks);
  ldr.set_v(kw.vs);
  const unsigned ks_lds = lds_addr(Ks), vs_lds = lds_addr(Vs);
  constexpr unsigned kTileBytes = Ldr::TILE * 2;

  int vcur = kw.valid();
  ldr.load_k(kw.kp, vcur, wave, ks_lds);
  ldr.load_v(kw.vp, vcur, wave, vs_lds);
  if (kw.advance()) {
    ldr.set_k(kw.ks);
    ldr.set_v(kw.vs);
  }

  const int prow = it.qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  const long long qtok = (long long)it.f * d.n + (row_ok ? prow : 0);
  bf16x8 qf[KS], df[KS];
  {
    const bf16_t* qp = (const bf16_t*)q.p + tok_off(q, it.b, qtok, it.h) + 8 * half;
    const bf16_t* dp = dos + ((long long)it.b * d.N + qtok) * d.hid + (long long)it.h * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * s));
      df[s] = __builtin_bit_cast(bf16x8, ldg16(dp + 16 * s));
    }
  }
  const long long bhn = ((long long)it.b * d.H + it.h) * d.N + qtok;
  const float l2 = lse[bhn], di = dvr[bhn];
  const int dsub = (lgrp & 1) * 16 + 4 * (j16 & 3);

  floatx16 dacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dacc[i] = zero16();

  wait_vmcnt<0>();
  tile_barrier();
  int buf = 0;
  for (;;) {
    const bool more = !kw.done();
    int vnext = 0;
    if (more) {  // next tile into the other buffer (last read one tile ago)
      vnext = kw.valid();
      ldr.load_k(kw.kp, vnext, wave, ks_lds + (buf ^ 1) * kTileBytes);
      ldr.load_v(kw.vp, vnext, wave, vs_lds + (buf ^ 1) * kTileBytes);
      if (kw.advance()) {
        ldr.set_k(kw.ks);
        ldr.set_v(kw.vs);
      }
    }
    floatx16 s[KB], dpv[KB];
    qk_tile<D, KB>(s, Ks[buf], qf, l32, half);
    qk_tile<D, KB>(dpv, Vs[buf], df, l32, half);
    if (vcur < BN) mask_tile<KB>(s, vcur, half);
    bf16x8 dsf[2 * KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hb + e], sl2, -l2));
          dsf[2 * kb + hb][e] = static_cast<__bf16>(p * (dpv[kb][8 * hb + e] - di));
        }
    pv_tile<D, KB>(dacc, Ks[buf], dsf, half, j16, dsub);
    if (!more) break;
    vcur = vnext;
    wait_vmcnt<0>();
    tile_barrier();
    buf ^= 1;
  }
  if (!row_ok) return;
  float* op = dq + ((long long)it.b * d.N + qtok) * d.hid + (long long)it.h * D;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = i * 32 + 8 * jg + 4 * half;
      *(float4*)(op + d0) = make_float4(dacc[i][4 * jg] * tau, dacc[i][4 * jg + 1] * tau, dacc[i][4 * jg + 2] * tau,
                                        dacc[i][4 * jg + 3] * tau);
    }
}

// ---------------------------------------------------------------------------
// dK, dV.  Work items: first the text key tiles (seen by every frame), then
// the video key tiles of each (key frame, batch, head), key frames in the
// forward's longest-first order.  32 keys per wave, NW waves; query tiles of
// 32 rows (Q and dO, double buffered in LDS).
template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void k_attn_bwd_dkv(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, const bf16_t* __restrict__ dos,
                    const float* __restrict__ lse, const float* __restrict__ dvr, float sl2, float tau,
                    int text_items, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dtk,
                    float* __restrict__ dtv) {
  constexpr int KS = D / 16, DB = D / 32, KT = 32 * NW, QT = 32;
  using Ldr = TileLoader<D, NW, 1>;  // one block of 32 query rows per tile
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][Ldr::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Ds[2][Ldr::TILE];
  __shared__ __attribute__((aligned(16))) float Ls[2][2 * QT];  // per tile: the rows' lse2, then their D
  __shared__ __attribute__((aligned(16))) bf16_t Vk[KT * D];     // this workgroup's value rows (B operand of dP)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;

  // ---- work item
  int b, h, g, ktile;
  bool text;
  int rlo[3], rhi[3], nr;
  {
    unsigned idx = blockIdx.x;
    if ((int)idx < text_items) {
      const int tt = (d.L + KT - 1) / KT;
      text = true;
      ktile = (int)(idx % tt);
      const int bh = (int)(idx / tt);
      h = bh % d.H;
      b = bh / d.H;
      g = 0;
      nr = 1;
      rlo[0] = 0;
      rhi[0] = d.T;
      rlo[1] = rhi[1] = rlo[2] = rhi[2] = 0;
    } else {
      idx -= text_items;
      const int tt = (d.n + KT - 1) / KT;
      text = false;
      ktile = (int)(idx % tt);
      const int grp = (int)(idx / tt);
      h = grp % d.H;
      b = (grp / d.H) % d.B;
      g = frame_by_cost(d.g, grp / (d.H * d.B));
      const SoftRanges sr = soft_ranges(d.g, g);
      nr = sr.n;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        rlo[i] = i < sr.n ? sr.lo[i] : 0;
        rhi[i] = i < sr.n ? sr.hi[i] : 0;
      }
    }
  }
  const int nkeys = text ? d.L : d.n;
  const int key = ktile * KT + wave * 32 + l32;
  const bool key_ok = key < nkeys;
  const int keyc = key_ok ? key : nkeys - 1;

  // K^T fragments of this lane's key (B operand of S) in registers; the
  // workgroup's V rows (B operand of dP) in LDS, which keeps the kernel at two
  // waves per SIMD
  bf16x8 kf[KS];
  {
    const bf16_t* kp = text ? (const bf16_t*)tk.p + tok_off(tk, b, keyc, h)
                            : (const bf16_t*)k.p + tok_off(k, b, (long long)g * d.n + keyc, h);
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = __builtin_bit_cast(bf16x8, ldg16(kp + 8 * half + 16 * s));
    constexpr int G = D / 8;
    for (int ci = tid; ci < KT * G; ci += 64 * NW) {
      const int r = ci / G, c = (ci % G) * 8;
      const int kr = min(ktile * KT + r, nkeys - 1);
      const bf16_t* vp = text ? (const bf16_t*)tv.p + tok_off(tv, b, kr, h)
                              : (const bf16_t*)v.p + tok_off(v, b, (long long)g * d.n + kr, h);
      *(uint4*)&Vk[Swz<D>::off(r, c)] = ldg16(vp + c);
    }
  }

  // ---- query walk: frames of the ranges, ceil(n / QT) tiles per frame
  const int tpf = (d.n + QT - 1) / QT;
  int nfr = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) nfr += i < nr ? rhi[i] - rlo[i] : 0;
  const int nsteps = nfr * tpf;
  auto frame_at = [&](int fi) {
    int f = rlo[0] + fi;
    const int l0 = rhi[0] - rlo[0], l1 = rhi[1] - rlo[1];
    if (nr > 1 && fi >= l0) f = rlo[1] + (fi - l0);
    if (nr > 2 && fi >= l0 + l1) f = rlo[2] + (fi - l0 - l1);
    return f;
  };
  const char* qbase = (const char*)((const bf16_t*)q.p + (long long)b * q.sb + (long long)h * q.sh);
  const char* dbase = (const char*)(dos + (long long)b * d.N * d.hid + (long long)h * D);
  Ldr ldr;
  ldr.init(wave, lane);
  ldr.set_k((unsigned)(q.st * 2));
  ldr.set_v((unsigned)(d.hid * 2));
  const unsigned qs_lds = lds_addr(Qs), ds_lds = lds_addr(Ds);
  constexpr unsigned kTileBytes = Ldr::TILE * 2;
  const float* lrow = lse + ((long long)b * d.H + h) * d.N;
  const float* drow = dvr + ((long long)b * d.H + h) * d.N;

  // Q and dO rows by direct-to-LDS loads (rows past the tile repeat its last
  // row); the rows' lse2 and D (one value per lane of wave 0) go through a
  // register and are written to LDS just before the tile's barrier
  float lsv = 0.f;
  auto issue = [&](int step, int buf) {
    const int f = frame_at(step / tpf), t0 = (step % tpf) * QT;
    const int valid = min(QT, d.n - t0);
    const long long tok = (long long)f * d.n + t0;
    ldr.load_k(qbase + tok * (q.st * 2), valid, wave, qs_lds + buf * kTileBytes);
    ldr.load_v(dbase + tok * ((long long)d.hid * 2), valid, wave, ds_lds + buf * kTileBytes);
    if (wave == 0) {  // rows past the tile: lse2 = +inf and D = 0, so P = dS = 0 there
      const bool ok = l32 < valid;
      const float vl = half == 0 ? lrow[tok + (ok ? l32 : 0)] : drow[tok + (ok ? l32 : 0)];
      lsv = ok ? vl : (half == 0 ? INFINITY : 0.f);
    }
  };
  auto publish = [&](int buf) {  // after this wave's loads landed, before the barrier
    if (wave == 0) Ls[buf][lane] = lsv;
  };

  floatx16 dka[DB], dva[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dka[i] = zero16();
    dva[i] = zero16();
  }
  const int dsub = (lgrp & 1) * 16 + 4 * (j16 & 3);

  if (nsteps > 0) issue(0, 0);
  wait_vmcnt<0>();
  publish(0);
  tile_barrier();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) issue(step + 1, buf ^ 1);
    floatx16 s = zero16(), dp = zero16();
    // S and dP chains interleaved; two k-steps of operand reads in flight
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      if (st % 2 == 0) __builtin_amdgcn_sched_barrier(0);
      const bf16x8 a = *(const bf16x8*)&Qs[buf][Swz<D>::off(l32, 16 * st + 8 * half)];
      const bf16x8 b = *(const bf16x8*)&Ds[buf][Swz<D>::off(l32, 16 * st + 8 * half)];
      const bf16x8 vb = *(const bf16x8*)&Vk[Swz<D>::off(wave * 32 + l32, 16 * st + 8 * half)];
      s = mfma32(a, kf[st], s);
      dp = mfma32(b, vb, dp);
    }
    // this lane's 16 query rows: 8 (j / 4) + 4 half + j % 4
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const float4 l4 = *(const float4*)&Ls[buf][8 * jg + 4 * half];
      const float4 d4 = *(const float4*)&Ls[buf][QT + 8 * jg + 4 * half];
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * jg + r;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j], sl2, -lv[r]));
        pf[j >> 3][j & 7] = static_cast<__bf16>(p);
        dsf[j >> 3][j & 7] = static_cast<__bf16>(p * (dp[j] - dvv[r]));
      }
    }
    // phase boundaries keep each phase's operand reads from being hoisted
    // into the previous one (register pressure at two waves per SIMD)
    __builtin_amdgcn_sched_barrier(0);
    pv_tile<D, 1>(dva, Ds[buf], pf, half, j16, dsub);
    __builtin_amdgcn_sched_barrier(0);
    pv_tile<D, 1>(dka, Qs[buf], dsf, half, j16, dsub);
    wait_vmcnt<0>();
    if (step + 1 < nsteps) publish(buf ^ 1);
    tile_barrier();
  }
  if (!key_ok) return;
  float* kout = text ? dtk + ((long long)b * d.L + key) * d.hid + (long long)h * D
                     : dk + ((long long)b * d.N + (long long)g * d.n + key) * d.hid + (long long)h * D;
  float* vout = text ? dtv + ((long long)b * d.L + key) * d.hid + (long long)h * D
                     : dv + ((long long)b * d.N + (long long)g * d.n + key) * d.hid + (long long)h * D;
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = i * 32 + 8 * jg + 4 * half;
      *(float4*)(kout + d0) = make_float4(dka[i][4 * jg] * tau, dka[i][4 * jg + 1] * tau, dka[i][4 * jg + 2] * tau,
                                          dka[i][4 * jg + 3] * tau);
      *(float4*)(vout + d0) = make_float4(dva[i][4 * jg], dva[i][4 * jg + 1], dva[i][4 * jg + 2], dva[i][4 * jg + 3]);
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_softmax_backward(const Dims& d, const BwdArgs& a, hipStream_t s) {
  const long long M = (long long)d.B * d.N;
  {
    const long long threads = M * d.hid / 8;
    const long long blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d.D == 128)
      hipLaunchKernelGGL(k_bwd_rowdot<128>, dim3((unsigned)blocks), dim3(256), 0, s, a.dos, a.os, M, d.H, d.N, a.dvr);
    else
      hipLaunchKernelGGL(k_bwd_rowdot<64>, dim3((unsigned)blocks), dim3(256), 0, s, a.dos, a.os, M, d.H, d.N, a.dvr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = 4, BM = 32 * NW;
    const long long grid = (long long)((d.n + BM - 1) / BM) * d.H * d.B * d.T;
    if (d.D == 128)
      hipLaunchKernelGGL((k_attn_bwd_dq<128, 2, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v,
                         a.tk, a.tv, a.dos, a.lse, a.dvr, a.scale_log2, a.tau, a.dq_s);
    else
      hipLaunchKernelGGL((k_attn_bwd_dq<64, 2, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v,
                         a.tk, a.tv, a.dos, a.lse, a.dvr, a.scale_log2, a.tau, a.dq_s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr int NW = 4, KT = 32 * NW;
    const int text_items = d.L > 0 ? ((d.L + KT - 1) / KT) * d.B * d.H : 0;
    const long long grid = text_items + (long long)((d.n + KT - 1) / KT) * d.H * d.B * d.T;
    if (d.D == 128)
      hipLaunchKernelGGL((k_attn_bwd_dkv<128, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v,
                         a.tk, a.tv, a.dos, a.lse, a.dvr, a.scale_log2, a.tau, text_items, a.dk_s, a.dv_s, a.dtk_s,
                         a.dtv_s);
    else
      hipLaunchKernelGGL((k_attn_bwd_dkv<64, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v,
                         a.tk, a.tv, a.dos, a.lse, a.dvr, a.scale_log2, a.tau, text_items, a.dk_s, a.dv_s, a.dtk_s,
                         a.dtv_s);
    return hipGetLastError();
  }
}

}  // namespace hyb
