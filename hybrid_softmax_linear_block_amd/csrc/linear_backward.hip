// Backward pass of the linear branch on MFMA.
//
// VDN-H3 article (tahou.com), section "分阶段适配预训练模型": stage A1 calibrates
// and stage A2 trains the new linear branch, so its gradients are the heart of
// both.  Forward (section "双分支混合注意力机制"): for query i of frame f,
//   num = phi(q)^T C_f, den = phi(q) . c_f + eps, O = num / den,
//   C_f = S_T + sum_{g in F(f)} S_g + sum_{g in B(f)} S_g (c_f likewise),
//   S_g = sum_{t in g} phi(k_t) v_t^T, z_g = sum_{t in g} phi(k_t).
// Reverse, in three steps:
//   1. per query token: dnum = dO / den, dden = -(dO . O) / den,
//      dphi(q) = C_f dnum + c_f dden, dq = dphi(q) phi'(q)   (k_lin_bwd_q);
//      per frame: dC_f = sum_i phi(q_i) dnum_i^T, dc_f = sum_i phi(q_i) dden_i
//      (the state-build kernel with per-token z weights);
//   2. every frame state collects dC_f from each f whose forward or backward
//      range holds it; the text state collects every dC_f (half through each
//      direction)  (k_lin_bwd_scan);
//   3. per key token of frame g (or text): dphi(k) = dS_g v + dz_g,
//      dv = dS_g^T phi(k), dk = dphi(k) phi'(k)  (k_lin_bwd_kv).
// Steps 1 and 3 add the softmax branch's fp32 gradients and write the final
// bf16 dq, dk, dv.  Products that carry a computed operand (the states,
// dnum, phi(q), phi(k)) split it into bf16 hi + lo and take three MFMAs
// (hi*hi, hi*lo, lo*hi), as the forward readout does.
#include "kernels_bf16.h"

namespace hyb {

__device__ __forceinline__ float dphi_f(float u) { return u > 0.f ? 1.f : __expf(u); }

// a = hi + lo with both parts bf16 (hi the nearest bf16, lo the rounded rest)
#define SPLIT_BF16(a, HI, LO)                                  \
  do {                                                         \
    const float a_ = (a);                                      \
    const __bf16 h_ = static_cast<__bf16>(a_);                 \
    HI = h_;                                                   \
    LO = static_cast<__bf16>(a_ - static_cast<float>(h_));     \
  } while (0)

__device__ __forceinline__ float4 load_bf16x4(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// ---------------------------------------------------------------------------
// Step 1, per query token.  Workgroup = (b, h, frame f, tile of tt tokens);
// the combined state C_f^T (hi + lo, [e][d]) and c_f sit in LDS; lane = token.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void k_lin_bwd_q(Dims d, Tensor4 q, const bf16_t* __restrict__ chi, const bf16_t* __restrict__ clo,
                 const float* __restrict__ cz, float eps, int tt, const float* __restrict__ dol,
                 const float* __restrict__ dqs, bf16_t* __restrict__ dq, int ldq, bf16_t* __restrict__ dnum,
                 float* __restrict__ dden) {
  constexpr int G = D / 8, KS = D / 16, DB = D / 32;
  using SW = Swz<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Sh[D * D];
  __shared__ __attribute__((aligned(16))) bf16_t Sl[D * D];
  __shared__ float Z[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const int dsub = (lgrp & 1) * 16 + 4 * (j16 & 3);
  const int tiles = (d.n + tt - 1) / tt;
  int w = blockIdx.x;
  const int tile = w % tiles; w /= tiles;
  const int f = w % d.T; w /= d.T;
  const int h = w % d.H;
  const int b = w / d.H;
  const long long fo = ((long long)b * d.H + h) * d.T + f;

  for (int gi = tid; gi < D * G; gi += 256) {
    const int row = gi / G, col = (gi % G) * 8;
    *(uint4*)&Sh[SW::off(row, col)] = ldg16(chi + fo * D * D + row * D + col);
    *(uint4*)&Sl[SW::off(row, col)] = ldg16(clo + fo * D * D + row * D + col);
  }
  if (tid < D) Z[tid] = cz[fo * D + tid];
  __syncthreads();

  const int p_end = min(d.n, (tile + 1) * tt);
  for (int p0 = tile * tt + wave * 32; p0 < p_end; p0 += 4 * 32) {
    // lanes past the tile's end redo token p0 (lane 0's token): they compute
    // the same values and store them to the same places, so no lane branches
    const int p = p0 + l32;
    const bool ok = p < p_end;
    const long long tok = (long long)f * d.n + (ok ? p : p0);
    const long long row = ((long long)b * d.N + tok) * d.hid + (long long)h * D;  // [M][hid] offset
    const long long qo = ((long long)b * d.N + tok) * ldq + (long long)h * D;      // output row of dq
    const bf16_t* qrow = (const bf16_t*)q.p + tok_off(q, b, tok, h);
    bf16x8 ph[KS], pl[KS];
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 u = ldg16(qrow + 8 * half + 16 * s);
      const uint32_t* uu = (const uint32_t*)&u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = phi_f(__uint_as_float(uu[i] << 16));
        const float a1 = phi_f(__uint_as_float(uu[i] & 0xffff0000u));
        const int dd = 16 * s + 8 * half + 2 * i;
        den = fmaf(a0, Z[dd], den);
        den = fmaf(a1, Z[dd + 1], den);
        SPLIT_BF16(a0, ph[s][2 * i], pl[s][2 * i]);
        SPLIT_BF16(a1, ph[s][2 * i + 1], pl[s][2 * i + 1]);
      }
    }
    den += __shfl_xor(den, 32);
    const float inv = 1.f / (den + eps);
    // O^T = C^T phi(q)^T / den (as the forward readout), then dnum = dO / den
    // as the B-operand fragments of the next product (C-layout order)
    bf16x8 nh[2 * DB], nl[2 * DB];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      // one block's operand reads in flight at a time (no hoisting across blocks)
      __builtin_amdgcn_sched_barrier(0);
      floatx16 acc = zero16();
      const int r = i * 32 + l32;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if (s % 2 == 0) __builtin_amdgcn_sched_barrier(0);
        const bf16x8 ah = *(const bf16x8*)&Sh[SW::off(r, 16 * s + 8 * half)];
        const bf16x8 al = *(const bf16x8*)&Sl[SW::off(r, 16 * s + 8 * half)];
        acc = mfma32(ah, ph[s], acc);
        acc = mfma32(ah, pl[s], acc);
        acc = mfma32(al, ph[s], acc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int e0 = i * 32 + 8 * jg + 4 * half;
        const float4 g4 = *(const float4*)(dol + row + e0);
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
        float nv[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int j = 4 * jg + rr;
          dot = fmaf(gv[rr], acc[j] * inv, dot);
          nv[rr] = gv[rr] * inv;
          SPLIT_BF16(nv[rr], nh[2 * i + (j >> 3)][j & 7], nl[2 * i + (j >> 3)][j & 7]);
        }
        *(uint2*)(dnum + row + e0) = make_uint2(pack_bf16x2(nv[0], nv[1]), pack_bf16x2(nv[2], nv[3]));
      }
    }
    dot += __shfl_xor(dot, 32);
    const float ddn = -dot * inv;
    dden[((long long)b * d.N + tok) * d.H + h] = ddn;
    // dphi(q)^T = C dnum, one 32-row block of d at a time: the C operand from
    // transposing reads of C^T [e][d]; then dq = (dphi(q) + c dden) phi'(q)
    // plus the softmax branch's part
#pragma unroll 1
    for (int i = 0; i < DB; ++i) {
      floatx16 acc = zero16();
      const int col = i * 32 + dsub;
#pragma unroll
      for (int kk = 0; kk < 2 * DB; ++kk) {
        if (kk % 2 == 0) __builtin_amdgcn_sched_barrier(0);
        const int kb0 = (kk >> 1) * 32 + (kk & 1) * 16 + 4 * half + (j16 >> 2);
        const bf16x8 ah = tr_pair(&Sh[SW::off(kb0, col)], &Sh[SW::off(kb0 + 8, col)]);
        const bf16x8 al = tr_pair(&Sl[SW::off(kb0, col)], &Sl[SW::off(kb0 + 8, col)]);
        acc = mfma32(ah, nh[kk], acc);
        acc = mfma32(ah, nl[kk], acc);
        acc = mfma32(al, nh[kk], acc);
      }
      {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = i * 32 + 8 * jg + 4 * half;
          const float4 q4 = load_bf16x4(qrow + d0);
          const float4 s4 = *(const float4*)(dqs + row + d0);
          const float o0 = (acc[4 * jg] + Z[d0] * ddn) * dphi_f(q4.x) + s4.x;
          const float o1 = (acc[4 * jg + 1] + Z[d0 + 1] * ddn) * dphi_f(q4.y) + s4.y;
          const float o2 = (acc[4 * jg + 2] + Z[d0 + 2] * ddn) * dphi_f(q4.z) + s4.z;
          const float o3 = (acc[4 * jg + 3] + Z[d0 + 3] * ddn) * dphi_f(q4.w) + s4.w;
          *(uint2*)(dq + qo + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Step 2.  One thread per (b, h, element) of a state (element < D*D: the
// [e][d] entry e*D + d; then z[d]).  Pass 1 reduces the per-split partials of
// dC_f into dcf (the thread's own column, re-read in pass 2); pass 2 sums, for
// every frame g, the dC_f of the frames whose forward or backward range holds
// g, and for the text (slot T) all of them.  Output dS [B*H][T+1][d][e] as bf16
// hi + lo (the layout step 3 reads) and dz [B*H][T+1][D] fp32.
template <int D>
__global__ __launch_bounds__(256) void k_lin_bwd_scan(Dims d, const float* __restrict__ part, int split,
                                                      float* __restrict__ dcf, bf16_t* __restrict__ dsh,
                                                      bf16_t* __restrict__ dsl, float* __restrict__ dsz) {
  constexpr int E = D * D + D;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.H * E) return;
  const int el = (int)(gid % E);
  const long long bh = gid / E;
  const float* pp = part + bh * (long long)d.T * split * E + el;
  float* cf = dcf + bh * (long long)d.T * E + el;
  float text = 0.f;
  for (int f = 0; f < d.T; ++f) {
    float s = 0.f;
    for (int p = 0; p < split; ++p) s += pp[(long long)(f * split + p) * E];
    cf[(long long)f * E] = s;
    text += s;
  }
  auto emit = [&](int g, float val) {
    const long long so = bh * (d.T + 1) + g;
    if (el < D * D) {
      const int e = el / D, dd = el % D;
      const bf16_t hi = f32_to_bf16(val);
      dsh[so * D * D + dd * D + e] = hi;
      dsl[so * D * D + dd * D + e] = f32_to_bf16(val - bf16_to_f32(hi));
    } else {
      dsz[so * D + (el - D * D)] = val;
    }
  };
  for (int g = 0; g < d.T; ++g) {
    float s = 0.f;
    for (int f = 0; f < d.T; ++f) {
      int flo, fhi, blo, bhi;
      linear_ranges(d.g, f, &flo, &fhi, &blo, &bhi);
      if ((g >= flo && g < fhi) || (g >= blo && g < bhi)) s += cf[(long long)f * E];
    }
    emit(g, s);
  }
  emit(d.T, text);
}

// ---------------------------------------------------------------------------
// Step 3, per key token.  Workgroup = (b, h, slot g in 0..T (T = text), tile
// of tt tokens); dS_g (hi + lo, [d][e]) and dz_g in LDS; lane = token.
//   dphi(k)^T = dS_g v^T (dS rows from LDS, v fragments from the token row)
//   dv^T      = dS_g^T phi(k)^T (dS^T by transposing LDS reads in natural k order)
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void k_lin_bwd_kv(Dims d, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, const bf16_t* __restrict__ dsh,
                  const bf16_t* __restrict__ dsl, const float* __restrict__ dsz, int tt,
                  const float* __restrict__ dks, const float* __restrict__ dvs, const float* __restrict__ dtks,
                  const float* __restrict__ dtvs, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int ldkv,
                  bf16_t* __restrict__ dtk, bf16_t* __restrict__ dtv) {
  constexpr int G = D / 8, KS = D / 16, DB = D / 32;
  using SW = Swz<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ah[D * D];
  __shared__ __attribute__((aligned(16))) bf16_t Al[D * D];
  __shared__ float Z[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const int dsub = (lgrp & 1) * 16 + 4 * (j16 & 3);
  const int ntok_max = max(d.n, d.L);
  const int tiles = (ntok_max + tt - 1) / tt;
  int w = blockIdx.x;
  const int tile = w % tiles; w /= tiles;
  const int g = w % (d.T + 1); w /= (d.T + 1);
  const int h = w % d.H;
  const int b = w / d.H;
  const bool text = g == d.T;
  const int ntok = text ? d.L : d.n;
  if (tile * tt >= ntok) return;  // whole workgroup leaves before any barrier
  const long long so = ((long long)b * d.H + h) * (d.T + 1) + g;

  for (int gi = tid; gi < D * G; gi += 256) {
    const int row = gi / G, col = (gi % G) * 8;
    *(uint4*)&Ah[SW::off(row, col)] = ldg16(dsh + so * D * D + row * D + col);
    *(uint4*)&Al[SW::off(row, col)] = ldg16(dsl + so * D * D + row * D + col);
  }
  if (tid < D) Z[tid] = dsz[so * D + tid];
  __syncthreads();

  const int p_end = min(ntok, (tile + 1) * tt);
  for (int p0 = tile * tt + wave * 32; p0 < p_end; p0 += 4 * 32) {
    const int p = p0 + l32;
    const bool ok = p < p_end;
    const int pc = ok ? p : p0;
    const bf16_t* krow = text ? (const bf16_t*)tk.p + tok_off(tk, b, pc, h)
                              : (const bf16_t*)k.p + tok_off(k, b, (long long)g * d.n + pc, h);
    const bf16_t* vrow = text ? (const bf16_t*)tv.p + tok_off(tv, b, pc, h)
                              : (const bf16_t*)v.p + tok_off(v, b, (long long)g * d.n + pc, h);
    // [M][hid] row offset of the token's head in the gradient buffers
    const long long tok_row = text ? ((long long)b * d.L + pc) : ((long long)b * d.N + (long long)g * d.n + pc);
    const long long orow = tok_row * d.hid + (long long)h * D;                       // fp32 partials
    const long long wrow = tok_row * (text ? d.hid : ldkv) + (long long)h * D;        // bf16 outputs
    bf16x8 vf[KS], ph[KS], pl[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      vf[s] = __builtin_bit_cast(bf16x8, ldg16(vrow + 8 * half + 16 * s));
      const uint4 u = ldg16(krow + 8 * half + 16 * s);
      const uint32_t* uu = (const uint32_t*)&u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        SPLIT_BF16(phi_f(__uint_as_float(uu[i] << 16)), ph[s][2 * i], pl[s][2 * i]);
        SPLIT_BF16(phi_f(__uint_as_float(uu[i] & 0xffff0000u)), ph[s][2 * i + 1], pl[s][2 * i + 1]);
      }
    }
    const float* ks_ = text ? dtks : dks;
    const float* vs_ = text ? dtvs : dvs;
    bf16_t* ko = text ? dtk : dk;
    bf16_t* vo = text ? dtv : dv;
    // dk
#pragma unroll 1
    for (int i = 0; i < DB; ++i) {
      floatx16 acc = zero16();
      const int r = i * 32 + l32;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 ah = *(const bf16x8*)&Ah[SW::off(r, 16 * s + 8 * half)];
        const bf16x8 al = *(const bf16x8*)&Al[SW::off(r, 16 * s + 8 * half)];
        acc = mfma32(ah, vf[s], acc);
        acc = mfma32(al, vf[s], acc);
      }
      if (ok) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = i * 32 + 8 * jg + 4 * half;
          const float4 k4 = load_bf16x4(krow + d0);
          const float4 s4 = *(const float4*)(ks_ + orow + d0);
          const float o0 = (acc[4 * jg] + Z[d0]) * dphi_f(k4.x) + s4.x;
          const float o1 = (acc[4 * jg + 1] + Z[d0 + 1]) * dphi_f(k4.y) + s4.y;
          const float o2 = (acc[4 * jg + 2] + Z[d0 + 2]) * dphi_f(k4.z) + s4.z;
          const float o3 = (acc[4 * jg + 3] + Z[d0 + 3]) * dphi_f(k4.w) + s4.w;
          *(uint2*)(ko + wrow + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
      }
    }
    // dv
#pragma unroll 1
    for (int i = 0; i < DB; ++i) {
      floatx16 acc = zero16();
      const int col = i * 32 + dsub;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int r0 = 16 * s + 8 * half + (j16 >> 2);
        const bf16x8 ah = tr_pair(&Ah[SW::off(r0, col)], &Ah[SW::off(r0 + 4, col)]);
        const bf16x8 al = tr_pair(&Al[SW::off(r0, col)], &Al[SW::off(r0 + 4, col)]);
        acc = mfma32(ah, ph[s], acc);
        acc = mfma32(ah, pl[s], acc);
        acc = mfma32(al, ph[s], acc);
      }
      if (ok) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int e0 = i * 32 + 8 * jg + 4 * half;
          const float4 s4 = *(const float4*)(vs_ + orow + e0);
          *(uint2*)(vo + wrow + e0) = make_uint2(pack_bf16x2(acc[4 * jg] + s4.x, acc[4 * jg + 1] + s4.y),
                                                 pack_bf16x2(acc[4 * jg + 2] + s4.z, acc[4 * jg + 3] + s4.w));
        }
      }
    }
  }
}

hipError_t launch_linear_backward(const Dims& d, const BwdArgs& a, hipStream_t s) {
  const int tt = 512;
  {
    const long long grid = (long long)d.B * d.H * d.T * ((d.n + tt - 1) / tt);
    if (d.D == 128)
      hipLaunchKernelGGL(k_lin_bwd_q<128>, dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.comb_hi, a.comb_lo,
                         a.comb_z, a.eps, tt, a.dol, a.dq_s, a.dq, a.ld_qkv, a.dnum, a.dden);
    else
      hipLaunchKernelGGL(k_lin_bwd_q<64>, dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.comb_hi, a.comb_lo,
                         a.comb_z, a.eps, tt, a.dol, a.dq_s, a.dq, a.ld_qkv, a.dnum, a.dden);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    hipError_t e = launch_states_weighted(d, a.q, a.dnum, a.dden, a.lin_split, a.lpart, s);
    if (e != hipSuccess) return e;
  }
  {
    const long long E = (long long)d.D * d.D + d.D;
    const long long n = (long long)d.B * d.H * E;
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (d.D == 128)
      hipLaunchKernelGGL(k_lin_bwd_scan<128>, dim3(grid), dim3(256), 0, s, d, a.lpart, a.lin_split, a.dcf, a.dsh,
                         a.dsl, a.dsz);
    else
      hipLaunchKernelGGL(k_lin_bwd_scan<64>, dim3(grid), dim3(256), 0, s, d, a.lpart, a.lin_split, a.dcf, a.dsh,
                         a.dsl, a.dsz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int ntok = d.n > d.L ? d.n : d.L;
    const long long grid = (long long)d.B * d.H * (d.T + 1) * ((ntok + tt - 1) / tt);
    if (d.D == 128)
      hipLaunchKernelGGL(k_lin_bwd_kv<128>, dim3((unsigned)grid), dim3(256), 0, s, d, a.k, a.v, a.tk, a.tv, a.dsh,
                         a.dsl, a.dsz, tt, a.dk_s, a.dv_s, a.dtk_s, a.dtv_s, a.dk, a.dv, a.ld_qkv, a.dtk, a.dtv);
    else
      hipLaunchKernelGGL(k_lin_bwd_kv<64>, dim3((unsigned)grid), dim3(256), 0, s, d, a.k, a.v, a.tk, a.tv, a.dsh,
                         a.dsl, a.dsz, tt, a.dk_s, a.dv_s, a.dtk_s, a.dtv_s, a.dk, a.dv, a.ld_qkv, a.dtk, a.dtv);
    return hipGetLastError();
  }
}

}  // namespace hyb
