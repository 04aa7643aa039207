// Linear branch of the hybrid layer: per-frame states, the prefix/suffix scan
// across frames, and the phi(Q) readout.
//
// VDN-H3 article (tahou.com), section "双分支混合注意力机制": the linear branch
// keeps a forward state summing the context before the local window and a
// backward state summing the context after it (window and anchor frames left
// out); text is written half into each state, and merging the two reads counts
// it once; the states are read at the query's position.  The article's intro
// calls this attention "updated frame by frame", which is what the per-frame
// states + scan do.  With phi(u) = elu(u) + 1:
//   S_g = sum_{t in g} phi(k_t) v_t^T,  z_g = sum_{t in g} phi(k_t)
//   comb(f) = S_T + sum_{g in F(f)} S_g + sum_{g in B(f)} S_g   (1/2 S_T + 1/2 S_T)
//   O_l = phi(q)^T comb(f) / (phi(q)^T z_comb(f) + eps)
#include "kernels_bf16.h"

namespace hyb {

// ---------------------------------------------------------------------------
// State build on MFMA: C[d][e] = sum_t phi(K)[t][d] V[t][e].  The contraction
// runs over tokens, so both operands come from row-major LDS tiles through
// the transposing LDS read.  phi(K) is a computed value: it is split into bf16
// hi + lo and both halves are multiplied (V is exact in bf16), so the states
// carry near-fp32 products -- the backward pass differentiates through
// C - c O, which cancels most of C and would magnify a bf16 rounding of phi(K).  One workgroup = (b, h, slot); a slot is one token
// split of one frame, or one split of the text.  Output per slot (fp32):
// S transposed [e][d] followed by z[d].  With ZW, z accumulates
// phi(K)[t][d] * zw[t] (per-token weights [B*N][H]); the backward pass uses
// this form for dC = sum phi(q) dnum^T and dc = sum phi(q) dden.
template <int D, bool ZW = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2))) void k_states_bf16(Dims d, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv,
                                                     int split, int ts, float* __restrict__ part, int slots,
                                                     const float* __restrict__ zw) {
  constexpr int G = D / 8, GPT = (64 * G) / 256, DB = D / 32;
  constexpr int NB = (DB * DB) / 4;  // 32x32 output blocks per wave
  using SW = Swz<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t Kl[64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[64 * D];
  __shared__ float zred[256 / G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5, grp = lane >> 4, j16 = lane & 15;

  int w = blockIdx.x;
  const int slot = w % slots; w /= slots;
  const int h = w % d.H;
  const int b = w / d.H;
  const bool text = slot >= d.T * split;
  long long t0;
  int cnt;
  if (!text) {
    const int g = slot / split, p = slot % split;
    t0 = (long long)g * d.n + (long long)p * ts;
    cnt = min(ts, d.n - p * ts);
  } else {
    const int p = slot - d.T * split;
    t0 = (long long)p * ts;
    cnt = min(ts, d.L - p * ts);
  }
  if (cnt < 0) cnt = 0;
  // select field by field (a select between the two structs would put them
  // in scratch memory)
  const long long kst = text ? tk.st : k.st, vst = text ? tv.st : v.st;
  const bf16_t* kbase = text ? (const bf16_t*)tk.p + tok_off(tk, b, t0, h) : (const bf16_t*)k.p + tok_off(k, b, t0, h);
  const bf16_t* vbase = text ? (const bf16_t*)tv.p + tok_off(tv, b, t0, h) : (const bf16_t*)v.p + tok_off(v, b, t0, h);

  // block assignment: wave covers output blocks (mb, nb) = blk / DB, blk % DB
  floatx16 acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = zero16();
  float zacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) zacc[i] = 0.f;

  const int ntile = (cnt + 63) >> 6;
  // tile loads go to registers one tile ahead: the next tile's loads are in
  // flight while the current tile is multiplied
  uint4 kr[GPT], vr[GPT];
  float wr[GPT];
  auto load = [&](int tile) {
    const int valid = min(64, cnt - tile * 64);
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int gi = tid + r * 256, row = gi / G, col = (gi % G) * 8;
      if (row < valid) {
        kr[r] = ldg16(kbase + (long long)(tile * 64 + row) * kst + col);
        vr[r] = ldg16(vbase + (long long)(tile * 64 + row) * vst + col);
        if constexpr (ZW) wr[r] = zw[((long long)b * d.N + t0 + tile * 64 + row) * d.H + h];
      } else {
        kr[r] = make_uint4(0, 0, 0, 0);
        vr[r] = make_uint4(0, 0, 0, 0);
        if constexpr (ZW) wr[r] = 0.f;
      }
    }
  };
  if (ntile > 0) load(0);
  for (int tile = 0; tile < ntile; ++tile) {
    const int valid = min(64, cnt - tile * 64);
    __syncthreads();  // previous tile's reads are done
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int gi = tid + r * 256, row = gi / G, col = (gi % G) * 8;
      const bool ok = row < valid;
      const uint32_t* u = (const uint32_t*)&kr[r];
      uint32_t o[4], ol[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = ok ? phi_f(__uint_as_float(u[i] << 16)) : 0.f;
        const float hi = ok ? phi_f(__uint_as_float(u[i] & 0xffff0000u)) : 0.f;
        if constexpr (ZW) {
          zacc[2 * i] = fmaf(lo, wr[r], zacc[2 * i]);
          zacc[2 * i + 1] = fmaf(hi, wr[r], zacc[2 * i + 1]);
        } else {
          zacc[2 * i] += lo;
          zacc[2 * i + 1] += hi;
        }
        o[i] = pack_bf16x2(lo, hi);
        ol[i] = pack_bf16x2(lo - bf16_to_f32((bf16_t)(o[i] & 0xffffu)), hi - bf16_to_f32((bf16_t)(o[i] >> 16)));
      }
      *(uint4*)&Ks[SW::off(row, col)] = make_uint4(o[0], o[1], o[2], o[3]);
      *(uint4*)&Kl[SW::off(row, col)] = make_uint4(ol[0], ol[1], ol[2], ol[3]);
      *(uint4*)&Vs[SW::off(row, col)] = vr[r];
    }
    __syncthreads();
    if (tile + 1 < ntile) load(tile + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      __builtin_amdgcn_sched_barrier(0);  // one 16-token step's operand reads in flight at a time
      const int r0 = kk * 16 + 4 * half + (j16 >> 2);
      const int csub = (grp & 1) * 16 + 4 * (j16 & 3);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int blk = wave * NB + i;
        const int mb = blk / DB, nb = blk % DB;
        const bf16x8 a = tr_pair(&Ks[SW::off(r0, mb * 32 + csub)], &Ks[SW::off(r0 + 8, mb * 32 + csub)]);
        const bf16x8 al = tr_pair(&Kl[SW::off(r0, mb * 32 + csub)], &Kl[SW::off(r0 + 8, mb * 32 + csub)]);
        const bf16x8 bb = tr_pair(&Vs[SW::off(r0, nb * 32 + csub)], &Vs[SW::off(r0 + 8, nb * 32 + csub)]);
        acc[i] = mfma32(a, bb, acc[i]);
        acc[i] = mfma32(al, bb, acc[i]);
      }
    }
  }

  float* out = part + ((long long)(b * d.H + h) * slots + slot) * (D * D + D);
  // acc[i]: lane holds column e = nb*32 + l32, rows d = mb*32 + 8*(j/4) + 4*half + j%4
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = wave * NB + i;
    const int mb = blk / DB, nb = blk % DB;
    const int e = nb * 32 + l32;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = mb * 32 + 8 * jg + 4 * half;
      *(float4*)(out + (long long)e * D + d0) =
          make_float4(acc[i][4 * jg], acc[i][4 * jg + 1], acc[i][4 * jg + 2], acc[i][4 * jg + 3]);
    }
  }
  // z: every thread owns granule column (tid % G); reduce over tid / G
  {
    const int c0 = (tid % G) * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) zred[tid / G][c0 + i] = zacc[i];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int r = 0; r < 256 / G; ++r) s += zred[r][tid];
      out[D * D + tid] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Scan across frames.  F(f) always starts at the first interior frame and
// B(f) always ends at the last, so with s_g the state of interior frame g
// (zero outside [i0, i1)):
//   comb(f) = text + P(fhi(f) - 1) + Q(blo(f)),
//   P(g) = sum_{j <= g} s_j (inclusive prefix),  Q(g) = sum_{j >= g} s_j (inclusive suffix),
// each term present only when F(f), B(f) are non-empty.
//
// One wave per 64 consecutive state elements of one (b, h) (element < D*D is
// S^T[e][d], element >= D*D is z[d]).  The frame states (sums of their split
// partials) are loaded coalesced, lane = element, into a wave-private LDS
// tile [frame][element]; the scans then run across lanes, lane = frame, as
// DPP prefix sums over groups of W lanes (W >= T; 64 / W elements per
// instruction), forward for P and over the reversed frame order for Q; the
// results go back through LDS so that each output frame is stored lane =
// element again: comb = hi + lo bf16 pair (transposed [e][d]) and z_comb in
// fp32.

// Inclusive prefix sum over each group of W consecutive lanes (W = 16, 32,
// 64): four row shifts inside each 16-lane row, then the row broadcasts of
// lanes 15 and 31 into the following rows.
template <int W>
__device__ __forceinline__ float group_prefix(float x) {
  static_assert(W == 16 || W == 32 || W == 64, "scan width");
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));  // row_shr:1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));  // row_shr:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));  // row_shr:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));  // row_shr:8
  if constexpr (W >= 32)  // lane 15 of rows 0 / 2 into rows 1 / 3
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
  if constexpr (W == 64)  // lane 31 into rows 2 and 3
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
  return x;
}

template <int D, int W>
__global__ __launch_bounds__(64) void k_scan_bf16(Dims d, const float* __restrict__ part, int split, int tsplit,
                                                  int slots, bf16_t* __restrict__ chi, bf16_t* __restrict__ clo,
                                                  float* __restrict__ cz) {
  // one wave per workgroup: W x 130 floats of LDS (8.3 KB at W = 16), small
  // enough to run beside the softmax kernel's workgroups
  constexpr int E = D * D + D, NCH = E / 64, RS = 65;  // chunks per (b, h); LDS row stride (floats)
  static_assert(E % 64 == 0 && (D * D) % 64 == 0, "a chunk is all S or all z");
  __shared__ float lds_[2][W * RS];
  const int lane = threadIdx.x;
  const long long gw = blockIdx.x;
  const long long bh = gw / NCH;
  const int e0 = (int)(gw % NCH) * 64, el = e0 + lane;
  float* A = lds_[0];   // frame states, then P in place
  float* Qt = lds_[1];  // Q
  const float* pp = part + bh * slots * (long long)E + el;
  const int T = d.T, i0 = interior_begin(d.g), i1 = interior_end(d.g);

  // frame states, lane = element (all frames' loads of one split in flight together)
  float text = 0.f;
  for (int p = 0; p < tsplit; ++p) text += pp[(long long)(T * split + p) * E];
  float sg[W];
#pragma unroll
  for (int g = 0; g < W; ++g) sg[g] = 0.f;
  for (int p = 0; p < split; ++p) {
#pragma unroll
    for (int g = 0; g < W; ++g)
      if (g >= i0 && g < i1) sg[g] += pp[(long long)(g * split + p) * E];
  }
#pragma unroll
  for (int g = 0; g < W; ++g) A[g * RS + lane] = sg[g];
  asm volatile("" ::: "memory");  // a wave's LDS operations run in order; keep the compiler from reordering

  // scans, lane = frame g of element column j
  constexpr int NG = 64 / W;  // element columns per instruction
  const int g = lane % W, r = lane / W;
#pragma unroll 4
  for (int jb = 0; jb < W; ++jb) {
    const int j = jb * NG + r;
    const float a = A[g * RS + j];
    const float ar = g < T ? A[(T - 1 - g) * RS + j] : 0.f;
    const float P = group_prefix<W>(a), R = group_prefix<W>(ar);
    asm volatile("" ::: "memory");
    A[g * RS + j] = P;
    if (g < T) Qt[(T - 1 - g) * RS + j] = R;
  }
  asm volatile("" ::: "memory");

  // combined states, lane = element
  for (int f = 0; f < T; ++f) {
    int flo, fhi, blo, bhi;
    linear_ranges(d.g, f, &flo, &fhi, &blo, &bhi);
    float val = text;
    if (fhi > flo) val += A[(fhi - 1) * RS + lane];
    if (bhi > blo) val += Qt[blo * RS + lane];
    const long long fo = bh * T + f;
    if (e0 < D * D) {
      const bf16_t hi = f32_to_bf16(val);
      chi[fo * D * D + el] = hi;
      clo[fo * D * D + el] = f32_to_bf16(val - bf16_to_f32(hi));
    } else {
      cz[fo * D + (el - D * D)] = val;
    }
  }
}

// The scan for layouts with more frames than one wave covers (T > 64), one
// thread per (b, h, element):
// pass 1 writes the forward part of every frame to the workspace (pre),
// pass 2 reads it back.
template <int D>
__global__ __launch_bounds__(256) void k_scan_pre_bf16(Dims d, const float* __restrict__ part, int split, int tsplit,
                                                   int slots, float* __restrict__ pre, bf16_t* __restrict__ chi,
                                                   bf16_t* __restrict__ clo, float* __restrict__ cz) {
  constexpr int E = D * D + D;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)d.B * d.H * E) return;
  const int el = (int)(gid % E);
  const long long bh = gid / E;
  const float* pp = part + bh * slots * (long long)E + el;
  auto frame_state = [&](int g) {
    float s = 0.f;
    for (int p = 0; p < split; ++p) s += pp[(long long)(g * split + p) * E];
    return s;
  };
  float text = 0.f;
  for (int p = 0; p < tsplit; ++p) text += pp[(long long)(d.T * split + p) * E];

  float* prow = pre + bh * (long long)d.T * E + el;
  const int i0 = interior_begin(d.g), i1 = interior_end(d.g);
  // pass 1: forward (exclusive prefix up to F's end)
  {
    float P = 0.f;
    int gp = i0;
    for (int f = 0; f < d.T; ++f) {
      int flo, fhi, blo, bhi;
      linear_ranges(d.g, f, &flo, &fhi, &blo, &bhi);
      float val = 0.f;
      if (fhi > flo) {
        while (gp < fhi) { P += frame_state(gp); ++gp; }
        val = P;
      }
      prow[(long long)f * E] = val;
    }
  }
  // pass 2: backward (exclusive suffix from B's start) + text, emit
  {
    float Q = 0.f;
    int gp = i1;
    for (int f = d.T - 1; f >= 0; --f) {
      int flo, fhi, blo, bhi;
      linear_ranges(d.g, f, &flo, &fhi, &blo, &bhi);
      float val = text + prow[(long long)f * E];
      if (bhi > blo) {
        while (gp > blo) { --gp; Q += frame_state(gp); }
        val += Q;
      }
      const long long fo = bh * d.T + f;
      if (el < D * D) {
        const bf16_t hi = f32_to_bf16(val);
        const float rem = val - bf16_to_f32(hi);
        chi[fo * D * D + el] = hi;
        clo[fo * D * D + el] = f32_to_bf16(rem);
      } else {
        cz[fo * D + (el - D * D)] = val;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Readout on MFMA: O^T[e][t] = sum_d comb^T[e][d] phi(Q)^T[d][t].  The comb
// state (hi + lo bf16) of the frame sits in LDS; phi(q) is split into bf16
// hi + lo in registers; three MFMAs per step (hi*hi, hi*lo, lo*hi) keep the
// product near fp32 accuracy.  Lane = one token; the normaliser
// phi(q).z + eps is a per-lane dot product.  Also emits sum_e O_l^2 per
// (token, head) for the RMSNorm.  Work items are 512-token tiles of one
// (b, h, frame).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2))) void k_readout_bf16(Dims d, Tensor4 q, const bf16_t* __restrict__ chi,
                                                      const bf16_t* __restrict__ clo, const float* __restrict__ cz,
                                                      float eps, int tt, uint16_t* __restrict__ ol,
                                                      float* __restrict__ ss) {
  constexpr int G = D / 8, KS = D / 16, DB = D / 32;
  using SW = Swz<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Sh[D * D];
  __shared__ __attribute__((aligned(16))) bf16_t Sl[D * D];
  __shared__ float Z[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int tiles = (d.n + tt - 1) / tt;
  // XCD-aware order: each XCD runs a contiguous range of (b, h, frame, tile)
  // items, so the tiles of one frame share one fetch of its state in that
  // XCD's L2
  int w = (int)xcd_remap(blockIdx.x, gridDim.x);
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
  // q rows of the next 32 tokens are loaded while the current ones are
  // multiplied (the loop is bound by load latency otherwise)
  auto load_q = [&](int pb, uint4 (&u)[KS]) {
    const int pq = min(pb + l32, p_end - 1);
    const bf16_t* qp = (const bf16_t*)q.p + tok_off(q, b, (long long)f * d.n + pq, h) + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) u[s] = ldg16(qp + 16 * s);
  };
  uint4 qr[KS];
  if (tile * tt + wave * 32 < p_end) load_q(tile * tt + wave * 32, qr);
  for (int p0 = tile * tt + wave * 32; p0 < p_end; p0 += 4 * 32) {
    const int p = p0 + l32;
    const bool ok = p < p_end;
    const long long tok = (long long)f * d.n + (ok ? p : p0);
    bf16x8 ph[KS], pl[KS];
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 u = qr[s];
      const uint32_t* uu = (const uint32_t*)&u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = phi_f(__uint_as_float(uu[i] << 16));
        const float a1 = phi_f(__uint_as_float(uu[i] & 0xffff0000u));
        const int dd = 16 * s + 8 * half + 2 * i;
        den = fmaf(a0, Z[dd], den);
        den = fmaf(a1, Z[dd + 1], den);
        const __bf16 h0 = static_cast<__bf16>(a0), h1 = static_cast<__bf16>(a1);
        ph[s][2 * i] = h0;
        ph[s][2 * i + 1] = h1;
        pl[s][2 * i] = static_cast<__bf16>(a0 - static_cast<float>(h0));
        pl[s][2 * i + 1] = static_cast<__bf16>(a1 - static_cast<float>(h1));
      }
    }
    if (p0 + 4 * 32 < p_end) load_q(p0 + 4 * 32, qr);
    den += __shfl_xor(den, 32);
    const float inv = 1.f / (den + eps);
    float sq = 0.f;
    uint16_t* op = ol + (((long long)b * d.N + tok) * d.H + h) * D;
    // one 32-row block of the state at a time (keeps the operand reads of a
    // single block in flight instead of all of them)
#pragma unroll 1
    for (int i = 0; i < DB; ++i) {
      floatx16 acc = zero16();
      const int row = i * 32 + l32;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 ah = *(const bf16x8*)&Sh[SW::off(row, 16 * s + 8 * half)];
        const bf16x8 al = *(const bf16x8*)&Sl[SW::off(row, 16 * s + 8 * half)];
        acc = mfma32(ah, ph[s], acc);
        acc = mfma32(ah, pl[s], acc);
        acc = mfma32(al, ph[s], acc);
      }
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int e0 = i * 32 + 8 * jg + 4 * half;
        float4 o4 = make_float4(acc[4 * jg] * inv, acc[4 * jg + 1] * inv, acc[4 * jg + 2] * inv,
                                acc[4 * jg + 3] * inv);
        sq += o4.x * o4.x + o4.y * o4.y + o4.z * o4.z + o4.w * o4.w;
        if (ok) store_f16x4(op + e0, o4.x, o4.y, o4.z, o4.w);
      }
    }
    sq += __shfl_xor(sq, 32);
    if (ok && half == 0) ss[((long long)b * d.N + tok) * d.H + h] = sq;
  }
}

hipError_t launch_states_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long ts = 64LL * ((((long long)d.n + 63) / 64 + a.state_split - 1) / a.state_split);
  const long long grid = (long long)d.B * d.H * a.state_slots;
  if (d.D == 128)
    hipLaunchKernelGGL((k_states_bf16<128, false>), dim3((unsigned)grid), dim3(256), 0, s, d, a.k, a.v, a.tk, a.tv,
                       a.state_split, (int)ts, a.part, a.state_slots, nullptr);
  else
    hipLaunchKernelGGL((k_states_bf16<64, false>), dim3((unsigned)grid), dim3(256), 0, s, d, a.k, a.v, a.tk, a.tv,
                       a.state_split, (int)ts, a.part, a.state_slots, nullptr);
  return hipGetLastError();
}

template <int D, int W>
static void launch_scan_t(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long waves = (long long)d.B * d.H * ((D * D + D) / 64);
  hipLaunchKernelGGL((k_scan_bf16<D, W>), dim3((unsigned)waves), dim3(64), 0, s, d, a.part, a.state_split,
                     a.text_split, a.state_slots, a.comb_hi, a.comb_lo, a.comb_z);
}

hipError_t launch_scan_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long E = (long long)d.D * d.D + d.D;
  const long long n = (long long)d.B * d.H * E;
  const unsigned grid = (unsigned)((n + 255) / 256);
  // the scan width (lanes per frame group) covers the frame count
  if (d.T <= 16) {
    if (d.D == 128) launch_scan_t<128, 16>(d, a, s); else launch_scan_t<64, 16>(d, a, s);
  } else if (d.T <= 32) {
    if (d.D == 128) launch_scan_t<128, 32>(d, a, s); else launch_scan_t<64, 32>(d, a, s);
  } else if (d.T <= 64) {
    if (d.D == 128) launch_scan_t<128, 64>(d, a, s); else launch_scan_t<64, 64>(d, a, s);
  } else if (d.D == 128) {
    hipLaunchKernelGGL(k_scan_pre_bf16<128>, dim3(grid), dim3(256), 0, s, d, a.part, a.state_split, a.text_split,
                       a.state_slots, a.pre, a.comb_hi, a.comb_lo, a.comb_z);
  } else {
    hipLaunchKernelGGL(k_scan_pre_bf16<64>, dim3(grid), dim3(256), 0, s, d, a.part, a.state_split, a.text_split,
                       a.state_slots, a.pre, a.comb_hi, a.comb_lo, a.comb_z);
  }
  return hipGetLastError();
}

// RMS factor of the linear branch per token: the per-head sums of squares
// from the readout, summed over heads in order, -> 1 / sqrt(mean + eps).
__global__ __launch_bounds__(256) void k_rms_rinv(const float* __restrict__ ss, long long M, int H, int hid, float eps,
                                                  float* __restrict__ rinv) {
  const long long m = (long long)blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  float tot = 0.f;
  for (int h = 0; h < H; ++h) tot += ss[m * H + h];
  rinv[m] = rsqrtf(tot / (float)hid + eps);
}

hipError_t launch_readout_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const int tt = 512;
  const long long grid = (long long)d.B * d.H * d.T * ((d.n + tt - 1) / tt);
  if (d.D == 128)
    hipLaunchKernelGGL(k_readout_bf16<128>, dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.comb_hi, a.comb_lo,
                       a.comb_z, a.eps, tt, a.ol, a.ss);
  else
    hipLaunchKernelGGL(k_readout_bf16<64>, dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.comb_hi, a.comb_lo,
                       a.comb_z, a.eps, tt, a.ol, a.ss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long M = (long long)d.B * d.N;
  hipLaunchKernelGGL(k_rms_rinv, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, a.ss, M, d.H, d.hid, a.eps,
                     a.rinv);
  return hipGetLastError();
}

// Weighted state build over the video tokens only (backward pass): per
// (b, h, frame split) partials of sum_t phi(q_t) dnum_t^T ([e][d]) and
// sum_t phi(q_t) dden_t.  dnum: [B*N][hid] bf16; dden: [B*N][H].
hipError_t launch_states_weighted(const Dims& d, Tensor4 q, const bf16_t* dnum, const float* dden, int split,
                                  float* part, hipStream_t s) {
  const long long ts = 64LL * ((((long long)d.n + 63) / 64 + split - 1) / split);
  const int slots = d.T * split;
  const long long grid = (long long)d.B * d.H * slots;
  Tensor4 dn;
  dn.p = dnum;
  dn.sb = d.N * d.hid;
  dn.st = d.hid;
  dn.sh = d.D;
  if (d.D == 128)
    hipLaunchKernelGGL((k_states_bf16<128, true>), dim3((unsigned)grid), dim3(256), 0, s, d, q, dn, q, dn, split,
                       (int)ts, part, slots, dden);
  else
    hipLaunchKernelGGL((k_states_bf16<64, true>), dim3((unsigned)grid), dim3(256), 0, s, d, q, dn, q, dn, split,
                       (int)ts, part, slots, dden);
  return hipGetLastError();
}

}  // namespace hyb
