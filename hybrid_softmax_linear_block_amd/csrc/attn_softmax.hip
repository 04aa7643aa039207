// Softmax branch of the hybrid layer on bf16 MFMA: block-sparse flash
// attention over the key frames S(f) of the query's frame plus all text tokens.
//
// VDN-H3 article (tahou.com), section "双分支混合注意力机制": exact softmax
// attention inside the local window (chunks of consecutive latent frames, a
// chunk seeing itself and its neighbouring chunks), the first/last frames as
// anchors read by every frame, and the text tokens visible from every frame.
// Frames outside S(f) are never loaded: the key sequence of a work item is the
// (at most three) contiguous frame ranges of S(f) followed by the text.
//
// Work item = (query frame, batch, head, query tile inside the frame).  Items
// of anchor frames (every frame visible, the longest) are issued first, and
// all tiles of one (frame, batch, head) run on one XCD so that their common
// key tiles are fetched into that XCD's L2 once.  Each wave owns 32 query
// rows.  Per 64-key tile:
//   S^T = K Q^T  (32x32x16 MFMA), so each lane holds 32 scores of ONE query
//   row: row max / sum are per-lane plus one exchange with lane l^32;
//   O^T += V^T P^T with P taken straight from the score registers and V^T
//   read from the row-major V tile by ds_read_b64_tr_b16 in the matching key
//   order -- no transposes anywhere.
// K/V tiles are double-buffered in LDS and filled by wave-wide direct-to-LDS
// loads; the 16-byte granules of each row are XOR-swizzled by row so that both
// read patterns are bank-conflict free.
//
// Two schedules:
//   k_attn_bf16     4 waves (128 rows) per workgroup, two workgroups per CU;
//                   the hardware overlaps one workgroup's matrix phase with
//                   the other's softmax.
//   k_attn_bf16_pp  8 waves (256 rows) in two groups that alternate phases at
//                   every barrier ("ping-pong"): while group A issues the
//                   MFMAs of S(t) and P V(t-1), group B runs its softmax on the
//                   vector ALUs, so each SIMD always holds one wave of each.
#include "kernels_bf16.h"

namespace hyb {

// Key sequence of one query frame: up to three contiguous video frame ranges
// of S(f) and the text, as 64-key tiles.  Kept in scalars (wave-uniform).
struct KeySeq {
  int st0, ln0, nt0, st1, ln1, nt1, st2, ln2, nt2, ntt, total;
};

__device__ __forceinline__ KeySeq key_sequence(const Dims& d, int f) {
  const SoftRanges sr = soft_ranges(d.g, f);
  KeySeq ks;
  ks.st0 = sr.lo[0] * d.n;
  ks.ln0 = (sr.hi[0] - sr.lo[0]) * d.n;
  ks.st1 = sr.n > 1 ? sr.lo[1] * d.n : 0;
  ks.ln1 = sr.n > 1 ? (sr.hi[1] - sr.lo[1]) * d.n : 0;
  ks.st2 = sr.n > 2 ? sr.lo[2] * d.n : 0;
  ks.ln2 = sr.n > 2 ? (sr.hi[2] - sr.lo[2]) * d.n : 0;
  ks.nt0 = (ks.ln0 + 63) >> 6;
  ks.nt1 = (ks.ln1 + 63) >> 6;
  ks.nt2 = (ks.ln2 + 63) >> 6;
  ks.ntt = (d.L + 63) >> 6;
  ks.total = ks.nt0 + ks.nt1 + ks.nt2 + ks.ntt;
  return ks;
}

// tile t -> first key, number of valid keys, text or video
__device__ __forceinline__ void locate(const KeySeq& ks, int L, int t, int& key0, int& valid, bool& text) {
  text = false;
  if (t < ks.nt0) { key0 = ks.st0 + t * 64; valid = min(64, ks.ln0 - t * 64); return; }
  t -= ks.nt0;
  if (t < ks.nt1) { key0 = ks.st1 + t * 64; valid = min(64, ks.ln1 - t * 64); return; }
  t -= ks.nt1;
  if (t < ks.nt2) { key0 = ks.st2 + t * 64; valid = min(64, ks.ln2 - t * 64); return; }
  t -= ks.nt2;
  text = true;
  key0 = t * 64;
  valid = min(64, L - t * 64);
}

__device__ __forceinline__ int tile_valid(const KeySeq& ks, int L, int t) {
  int key0, valid;
  bool text;
  locate(ks, L, t, key0, valid, text);
  return valid;
}

// Work item of workgroup blockIdx.x.  A group = all query tiles of one
// (frame, b, h).  Groups are ordered longest first (anchor frames) and dealt
// to the 8 XCDs round-robin; within an XCD a group's tiles run back to back.
// (Workgroup i is dispatched to XCD i % 8.)
struct Item {
  int qt, h, b, f;
};

__device__ __forceinline__ Item decode_item(const Dims& d, int qtiles) {
  const unsigned ngroups = (unsigned)d.T * d.B * d.H;
  const unsigned nfull = (ngroups / 8u) * 8u * (unsigned)qtiles;
  unsigned grp, qtu;
  if (blockIdx.x < nfull) {
    const unsigned local = blockIdx.x >> 3;
    grp = (local / qtiles) * 8u + (blockIdx.x & 7u);
    qtu = local % qtiles;
  } else {
    grp = blockIdx.x / qtiles;
    qtu = blockIdx.x % qtiles;
  }
  Item it;
  it.qt = (int)qtu;
  it.h = grp % d.H;
  it.b = (grp / d.H) % d.B;
  it.f = frame_by_cost(d.g, (int)(grp / ((unsigned)d.H * d.B)));
  return it;
}

// Lazy rescaling: the running maximum only moves when a row's tile maximum
// exceeds it by more than 2^8 (log2 units); probabilities then stay <= 2^8,
// exact enough in bf16 and fp32, and the O rescale is skipped on most tiles.
constexpr float kRescaleSlack = 8.f;

// Per-lane LDS byte addresses in a swizzled [rows][D] bf16 tile.  Because
// the swizzle XORs the granule index and the row offset has zero granule
// bits, an address splits into a per-lane base XOR a per-step constant:
//   K/Q fragment (row, granule 2s + half):  kq_base(row, half) ^ (32 s)
//   V transposing read (row rr + 16 m, granule 4 i + c, byte 8 b):
//                                            v_base(rr, c, b) ^ (64 i) + 16 m rows
template <int D>
struct LaneAddr {
  __device__ static __forceinline__ unsigned kq_base(int row, int half) {
    return (unsigned)(row * 2 * D + 16 * (half ^ Swz<D>::key(row)));
  }
  __device__ static __forceinline__ unsigned v_base(int rr, int c, int bsel) {
    return (unsigned)(rr * 2 * D + 16 * (c ^ Swz<D>::key(rr)) + 8 * bsel);
  }
};

// Keeps a value opaque to loop-invariant code motion, so that addresses
// derived from it are recomputed per use (one v_xor) instead of being
// precomputed into dozens of registers.
__device__ __forceinline__ unsigned opaque(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Tile loader shared by the two kernels.
template <int D, int NW>
struct TileCtx {
  static constexpr int G = D / 8;           // 16-byte granules per row
  static constexpr int RPC = 64 / G;        // rows per 1 KB chunk (one wave-wide LDS-DMA load)
  static constexpr int CHUNKS = 64 / RPC;   // chunks per 64-key tile
  static constexpr int CPW = CHUNKS / NW;   // chunks per wave
  static constexpr int TILE = 64 * D;       // elements per tile
  static_assert(CHUNKS % NW == 0, "tile chunks must split evenly over waves");

  unsigned lrow[CPW], lcol[CPW];  // per chunk: row in tile, byte offset of the logical granule
  unsigned kst2, vst2, tkst2, tvst2;

  __device__ __forceinline__ void init(int wave, int lane, const Tensor4& k, const Tensor4& v, const Tensor4& tk,
                                       const Tensor4& tv) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      lrow[i] = (unsigned)((wave * CPW + i) * RPC + lane / G);
      lcol[i] = (unsigned)(((lane % G) ^ Swz<D>::key((int)lrow[i])) * 16);
    }
    kst2 = (unsigned)(k.st * 2);  // byte strides (< 2^18, host-checked)
    vst2 = (unsigned)(v.st * 2);
    tkst2 = (unsigned)(tk.st * 2);
    tvst2 = (unsigned)(tv.st * 2);
  }

  // Wave-wide direct-to-LDS loads of this wave's chunks of tile t.  Lane l of
  // a chunk fills row (l / G), physical granule (l % G), which holds logical
  // granule (l % G) ^ swizzle(row).  Rows past the tile's valid keys repeat the
  // last valid row (their scores are masked to -inf).
  __device__ __forceinline__ void load(const KeySeq& ks, const Dims& d, int b, int h, int wave, const Tensor4& x,
                                       const Tensor4& tx, unsigned st_x, unsigned st_t, bf16_t* dst, int t) const {
    int key0, valid;
    bool text;
    locate(ks, d.L, t, key0, valid, text);
    const Tensor4& src = text ? tx : x;
    const char* base = (const char*)((const bf16_t*)src.p + tok_off(src, b, key0, h));
    const unsigned st2 = text ? st_t : st_x;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const unsigned rs = valid == 64 ? lrow[i] : min(lrow[i], (unsigned)(valid - 1));
      dma16(base, __umul24(rs, st2) + lcol[i], dst + (wave * CPW + i) * RPC * D);
    }
  }
};

// Softmax of one 32 x 64 score block held as S^T in two 32x32 accumulators:
// masks keys >= valid, updates the lazily rescaled running max and the lane's
// partial row sum, rescales O when the max moved, and emits P as the four bf16
// B-operand fragments of the P V product.
template <int DB>
__device__ __forceinline__ void softmax_tile(floatx16 (&s)[2], int valid, int half, float sl2, float& m_run,
                                             float& l_run, floatx16 (&oacc)[DB], bf16x8 (&pf)[4]) {
  if (valid < 64) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        if (key >= valid) s[kb][j] = -INFINITY;
      }
  }
  float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
  float m1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
  for (int j = 3; j < 15; j += 2) {
    m0 = fmaxf(fmaxf(m0, s[0][j]), s[0][j + 1]);
    m1 = fmaxf(fmaxf(m1, s[1][j]), s[1][j + 1]);
  }
  float mx = fmaxf(fmaxf(m0, s[0][15]), fmaxf(m1, s[1][15]));
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
  const bool grow = mx > m_run + kRescaleSlack;
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;
  }
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      bf16x8 p;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hb + e], sl2, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hb + e + 1], sl2, -m_run));
        ls0 += p0;
        ls1 += p1;
        p[e] = static_cast<__bf16>(p0);
        p[e + 1] = static_cast<__bf16>(p1);
      }
      pf[2 * kb + hb] = p;
    }
  l_run += ls0 + ls1;
}

// O^T += V^T P^T for one 64-key tile; vt = the tile's LDS bytes.
template <int D>
__device__ __forceinline__ void pv_tile(const char* vt, unsigned vb0, unsigned vb1, const bf16x8 (&pf)[4],
                                        floatx16 (&oacc)[D / 32]) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int m = (kk >> 1) * 2 + (kk & 1);  // row offset in units of 16 rows
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      const bf16x8 a = tr_pair((const bf16_t*)(vt + ((vb0 ^ (64u * i)) + m * 32 * D)),
                               (const bf16_t*)(vt + ((vb1 ^ (64u * i)) + m * 32 * D)));
      oacc[i] = mfma32(a, pf[kk], oacc[i]);
    }
  }
}

// S^T = K Q^T for one 64-key tile (two 32-key blocks); kt = the K tile's LDS
// bytes; Q fragments from registers.
template <int D>
__device__ __forceinline__ void qk_tile(const char* kt, unsigned kb0, const bf16x8 (&qf)[D / 16],
                                        floatx16 (&s)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = zero16();
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8 a = *(const bf16x8*)(kt + ((kb0 ^ (32u * st)) + kb * 64 * D));
      s[kb] = mfma32(a, qf[st], s[kb]);
    }
  }
}

// Normalise O^T by the row sum and store fp32 [B*N][H][D].
template <int D>
__device__ __forceinline__ void store_rows(const floatx16 (&oacc)[D / 32], float l_run, bool row_ok, float* op,
                                           int half) {
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (!row_ok) return;
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = i * 32 + 8 * jg + 4 * half;
      *(float4*)(op + d0) = make_float4(oacc[i][4 * jg] * inv, oacc[i][4 * jg + 1] * inv,
                                        oacc[i][4 * jg + 2] * inv, oacc[i][4 * jg + 3] * inv);
    }
}

// ---------------------------------------------------------------------------
// Plain schedule: 4 waves, 128 query rows, two workgroups per CU.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, float sl2,
                 float* __restrict__ os) {
  constexpr int NW = 4, BM = 32 * NW, KS = D / 16, DB = D / 32;
  using Ctx = TileCtx<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ctx::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][Ctx::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const Item it = decode_item(d, (d.n + BM - 1) / BM);
  const KeySeq ks = key_sequence(d, it.f);

  Ctx ctx;
  ctx.init(wave, lane, k, v, tk, tv);
  ctx.load(ks, d, it.b, it.h, wave, k, tk, ctx.kst2, ctx.tkst2, Ks[0], 0);
  ctx.load(ks, d, it.b, it.h, wave, v, tv, ctx.vst2, ctx.tvst2, Vs[0], 0);

  const int prow = it.qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  const long long qtok = (long long)it.f * d.n + (row_ok ? prow : 0);
  bf16x8 qf[KS];
  {
    const bf16_t* qp = (const bf16_t*)q.p + tok_off(q, it.b, qtok, it.h) + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * s));
  }
  const unsigned kbase = LaneAddr<D>::kq_base(l32, half);
  const int rr = 4 * half + (j16 >> 2);
  const int vc = 2 * (lgrp & 1) + ((j16 & 3) >> 1);
  const unsigned vbase0 = LaneAddr<D>::v_base(rr, vc, j16 & 1);
  const unsigned vbase1 = LaneAddr<D>::v_base(rr + 8, vc, j16 & 1);

  floatx16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  wait_vmcnt<0>();
  tile_barrier();

  for (int t = 0; t < ks.total; ++t) {
    const int buf = t & 1;
    if (t + 1 < ks.total) {
      ctx.load(ks, d, it.b, it.h, wave, k, tk, ctx.kst2, ctx.tkst2, Ks[buf ^ 1], t + 1);
      ctx.load(ks, d, it.b, it.h, wave, v, tv, ctx.vst2, ctx.tvst2, Vs[buf ^ 1], t + 1);
    }
    floatx16 s[2];
    qk_tile<D>((const char*)Ks[buf], opaque(kbase), qf, s);
    bf16x8 pf[4];
    softmax_tile<DB>(s, tile_valid(ks, d.L, t), half, sl2, m_run, l_run, oacc, pf);
    pv_tile<D>((const char*)Vs[buf], opaque(vbase0), opaque(vbase1), pf, oacc);
    wait_vmcnt<0>();  // this wave's loads of tile t+1 landed
    tile_barrier();
  }
  store_rows<D>(oacc, l_run, row_ok, os + (((long long)it.b * d.N + qtok) * d.H + it.h) * D, half);
}

// ---------------------------------------------------------------------------
// Ping-pong schedule: 8 waves, 256 query rows, one workgroup per CU; Q tile in
// LDS.  Phase p: all waves fetch K(t+1), V(t) when p = 2t is even; a group in
// its own phase 2t issues P V(t-1) and S(t), in phase 2t+1 runs softmax(t).
// Group B runs one phase behind group A.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16_pp(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, float sl2,
                    float* __restrict__ os) {
  constexpr int NW = 8, BM = 256, KS = D / 16, DB = D / 32;
  using Ctx = TileCtx<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ctx::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][Ctx::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Qs[BM * D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gab = wave >> 2;  // 0: group A, 1: group B (one phase behind)
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const Item it = decode_item(d, (d.n + BM - 1) / BM);
  const KeySeq ks = key_sequence(d, it.f);
  const int T = ks.total;

  Ctx ctx;
  ctx.init(wave, lane, k, v, tk, tv);
  ctx.load(ks, d, it.b, it.h, wave, k, tk, ctx.kst2, ctx.tkst2, Ks[0], 0);
  {  // Q tile -> LDS: each wave loads its own 32 rows
    const int valid = min(BM, d.n - it.qt * BM);
    const char* qb = (const char*)((const bf16_t*)q.p + tok_off(q, it.b, (long long)it.f * d.n + it.qt * BM, it.h));
    const unsigned qst2 = (unsigned)(q.st * 2);
#pragma unroll
    for (int i = 0; i < 32 / Ctx::RPC; ++i) {
      const unsigned r = (unsigned)(wave * 32 + i * Ctx::RPC + lane / Ctx::G);
      const unsigned rs = min(r, (unsigned)(valid - 1));
      const unsigned col = (unsigned)(((lane % Ctx::G) ^ Swz<D>::key((int)r)) * 16);
      dma16(qb, __umul24(rs, qst2) + col, Qs + (wave * 32 + i * Ctx::RPC) * D);
    }
  }
  const int prow = it.qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  const long long qtok = (long long)it.f * d.n + (row_ok ? prow : 0);
  const unsigned kbase = LaneAddr<D>::kq_base(l32, half);
  const unsigned qbase = LaneAddr<D>::kq_base(wave * 32 + l32, half);
  const int rr = 4 * half + (j16 >> 2);
  const int vc = 2 * (lgrp & 1) + ((j16 & 3) >> 1);
  const unsigned vbase0 = LaneAddr<D>::v_base(rr, vc, j16 & 1);
  const unsigned vbase1 = LaneAddr<D>::v_base(rr + 8, vc, j16 & 1);

  floatx16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  floatx16 sacc[2];
  bf16x8 pf[4];
  float m_run = -INFINITY, l_run = 0.f;

  wait_vmcnt<0>();
  tile_barrier();

  for (int p = 0; p < 2 * T + 2; ++p) {
    if ((p & 1) == 0) {  // all waves: fetch K(t+1) and V(t), t = p / 2
      const int t = p >> 1;
      if (t + 1 < T) ctx.load(ks, d, it.b, it.h, wave, k, tk, ctx.kst2, ctx.tkst2, Ks[(t + 1) & 1], t + 1);
      if (t < T) ctx.load(ks, d, it.b, it.h, wave, v, tv, ctx.vst2, ctx.tvst2, Vs[t & 1], t);
    }
    const int ph = p - gab;  // this group's own phase
    if (ph >= 0 && (ph & 1) == 0) {
      // ---- matrix phase: P V(t-1), then S(t)
      const int t = ph >> 1;
      __builtin_amdgcn_s_setprio(1);
      if (t >= 1) pv_tile<D>((const char*)Vs[(t - 1) & 1], opaque(vbase0), opaque(vbase1), pf, oacc);
      if (t < T) {
        const char* kt = (const char*)Ks[t & 1];
        const char* qt_ = (const char*)Qs;
        const unsigned kb0 = opaque(kbase), qb0 = opaque(qbase);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sacc[kb] = zero16();
#pragma unroll
          for (int st = 0; st < KS; ++st) {
            const bf16x8 a = *(const bf16x8*)(kt + ((kb0 ^ (32u * st)) + kb * 64 * D));
            const bf16x8 qv = *(const bf16x8*)(qt_ + (qb0 ^ (32u * st)));
            sacc[kb] = mfma32(a, qv, sacc[kb]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
    } else if (ph >= 0 && (ph >> 1) < T) {
      // ---- vector phase: softmax of S(t) -> P(t)
      softmax_tile<DB>(sacc, tile_valid(ks, d.L, ph >> 1), half, sl2, m_run, l_run, oacc, pf);
    }
    if (p & 1) wait_vmcnt<0>();  // this wave's loads of the previous even phase landed
    tile_barrier();
  }
  store_rows<D>(oacc, l_run, row_ok, os + (((long long)it.b * d.N + qtok) * d.H + it.h) * D, half);
}

template <int D>
static hipError_t launch_attn(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long grid = (long long)((d.n + 127) / 128) * d.H * d.B * d.T;
  hipLaunchKernelGGL((k_attn_bf16<D>), dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.k, a.v, a.tk, a.tv,
                     a.scale_log2, a.os);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_attn_pp(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long grid = (long long)((d.n + 255) / 256) * d.H * d.B * d.T;
  hipLaunchKernelGGL((k_attn_bf16_pp<D>), dim3((unsigned)grid), dim3(512), 0, s, d, a.q, a.k, a.v, a.tk, a.tv,
                     a.scale_log2, a.os);
  return hipGetLastError();
}

hipError_t launch_softmax_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  if (d.D == 128) return launch_attn<128>(d, a, s);
  if (d.D == 64) return launch_attn<64>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hyb
