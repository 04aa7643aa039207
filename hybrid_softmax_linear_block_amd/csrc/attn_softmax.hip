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
// K/V tiles (KB blocks of 32 keys) are double-buffered in LDS and filled by
// wave-wide direct-to-LDS loads; the 16-byte granules of each row are
// XOR-swizzled by row so that both read patterns are bank-conflict free.
// 4 waves (128 query rows) per workgroup and several workgroups per CU: the
// hardware overlaps one workgroup's matrix phase with another's softmax.
#include "kernels_bf16.h"

namespace hyb {

// Key sequence of one query frame: up to three contiguous video frame ranges
// of S(f) and the text, as 64-key tiles.  Kept in scalars (wave-uniform).
struct KeySeq {
  int st0, ln0, nt0, st1, ln1, nt1, st2, ln2, nt2, ntt, total;
};

template <int BN>
__device__ __forceinline__ KeySeq key_sequence(const Dims& d, int f) {
  const SoftRanges sr = soft_ranges(d.g, f);
  KeySeq ks;
  ks.st0 = sr.lo[0] * d.n;
  ks.ln0 = (sr.hi[0] - sr.lo[0]) * d.n;
  ks.st1 = sr.n > 1 ? sr.lo[1] * d.n : 0;
  ks.ln1 = sr.n > 1 ? (sr.hi[1] - sr.lo[1]) * d.n : 0;
  ks.st2 = sr.n > 2 ? sr.lo[2] * d.n : 0;
  ks.ln2 = sr.n > 2 ? (sr.hi[2] - sr.lo[2]) * d.n : 0;
  ks.nt0 = (ks.ln0 + BN - 1) / BN;
  ks.nt1 = (ks.ln1 + BN - 1) / BN;
  ks.nt2 = (ks.ln2 + BN - 1) / BN;
  ks.ntt = (d.L + BN - 1) / BN;
  ks.total = ks.nt0 + ks.nt1 + ks.nt2 + ks.ntt;
  return ks;
}

// tile t (BN keys) -> first key, number of valid keys, text or video
template <int BN>
__device__ __forceinline__ void locate(const KeySeq& ks, int L, int t, int& key0, int& valid, bool& text) {
  text = false;
  if (t < ks.nt0) { key0 = ks.st0 + t * BN; valid = min(BN, ks.ln0 - t * BN); return; }
  t -= ks.nt0;
  if (t < ks.nt1) { key0 = ks.st1 + t * BN; valid = min(BN, ks.ln1 - t * BN); return; }
  t -= ks.nt1;
  if (t < ks.nt2) { key0 = ks.st2 + t * BN; valid = min(BN, ks.ln2 - t * BN); return; }
  t -= ks.nt2;
  text = true;
  key0 = t * BN;
  valid = min(BN, L - t * BN);
}

template <int BN>
__device__ __forceinline__ int tile_valid(const KeySeq& ks, int L, int t) {
  int key0, valid;
  bool text;
  locate<BN>(ks, L, t, key0, valid, text);
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

// Tile loader: a tile is KB blocks of 32 keys.
template <int D, int NW, int KB>
struct TileCtx {
  static constexpr int G = D / 8;           // 16-byte granules per row
  static constexpr int BN = 32 * KB;       // keys per tile
  static constexpr int RPC = 64 / G;        // rows per 1 KB chunk (one wave-wide LDS-DMA load)
  static constexpr int CHUNKS = BN / RPC;   // chunks per tile
  static constexpr int CPW = CHUNKS / NW;   // chunks per wave
  static constexpr int TILE = BN * D;       // elements per tile
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
    locate<BN>(ks, d.L, t, key0, valid, text);
    const Tensor4& src = text ? tx : x;
    const char* base = (const char*)((const bf16_t*)src.p + tok_off(src, b, key0, h));
    const unsigned st2 = text ? st_t : st_x;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const unsigned rs = valid == BN ? lrow[i] : min(lrow[i], (unsigned)(valid - 1));
      dma16(base, __umul24(rs, st2) + lcol[i], dst + (wave * CPW + i) * RPC * D);
    }
  }
};

// Softmax of one 32 x (32 KB) score block held as S^T in KB 32x32
// accumulators: masks keys >= valid, updates the lazily rescaled running max
// and the lane's partial row sum, rescales O when the max moved, and emits P as
// the 2 KB bf16 B-operand fragments of the P V product.
template <int KB, int DB>
__device__ __forceinline__ void softmax_tile(floatx16 (&s)[KB], int valid, int half, float sl2, float& m_run,
                                             float& l_run, floatx16 (&oacc)[DB], bf16x8 (&pf)[2 * KB]) {
  if (valid < 32 * KB) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        if (key >= valid) s[kb][j] = -INFINITY;
      }
  }
  float mk[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    mk[kb] = fmaxf(fmaxf(s[kb][0], s[kb][1]), s[kb][2]);
#pragma unroll
    for (int j = 3; j < 15; j += 2) mk[kb] = fmaxf(fmaxf(mk[kb], s[kb][j]), s[kb][j + 1]);
    mk[kb] = fmaxf(mk[kb], s[kb][15]);
  }
  float mx = mk[0];
#pragma unroll
  for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, mk[kb]);
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
  for (int kb = 0; kb < KB; ++kb)
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
// 4 waves, 128 query rows per workgroup; WPE workgroups' waves per SIMD.
template <int D, int KB, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WPE, WPE)))
void k_attn_bf16(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, float sl2,
                 float* __restrict__ os) {
  constexpr int NW = 4, BM = 32 * NW, KS = D / 16, DB = D / 32, BN = 32 * KB;
  using Ctx = TileCtx<D, NW, KB>;
  using SW = Swz<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ctx::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][Ctx::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const Item it = decode_item(d, (d.n + BM - 1) / BM);
  const KeySeq ks = key_sequence<BN>(d, it.f);

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
  const int dsub = (lgrp & 1) * 16 + 4 * (j16 & 3);

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
    // ---- S^T = K Q^T: KB blocks of 32 keys
    floatx16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = zero16();
      const int row = kb * 32 + l32;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bf16x8 a = *(const bf16x8*)&Ks[buf][SW::off(row, 16 * st + 8 * half)];
        s[kb] = mfma32(a, qf[st], s[kb]);
      }
    }
    bf16x8 pf[2 * KB];
    softmax_tile<KB, DB>(s, tile_valid<BN>(ks, d.L, t), half, sl2, m_run, l_run, oacc, pf);
    // ---- O^T += V^T P^T; V^T operand via transposing LDS reads
#pragma unroll
    for (int kk = 0; kk < 2 * KB; ++kk) {
      const int kb0 = (kk >> 1) * 32 + (kk & 1) * 16 + 4 * half + (j16 >> 2);
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const int col = i * 32 + dsub;
        const bf16x8 a = tr_pair(&Vs[buf][SW::off(kb0, col)], &Vs[buf][SW::off(kb0 + 8, col)]);
        oacc[i] = mfma32(a, pf[kk], oacc[i]);
      }
    }
    wait_vmcnt<0>();  // this wave's loads of tile t+1 landed
    tile_barrier();
  }
  store_rows<D>(oacc, l_run, row_ok, os + (((long long)it.b * d.N + qtok) * d.H + it.h) * D, half);
}

template <int D, int KB, int WPE>
static hipError_t launch_attn(const Dims& d, const Bf16Args& a, hipStream_t s) {
  const long long grid = (long long)((d.n + 127) / 128) * d.H * d.B * d.T;
  hipLaunchKernelGGL((k_attn_bf16<D, KB, WPE>), dim3((unsigned)grid), dim3(256), 0, s, d, a.q, a.k, a.v, a.tk,
                     a.tv, a.scale_log2, a.os);
  return hipGetLastError();
}

hipError_t launch_softmax_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  if (d.D == 128) return launch_attn<128, 2, 2>(d, a, s);
  if (d.D == 64) return launch_attn<64, 2, 2>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hyb
