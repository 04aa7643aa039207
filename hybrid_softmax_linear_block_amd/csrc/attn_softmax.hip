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
// 4 waves (128 query rows) per workgroup, two workgroups per CU.  The loop is
// software-pipelined (S of the next tile is computed while the current
// tile's probabilities are formed) so that each wave's instruction stream
// mixes matrix and vector work evenly.
#include <type_traits>

#include "attn_tiles.h"
#include "work_items.h"

namespace hyb {

// Lazy rescaling: the running maximum only moves when a row's tile maximum
// exceeds it by more than 2^8 (log2 units); probabilities then stay <= 2^8,
// exact enough in bf16 and fp32, and the O rescale is skipped on most tiles.
constexpr float kRescaleSlack = 8.f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Softmax of one 32 x (32 KB) score block held as S^T in KB 32x32
// accumulators, in four steps: mask keys >= valid (mask_tile), row maximum,
// lazy rescale of the running state, and the probabilities P as the 2 KB bf16
// B-operand fragments of the P V product (plus their row sum).

// Row maximum in log2 units (scaled by sl2), combined over both lane halves.
template <int KB>
__device__ __forceinline__ float tile_max(const floatx16 (&s)[KB], float sl2) {
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
  return xor32_max(mx) * sl2;
}

// Lazy rescale: move the running maximum only when the tile maximum exceeds it
// by more than the slack, and then scale O and the row sum.
template <int DB>
__device__ __forceinline__ void rescale(float mx, float& m_run, float& l_run, floatx16 (&oacc)[DB]) {
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
}

// P = exp2(S sl2 - m) in bf16; the row sum accumulates the bf16-rounded
// probabilities (the weights the P V product uses), two at a time with a bf16
// dot product against (1, 1).
template <int KB>
__device__ __forceinline__ void exp_tile(const floatx16 (&s)[KB], float sl2, float m_run, float& l_run,
                                         bf16x8 (&pf)[2 * KB]) {
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      bf16x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[kb][8 * hb + e], sl2, -m_run)));
      pf[2 * kb + hb] = p;
      const uint4 pw = __builtin_bit_cast(uint4, p);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.x), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.y), ones, ls1, false);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.z), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw.w), ones, ls1, false);
    }
  l_run += ls0 + ls1;
}

// Normalise O^T by the row sum and store fp16 [B*N][H][D].  O is a convex
// combination of value rows, so it lies in the fp16 range whenever V does.
// With lse non-null, also the row's log2-sum-exp2 of the scaled scores,
// m + log2(sum), which the backward pass uses to recompute P.
template <int D>
__device__ __forceinline__ void store_rows(const floatx16 (&oacc)[D / 32], float m_run, float l_run, bool row_ok,
                                           uint16_t* op, float* lse, int half) {
  const float l_tot = xor32_sum(l_run);
  const float inv = 1.f / l_tot;
  if (!row_ok) return;
  if (lse && half == 0) *lse = m_run + __log2f(l_tot);
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = i * 32 + 8 * jg + 4 * half;
      store_f16x4(op + d0, oacc[i][4 * jg] * inv, oacc[i][4 * jg + 1] * inv, oacc[i][4 * jg + 2] * inv,
                  oacc[i][4 * jg + 3] * inv);
    }
}

// ---------------------------------------------------------------------------
// Software-pipelined schedule, same work split.  Iteration t issues the
// S = K Q^T MFMAs of tile t+1 interleaved with the exp work of tile t, then
// the P V MFMAs of tile t interleaved with the row maximum of tile t+1, so each
// wave's instruction stream mixes matrix and vector work evenly (the order is
// pinned with scheduling-group barriers).  The row maximum is taken before the
// tail mask: padded key rows repeat the last valid key, so they cannot raise
// it.  K tiles are loaded two tiles ahead and V tiles one tile ahead, with one
// barrier per tile.
// NW waves (32 query rows each) per workgroup; PF: LDS operand reads issued
// ahead of the MFMA that consumes them.
template <int D, int KB, int NW, int PF>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16_sp(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, float sl2,
                    uint16_t* __restrict__ os, float* __restrict__ lse) {
  constexpr int BM = 32 * NW, KS = D / 16, DB = D / 32, BN = 32 * KB;
  constexpr int NMF = KB * KS;  // MFMAs per S tile (= per P V tile)
  using Ldr = TileLoader<D, NW, KB>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ldr::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][Ldr::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5, j16 = lane & 15, lgrp = lane >> 4;
  const Item it = decode_item(d, (d.n + BM - 1) / BM);

  // kwk: next K tile to load, kwv: next V tile to load.  S(f) always holds
  // the query's own frame, so there is at least one tile.
  KeyWalk<BN> kwk;
  kwk.init(d, it.f, it.b, it.h, k, v, tk, tv);
  KeyWalk<BN> kwv = kwk;
  Ldr ldr;
  ldr.init(wave, lane);
  ldr.set_k(kwk.ks);
  ldr.set_v(kwv.vs);
  const unsigned ks_lds = lds_addr(Ks), vs_lds = lds_addr(Vs);
  constexpr unsigned kTileBytes = Ldr::TILE * 2;

  const int valid0 = kwk.valid();
  ldr.load_k(kwk.kp, valid0, wave, ks_lds);
  if (kwk.advance()) ldr.set_k(kwk.ks);
  ldr.load_v(kwv.vp, valid0, wave, vs_lds);
  if (kwv.advance()) ldr.set_v(kwv.vs);
  int vnext = 0;
  if (!kwk.done()) {
    vnext = kwk.valid();
    ldr.load_k(kwk.kp, vnext, wave, ks_lds + kTileBytes);
    if (kwk.advance()) ldr.set_k(kwk.ks);
  }

  const int prow = it.qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  // a wave whose 32 rows all lie past the frame's end (the second half of a
  // frame's last tile when n % BM == 64) only loads tiles and joins barriers
  const bool idle = it.qt * BM + wave * 32 >= d.n;
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
  floatx16 s[KB];
  float mx = 0.f;
  if (!idle) {
    qk_tile<D, KB>(s, Ks[0], qf, l32, half);
    mx = tile_max<KB>(s, sl2);
  }
  int vcur = valid0;
  tile_barrier();  // K buffer 0 is refilled below

  auto step = [&](auto bufc) -> bool {
    constexpr int BUF = decltype(bufc)::value;
    if (kwv.done()) return false;  // no tile t + 1
    // K_{t+2} -> K buffer of tile t, V_{t+1} -> V buffer of tile t-1
    int vk = 0;
    if (!kwk.done()) {
      vk = kwk.valid();
      ldr.load_k(kwk.kp, vk, wave, ks_lds + BUF * kTileBytes);
      if (kwk.advance()) ldr.set_k(kwk.ks);
    }
    ldr.load_v(kwv.vp, kwv.valid(), wave, vs_lds + (BUF ^ 1) * kTileBytes);
    if (kwv.advance()) ldr.set_v(kwv.vs);
    if (idle) {
      vcur = vnext;
      vnext = vk;
      wait_vmcnt<0>();
      tile_barrier();
      return true;
    }

    rescale<DB>(mx, m_run, l_run, oacc);
    if (vcur < BN) mask_tile<KB>(s, vcur, half);
    // S(t+1) = K(t+1) Q^T  ||  P(t) = exp(S(t))
    floatx16 sn[KB];
    qk_tile<D, KB>(sn, Ks[BUF ^ 1], qf, l32, half);
    bf16x8 pf[2 * KB];
    exp_tile<KB>(s, sl2, m_run, l_run, pf);
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // LDS reads ahead
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
    }
    // O += P(t) V(t)  ||  row max of S(t+1)
    pv_tile<D, KB>(oacc, Vs[BUF], pf, half, j16, dsub);
    mx = tile_max<KB>(sn, sl2);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);  // LDS reads ahead
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = sn[kb];
    vcur = vnext;
    vnext = vk;
    wait_vmcnt<0>();  // this wave's loads of K_{t+2}, V_{t+1} landed
    tile_barrier();
    return true;
  };
  int last = 0;
  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) {
      last = 1;
      break;
    }
  }
  if (idle) return;
  rescale<DB>(mx, m_run, l_run, oacc);
  if (vcur < BN) mask_tile<KB>(s, vcur, half);
  bf16x8 pf[2 * KB];
  exp_tile<KB>(s, sl2, m_run, l_run, pf);
  pv_tile<D, KB>(oacc, last ? Vs[1] : Vs[0], pf, half, j16, dsub);
  store_rows<D>(oacc, m_run, l_run, row_ok, os + (((long long)it.b * d.N + qtok) * d.H + it.h) * D,
                lse ? lse + ((long long)it.b * d.H + it.h) * d.N + qtok : nullptr, half);
}

template <int D, int KB, int NW, int PF>
static hipError_t launch_attn_sp(const Dims& d, const Bf16Args& a, hipStream_t s) {
  constexpr int BM = 32 * NW;
  const long long grid = (long long)((d.n + BM - 1) / BM) * d.H * d.B * d.T;
  hipLaunchKernelGGL((k_attn_bf16_sp<D, KB, NW, PF>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v,
                     a.tk, a.tv, a.scale_log2, a.os, a.lse);
  return hipGetLastError();
}

hipError_t launch_softmax_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  if (d.D == 128) return launch_attn_sp<128, 2, 4, 2>(d, a, s);
  if (d.D == 64) return launch_attn_sp<64, 2, 4, 2>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hyb
