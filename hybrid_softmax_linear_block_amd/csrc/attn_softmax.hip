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
// Work item = (query frame, batch, head, BM-row query tile inside the frame);
// items of anchor frames (every frame visible, the longest) are issued first.
// Each wave owns 32 query rows.  Per 64-key tile:
//   S^T = K Q^T  (32x32x16 MFMA, K from LDS, Q^T fragments in registers),
//   so each lane holds 32 scores of ONE query row -> row max/sum are per lane
//   plus one exchange with lane l^32;
//   O^T += V^T P^T with P taken straight from the score registers and V^T
//   read from the row-major V tile by ds_read_b64_tr_b16 in the matching key
//   order -- no transposes anywhere.
// K/V tiles are double-buffered in LDS (one barrier per tile) and prefetched
// into registers one tile ahead.
#include "kernels_bf16.h"

namespace hyb {

struct KeySeq {
  int nseg;
  int start[4], len[4], tiles[4];
  bool text[4];
  int total;
};

__device__ __forceinline__ KeySeq key_sequence(const Dims& d, int f) {
  KeySeq ks;
  const SoftRanges sr = soft_ranges(d.g, f);
  ks.nseg = 0;
  ks.total = 0;
  for (int r = 0; r < sr.n; ++r) {
    ks.start[ks.nseg] = sr.lo[r] * d.n;
    ks.len[ks.nseg] = (sr.hi[r] - sr.lo[r]) * d.n;
    ks.text[ks.nseg] = false;
    ++ks.nseg;
  }
  if (d.L > 0) {
    ks.start[ks.nseg] = 0;
    ks.len[ks.nseg] = d.L;
    ks.text[ks.nseg] = true;
    ++ks.nseg;
  }
  for (int s = 0; s < ks.nseg; ++s) {
    ks.tiles[s] = (ks.len[s] + 63) >> 6;
    ks.total += ks.tiles[s];
  }
  return ks;
}

// frame visiting order: anchors first (they see every frame), then the rest
__device__ __forceinline__ int frame_by_cost(const FrameGeom& g, int i) {
  const bool a0 = g.af;
  const bool a1 = g.al && !(g.af && g.T == 1);
  if (a0) { if (i == 0) return 0; --i; }
  if (a1) { if (i == 0) return g.T - 1; --i; }
  return interior_begin(g) + i;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_bf16(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk,
                                                        Tensor4 tv, float sl2, float* __restrict__ os) {
  constexpr int BM = 32 * NW;
  constexpr int NT = 64 * NW;
  constexpr int G = D / 8;                 // 16-byte granules per row
  constexpr int GPT = (64 * G) / NT;       // granules per thread per tile
  constexpr int KS = D / 16;               // k-steps of Q K^T
  constexpr int DB = D / 32;               // 32-wide d blocks of O^T
  static_assert((64 * G) % NT == 0, "tile granules must split evenly");
  using SW = Swz<D>;

  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][64 * D];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][64 * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;

  // ---- decode the work item (anchors first, longest work first)
  const int qtiles = (d.n + BM - 1) / BM;
  unsigned w = blockIdx.x;
  const int qt = w % qtiles; w /= qtiles;
  const int h = w % d.H; w /= d.H;
  const int b = w % d.B; w /= d.B;
  const int f = frame_by_cost(d.g, (int)w);

  const KeySeq ks = key_sequence(d, f);

  // ---- Q^T fragments (B operand): lane holds row l32, d = 16*s + 8*half + 0..7
  const int prow = qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  const long long qtok = (long long)f * d.n + (row_ok ? prow : 0);
  bf16x8 qf[KS];
  {
    const bf16_t* qp = (const bf16_t*)q.p + tok_off(q, b, qtok, h) + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 u = row_ok ? ldg16(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  floatx16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // running max in log2 units (already scaled)
  float l_run = 0.f;        // this lane's partial row sum

  uint4 kreg[GPT], vreg[GPT];
  int cur_valid = 0, nxt_valid = 0;

  auto fetch = [&](int t, int& valid) {
    int s = 0, lt = t;
    while (s < ks.nseg - 1 && lt >= ks.tiles[s]) { lt -= ks.tiles[s]; ++s; }
    const int key0 = ks.start[s] + lt * 64;
    valid = min(64, ks.len[s] - lt * 64);
    const Tensor4& kt = ks.text[s] ? tk : k;
    const Tensor4& vt = ks.text[s] ? tv : v;
    const bf16_t* kb = (const bf16_t*)kt.p + tok_off(kt, b, key0, h);
    const bf16_t* vb = (const bf16_t*)vt.p + tok_off(vt, b, key0, h);
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int gi = tid + r * NT;
      const int row = gi / G, col = (gi % G) * 8;
      if (row < valid) {
        kreg[r] = ldg16(kb + (long long)row * kt.st + col);
        vreg[r] = ldg16(vb + (long long)row * vt.st + col);
      } else {
        kreg[r] = make_uint4(0, 0, 0, 0);
        vreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int r = 0; r < GPT; ++r) {
      const int gi = tid + r * NT;
      const int row = gi / G, col = (gi % G) * 8;
      *(uint4*)&Ks[buf][SW::off(row, col)] = kreg[r];
      *(uint4*)&Vs[buf][SW::off(row, col)] = vreg[r];
    }
  };

  fetch(0, cur_valid);
  stash(0);
  __syncthreads();

  for (int t = 0; t < ks.total; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ks.total;
    if (more) fetch(t + 1, nxt_valid);

    // ---- scores S^T for two 32-key blocks
    floatx16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = zero16();
      const int row = kb * 32 + l32;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *(const bf16x8*)&Ks[buf][SW::off(row, 16 * s + 8 * half)];
        sacc[kb] = mfma32(a, qf[s], sacc[kb]);
      }
    }
    if (cur_valid < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
          if (key >= cur_valid) sacc[kb][j] = -INFINITY;
        }
    }
    // ---- online softmax (per lane = per query row)
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[i][j] *= alpha;

    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        bf16x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = exp2f(fmaf(sacc[kb][8 * hb + e], sl2, -m_new));
          l_run += pv;
          p[e] = static_cast<__bf16>(pv);
        }
        pf[2 * kb + hb] = p;
      }

    // ---- O^T += V^T P^T; V^T operand via transposing LDS reads
    const int grp = lane >> 4, j16 = lane & 15;
    const int dsub = (grp & 1) * 16 + 4 * (j16 & 3);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb0 = (kk >> 1) * 32 + (kk & 1) * 16 + 4 * half + (j16 >> 2);
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const int col = i * 32 + dsub;
        const bf16x8 a = tr_pair(&Vs[buf][SW::off(kb0, col)], &Vs[buf][SW::off(kb0 + 8, col)]);
        oacc[i] = mfma32(a, pf[kk], oacc[i]);
      }
    }

    if (more) stash(buf ^ 1);
    cur_valid = nxt_valid;
    __syncthreads();
  }

  // ---- normalise and store (fp32, [B*N][H][D])
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (row_ok) {
    float* op = os + (((long long)b * d.N + qtok) * d.H + h) * D;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = i * 32 + 8 * jg + 4 * half;
        float4 o4 = make_float4(oacc[i][4 * jg] * inv, oacc[i][4 * jg + 1] * inv, oacc[i][4 * jg + 2] * inv,
                                oacc[i][4 * jg + 3] * inv);
        *(float4*)(op + d0) = o4;
      }
  }
}

template <int D, int NW>
static hipError_t launch_attn(const Dims& d, const Bf16Args& a, hipStream_t s) {
  constexpr int BM = 32 * NW;
  const long long qtiles = (d.n + BM - 1) / BM;
  const long long grid = qtiles * d.H * d.B * d.T;
  hipLaunchKernelGGL((k_attn_bf16<D, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, d, a.q, a.k, a.v, a.tk, a.tv,
                     a.scale_log2, a.os);
  return hipGetLastError();
}

hipError_t launch_softmax_bf16(const Dims& d, const Bf16Args& a, hipStream_t s) {
  if (d.D == 128) return launch_attn<128, 4>(d, a, s);
  if (d.D == 64) return launch_attn<64, 4>(d, a, s);
  return hipErrorInvalidValue;
}

}  // namespace hyb
