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

typedef __attribute__((address_space(3))) void lds_void;

// Lazy rescaling: the running maximum only moves when a row's tile maximum
// exceeds it by more than 2^8 (log2 units); probabilities then stay <= 2^8,
// exact enough in bf16 and fp32, and the O rescale is skipped on most tiles.
constexpr float kRescaleSlack = 8.f;

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void k_attn_bf16(Dims d, Tensor4 q, Tensor4 k, Tensor4 v, Tensor4 tk, Tensor4 tv, float sl2,
                 float* __restrict__ os) {
  constexpr int BM = 32 * NW;
  constexpr int G = D / 8;                 // 16-byte granules per row
  constexpr int RPC = 64 / G;              // rows per 1 KB chunk (one wave-wide LDS-DMA load)
  constexpr int CHUNKS = 64 / RPC;         // chunks per 64-key tile
  constexpr int CPW = CHUNKS / NW;         // chunks per wave
  constexpr int KS = D / 16;               // k-steps of Q K^T
  constexpr int DB = D / 32;               // 32-wide d blocks of O^T
  static_assert(CHUNKS % NW == 0, "tile chunks must split evenly over waves");
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

  // ---- K and V tiles: wave-wide direct-to-LDS loads of 1 KB chunks; lane l
  // of a chunk fills row (l / G), physical granule (l % G), which holds the
  // logical granule (l % G) ^ swizzle(row).  Rows past the tile's valid keys
  // repeat the last valid row (their scores are masked to -inf).
  auto issue = [&](int t, int buf) -> int {
    int key0, valid;
    bool text;
    locate(ks, d.L, t, key0, valid, text);
    const Tensor4& kt = text ? tk : k;
    const Tensor4& vt = text ? tv : v;
    const bf16_t* kb = (const bf16_t*)kt.p + tok_off(kt, b, key0, h);
    const bf16_t* vb = (const bf16_t*)vt.p + tok_off(vt, b, key0, h);
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = wave * CPW + i;
      const int r = c * RPC + lane / G;
      const int gl = (lane % G) ^ SW::key(r);
      const int rs = min(r, valid - 1);
      __builtin_amdgcn_global_load_lds((const void*)(kb + (long long)rs * kt.st + gl * 8),
                                       (lds_void*)&Ks[buf][c * RPC * D], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + (long long)rs * vt.st + gl * 8),
                                       (lds_void*)&Vs[buf][c * RPC * D], 16, 0, 0);
    }
    return valid;
  };

  int cur_valid = issue(0, 0);

  // ---- Q^T fragments (B operand): lane holds row l32, d = 16*s + 8*half + 0..7
  const int prow = qt * BM + wave * 32 + l32;
  const bool row_ok = prow < d.n;
  const long long qtok = (long long)f * d.n + (row_ok ? prow : 0);
  bf16x8 qf[KS];
  {
    const bf16_t* qp = (const bf16_t*)q.p + tok_off(q, b, qtok, h) + 8 * half;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * s));
  }

  floatx16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // running max in log2 units (already scaled)
  float l_run = 0.f;        // this lane's partial row sum

  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 landed in LDS
  __syncthreads();

  const int grp = lane >> 4, j16 = lane & 15;
  const int dsub = (grp & 1) * 16 + 4 * (j16 & 3);

  for (int t = 0; t < ks.total; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ks.total;
    int nxt_valid = 0;
    if (more) nxt_valid = issue(t + 1, buf ^ 1);

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
    // ---- online softmax (per lane = per query row), lazily rescaled
    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, fmaxf(sacc[0][j], sacc[1][j]));
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

    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        bf16x8 p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * hb + e], sl2, -m_run));
          l_run += pv;
          p[e] = static_cast<__bf16>(pv);
        }
        pf[2 * kb + hb] = p;
      }

    // ---- O^T += V^T P^T; V^T operand via transposing LDS reads
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

    cur_valid = nxt_valid;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile landed
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
