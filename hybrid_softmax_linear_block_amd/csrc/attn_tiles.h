// Tile machinery shared by the softmax-branch kernels (forward and
// backward): the walk over the key frames S(f) of a query frame plus the
// text, the direct-to-LDS tile loader, the tail mask, and the two MFMA tile
// products (S^T = K Q^T from a row-major LDS tile and register fragments;
// O^T += V^T P^T with V^T read by transposing LDS reads in the key order of
// the score registers).
#pragma once
#include "kernels_bf16.h"

namespace hyb {

// Walk over the keys of one work item in tiles of BN keys: up to three video
// frame ranges of S(f) (one tensor, one stride), then the text tokens (own
// tensor and stride).  Everything here is wave-uniform and lives in SGPRs;
// the common step is one pointer bump per tensor, segment changes (at most
// four per item) take the slow branch.
template <int BN>
struct KeyWalk {
  const char *kvid, *vvid, *ktxt, *vtxt;  // (b, h) bases of the key/value tensors
  unsigned kstv, vstv, kstt, vstt;         // byte strides per token
  int st[3], ln[3], L;                     // video ranges of S(f) in keys (constant indices only)
  const char *kp, *vp;                     // first key of the current tile
  unsigned ks, vs;                         // strides of the current segment
  int rem, seg;                            // keys left from kp in the segment; 0..2 video, 3 text, 4 done

  __device__ __forceinline__ void init(const Dims& d, int f, int b, int h, const Tensor4& k, const Tensor4& v,
                                       const Tensor4& tk, const Tensor4& tv) {
    const SoftRanges sr = soft_ranges(d.g, f);
    kvid = (const char*)((const bf16_t*)k.p + (long long)b * k.sb + (long long)h * k.sh);
    vvid = (const char*)((const bf16_t*)v.p + (long long)b * v.sb + (long long)h * v.sh);
    ktxt = (const char*)((const bf16_t*)tk.p + (long long)b * tk.sb + (long long)h * tk.sh);
    vtxt = (const char*)((const bf16_t*)tv.p + (long long)b * tv.sb + (long long)h * tv.sh);
    kstv = (unsigned)(k.st * 2);  // byte strides (< 2^18, host-checked)
    vstv = (unsigned)(v.st * 2);
    kstt = (unsigned)(tk.st * 2);
    vstt = (unsigned)(tv.st * 2);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      st[i] = sr.n > i ? sr.lo[i] * d.n : 0;
      ln[i] = sr.n > i ? (sr.hi[i] - sr.lo[i]) * d.n : 0;
    }
    L = d.L;
    open_from(0);
  }

  // position at the first key of the first non-empty segment >= s0
  __device__ __forceinline__ void open_from(int s0) {
    seg = 4;
    rem = 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (seg == 4 && i >= s0 && ln[i] > 0) {
        seg = i;
        kp = kvid + (unsigned long long)(unsigned)st[i] * kstv;
        vp = vvid + (unsigned long long)(unsigned)st[i] * vstv;
        ks = kstv;
        vs = vstv;
        rem = ln[i];
      }
    }
    if (seg == 4 && s0 <= 3 && L > 0) {
      seg = 3;
      kp = ktxt;
      vp = vtxt;
      ks = kstt;
      vs = vstt;
      rem = L;
    }
  }

  __device__ __forceinline__ bool done() const { return seg == 4; }
  __device__ __forceinline__ int valid() const { return min(BN, rem); }
  // step to the next tile; true when that opened a new segment (or ended)
  __device__ __forceinline__ bool advance() {
    rem -= BN;
    if (rem > 0) {
      kp += BN * ks;
      vp += BN * vs;
      return false;
    }
    open_from(seg + 1);
    return true;
  }
};

// Tile loader: a tile is KB blocks of 32 keys; each of the NW waves fills
// CPW chunks of RPC rows (1 KB, one wave-wide direct-to-LDS load per chunk).
template <int D, int NW, int KB>
struct TileLoader {
  static constexpr int G = D / 8;           // 16-byte granules per row
  static constexpr int BN = 32 * KB;        // keys per tile
  static constexpr int RPC = 64 / G;        // rows per chunk
  static constexpr int CHUNKS = BN / RPC;   // chunks per tile
  static constexpr int CPW = CHUNKS / NW;   // chunks per wave
  static constexpr int TILE = BN * D;       // elements per tile
  static_assert(CHUNKS % NW == 0, "tile chunks must split evenly over waves");

  unsigned lrow[CPW], lcol[CPW];  // per chunk: row in tile, byte offset of the logical granule
  unsigned koff[CPW], voff[CPW];  // per chunk: lane byte offset of a full tile at the current strides
  unsigned kst, vst;              // current byte strides

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      lrow[i] = (unsigned)((wave * CPW + i) * RPC + lane / G);
      lcol[i] = (unsigned)(((lane % G) ^ Swz<D>::key((int)lrow[i])) * 16);
    }
  }
  __device__ __forceinline__ void set_k(unsigned st2) {
    kst = st2;
#pragma unroll
    for (int i = 0; i < CPW; ++i) koff[i] = __umul24(lrow[i], st2) + lcol[i];
  }
  __device__ __forceinline__ void set_v(unsigned st2) {
    vst = st2;
#pragma unroll
    for (int i = 0; i < CPW; ++i) voff[i] = __umul24(lrow[i], st2) + lcol[i];
  }

  // Lane l of a chunk fills row (l / G), physical granule (l % G), which holds
  // logical granule (l % G) ^ swizzle(row).  Rows past the tile's valid keys
  // repeat the last valid row (their scores are masked to -inf).
  // dst: LDS byte address of the tile
  __device__ __forceinline__ void load(const char* base, const unsigned (&off)[CPW], unsigned st2, int valid,
                                       int wave, unsigned dst) const {
    if (valid == BN) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) dma16(base, off[i], dst + (wave * CPW + i) * RPC * D * 2);
    } else {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const unsigned rs = min(lrow[i], (unsigned)(valid - 1));
        dma16(base, __umul24(rs, st2) + lcol[i], dst + (wave * CPW + i) * RPC * D * 2);
      }
    }
  }
  __device__ __forceinline__ void load_k(const char* base, int valid, int wave, unsigned dst) const {
    load(base, koff, kst, valid, wave, dst);
  }
  __device__ __forceinline__ void load_v(const char* base, int valid, int wave, unsigned dst) const {
    load(base, voff, vst, valid, wave, dst);
  }
};

// Keys >= valid -> -inf.  key = c + 4 * half with c a compile-time constant
// per element; the key is masked when 4 * half - (valid - c) >= 0.  The sign
// of that difference becomes a bit mask that selects -inf, all in VGPRs (no
// per-element compare masks held in scalar registers).
template <int KB>
__device__ __forceinline__ void mask_tile(floatx16 (&s)[KB], int valid, int half) {
  const int kbase = 4 * half;
  const unsigned ninf = 0xff800000u;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int lim = valid - (kb * 32 + 8 * (j >> 2) + (j & 3));
      unsigned bits = __float_as_uint(s[kb][j]), m;
      asm("v_sub_u32 %0, %2, %3\n\t"
          "v_ashrrev_i32 %0, 31, %0\n\t"
          "v_bfi_b32 %1, %0, %1, %4"
          : "=&v"(m), "+v"(bits)
          : "v"(kbase), "s"(lim), "s"(ninf));
      s[kb][j] = __uint_as_float(bits);
    }
}

// S^T = K Q^T for one tile: KB blocks of 32 keys; K rows from the swizzled
// LDS tile, Q^T fragments from registers.
template <int D, int KB>
__device__ __forceinline__ void qk_tile(floatx16 (&s)[KB], const bf16_t* kt, const bf16x8 (&qf)[D / 16], int l32,
                                        int half) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) s[kb] = zero16();
  // step-major: the KB accumulation chains alternate, so each MFMA's K operand
  // read has the previous step's MFMAs to hide behind
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 a = *(const bf16x8*)&kt[Swz<D>::off(kb * 32 + l32, 16 * st + 8 * half)];
      s[kb] = mfma32(a, qf[st], s[kb]);
    }
}

// O^T += V^T P^T for one tile; the V^T operand comes from transposing LDS
// reads in the key order of the P fragments.
template <int D, int KB>
__device__ __forceinline__ void pv_tile(floatx16 (&oacc)[D / 32], const bf16_t* vt, const bf16x8 (&pf)[2 * KB],
                                        int half, int j16, int dsub) {
#pragma unroll
  for (int kk = 0; kk < 2 * KB; ++kk) {
    const int kb0 = (kk >> 1) * 32 + (kk & 1) * 16 + 4 * half + (j16 >> 2);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int col = i * 32 + dsub;
      const bf16x8 a = tr_pair(&vt[Swz<D>::off(kb0, col)], &vt[Swz<D>::off(kb0 + 8, col)]);
      oacc[i] = mfma32(a, pf[kk], oacc[i]);
    }
  }
}

}  // namespace hyb
