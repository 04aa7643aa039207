// Closed-form frame sets of the hybrid layer, shared by the host table export
// and the kernels (which derive their key-frame ranges from blockIdx).
//
// VDN-H3 article (tahou.com), section "双分支混合注意力机制": consecutive
// latent frames are grouped into chunks; a chunk attends (softmax) to itself
// and its neighbouring chunks; the first and last frames are anchors read by
// every frame; the forward / backward linear states cover the frames before /
// after the window, leaving out window and anchor frames.  Chunk size C and
// radius R: (C=1, R=1) is the article's frame-7 example, (C=5, R=1) its
// chunk description.  Chunks are formed over the non-anchor frames in order;
// an anchor frame as a query sees every frame and has empty linear ranges.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define HYB_HD __host__ __device__ inline
#else
#define HYB_HD inline
#endif

namespace hyb {

struct FrameGeom {
  int T, C, R, af, al;  // frames, chunk size, chunk radius, anchor flags
};

// Interior (non-anchor) frames form the half-open range [i0, i1).
HYB_HD int interior_begin(const FrameGeom& g) { return g.af ? 1 : 0; }
HYB_HD int interior_end(const FrameGeom& g) {
  int i1 = g.al ? g.T - 1 : g.T;
  int i0 = interior_begin(g);
  return i1 < i0 ? i0 : i1;
}
HYB_HD bool is_anchor(const FrameGeom& g, int f) {
  return (g.af && f == 0) || (g.al && f == g.T - 1);
}

// Up to three ascending, disjoint half-open frame ranges whose union is the
// softmax key-frame set S(f).
struct SoftRanges {
  int n;
  int lo[3], hi[3];
};

HYB_HD SoftRanges soft_ranges(const FrameGeom& g, int f) {
  // built with constant indices only, so device code keeps it in registers
  SoftRanges s;
  s.n = 0;
  s.lo[0] = s.hi[0] = s.lo[1] = s.hi[1] = s.lo[2] = s.hi[2] = 0;
  if (is_anchor(g, f)) {
    s.lo[0] = 0;
    s.hi[0] = g.T;
    s.n = 1;
    return s;
  }
  const int i0 = interior_begin(g), i1 = interior_end(g);
  const int c = (f - i0) / g.C;
  const int clo = c - g.R < 0 ? 0 : c - g.R;
  const long long w0 = (long long)i0 + (long long)clo * g.C;
  long long w1 = (long long)i0 + ((long long)c + g.R + 1) * g.C;
  if (w1 > i1) w1 = i1;
  if (g.af) {
    s.lo[0] = 0; s.hi[0] = 1;
    s.lo[1] = (int)w0; s.hi[1] = (int)w1;
    s.n = 2;
  } else {
    s.lo[0] = (int)w0; s.hi[0] = (int)w1;
    s.n = 1;
  }
  if (g.al) {  // f is interior, so T - 1 >= 1 is a distinct anchor
    if (s.n == 2) { s.lo[2] = g.T - 1; s.hi[2] = g.T; }
    else { s.lo[1] = g.T - 1; s.hi[1] = g.T; }
    ++s.n;
  }
  return s;
}

// Forward range F(f) = interior frames in chunks before the window;
// backward range B(f) = interior frames in chunks after it.  Empty -> {0,0}.
HYB_HD void linear_ranges(const FrameGeom& g, int f, int* f_lo, int* f_hi, int* b_lo, int* b_hi) {
  *f_lo = *f_hi = *b_lo = *b_hi = 0;
  if (is_anchor(g, f)) return;
  const int i0 = interior_begin(g), i1 = interior_end(g);
  const int c = (f - i0) / g.C;
  if (c - g.R > 0) {
    long long e = (long long)i0 + (long long)(c - g.R) * g.C;
    *f_lo = i0;
    *f_hi = (int)(e < i1 ? e : i1);
  }
  long long s = (long long)i0 + ((long long)c + g.R + 1) * g.C;
  if (s < i1) {
    *b_lo = (int)s;
    *b_hi = i1;
  }
}

HYB_HD int soft_frame_count(const FrameGeom& g, int f) {
  SoftRanges s = soft_ranges(g, f);
  int n = 0;
  for (int i = 0; i < s.n; ++i) n += s.hi[i] - s.lo[i];
  return n;
}

// Query-frame visiting order of the softmax kernels: anchors first (they see
// every frame, the longest work items), then the interior frames.
HYB_HD int frame_by_cost(const FrameGeom& g, int i) {
  const bool a0 = g.af;
  const bool a1 = g.al && !(g.af && g.T == 1);
  if (a0) { if (i == 0) return 0; --i; }
  if (a1) { if (i == 0) return g.T - 1; --i; }
  return interior_begin(g) + i;
}

}  // namespace hyb
