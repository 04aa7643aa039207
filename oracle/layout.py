"""Frame sets of the hybrid layer (oracle, test infrastructure only).

Source: VDN-H3 article (tahou.com), section "双分支混合注意力机制":
  * local softmax branch: consecutive latent frames are grouped into chunks
    (5 frames in the base model); a chunk attends to itself and its
    neighbouring chunks; the first and last frames are boundary anchors that
    every frame reads and that also interact with the other frames;
  * linear branch: a forward state over the frames before the local window and
    a backward state over the frames after it, both leaving out the window and
    the anchor frames;
  * worked example: frame 7 of 0..14 keeps 6, 7, 8 and anchors 0, 14 in the
    softmax branch; forward state 1-5, backward state 9-13.

One rule covers both the chunked text and the worked example: chunk size C,
chunk radius R.  (C=1, R=1) is the worked example; (C=5, R=1) the chunk text.

Readings taken where the article is silent:
  * chunks are formed over the non-anchor ("interior") frames in order,
    starting at the first interior frame; the last chunk may be short;
  * an anchor frame used as a query attends to every frame, and its linear
    states hold text only (the article says anchors interact with the others);
  * a frame in both the window and the anchor set counts once (set union);
  * an empty forward/backward range is reported as the pair (0, 0).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Layout:
    batch: int
    frames: int
    tokens_per_frame: int
    text_tokens: int
    heads: int
    head_dim: int
    chunk_frames: int = 1
    chunk_radius: int = 1
    anchor_first: bool = True
    anchor_last: bool = True

    @property
    def n_video(self):
        return self.frames * self.tokens_per_frame

    @property
    def hidden(self):
        return self.heads * self.head_dim


def anchor_frames(T, anchor_first, anchor_last):
    a = set()
    if anchor_first:
        a.add(0)
    if anchor_last:
        a.add(T - 1)
    return a


def frame_sets(T, C, R, anchor_first=True, anchor_last=True):
    """Return, per query frame f, the triple (S(f), F(f), B(f)) as Python sets.

    S(f): key frames of the softmax branch; F(f): frames summed into the forward
    linear state; B(f): frames summed into the backward linear state.
    """
    if T < 1 or C < 1 or R < 0:
        raise ValueError("need T >= 1, C >= 1, R >= 0")
    A = anchor_frames(T, anchor_first, anchor_last)
    interior = [g for g in range(T) if g not in A]
    chunk = {g: i // C for i, g in enumerate(interior)}
    out = []
    for f in range(T):
        if f in A:
            out.append((set(range(T)), set(), set()))
            continue
        cf = chunk[f]
        window = {g for g in interior if abs(chunk[g] - cf) <= R}
        S = window | A
        F = {g for g in interior if chunk[g] < cf - R}
        B = {g for g in interior if chunk[g] > cf + R}
        out.append((S, F, B))
    return out


def _as_range(s):
    if not s:
        return (0, 0)
    lo, hi = min(s), max(s) + 1
    if set(range(lo, hi)) != s:
        raise AssertionError("linear-state frame set is not contiguous: %r" % sorted(s))
    return (lo, hi)


def tables(T, C, R, anchor_first=True, anchor_last=True):
    """Integer tables in the form the library's table call fills.

    soft_frames: T x T, ascending key frames of S(f), padded with -1
    soft_count:  T
    fwd, bwd:    T x 2 half-open frame ranges [lo, hi); (0, 0) when empty
    """
    sets = frame_sets(T, C, R, anchor_first, anchor_last)
    soft_frames = [[-1] * T for _ in range(T)]
    soft_count = [0] * T
    fwd = [[0, 0] for _ in range(T)]
    bwd = [[0, 0] for _ in range(T)]
    for f, (S, F, B) in enumerate(sets):
        s = sorted(S)
        soft_frames[f][:len(s)] = s
        soft_count[f] = len(s)
        fwd[f] = list(_as_range(F))
        bwd[f] = list(_as_range(B))
    return soft_frames, soft_count, fwd, bwd
