"""Seeded synthetic inputs for the hybrid attention layer.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage type the device reads (bf16 round-to-nearest-even,
or float32 as drawn) and describes the workload shapes.  Both the fp64 oracle
(in the tests) and the HIP library consume the same rounded values.

Workloads (the article measures 768p, ~14.4 s video; the latent grid below
stands in for it):
  1 tiny-fp32    B1, 15 frames x 64 tokens (8x8), H2 x D32, 16 text, fp32,
                 all activations N(0,1)
  2 small-bf16   B1, 15 x 1024 (32x32), H8 x D64, 128 text, bf16,
                 q/k/v/text ~ N(0,1) * D^-1/4, x ~ N(0,1)
  3 768p-bf16    B1, 15 x 4032 (48x84), H24 x D128, 512 text, bf16, N(0,1)
  4 chunked-bf16 B1, 31 x 4032, H24 x D128, 512 text, 5-frame chunks,
                 anchors 0/30, recipe of workload 2
  5 fp8-softmax  B2, otherwise workload 2; softmax-branch Q/K/V quantised to
                 e4m3 by the library; 1% of q/k/v/text entries scaled x8
All weights ~ N(0, 0.02^2), RMSNorm weight 1.  Draw order from
numpy Generator(PCG64(seed)): x, q, k, v, text_k, text_v, w_gs, w_gl, w_os,
w_ol; outliers come from a second generator seeded seed + 1000.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
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
    act: str = "bf16"          # storage type of x, q, k, v, text, weights, y
    soft: str = "bf16"         # precision of the softmax branch's Q/K/V
    qkv_scale: float = 1.0     # multiplier on q, k, v, text_k, text_v draws
    outlier_frac: float = 0.0  # fraction of q/k/v/text entries scaled x8
    weight_std: float = 0.02
    seed: int = 0

    @property
    def n_video(self):
        return self.frames * self.tokens_per_frame

    @property
    def hidden(self):
        return self.heads * self.head_dim

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("tiny-fp32", 1, 15, 64, 16, 2, 32, act="f32", soft="f32", seed=1),
    2: Workload("small-bf16", 1, 15, 1024, 128, 8, 64, qkv_scale=64 ** -0.25, seed=2),
    3: Workload("768p-bf16", 1, 15, 4032, 512, 24, 128, seed=3),
    4: Workload("chunked-768p-bf16", 1, 31, 4032, 512, 24, 128, chunk_frames=5,
                qkv_scale=128 ** -0.25, seed=4),
    5: Workload("fp8-softmax", 2, 15, 1024, 128, 8, 64, soft="fp8", qkv_scale=64 ** -0.25,
                outlier_frac=0.01, seed=5),
}


def round_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a, act):
    if act == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    return bf16_bits_to_f32(round_bf16_bits(a))


def make_inputs(w: Workload, seed=None):
    """Return a dict of float32 arrays whose values are exact in ``w.act``.

    Shapes: x [B,N,hid]; q, k, v [B,N,H,D]; text_k, text_v [B,L,H,D];
    w_gs, w_gl, w_os, w_ol [hid,hid] ([in][out]); rms_w [hid].
    """
    seed = w.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed))
    B, N, L, H, D, hid = w.batch, w.n_video, w.text_tokens, w.heads, w.head_dim, w.hidden

    def normal(shape, scale=1.0):
        a = g.standard_normal(size=shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return a

    out = {"x": normal((B, N, hid))}
    for name, shape in (("q", (B, N, H, D)), ("k", (B, N, H, D)), ("v", (B, N, H, D)),
                        ("text_k", (B, L, H, D)), ("text_v", (B, L, H, D))):
        out[name] = normal(shape, w.qkv_scale)
    for name in ("w_gs", "w_gl", "w_os", "w_ol"):
        out[name] = normal((hid, hid), w.weight_std)
    if w.outlier_frac > 0:
        g2 = np.random.Generator(np.random.PCG64(seed + 1000))
        for name in ("q", "k", "v", "text_k", "text_v"):
            a = out[name]
            m = g2.random(size=a.shape) < w.outlier_frac
            a[m] *= np.float32(8.0)
    for name in list(out):
        out[name] = _store(out[name], w.act)
    out["rms_w"] = np.ones((hid,), dtype=np.float32)
    return out


def make_projection_weights(w: Workload, seed=None):
    """Seeded Q/K/V projection weights w_q, w_k, w_v [hid, hid] ([in][out]),
    ~ N(0, weight_std^2), exact in ``w.act``; drawn from PCG64(seed + 3000) so
    that the layer inputs of ``make_inputs`` are unchanged."""
    seed = w.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed + 3000))
    hid = w.hidden
    out = {}
    for name in ("w_q", "w_k", "w_v"):
        a = g.standard_normal(size=(hid, hid), dtype=np.float32) * np.float32(w.weight_std)
        out[name] = _store(a, w.act)
    return out


def make_ffn_weights(w: Workload, seed=None, expansion=4):
    """Seeded feed-forward weights of the block: w_n [hid] = 1 + 0.1 N(0, 1)
    (RMSNorm weight), w_1 [hid, F], w_2 [F, hid] ~ N(0, weight_std^2) with
    F = expansion * hid, exact in ``w.act``; drawn from PCG64(seed + 5000)."""
    seed = w.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed + 5000))
    hid = w.hidden
    F = expansion * hid
    w_n = np.float32(1.0) + np.float32(0.1) * g.standard_normal(size=hid, dtype=np.float32)
    w_1 = g.standard_normal(size=(hid, F), dtype=np.float32) * np.float32(w.weight_std)
    w_2 = g.standard_normal(size=(F, hid), dtype=np.float32) * np.float32(w.weight_std)
    return {"w_n": _store(w_n, w.act), "w_1": _store(w_1, w.act), "w_2": _store(w_2, w.act)}


def make_grad_output(w: Workload, seed=None):
    """Seeded gradient of the layer output, dy [B, N, hid] ~ N(0, 1), exact in
    ``w.act``; drawn from PCG64(seed + 4000)."""
    seed = w.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed + 4000))
    a = g.standard_normal(size=(w.batch, w.n_video, w.hidden), dtype=np.float32)
    return _store(a, w.act)


def sample_tokens(w: Workload, per_frame=64, seed=None):
    """Seeded sorted sample of video-token indices: ``per_frame`` tokens from
    every frame, always including each frame's first and last token."""
    seed = w.seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(seed + 2000))
    n = w.tokens_per_frame
    out = []
    for f in range(w.frames):
        k = min(per_frame, n)
        pick = set(g.choice(n, size=k, replace=False).tolist()) | {0, n - 1}
        out.extend(f * n + p for p in sorted(pick))
    return np.asarray(sorted(out), dtype=np.int64)
