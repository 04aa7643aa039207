"""fp8 (OCP e4m3) emulation of the softmax branch (oracle, test
infrastructure only).

The VDN-H3 article's performance section reports an "FP8 version" without
saying which operations are fp8.  The library's reading: the softmax
branch's Q, K, V (video and text) are quantised per (tensor, batch, head)
with scale s = absmax / 448 and both products run on fp8 inputs.  This module
computes what that quantised problem gives in exact arithmetic, so that the
GPU's fp8 kernel can be checked against the computation it is meant to do,
while the layer output is checked against the unquantised oracle.

Decisions that pick a quantised code are taken in float32, as the kernel
takes them: s = float32(absmax) / 448, inv = 1 / s, x * inv in float32, then
round-to-nearest-even to e4m3 with saturation at +-448.

e4m3 (OCP FP8 E4M3): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
normal numbers 2^-6 .. 448, subnormals in steps of 2^-9, no infinities.

Pinned by tests/test_oracle_fp8.py against torch's float8_e4m3fn conversion
and by closed forms of the format (max, min subnormal, ties to even).
"""
import math

import numpy as np

from .layout import frame_sets

E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest e4m3 value (ties to even), saturated to +-448; float64 in/out."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade, floored at the subnormal binade (2^-6)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3.0)            # 3 mantissa bits
    q = np.round(a / step) * step      # np.round: half to even
    return np.sign(x) * np.minimum(q, E4M3_MAX)


def quantise(x, axes=(1, 3)):
    """Per-(batch, head) quantisation of a [B, tokens, H, D] tensor.
    Returns (dequantised values float64, scales float32 [B, H])."""
    x32 = np.asarray(x, np.float32)
    amax = np.max(np.abs(x32), axis=axes, keepdims=True)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    codes = round_e4m3((x32 * inv).astype(np.float32))
    return codes * s.astype(np.float64), s.reshape(s.shape[0], s.shape[2])


def softmax_branch_fp8(q, k, v, text_k, text_v, lay, scale=None, tokens=None, p_scale=256.0):
    """Softmax branch on the quantised inputs, in float64, with the
    probabilities rounded to e4m3 (after scaling by p_scale) in the P V
    product and exact in the normaliser."""
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    qq, _ = quantise(q)
    kq, _ = quantise(k)
    vq, _ = quantise(v)
    tkq, _ = quantise(text_k) if text_k.shape[1] else (np.zeros(text_k.shape), None)
    tvq, _ = quantise(text_v) if text_v.shape[1] else (np.zeros(text_v.shape), None)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    rows = np.arange(N) if tokens is None else np.asarray(tokens)
    out = np.zeros((B, rows.size, H, D))
    frame_of = rows // n
    for f in range(lay.frames):
        sel = np.nonzero(frame_of == f)[0]
        if sel.size == 0:
            continue
        kt = np.concatenate([np.arange(g * n, (g + 1) * n) for g in sorted(sets[f][0])])
        for b in range(B):
            for h in range(H):
                K = np.concatenate([kq[b, kt, h], tkq[b, :, h]])
                V = np.concatenate([vq[b, kt, h], tvq[b, :, h]])
                s = tau * (qq[b, rows[sel], h] @ K.T)
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                pq = round_e4m3(p * p_scale) / p_scale
                out[b, sel, h] = (pq @ V) / p.sum(axis=1, keepdims=True)
    return out


def scales(inp):
    """float32 dequantisation scales [5, B, H] of q, k, v, text_k, text_v."""
    out = []
    for name in ("q", "k", "v", "text_k", "text_v"):
        x = inp[name]
        if x.shape[1] == 0:
            out.append(np.ones((x.shape[0], x.shape[2]), np.float32))
        else:
            out.append(quantise(x)[1])
    return np.stack(out)
