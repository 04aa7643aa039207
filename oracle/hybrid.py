"""fp64 definition of the VDN-H3 hybrid attention layer (oracle, test
infrastructure only).

Source: VDN-H3 article (tahou.com, article 216474224916730885).
  * section "双分支混合注意力机制" (dual-branch hybrid attention): the softmax
    branch over the local window plus anchors plus text; the linear branch
    with a forward state over the frames before the window and a backward
    state over the frames after it; text visible from every frame in the
    softmax branch and written half into each linear state, so that merging
    the two reads counts it once; states are read at the query's position;
  * section "自适应门控融合双分支输出" (adaptive gated fusion): one
    content-dependent sigmoid gate per branch, RMSNorm on the linear branch
    before its element-wise gate, one output projection per branch, summed
    into the residual stream.

Readings taken where the article is silent (the library implements the same):
  * softmax scale tau = 1/sqrt(D); text tokens are keys/values only;
  * feature map phi(u) = elu(u) + 1 (alpha = 1) on Q and K; V is raw;
  * the two linear reads share one normaliser:
        O_l = phi(q)^T (S+ + S-) / (phi(q)^T (z+ + z-) + eps),  eps = 1e-6,
    so the two text halves add up to one text contribution;
  * "aligned with the query position" = the states are chosen by the query's
    frame; no positional transform or decay is applied;
  * gates are element-wise over the hidden size, computed from the layer
    input x with no bias:  g = sigmoid(x W);
  * RMSNorm runs per token over the full hidden size of the concatenated
    head outputs, with weight w and the same eps;
  * weights are [in][out] row-major (y = x W); the layer returns y = x + delta.
"""
import math

import numpy as np

from .layout import frame_sets

_ROW_BLOCK = 512


def phi(u):
    """elu(u) + 1: u + 1 for u > 0, exp(u) otherwise."""
    u = np.asarray(u, dtype=np.float64)
    return np.where(u > 0, u + 1.0, np.exp(np.minimum(u, 0.0)))


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-np.asarray(u, dtype=np.float64)))


def _rows(lay, tokens):
    if tokens is None:
        return np.arange(lay.n_video)
    t = np.asarray(tokens, dtype=np.int64)
    if t.ndim != 1 or (t.size and (t.min() < 0 or t.max() >= lay.n_video)):
        raise ValueError("token sample out of range")
    return t


def softmax_branch(q, k, v, text_k, text_v, lay, scale=None, tokens=None):
    """O_s = softmax over K(f) of tau q.k, applied to V, for every query token.

    K(f) = video tokens of the key frames S(f) of the query's frame f, plus all
    text tokens.  q, k, v: [B, N, H, D]; text_k, text_v: [B, L, H, D].
    Returns [B, len(tokens), H, D] (all N video tokens when tokens is None).
    """
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius,
                      lay.anchor_first, lay.anchor_last)
    rows = _rows(lay, tokens)
    out = np.zeros((B, rows.size, H, D))
    frame_of = rows // n
    for f in range(lay.frames):
        sel = np.nonzero(frame_of == f)[0]
        if sel.size == 0:
            continue
        key_tok = np.concatenate([np.arange(g * n, (g + 1) * n) for g in sorted(sets[f][0])])
        for b in range(B):
            for h in range(H):
                K = np.concatenate([np.asarray(k[b, key_tok, h], np.float64),
                                    np.asarray(text_k[b, :, h], np.float64)])
                V = np.concatenate([np.asarray(v[b, key_tok, h], np.float64),
                                    np.asarray(text_v[b, :, h], np.float64)])
                for s0 in range(0, sel.size, _ROW_BLOCK):
                    ii = sel[s0:s0 + _ROW_BLOCK]
                    Q = np.asarray(q[b, rows[ii], h], np.float64)
                    s = tau * (Q @ K.T)
                    s -= s.max(axis=1, keepdims=True)
                    p = np.exp(s)
                    out[b, ii, h] = (p @ V) / p.sum(axis=1, keepdims=True)
    return out


def linear_states(k, v, text_k, text_v, lay):
    """Per-frame states S_g = sum_{t in g} phi(k_t) v_t^T, z_g = sum phi(k_t),
    and the text state (S_T, z_T) over all text tokens.

    Returns S [B, H, T, D, D], z [B, H, T, D], S_T [B, H, D, D], z_T [B, H, D].
    """
    B, N, H, D = k.shape
    n, T = lay.tokens_per_frame, lay.frames
    S = np.zeros((B, H, T, D, D))
    z = np.zeros((B, H, T, D))
    ST = np.zeros((B, H, D, D))
    zT = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            for g in range(T):
                pk = phi(k[b, g * n:(g + 1) * n, h])
                S[b, h, g] = pk.T @ np.asarray(v[b, g * n:(g + 1) * n, h], np.float64)
                z[b, h, g] = pk.sum(axis=0)
            pk = phi(text_k[b, :, h])
            ST[b, h] = pk.T @ np.asarray(text_v[b, :, h], np.float64)
            zT[b, h] = pk.sum(axis=0)
    return S, z, ST, zT


def directional_states(states, lay):
    """Forward and backward states per query frame (each with half the text).

    Returns (Sf, zf, Sb, zb) with shapes [B, H, T, D, D] / [B, H, T, D].
    """
    S, z, ST, zT = states
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius,
                      lay.anchor_first, lay.anchor_last)
    Sf = np.zeros_like(S)
    Sb = np.zeros_like(S)
    zf = np.zeros_like(z)
    zb = np.zeros_like(z)
    for f, (_, F, Bk) in enumerate(sets):
        Sf[:, :, f] = 0.5 * ST
        zf[:, :, f] = 0.5 * zT
        Sb[:, :, f] = 0.5 * ST
        zb[:, :, f] = 0.5 * zT
        for g in F:
            Sf[:, :, f] += S[:, :, g]
            zf[:, :, f] += z[:, :, g]
        for g in Bk:
            Sb[:, :, f] += S[:, :, g]
            zb[:, :, f] += z[:, :, g]
    return Sf, zf, Sb, zb


def linear_branch(q, states, lay, eps=1e-6, tokens=None):
    """O_l[i] = phi(q_i)^T (S+ + S-) / (phi(q_i)^T (z+ + z-) + eps) for the
    forward/backward states of the query's frame.  Returns [B, len(tokens), H, D].
    """
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    Sf, zf, Sb, zb = directional_states(states, lay)
    rows = _rows(lay, tokens)
    out = np.zeros((B, rows.size, H, D))
    frame_of = rows // n
    for f in range(lay.frames):
        sel = np.nonzero(frame_of == f)[0]
        if sel.size == 0:
            continue
        for b in range(B):
            for h in range(H):
                pq = phi(q[b, rows[sel], h])
                num = pq @ (Sf[b, h, f] + Sb[b, h, f])
                den = pq @ (zf[b, h, f] + zb[b, h, f]) + eps
                out[b, sel, h] = num / den[:, None]
    return out


def epilogue(x, o_s, o_l, w_gs, w_gl, w_os, w_ol, rms_w, eps=1e-6):
    """Gated fusion of the two branches into the residual stream.

    x: [B, M, hid]; o_s, o_l: [B, M, H, D] (heads concatenated into hid, head
    major).  Returns dict with g_s, g_l, r (RMSNorm of the linear branch),
    delta and y = x + delta.
    """
    x = np.asarray(x, np.float64)
    B, M, hid = x.shape
    os_ = np.asarray(o_s, np.float64).reshape(B, M, hid)
    ol_ = np.asarray(o_l, np.float64).reshape(B, M, hid)
    g_s = sigmoid(x @ np.asarray(w_gs, np.float64))
    g_l = sigmoid(x @ np.asarray(w_gl, np.float64))
    ms = np.mean(ol_ * ol_, axis=-1, keepdims=True)
    r = ol_ * np.asarray(rms_w, np.float64) / np.sqrt(ms + eps)
    delta = (g_s * os_) @ np.asarray(w_os, np.float64) + (g_l * r) @ np.asarray(w_ol, np.float64)
    return {"g_s": g_s, "g_l": g_l, "r": r, "delta": delta, "y": x + delta}


def hybrid_forward(inp, lay, scale=None, eps=1e-6, tokens=None):
    """The whole layer.  ``inp`` maps names to arrays: x [B,N,hid];
    q, k, v [B,N,H,D]; text_k, text_v [B,L,H,D]; w_gs, w_gl, w_os, w_ol
    [hid,hid]; rms_w [hid].  With ``tokens`` the outputs are evaluated only at
    those video tokens (the states still use every token).
    """
    rows = _rows(lay, tokens)
    o_s = softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"],
                         lay, scale=scale, tokens=rows)
    st = linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    o_l = linear_branch(inp["q"], st, lay, eps=eps, tokens=rows)
    ep = epilogue(np.asarray(inp["x"])[:, rows], o_s, o_l, inp["w_gs"], inp["w_gl"],
                  inp["w_os"], inp["w_ol"], inp["rms_w"], eps=eps)
    ep.update({"o_s": o_s, "o_l": o_l, "tokens": rows})
    return ep
