"""fp64 gradient of the hybrid attention layer (oracle, test infrastructure
only).

Source: VDN-H3 article (tahou.com, article 216474224916730885), section
"分阶段适配预训练模型" (staged adaptation).  Stage A1 calibrates the new
linear branch of every layer, stage A2 trains it end to end inside the
otherwise frozen denoiser (softmax branch, Q/K/V/O projections and FFN
frozen), and stage B adds LoRA adapters to the Q/K/V and output projections
and lets the softmax gate train too.  Every stage therefore runs the layer's
backward pass: gradients of the activations (to reach earlier layers and the
projections' adapters) and of the layer's own weights.

What is computed is the plain chain-rule derivative of the forward
definition in ``oracle/hybrid.py`` (same readings: tau = 1/sqrt(D),
phi = elu + 1 on Q and K, one shared linear normaliser, element-wise gates
from x, RMSNorm over the full hidden size), for the scalar loss
L = sum(dy * y).  Nothing here is blocked, fused or reordered beyond the
definitions; each function follows one forward function in reverse.

Pinned by tests/test_oracle_backward.py: central finite differences of the
forward oracle along random directions, for every input tensor and on two
frame layouts (with the window, the anchors and non-empty forward and
backward states), and by mutations of this module that the finite
differences must catch.
"""
import math

import numpy as np

from .hybrid import directional_states, linear_states, phi, sigmoid
from .layout import frame_sets


def dphi(u):
    """Derivative of elu(u) + 1: 1 for u > 0, exp(u) otherwise (continuous at 0)."""
    u = np.asarray(u, np.float64)
    return np.where(u > 0, 1.0, np.exp(np.minimum(u, 0.0)))


def _key_tokens(lay, keyframes):
    n = lay.tokens_per_frame
    return np.concatenate([np.arange(g * n, (g + 1) * n) for g in sorted(keyframes)])


def softmax_lse(q, k, text_k, lay, scale=None):
    """Log-sum-exp of the scaled scores of every query row over its key set
    K(f): lse[b, i, h] = log sum_j exp(tau q_i . k_j)."""
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    out = np.zeros((B, N, H))
    for f in range(lay.frames):
        kt = _key_tokens(lay, sets[f][0])
        rows = np.arange(f * n, (f + 1) * n)
        for b in range(B):
            for h in range(H):
                K = np.concatenate([np.asarray(k[b, kt, h], np.float64), np.asarray(text_k[b, :, h], np.float64)])
                s = tau * (np.asarray(q[b, rows, h], np.float64) @ K.T)
                m = s.max(axis=1)
                out[b, rows, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def softmax_backward(q, k, v, text_k, text_v, lay, d_os, scale=None):
    """Gradients of the softmax branch O_s with respect to q, k, v and the
    text keys/values, given dL/dO_s.  Per query frame f and (b, h):
      P = softmax(tau Q K^T) over K(f), dP = dO V^T,
      dS = P * (dP - rowsum(dO * O)),  dQ = tau dS K,
      dK = tau dS^T Q,  dV = P^T dO  (scattered back to the key tokens)."""
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    dq = np.zeros((B, N, H, D))
    dk = np.zeros((B, N, H, D))
    dv = np.zeros((B, N, H, D))
    dtk = np.zeros(text_k.shape)
    dtv = np.zeros(text_v.shape)
    for f in range(lay.frames):
        kt = _key_tokens(lay, sets[f][0])
        nv = kt.size
        rows = np.arange(f * n, (f + 1) * n)
        for b in range(B):
            for h in range(H):
                K = np.concatenate([np.asarray(k[b, kt, h], np.float64), np.asarray(text_k[b, :, h], np.float64)])
                V = np.concatenate([np.asarray(v[b, kt, h], np.float64), np.asarray(text_v[b, :, h], np.float64)])
                Q = np.asarray(q[b, rows, h], np.float64)
                dO = np.asarray(d_os[b, rows, h], np.float64)
                s = tau * (Q @ K.T)
                s -= s.max(axis=1, keepdims=True)
                P = np.exp(s)
                P /= P.sum(axis=1, keepdims=True)
                O = P @ V
                dP = dO @ V.T
                dS = P * (dP - np.sum(dO * O, axis=1, keepdims=True))
                dq[b, rows, h] += tau * (dS @ K)
                dK = tau * (dS.T @ Q)
                dV = P.T @ dO
                dk[b, kt, h] += dK[:nv]
                dv[b, kt, h] += dV[:nv]
                dtk[b, :, h] += dK[nv:]
                dtv[b, :, h] += dV[nv:]
    return dq, dk, dv, dtk, dtv


def linear_backward(q, k, v, text_k, text_v, lay, d_ol, eps=1e-6):
    """Gradients of the linear branch O_l with respect to q, k, v and the text
    keys/values, given dL/dO_l.

    Forward (per query i of frame f): C_f = S+_f + S-_f, c_f = z+_f + z-_f,
    num = phi(q)^T C_f, den = phi(q) . c_f + eps, O = num / den.
    Reverse: dnum = dO / den, dden = -(dO . O) / den,
    dphi(q) = C_f dnum + c_f dden, and the combined state of frame f collects
    dC_f = sum_i phi(q_i) dnum_i^T, dc_f = sum_i phi(q_i) dden_i.  Each frame
    state S_g receives dC_f from every f whose forward or backward range holds
    g; the text state receives half of dC_f through each direction; finally
    S_g = sum_t phi(k_t) v_t^T, z_g = sum_t phi(k_t) give
    dphi(k_t) = dS_g v_t + dz_g and dv_t = dS_g^T phi(k_t)."""
    B, N, H, D = q.shape
    n, T = lay.tokens_per_frame, lay.frames
    st = linear_states(k, v, text_k, text_v, lay)
    Sf, zf, Sb, zb = directional_states(st, lay)
    sets = frame_sets(T, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    dq = np.zeros((B, N, H, D))
    dC = np.zeros((B, H, T, D, D))
    dc = np.zeros((B, H, T, D))
    for f in range(T):
        rows = np.arange(f * n, (f + 1) * n)
        for b in range(B):
            for h in range(H):
                C = Sf[b, h, f] + Sb[b, h, f]
                c = zf[b, h, f] + zb[b, h, f]
                qr = np.asarray(q[b, rows, h], np.float64)
                pq = phi(qr)
                num = pq @ C
                den = pq @ c + eps
                O = num / den[:, None]
                dO = np.asarray(d_ol[b, rows, h], np.float64)
                dnum = dO / den[:, None]
                dden = -np.sum(dO * O, axis=1) / den
                dpq = dnum @ C.T + dden[:, None] * c[None, :]
                dq[b, rows, h] = dpq * dphi(qr)
                dC[b, h, f] = pq.T @ dnum
                dc[b, h, f] = pq.T @ dden
    # through the directional states (forward and backward ranges, half text each)
    dS = np.zeros((B, H, T, D, D))
    dz = np.zeros((B, H, T, D))
    dST = np.zeros((B, H, D, D))
    dzT = np.zeros((B, H, D))
    for f, (_, F, Bk) in enumerate(sets):
        for rng in (F, Bk):
            dST += 0.5 * dC[:, :, f]
            dzT += 0.5 * dc[:, :, f]
            for g in rng:
                dS[:, :, g] += dC[:, :, f]
                dz[:, :, g] += dc[:, :, f]
    # through the per-frame and text states
    dk = np.zeros((B, N, H, D))
    dv = np.zeros((B, N, H, D))
    dtk = np.zeros(text_k.shape)
    dtv = np.zeros(text_v.shape)
    for b in range(B):
        for h in range(H):
            for g in range(T):
                rows = np.arange(g * n, (g + 1) * n)
                kr = np.asarray(k[b, rows, h], np.float64)
                vr = np.asarray(v[b, rows, h], np.float64)
                pk = phi(kr)
                dk[b, rows, h] = (vr @ dS[b, h, g].T + dz[b, h, g][None, :]) * dphi(kr)
                dv[b, rows, h] = pk @ dS[b, h, g]
            kr = np.asarray(text_k[b, :, h], np.float64)
            vr = np.asarray(text_v[b, :, h], np.float64)
            dtk[b, :, h] = (vr @ dST[b, h].T + dzT[b, h][None, :]) * dphi(kr)
            dtv[b, :, h] = phi(kr) @ dST[b, h]
    return dq, dk, dv, dtk, dtv


def epilogue_backward(x, o_s, o_l, w_gs, w_gl, w_os, w_ol, rms_w, dy, eps=1e-6):
    """Gradients of y = x + (G_s O_s) W_os + (G_l R) W_ol with G = sigmoid(x W_g)
    and R = O_l w / sqrt(mean(O_l^2) + eps), given dy = dL/dy.

    Returns dict: dx, dw_gs, dw_gl, dw_os, dw_ol, drms_w, d_os, d_ol
    (d_os, d_ol shaped [B, M, hid])."""
    x = np.asarray(x, np.float64)
    B, M, hid = x.shape
    dy = np.asarray(dy, np.float64).reshape(B * M, hid)
    xf = x.reshape(B * M, hid)
    os_ = np.asarray(o_s, np.float64).reshape(B * M, hid)
    ol_ = np.asarray(o_l, np.float64).reshape(B * M, hid)
    w_gs, w_gl, w_os, w_ol = (np.asarray(a, np.float64) for a in (w_gs, w_gl, w_os, w_ol))
    w = np.asarray(rms_w, np.float64)
    g_s = sigmoid(xf @ w_gs)
    g_l = sigmoid(xf @ w_gl)
    rinv = 1.0 / np.sqrt(np.mean(ol_ * ol_, axis=1, keepdims=True) + eps)
    r = ol_ * w * rinv
    a_s = g_s * os_
    a_l = g_l * r
    # output projections
    dw_os = a_s.T @ dy
    dw_ol = a_l.T @ dy
    da_s = dy @ w_os.T
    da_l = dy @ w_ol.T
    # element-wise gates
    d_os = da_s * g_s
    dz_s = da_s * os_ * g_s * (1.0 - g_s)
    dr = da_l * g_l
    dz_l = da_l * r * g_l * (1.0 - g_l)
    # gate projections and the residual
    dw_gs = xf.T @ dz_s
    dw_gl = xf.T @ dz_l
    dx = dy + dz_s @ w_gs.T + dz_l @ w_gl.T
    # RMSNorm: d rinv / d O_l[j] = -rinv^3 O_l[j] / hid
    drms_w = np.sum(dr * ol_ * rinv, axis=0)
    d_ol = dr * w * rinv - ol_ * rinv ** 3 / hid * np.sum(dr * w * ol_, axis=1, keepdims=True)
    return {"dx": dx.reshape(B, M, hid), "dw_gs": dw_gs, "dw_gl": dw_gl, "dw_os": dw_os, "dw_ol": dw_ol,
            "drms_w": drms_w, "d_os": d_os.reshape(B, M, hid), "d_ol": d_ol.reshape(B, M, hid)}


def hybrid_backward(inp, lay, dy, scale=None, eps=1e-6):
    """All gradients of L = sum(dy * y) for the layer: the forward of
    ``hybrid.hybrid_forward`` followed by the three reverse steps above.

    Returns dict with dx, dq, dk, dv, dtext_k, dtext_v, dw_gs, dw_gl, dw_os,
    dw_ol, drms_w and the intermediates d_os, d_ol [B, N, H, D] and lse
    [B, N, H]."""
    from .hybrid import linear_branch, softmax_branch
    B, N, H, D = inp["q"].shape
    o_s = softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, scale=scale)
    st = linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    o_l = linear_branch(inp["q"], st, lay, eps=eps)
    ep = epilogue_backward(inp["x"], o_s, o_l, inp["w_gs"], inp["w_gl"], inp["w_os"], inp["w_ol"], inp["rms_w"],
                           dy, eps=eps)
    d_os = ep["d_os"].reshape(B, N, H, D)
    d_ol = ep["d_ol"].reshape(B, N, H, D)
    sq, sk, sv, stk, stv = softmax_backward(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, d_os,
                                            scale=scale)
    lq, lk, lv, ltk, ltv = linear_backward(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, d_ol,
                                           eps=eps)
    out = {k_: ep[k_] for k_ in ("dx", "dw_gs", "dw_gl", "dw_os", "dw_ol", "drms_w")}
    out.update({"dq": sq + lq, "dk": sk + lk, "dv": sv + lv, "dtext_k": stk + ltk, "dtext_v": stv + ltv,
                "d_os": d_os, "d_ol": d_ol,
                "lse": softmax_lse(inp["q"], inp["k"], inp["text_k"], lay, scale=scale)})
    return out


def dq_dx_at(inp, lay, dy, tokens, states=None, scale=None, eps=1e-6):
    """dq and dx at a sample of video tokens only (each is a function of its
    own row given the layer's frame states): the epilogue backward of those
    rows, then the softmax rows' dQ over their key sets and the linear
    readout's dq.  Returns (dq [B, len, H, D], dx [B, len, hid])."""
    from .hybrid import linear_branch, softmax_branch
    q, k, v, tk, tv = inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"]
    B, N, H, D = q.shape
    n = lay.tokens_per_frame
    tau = 1.0 / math.sqrt(D) if not scale else float(scale)
    rows = np.asarray(tokens, np.int64)
    st = states if states is not None else linear_states(k, v, tk, tv, lay)
    o_s = softmax_branch(q, k, v, tk, tv, lay, scale=scale, tokens=rows)
    o_l = linear_branch(q, st, lay, eps=eps, tokens=rows)
    ep = epilogue_backward(np.asarray(inp["x"])[:, rows], o_s, o_l, inp["w_gs"], inp["w_gl"], inp["w_os"],
                           inp["w_ol"], inp["rms_w"], np.asarray(dy)[:, rows], eps=eps)
    d_os = ep["d_os"].reshape(B, rows.size, H, D)
    d_ol = ep["d_ol"].reshape(B, rows.size, H, D)
    sets = frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    Sf, zf, Sb, zb = directional_states(st, lay)
    dq = np.zeros((B, rows.size, H, D))
    for f in range(lay.frames):
        sel = np.nonzero(rows // n == f)[0]
        if sel.size == 0:
            continue
        kt = _key_tokens(lay, sets[f][0])
        for b in range(B):
            for h in range(H):
                K = np.concatenate([np.asarray(k[b, kt, h], np.float64), np.asarray(tk[b, :, h], np.float64)])
                V = np.concatenate([np.asarray(v[b, kt, h], np.float64), np.asarray(tv[b, :, h], np.float64)])
                C = Sf[b, h, f] + Sb[b, h, f]
                c = zf[b, h, f] + zb[b, h, f]
                for i in sel:
                    qi = np.asarray(q[b, rows[i], h], np.float64)
                    sc = tau * (K @ qi)
                    p = np.exp(sc - sc.max())
                    p /= p.sum()
                    dO = d_os[b, i, h]
                    ds = p * (V @ dO - np.dot(dO, o_s[b, i, h]))
                    pq = phi(qi)
                    den = pq @ c + eps
                    O = (pq @ C) / den
                    g = d_ol[b, i, h]
                    dpq = C @ (g / den) - c * (np.dot(g, O) / den)
                    dq[b, i, h] = tau * (ds @ K) + dpq * dphi(qi)
    return dq, ep["dx"]


def block_backward(inp, lay, proj, dy, scale=None, eps=1e-6):
    """Gradients of L = sum(dy * y) for the layer with its Q/K/V projection,
    y = layer(x; q, k, v = x W_q, x W_k, x W_v) (oracle/projection.py; no
    rounding between the steps here).  The layer's gradients, then through
    the projection: dx += dq W_q^T + dk W_k^T + dv W_v^T and
    dW_q = x^T dq (likewise k, v), heads flattened into the hidden axis.
    Returns the layer's dict with dx replaced and dw_q, dw_k, dw_v added."""
    from .projection import qkv_projection
    x = np.asarray(inp["x"], np.float64)
    B, N, hid = x.shape
    q, k, v = qkv_projection(x, proj["w_q"], proj["w_k"], proj["w_v"], lay.heads)
    g = hybrid_backward(dict(inp, q=q, k=k, v=v), lay, dy, scale=scale, eps=eps)
    xf = x.reshape(B * N, hid)
    dx = g["dx"].reshape(B * N, hid)
    for name, dname in (("w_q", "dq"), ("w_k", "dk"), ("w_v", "dv")):
        d = g[dname].reshape(B * N, hid)
        dx = dx + d @ np.asarray(proj[name], np.float64).T
        g["d" + name] = xf.T @ d
    g["dx"] = dx.reshape(B, N, hid)
    return g


def key_side_grads(inp, lay, dy, heads, scale=None, eps=1e-6, rows_per_block=4096, log=None):
    """Key-side gradients of the layer for a subset of heads, at sizes where
    hybrid_backward would be slow: dk, dv [B, N, len(heads), D] and dtext_k,
    dtext_v [B, L, len(heads), D] for those heads, and the weight gradients
    dw_gl, dw_ol [hid, hid] and drms_w [hid], which do not involve O_s.

    dL/dO_s and dL/dO_l come from epilogue_backward run on row blocks (its
    d_os = (dy W_os^T) G_s and d_ol, dw_gl, dw_ol, drms_w never read O_s,
    which is passed as zeros; the weight gradients are sums over rows); the
    softmax and linear reverse steps then run on the chosen heads alone,
    since both branches are independent per (batch, head).  ``log``, if
    given, is called with a short message after each of those steps."""
    from .hybrid import linear_branch
    log = log or (lambda msg: None)
    q, k, v, tk, tv = (np.asarray(inp[n]) for n in ("q", "k", "v", "text_k", "text_v"))
    B, N, H, D = q.shape
    hid = H * D
    st = linear_states(k, v, tk, tv, lay)
    o_l = linear_branch(q, st, lay, eps=eps).reshape(B, N, hid)
    log("linear branch forward done")
    x = np.asarray(inp["x"])
    dyv = np.asarray(dy)
    d_os = np.zeros((B, N, len(heads), D))
    d_ol = np.zeros((B, N, len(heads), D))
    dw_gl = np.zeros((hid, hid))
    dw_ol = np.zeros((hid, hid))
    drms_w = np.zeros(hid)
    for r0 in range(0, N, rows_per_block):
        sl = slice(r0, min(N, r0 + rows_per_block))
        ep = epilogue_backward(x[:, sl], np.zeros((B, sl.stop - r0, hid)), o_l[:, sl], inp["w_gs"], inp["w_gl"],
                               inp["w_os"], inp["w_ol"], inp["rms_w"], dyv[:, sl], eps=eps)
        d_os[:, sl] = ep["d_os"].reshape(B, -1, H, D)[:, :, heads]
        d_ol[:, sl] = ep["d_ol"].reshape(B, -1, H, D)[:, :, heads]
        dw_gl += ep["dw_gl"]
        dw_ol += ep["dw_ol"]
        drms_w += ep["drms_w"]
        log("epilogue reverse: rows %d of %d" % (sl.stop, N))
    sub = [np.ascontiguousarray(a[:, :, heads]) for a in (q, k, v, tk, tv)]
    _, sk, sv, stk, stv = softmax_backward(*sub, lay, d_os, scale=scale)
    log("softmax branch reverse done")
    _, lk, lv, ltk, ltv = linear_backward(*sub, lay, d_ol, eps=eps)
    log("linear branch reverse done")
    return {"dk": sk + lk, "dv": sv + lv, "dtext_k": stk + ltk, "dtext_v": stv + ltv,
            "dw_gl": dw_gl, "dw_ol": dw_ol, "drms_w": drms_w}
