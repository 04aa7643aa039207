"""Independent checks that pin the fp64 oracle to the article and to
mathematics, not to itself.  Each check recomputes the quantity by a
different route (token-level masks instead of frame-set gathers, quadratic
linear attention instead of states, library SDPA, closed forms) and raises
AssertionError on mismatch, so the mutation tests can plant mistakes in the
oracle and watch a check fail.
"""
import math

import numpy as np
from scipy.special import logsumexp

import oracle
from oracle import layout as olayout


def read_golden(path):
    cases, meta, cur = [], {}, None
    for line in open(path, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        vals = [int(x) for x in vals]
        if key == "query_frame":
            cur = {"f": vals[0]}
            cases.append(cur)
        elif cur is not None:
            cur[key] = set(vals)
        else:
            meta[key] = vals
    return meta, cases


def token_masks(lay):
    """Token-level visibility built from the golden-free rule statement:
    softmax mask [N, N] and linear mask [N, N] (video keys only)."""
    n, T = lay.tokens_per_frame, lay.frames
    sets = olayout.frame_sets(T, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    fr = np.arange(T * n) // n
    soft = np.zeros((T * n, T * n), bool)
    lin = np.zeros((T * n, T * n), bool)
    for i in range(T * n):
        S, F, B = sets[fr[i]]
        soft[i] = np.isin(fr, list(S))
        lin[i] = np.isin(fr, list(F | B))
    return soft, lin


def brute_softmax(q, k, v, tk, tv, lay):
    """Dense masked softmax: all N + L keys, masked by the token mask; the
    normaliser through logsumexp (no max subtraction)."""
    B, N, H, D = q.shape
    soft, _ = token_masks(lay)
    L = tk.shape[1]
    mask = np.concatenate([soft, np.ones((N, L), bool)], axis=1)
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            K = np.concatenate([k[b, :, h], tk[b, :, h]]).astype(np.float64)
            V = np.concatenate([v[b, :, h], tv[b, :, h]]).astype(np.float64)
            s = (q[b, :, h].astype(np.float64) @ K.T) / math.sqrt(D)
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - logsumexp(s, axis=1, keepdims=True))
            out[b, :, h] = p @ V
    return out


def _phi_scalar(u):
    return u + 1.0 if u > 0 else math.exp(u)


def brute_linear(q, k, v, tk, tv, lay, eps=1e-6):
    """Quadratic masked linear attention: every visible video key weight 1,
    every text key weight 1/2 + 1/2, one shared normaliser."""
    B, N, H, D = q.shape
    _, lin = token_masks(lay)
    L = tk.shape[1]
    vphi = np.vectorize(_phi_scalar)
    w = np.concatenate([lin.astype(np.float64), np.full((N, L), 0.5) + np.full((N, L), 0.5)], axis=1)
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            K = vphi(np.concatenate([k[b, :, h], tk[b, :, h]]).astype(np.float64))
            V = np.concatenate([v[b, :, h], tv[b, :, h]]).astype(np.float64)
            a = (vphi(q[b, :, h].astype(np.float64)) @ K.T) * w
            out[b, :, h] = (a @ V) / (a.sum(axis=1, keepdims=True) + eps)
    return out


def check_close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    if not err <= tol * scale:
        raise AssertionError("%s: max err %.3e > %.1e" % (what, err, tol * scale))


def tiny_inputs(lay, seed, L=None, integer=False):
    g = np.random.Generator(np.random.PCG64(seed))
    B, N, H, D = lay.batch, lay.n_video, lay.heads, lay.head_dim
    L = lay.text_tokens if L is None else L
    if integer:
        def draw(shape, lo, hi):
            return g.integers(lo, hi, size=shape).astype(np.float64)
        inp = {"q": draw((B, N, H, D), 0, 3), "k": draw((B, N, H, D), 0, 4),
               "v": draw((B, N, H, D), -3, 4), "text_k": draw((B, L, H, D), 0, 4),
               "text_v": draw((B, L, H, D), -3, 4)}
    else:
        inp = {nm: g.standard_normal(shape) for nm, shape in
               (("q", (B, N, H, D)), ("k", (B, N, H, D)), ("v", (B, N, H, D)),
                ("text_k", (B, L, H, D)), ("text_v", (B, L, H, D)))}
    hid = H * D
    inp["x"] = g.standard_normal((B, N, hid))
    for nm in ("w_gs", "w_gl", "w_os", "w_ol"):
        inp[nm] = 0.2 * g.standard_normal((hid, hid))
    inp["rms_w"] = np.ones(hid)
    return inp


# --- the pins, as callables ------------------------------------------------

def pin_worked_example(path):
    meta, cases = read_golden(path)
    T, C, R = meta["frames"][0], meta["chunk_frames"][0], meta["chunk_radius"][0]
    anchors = set(meta["anchors"])
    sets = oracle.frame_sets(T, C, R, 0 in anchors, (T - 1) in anchors)
    for c in cases:
        S, F, B = sets[c["f"]]
        if (S, F, B) != (c["softmax"], c["forward"], c["backward"]):
            raise AssertionError("frame %d: got S=%s F=%s B=%s" % (c["f"], sorted(S), sorted(F), sorted(B)))


def pin_text_once(lay, seed=0):
    """Integer inputs, K >= 0 so phi(k) = k + 1 exactly: for every query frame,
    S+ + S- + sum_{g in S(f)} S_g equals sum_all S_g + S_T exactly."""
    inp = tiny_inputs(lay, seed, integer=True)
    st = oracle.linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    S, z, ST, zT = st
    Sf, zf, Sb, zb = oracle.hybrid.directional_states(st, lay)
    sets = oracle.frame_sets(lay.frames, lay.chunk_frames, lay.chunk_radius, lay.anchor_first, lay.anchor_last)
    # phi(k) = k + 1 for k >= 0: the exact per-frame sums, computed directly
    kk = inp["k"] + 1.0
    n = lay.tokens_per_frame
    tot = np.einsum("bnhd,bnhe->bhde", kk, inp["v"]) + np.einsum("blhd,blhe->bhde", inp["text_k"] + 1.0, inp["text_v"])
    for f, (Sset, _, _) in enumerate(sets):
        win = sum((np.einsum("bnhd,bnhe->bhde", kk[:, g * n:(g + 1) * n], inp["v"][:, g * n:(g + 1) * n]) for g in Sset))
        lhs = Sf[:, :, f] + Sb[:, :, f] + win
        if not np.array_equal(lhs, tot):
            raise AssertionError("text-once invariant broken at frame %d" % f)


def pin_softmax_bruteforce(lay, seed=0, L=None):
    inp = tiny_inputs(lay, seed, L=L)
    a = oracle.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    b = brute_softmax(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    check_close(a, b, 1e-12, "softmax vs dense masked brute force")


def pin_linear_bruteforce(lay, seed=0, L=None):
    inp = tiny_inputs(lay, seed, L=L)
    st = oracle.linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    a = oracle.linear_branch(inp["q"], st, lay)
    b = brute_linear(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    check_close(a, b, 1e-12, "linear vs quadratic masked brute force")


def pin_sdpa(lay, seed=0):
    """All frames visible (radius covers every chunk): the softmax branch is
    plain attention over all video + text keys -> torch SDPA in float64."""
    import torch
    import torch.nn.functional as Fnn
    inp = tiny_inputs(lay, seed)
    a = oracle.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    q = torch.from_numpy(inp["q"]).permute(0, 2, 1, 3)
    k = torch.from_numpy(np.concatenate([inp["k"], inp["text_k"]], axis=1)).permute(0, 2, 1, 3)
    v = torch.from_numpy(np.concatenate([inp["v"], inp["text_v"]], axis=1)).permute(0, 2, 1, 3)
    b = Fnn.scaled_dot_product_attention(q, k, v).permute(0, 2, 1, 3).numpy()
    check_close(a, b, 1e-12, "softmax vs torch SDPA")


def pin_onehot_gate(seed=0):
    """W_gs with one nonzero entry [i0][j0] = a: g_s[:, j0] = sigmoid(a x[:, i0]),
    every other column exactly 1/2 (pins the [in][out] orientation)."""
    g = np.random.Generator(np.random.PCG64(seed))
    B, M, H, D = 1, 5, 2, 4
    hid = H * D
    x = g.standard_normal((B, M, hid))
    o = g.standard_normal((B, M, H, D))
    W = np.zeros((hid, hid))
    i0, j0, a = 1, 6, 0.75
    W[i0, j0] = a
    Z = np.zeros((hid, hid))
    ep = oracle.epilogue(x, o, o, W, Z, Z, Z, np.ones(hid))
    want = np.full((B, M, hid), 0.5)
    for m in range(M):
        want[0, m, j0] = 1.0 / (1.0 + math.exp(-a * x[0, m, i0]))
    check_close(ep["g_s"], want, 1e-15, "one-hot gate")
    if not np.all(ep["g_l"] == 0.5):
        raise AssertionError("zero gate weight must give exactly 1/2")


def pin_onehot_out(seed=0):
    """W_os one-hot [i0][j0] = 1, W_ol = 0, W_gs = 0 (gate 1/2):
    delta[:, j0] = O_s[:, i0] / 2 and every other column 0."""
    g = np.random.Generator(np.random.PCG64(seed))
    B, M, H, D = 1, 4, 2, 4
    hid = H * D
    x = g.standard_normal((B, M, hid))
    os_ = g.standard_normal((B, M, H, D))
    ol = g.standard_normal((B, M, H, D))
    Z = np.zeros((hid, hid))
    W = np.zeros((hid, hid))
    i0, j0 = 5, 2
    W[i0, j0] = 1.0
    ep = oracle.epilogue(x, os_, ol, Z, Z, W, Z, np.ones(hid))
    want = np.zeros((B, M, hid))
    want[0, :, j0] = 0.5 * os_.reshape(B, M, hid)[0, :, i0]
    check_close(ep["delta"], want, 1e-15, "one-hot output projection")
    check_close(ep["y"], x + want, 1e-15, "residual")


def pin_rms_scope():
    """Linear-branch output constant per head (c_h): RMSNorm over the whole
    hidden size gives w * c_h / sqrt(mean over heads of c_h^2 + eps)."""
    B, M, H, D = 1, 3, 3, 4
    hid = H * D
    c = np.array([1.0, -2.0, 3.0])
    ol = np.broadcast_to(c[None, None, :, None], (B, M, H, D)).copy()
    w = np.linspace(0.5, 1.5, hid)
    Z = np.zeros((hid, hid))
    ep = oracle.epilogue(np.zeros((B, M, hid)), ol, ol, Z, Z, Z, Z, w)
    rms = math.sqrt((1.0 + 4.0 + 9.0) / 3.0 + 1e-6)
    want = (np.repeat(c, D) / rms * w)[None, None, :].repeat(M, axis=1)
    check_close(ep["r"], want, 1e-15, "RMSNorm scope")
