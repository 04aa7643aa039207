"""Pins of the oracle's backward pass (CPU): central finite differences of the
forward oracle along random directions, per input tensor and per reverse
step, plus planted mistakes that the finite differences must catch."""
import math

import numpy as np
import pytest

import oracle
import oracle.backward as BW
from oracle.layout import Layout

# 7 frames of 3 tokens, window +-1 frame, anchors 0 and 6: interior frames have
# non-empty forward and backward ranges; chunked layout with a short last chunk
LAYOUTS = [Layout(1, 7, 3, 4, 2, 4), Layout(2, 9, 2, 3, 1, 3, chunk_frames=2),
           Layout(1, 6, 2, 0, 2, 3, chunk_radius=0, anchor_first=False)]
NAMES = ("x", "q", "k", "v", "text_k", "text_v", "w_gs", "w_gl", "w_os", "w_ol", "rms_w")
GRAD = {"x": "dx", "q": "dq", "k": "dk", "v": "dv", "text_k": "dtext_k", "text_v": "dtext_v", "w_gs": "dw_gs",
        "w_gl": "dw_gl", "w_os": "dw_os", "w_ol": "dw_ol", "rms_w": "drms_w"}


def make(lay, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    B, N, H, D, L, hid = lay.batch, lay.n_video, lay.heads, lay.head_dim, lay.text_tokens, lay.hidden
    inp = {"x": g.standard_normal((B, N, hid)),
           "q": g.standard_normal((B, N, H, D)), "k": g.standard_normal((B, N, H, D)),
           "v": g.standard_normal((B, N, H, D)),
           "text_k": g.standard_normal((B, L, H, D)), "text_v": g.standard_normal((B, L, H, D)),
           "rms_w": 1.0 + 0.3 * g.standard_normal(hid)}
    for w in ("w_gs", "w_gl", "w_os", "w_ol"):
        inp[w] = g.standard_normal((hid, hid)) / math.sqrt(hid)
    dy = g.standard_normal((B, N, hid))
    return inp, dy


def loss(inp, lay, dy):
    return float(np.sum(dy * oracle.hybrid_forward(inp, lay)["y"]))


def fd(fun, inp, name, u, h=1e-5):
    a = dict(inp)
    a[name] = inp[name] + h * u
    lp = fun(a)
    a[name] = inp[name] - h * u
    lm = fun(a)
    return (lp - lm) / (2 * h)


def check_direction(fun, inp, name, grad, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    u = g.standard_normal(inp[name].shape)
    num = fd(fun, inp, name, u)
    an = float(np.sum(grad * u))
    scale = float(np.sum(np.abs(grad * u))) + 1e-12
    return abs(num - an) / scale, num, an


@pytest.mark.parametrize("li", range(len(LAYOUTS)))
def test_layer_gradients_match_finite_differences(li):
    lay = LAYOUTS[li]
    inp, dy = make(lay, 100 + li)
    gr = BW.hybrid_backward(inp, lay, dy)
    for j, name in enumerate(NAMES):
        if inp[name].size == 0:
            assert gr[GRAD[name]].size == 0
            continue
        err, num, an = check_direction(lambda a: loss(a, lay, dy), inp, name, gr[GRAD[name]], 7 * li + j)
        assert err < 1e-7, (name, num, an, err)


@pytest.mark.parametrize("li", range(len(LAYOUTS)))
def test_each_reverse_step_matches_finite_differences(li):
    """Each reverse step against the finite differences of its own forward
    function (softmax branch, linear branch, epilogue)."""
    lay = LAYOUTS[li]
    inp, dy = make(lay, 200 + li)
    B, N, H, D = inp["q"].shape
    g = np.random.Generator(np.random.PCG64(300 + li))
    d_os = g.standard_normal((B, N, H, D))
    d_ol = g.standard_normal((B, N, H, D))
    names = ("q", "k", "v", "text_k", "text_v")

    def l_soft(a):
        return float(np.sum(d_os * oracle.softmax_branch(a["q"], a["k"], a["v"], a["text_k"], a["text_v"], lay)))

    def l_lin(a):
        st = oracle.linear_states(a["k"], a["v"], a["text_k"], a["text_v"], lay)
        return float(np.sum(d_ol * oracle.linear_branch(a["q"], st, lay)))

    sg = BW.softmax_backward(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, d_os)
    lg = BW.linear_backward(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, d_ol)
    for j, name in enumerate(names):
        if inp[name].size == 0:
            continue
        err, num, an = check_direction(l_soft, inp, name, sg[j], 11 * li + j)
        assert err < 1e-7, ("softmax", name, num, an)
        err, num, an = check_direction(l_lin, inp, name, lg[j], 13 * li + j)
        assert err < 1e-7, ("linear", name, num, an)
    # epilogue, with the branch outputs as its inputs
    ep_in = {"x": inp["x"], "o_s": g.standard_normal((B, N, H, D)), "o_l": g.standard_normal((B, N, H, D)),
             **{w: inp[w] for w in ("w_gs", "w_gl", "w_os", "w_ol", "rms_w")}}

    def l_epi(a):
        return float(np.sum(dy * oracle.epilogue(a["x"], a["o_s"], a["o_l"], a["w_gs"], a["w_gl"], a["w_os"],
                                                 a["w_ol"], a["rms_w"])["y"]))
    eg = BW.epilogue_backward(ep_in["x"], ep_in["o_s"], ep_in["o_l"], inp["w_gs"], inp["w_gl"], inp["w_os"],
                              inp["w_ol"], inp["rms_w"], dy)
    pairs = {"x": "dx", "o_s": "d_os", "o_l": "d_ol", "w_gs": "dw_gs", "w_gl": "dw_gl", "w_os": "dw_os",
             "w_ol": "dw_ol", "rms_w": "drms_w"}
    for j, (name, gname) in enumerate(pairs.items()):
        gv = eg[gname].reshape(ep_in[name].shape)
        err, num, an = check_direction(l_epi, ep_in, name, gv, 17 * li + j)
        assert err < 1e-7, ("epilogue", name, num, an)


def test_lse_closed_forms():
    """q = 0: every score is 0, so lse = log |K(f)| (key-set size, text
    included); a single key frame with identical keys shifts it by tau q.k."""
    lay = Layout(1, 7, 3, 4, 2, 4)
    inp, _ = make(lay, 5)
    q0 = np.zeros_like(inp["q"])
    lse = BW.softmax_lse(q0, inp["k"], inp["text_k"], lay)
    sets = oracle.frame_sets(7, 1, 1)
    for f in range(7):
        nk = len(sets[f][0]) * 3 + 4
        assert np.allclose(lse[0, 3 * f:3 * f + 3], math.log(nk), rtol=0, atol=1e-14)
    # constant keys c: lse = tau q.c + log |K(f)|
    c = np.random.Generator(np.random.PCG64(6)).standard_normal(4)
    kc = np.broadcast_to(c, inp["k"].shape).copy()
    tkc = np.broadcast_to(c, inp["text_k"].shape).copy()
    lse = BW.softmax_lse(inp["q"], kc, tkc, lay)
    for f in range(7):
        nk = len(sets[f][0]) * 3 + 4
        ref = 0.5 * np.einsum("nhd,d->nh", inp["q"][0, 3 * f:3 * f + 3], c) + math.log(nk)
        assert np.allclose(lse[0, 3 * f:3 * f + 3], ref, rtol=0, atol=1e-12)


def test_dphi_closed_form():
    u = np.array([-3.0, -0.5, 0.0, 0.25, 4.0])
    assert np.array_equal(BW.dphi(u), np.array([math.exp(-3.0), math.exp(-0.5), 1.0, 1.0, 1.0]))


# ---- planted mistakes: each must fail the finite-difference pin

MUTATIONS = {
    # the RMSNorm correction term dropped
    "rms_no_correction": ("epilogue_backward", "d_ol = dr * w * rinv - ol_ * rinv ** 3 / hid * np.sum(dr * w * ol_, "
                          "axis=1, keepdims=True)", "d_ol = dr * w * rinv"),
    # sigmoid derivative taken as G instead of G (1 - G)
    "sigmoid_deriv": ("epilogue_backward", "dz_s = da_s * os_ * g_s * (1.0 - g_s)", "dz_s = da_s * os_ * g_s"),
    # softmax: rowsum(dO * O) not subtracted
    "softmax_no_delta": ("softmax_backward", "dS = P * (dP - np.sum(dO * O, axis=1, keepdims=True))",
                         "dS = P * dP"),
    # linear: the normaliser's gradient dropped
    "linear_no_dden": ("linear_backward", "dpq = dnum @ C.T + dden[:, None] * c[None, :]", "dpq = dnum @ C.T"),
    # linear: phi'(q) forgotten
    "linear_no_dphi_q": ("linear_backward", "dq[b, rows, h] = dpq * dphi(qr)", "dq[b, rows, h] = dpq"),
    # linear: text state receives half of the gradient
    "text_half": ("linear_backward", "dST += 0.5 * dC[:, :, f]", "dST += 0.25 * dC[:, :, f]"),
    # linear: the backward range forgotten for the frame states
    "forward_range_only": ("linear_backward", "for rng in (F, Bk):\n            dST += 0.5 * dC[:, :, f]\n"
                           "            dzT += 0.5 * dc[:, :, f]\n            for g in rng:",
                           "for rng in (F, Bk):\n            dST += 0.5 * dC[:, :, f]\n"
                           "            dzT += 0.5 * dc[:, :, f]\n            for g in (F if rng is F else ()):"),
    # linear: S_g used untransposed in dphi(k)
    "states_transposed": ("linear_backward", "(vr @ dS[b, h, g].T + dz[b, h, g][None, :])",
                          "(vr @ dS[b, h, g] + dz[b, h, g][None, :])"),
}


def _mutated_module(old, new):
    import inspect
    import types
    src = inspect.getsource(BW)
    assert old in src, old
    mod = types.ModuleType("oracle.backward_mut")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "backward_mut", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mut", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(mut):
    _, old, new = MUTATIONS[mut]
    M = _mutated_module(old, new)
    caught = False
    for li, lay in enumerate(LAYOUTS[:2]):
        inp, dy = make(lay, 400 + li)
        gr = M.hybrid_backward(inp, lay, dy)
        for j, name in enumerate(NAMES):
            if inp[name].size == 0:
                continue
            err, _, _ = check_direction(lambda a: loss(a, lay, dy), inp, name, gr[GRAD[name]], 19 * li + j)
            if err > 1e-5:
                caught = True
                break
        if caught:
            break
    assert caught, mut


def test_dq_dx_at_sampled_tokens_equal_full_backward():
    """The per-token form used at full size equals the full backward on the
    sampled rows (it restates the same reverse steps one row at a time)."""
    lay = LAYOUTS[1]
    inp, dy = make(lay, 500)
    full = BW.hybrid_backward(inp, lay, dy)
    tok = np.array([0, 3, 7, 10, lay.n_video - 1])
    dq, dx = BW.dq_dx_at(inp, lay, dy, tok)
    assert np.allclose(dq, full["dq"][:, tok], rtol=1e-10, atol=1e-12)
    assert np.allclose(dx, full["dx"][:, tok], rtol=1e-10, atol=1e-12)


def test_key_side_grads_equal_full_backward():
    """The head-subset form used at full size equals the full backward on
    those heads (row blocks smaller than the token count, so the weight
    gradients are summed over several blocks)."""
    for lay in LAYOUTS[:2]:
        inp, dy = make(lay, 510)
        full = BW.hybrid_backward(inp, lay, dy, scale=0.4)
        heads = [lay.heads - 1] if lay.heads > 1 else [0]
        part = BW.key_side_grads(inp, lay, dy, heads, scale=0.4, rows_per_block=7)
        for name in ("dk", "dv", "dtext_k", "dtext_v"):
            assert np.allclose(part[name], full[name][:, :, heads], rtol=1e-10, atol=1e-12), name
        for name in ("dw_gl", "dw_ol", "drms_w"):
            assert np.allclose(part[name], full[name], rtol=1e-10, atol=1e-12), name


def test_block_gradients_match_finite_differences():
    """Through the Q/K/V projection: dx and the projection weights' gradients
    against central differences of the block forward."""
    from oracle.projection import qkv_projection
    lay = LAYOUTS[0]
    inp, dy = make(lay, 600)
    g = np.random.Generator(np.random.PCG64(601))
    hid = lay.hidden
    proj = {n: g.standard_normal((hid, hid)) / math.sqrt(hid) for n in ("w_q", "w_k", "w_v")}

    def block_loss(a):
        q, k, v = qkv_projection(a["x"], a["w_q"], a["w_k"], a["w_v"], lay.heads)
        return float(np.sum(dy * oracle.hybrid_forward(dict(a, q=q, k=k, v=v), lay)["y"]))
    gr = BW.block_backward(inp, lay, proj, dy)
    full = dict(inp, **proj)
    for j, (name, gname) in enumerate((("x", "dx"), ("w_q", "dw_q"), ("w_k", "dw_k"), ("w_v", "dw_v"),
                                       ("text_k", "dtext_k"), ("w_gl", "dw_gl"))):
        err, num, an = check_direction(block_loss, full, name, gr[gname], 700 + j)
        assert err < 1e-7, (name, num, an)
