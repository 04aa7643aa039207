"""Pins of the oracle's softmax branch, linear branch and epilogue (CPU)."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle.layout import Layout
from tests import pins

LAYOUTS = [
    Layout(1, 7, 3, 4, 2, 4, chunk_frames=1, chunk_radius=1),
    Layout(2, 9, 2, 3, 1, 3, chunk_frames=2, chunk_radius=1),
    Layout(1, 8, 2, 0, 1, 4, chunk_frames=1, chunk_radius=0, anchor_first=False, anchor_last=False),
    Layout(1, 11, 2, 5, 1, 2, chunk_frames=3, chunk_radius=1, anchor_first=True, anchor_last=False),
    Layout(1, 1, 5, 2, 1, 4),
    Layout(1, 2, 3, 2, 1, 4),
]


@pytest.mark.parametrize("lay", LAYOUTS)
def test_softmax_matches_dense_masked_bruteforce(lay):
    pins.pin_softmax_bruteforce(lay, seed=11)


@pytest.mark.parametrize("lay", LAYOUTS)
def test_linear_matches_quadratic_bruteforce(lay):
    pins.pin_linear_bruteforce(lay, seed=12)


@pytest.mark.parametrize("lay", LAYOUTS)
def test_text_counted_once_exact(lay):
    pins.pin_text_once(lay, seed=13)


def test_softmax_all_frames_visible_is_sdpa():
    pins.pin_sdpa(Layout(1, 6, 3, 4, 2, 8, chunk_frames=1, chunk_radius=6), seed=14)
    pins.pin_sdpa(Layout(1, 5, 4, 0, 1, 4, chunk_frames=2, chunk_radius=3, anchor_first=False, anchor_last=False), seed=15)


def test_constant_v_closed_forms():
    lay = Layout(1, 6, 3, 4, 2, 4)
    inp = pins.tiny_inputs(lay, 16)
    c = np.array([0.5, -1.25, 2.0, 3.0])
    inp["v"][:] = c
    inp["text_v"][:] = c
    o = oracle.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    pins.check_close(o, np.broadcast_to(c, o.shape), 1e-14, "softmax constant V")
    st = oracle.linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    ol = oracle.linear_branch(inp["q"], st, lay)
    # visible weights w_j = phi(q).phi(k_j): sum(w c) / (sum(w) + eps) = c * W / (W + eps)
    wsum = _visible_weight_sums(inp, lay)
    want = c[None, None, None, :] * (wsum / (wsum + 1e-6))[..., None]
    pins.check_close(ol, want, 1e-13, "linear constant V")


def _visible_weight_sums(inp, lay):
    # sum over visible keys of phi(q).phi(k), by direct token loops
    _, lin = pins.token_masks(lay)
    B, N, H, D = inp["q"].shape
    out = np.zeros((B, N, H))
    ph = lambda a: np.array([[pins._phi_scalar(t) for t in row] for row in a])
    for b in range(B):
        for h in range(H):
            pq = ph(inp["q"][b, :, h])
            pk = ph(inp["k"][b, :, h])
            pt = ph(inp["text_k"][b, :, h])
            for i in range(N):
                out[b, i, h] = (pq[i] @ pk[lin[i]].T).sum() + (pq[i] @ pt.T).sum()
    return out


def test_phi_closed_forms():
    u = np.array([-30.0, -2.5, -1e-9, 0.0, 1e-9, 0.5, 7.0])
    got = oracle.phi(u)
    want = [math.exp(-30.0), math.exp(-2.5), math.exp(-1e-9), 1.0, 1.0 + 1e-9, 1.5, 8.0]
    assert np.allclose(got, want, rtol=1e-15, atol=0)


def test_anchor_rows_linear_is_text_only_and_zero_without_text():
    lay = Layout(1, 6, 3, 3, 1, 4)
    inp = pins.tiny_inputs(lay, 17)
    st = oracle.linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    a = oracle.linear_branch(inp["q"], st, lay)
    inp2 = dict(inp)
    inp2["k"] = inp["k"] * 3.0 + 1.0
    inp2["v"] = -inp["v"]
    st2 = oracle.linear_states(inp2["k"], inp2["v"], inp2["text_k"], inp2["text_v"], lay)
    b = oracle.linear_branch(inp2["q"], st2, lay)
    n = lay.tokens_per_frame
    anchor_rows = list(range(0, n)) + list(range(5 * n, 6 * n))
    assert np.array_equal(a[:, anchor_rows], b[:, anchor_rows])
    lay0 = Layout(1, 6, 3, 0, 1, 4)
    inp0 = pins.tiny_inputs(lay0, 18)
    st0 = oracle.linear_states(inp0["k"], inp0["v"], inp0["text_k"], inp0["text_v"], lay0)
    o0 = oracle.linear_branch(inp0["q"], st0, lay0)
    assert np.all(o0[:, anchor_rows] == 0.0)
    # frame 1 and frame 4 have an empty forward / backward side respectively,
    # frames 1..4 with radius 1 and 4 interior frames: frame 1 sees F=0,B={3,4}
    assert oracle.frame_sets(6, 1, 1)[1][1] == set()


def test_symmetries():
    lay = Layout(1, 5, 4, 3, 1, 4)
    inp = pins.tiny_inputs(lay, 19)
    ref = oracle.hybrid_forward(inp, lay)
    g = np.random.Generator(np.random.PCG64(3))
    n = lay.tokens_per_frame
    perm = np.concatenate([f * n + g.permutation(n) for f in range(lay.frames)])
    p = dict(inp)
    for nm in ("x", "q", "k", "v"):
        p[nm] = inp[nm][:, perm]
    out = oracle.hybrid_forward(p, lay)
    for key in ("o_s", "o_l", "y"):
        pins.check_close(out[key], ref[key][:, perm], 1e-12, "in-frame permutation " + key)
    tp = g.permutation(lay.text_tokens)
    p = dict(inp)
    p["text_k"] = inp["text_k"][:, tp]
    p["text_v"] = inp["text_v"][:, tp]
    out = oracle.hybrid_forward(p, lay)
    for key in ("o_s", "o_l", "y"):
        pins.check_close(out[key], ref[key], 1e-12, "text permutation " + key)


def test_epilogue_closed_forms():
    pins.pin_onehot_gate()
    pins.pin_onehot_out()
    pins.pin_rms_scope()
    lay = Layout(1, 4, 2, 2, 2, 2)
    inp = pins.tiny_inputs(lay, 20)
    for nm in ("w_os", "w_ol"):
        inp[nm] = np.zeros_like(inp[nm])
    out = oracle.hybrid_forward(inp, lay)
    assert np.array_equal(out["y"], inp["x"])


def test_token_sample_matches_full():
    lay = Layout(2, 5, 6, 3, 2, 4, chunk_frames=2)
    inp = pins.tiny_inputs(lay, 21)
    full = oracle.hybrid_forward(inp, lay)
    rows = np.array([0, 5, 6, 13, 29])
    part = oracle.hybrid_forward(inp, lay, tokens=rows)
    for key in ("o_s", "o_l", "y", "delta", "g_s", "g_l"):
        pins.check_close(part[key], full[key][:, rows], 1e-13, key)
