"""Pins of the DiT-block oracle (CPU): the GELU, the RMSNorm, the residual
feed-forward and its composition with the layer."""
import math

import numpy as np
import torch

from oracle import dit
from oracle.layout import Layout


def test_gelu_matches_torch_tanh_gelu_and_limits():
    g = np.random.Generator(np.random.PCG64(31))
    u = np.concatenate([g.standard_normal(20000) * s for s in (0.1, 1.0, 6.0)])
    ref = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    assert np.allclose(dit.gelu_tanh(u), ref, rtol=1e-14, atol=1e-15)
    assert dit.gelu_tanh(0.0) == 0.0
    assert abs(dit.gelu_tanh(12.0) - 12.0) < 1e-12          # tanh -> 1
    assert abs(dit.gelu_tanh(-12.0)) < 1e-30                  # tanh -> -1
    # odd part: gelu(u) - gelu(-u) = u
    assert np.allclose(dit.gelu_tanh(u) - dit.gelu_tanh(-u), u, rtol=0, atol=1e-12)


def test_rmsnorm_hand_example_and_scale_invariance():
    y = np.array([[3.0, 4.0]])
    out = dit.rmsnorm(y, np.array([1.0, 2.0]), eps=0.0)
    r = math.sqrt(12.5)
    assert np.allclose(out, [[3.0 / r, 8.0 / r]], rtol=1e-15, atol=0)
    g = np.random.Generator(np.random.PCG64(32))
    y = g.standard_normal((5, 64))
    w = g.standard_normal(64)
    assert np.allclose(dit.rmsnorm(7.5 * y, w, eps=0.0), dit.rmsnorm(y, w, eps=0.0), rtol=1e-13, atol=1e-14)
    # unit weight: every row has mean square 1
    assert np.allclose(np.mean(dit.rmsnorm(y, np.ones(64), eps=0.0) ** 2, axis=-1), 1.0, rtol=1e-13)


def test_ffn_zero_and_identity_weights():
    g = np.random.Generator(np.random.PCG64(33))
    hid = 16
    y = g.standard_normal((2, 7, hid))
    w_n = 1.0 + 0.1 * g.standard_normal(hid)
    # W_2 = 0: exactly the residual
    assert np.array_equal(dit.ffn(y, w_n, g.standard_normal((hid, 4 * hid)), np.zeros((4 * hid, hid))), y)
    # W_1 = W_2 = I (F = hid): y + gelu(rmsnorm(y))
    z = dit.ffn(y, w_n, np.eye(hid), np.eye(hid))
    assert np.allclose(z, y + dit.gelu_tanh(dit.rmsnorm(y, w_n)), rtol=1e-15, atol=1e-15)
    # one-hot W_1 (column permutation p) and W_2 = its transpose undo each other
    p = np.roll(np.arange(hid), 3)
    w1 = np.zeros((hid, hid))
    w1[np.arange(hid), p] = 1.0
    z = dit.ffn(y, w_n, w1, w1.T)
    assert np.allclose(z, y + dit.gelu_tanh(dit.rmsnorm(y, w_n)), rtol=1e-15, atol=1e-15)


def test_block_composition():
    """z = ffn(round(layer(projections))) and with W_2 = 0 the block is the
    layer with its projection."""
    from oracle import hybrid_forward
    from oracle.projection import qkv_projection, round_bf16
    lay = Layout(1, 5, 3, 2, 2, 4)
    g = np.random.Generator(np.random.PCG64(34))
    hid = lay.hidden
    inp = {"x": g.standard_normal((1, lay.n_video, hid)),
           "text_k": g.standard_normal((1, 2, 2, 4)), "text_v": g.standard_normal((1, 2, 2, 4)),
           "rms_w": np.ones(hid)}
    for w in ("w_gs", "w_gl", "w_os", "w_ol"):
        inp[w] = 0.3 * g.standard_normal((hid, hid))
    proj = {n: 0.3 * g.standard_normal((hid, hid)) for n in ("w_q", "w_k", "w_v")}
    fw = {"w_n": np.ones(hid), "w_1": 0.2 * g.standard_normal((hid, 4 * hid)), "w_2": np.zeros((4 * hid, hid))}
    out = dit.dit_block(inp, lay, proj, fw)
    q, k, v = (round_bf16(t) for t in qkv_projection(inp["x"], proj["w_q"], proj["w_k"], proj["w_v"], 2))
    y = round_bf16(hybrid_forward(dict(inp, q=q, k=k, v=v), lay)["y"])
    assert np.array_equal(out["z"], y)
    fw["w_2"] = 0.2 * g.standard_normal((4 * hid, hid))
    out = dit.dit_block(inp, lay, proj, fw)
    assert np.allclose(out["z"], dit.ffn(y, fw["w_n"], fw["w_1"], fw["w_2"]), rtol=1e-15, atol=1e-15)
