"""Pins of the Q/K/V projection in the oracle (CPU)."""
import numpy as np
import torch

from oracle import projection as proj


def test_one_hot_weights_pin_orientation_and_head_split():
    # W[i, p(i)] = 1 with a non-symmetric permutation p: output feature p(i)
    # must equal input feature i ([in][out] weights, y = x W)
    B, N, H, D = 2, 5, 3, 4
    hid = H * D
    g = np.random.Generator(np.random.PCG64(11))
    x = g.standard_normal((B, N, hid))
    p = np.roll(np.arange(hid), 5)
    w = np.zeros((hid, hid))
    w[np.arange(hid), p] = 1.0
    y = proj.project(x, w, H)
    assert y.shape == (B, N, H, D)
    flat = y.reshape(B, N, hid)
    for i in range(hid):
        assert np.array_equal(flat[:, :, p[i]], x[:, :, i])
    # head h, dim d is feature h * D + d
    for h in range(H):
        for d in range(D):
            assert np.array_equal(y[:, :, h, d], flat[:, :, h * D + d])


def test_identity_weight_gives_feature_index_per_head():
    B, N, H, D = 1, 3, 4, 8
    hid = H * D
    x = np.tile(np.arange(hid, dtype=np.float64), (B, N, 1)) + 1000.0 * np.arange(N)[None, :, None]
    y = proj.project(x, np.eye(hid), H)
    for h in range(H):
        for d in range(D):
            assert np.all(y[0, :, h, d] == h * D + d + 1000.0 * np.arange(N))


def test_diagonal_weights_scale_each_feature():
    B, N, H, D = 1, 4, 2, 8
    hid = H * D
    g = np.random.Generator(np.random.PCG64(12))
    x = g.standard_normal((B, N, hid))
    c = np.linspace(-2.0, 3.0, hid)
    y = proj.project(x, np.diag(c), H).reshape(B, N, hid)
    assert np.array_equal(y, x * c)


def test_two_token_hand_example():
    # hid = 2, one head: q = [x0 w00 + x1 w10, x0 w01 + x1 w11]
    x = np.array([[[1.0, 2.0], [-3.0, 0.5]]])
    w = np.array([[2.0, -1.0], [0.25, 4.0]])
    q = proj.project(x, w, 1)[:, :, 0, :]
    assert np.array_equal(q, np.array([[[2.5, 7.0], [-5.875, 5.0]]]))


def test_qkv_projection_uses_each_weight_once():
    B, N, H, D = 1, 3, 2, 4
    hid = H * D
    x = np.ones((B, N, hid))
    q, k, v = proj.qkv_projection(x, 1 * np.eye(hid), 2 * np.eye(hid), 3 * np.eye(hid), H)
    assert np.all(q == 1) and np.all(k == 2) and np.all(v == 3)


def test_absmax_per_head_constructed():
    t = np.zeros((2, 6, 3, 4))
    t[0, 2, 1, 3] = -7.5       # negative extreme counts by magnitude
    t[0, 5, 1, 0] = 7.25
    t[1, 0, 0, 0] = 0.125
    t[1, 4, 2, 2] = 3.0
    m = proj.absmax_per_head(t)
    assert np.array_equal(m, np.array([[0.0, 7.5, 0.0], [0.125, 0.0, 3.0]]))


def test_round_bf16_matches_torch_bfloat16():
    g = np.random.Generator(np.random.PCG64(13))
    x = np.concatenate([g.standard_normal(50000) * s for s in (1e-3, 1.0, 300.0)])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(proj.round_bf16(x32), ref)
