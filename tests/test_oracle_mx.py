"""Pins of oracle/mx.py (MX e4m3 GEMM emulation) against the block format's
definition, torch's e4m3 conversion, closed forms and brute force."""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx
from oracle.layout import Layout


def test_exponent_closed_forms():
    # 448 = 1.75 * 2^8 fits scale 2^0 exactly; anything above needs 2^1
    cases = {448.0: 0, np.nextafter(448.0, np.inf): 1, 1.0: -8, 1.75: -8, 1.7500001: -7, 2.0 ** 100: 92,
             0.0: -127, 1e-300: -127, 448.0 * 2.0 ** -127: -127, 448.0 * 2.0 ** -126: -126, 3.0e38: 120}
    for a, s in cases.items():
        assert int(mx.mx_exponent(a)) == s, (a, int(mx.mx_exponent(a)), s)


def test_exponent_is_minimal_by_brute_force():
    rng = np.random.default_rng(0)
    a = np.exp(rng.uniform(-60, 60, 20000)) * rng.choice([1.0, 448.0, 0.875], 20000)
    s = mx.mx_exponent(a)
    for ai, si in zip(a, s):
        cands = [t for t in range(-127, 128) if ai <= 448.0 * 2.0 ** t]
        assert si == cands[0]


def test_elements_match_torch_e4m3():
    """Element rounding = torch's float8_e4m3fn conversion of value / 2^s
    (round to nearest even; no value exceeds 448 by construction)."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    el, s = mx.mx_quantise(x.astype(np.float64), axis=-1)
    assert s.shape == (64, 8)
    scaled = x.reshape(64, 8, 32).astype(np.float64) * np.exp2(-s.astype(np.float64))[..., None]
    assert np.abs(scaled).max() <= 448.0
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(el.reshape(64, 8, 32), ref)


def test_representable_blocks_round_trip_exactly():
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    rng = np.random.default_rng(2)
    blocks = rng.choice(vals, (50, 32)) * rng.choice([-1.0, 1.0], (50, 32))
    blocks[:, 5] = 448.0  # block maximum 448: exponent 0 after the shift below
    shift = rng.integers(-20, 20, 50)
    a = blocks * np.exp2(shift)[:, None]
    el, s = mx.mx_quantise(a)
    np.testing.assert_array_equal(s[:, 0], shift)
    np.testing.assert_array_equal(mx.mx_dequantise(el, s), a)


def test_block_extent_and_axis():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 96))
    b = a.copy()
    b[:, 40] *= 1000.0  # block 1 of each row
    ea, sa = mx.mx_quantise(a)
    eb, sb = mx.mx_quantise(b)
    np.testing.assert_array_equal(ea[:, :32], eb[:, :32])
    np.testing.assert_array_equal(ea[:, 64:], eb[:, 64:])
    assert np.all(sb[:, 1] > sa[:, 1]) and np.array_equal(sa[:, [0, 2]], sb[:, [0, 2]])
    # weights: blocks along the input axis (0) of each output column
    w = rng.standard_normal((64, 8)) * 0.02
    w2 = w.copy()
    w2[5, 3] = 10.0
    d = mx.mx_round(w2, 0) - mx.mx_round(w, 0)
    changed = np.argwhere(d != 0)
    assert set(changed[:, 1]) <= {3} and changed[:, 0].max() < 32


def test_error_bound():
    """|MX(a) - a| <= 2^-4 |a| for elements in e4m3's normal range
    (|a| >= 2^-6 2^s) and <= 2^-10 2^s (half the subnormal step) below it."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-5, 5, (200, 1)))
    el, s = mx.mx_quantise(a)
    q = mx.mx_dequantise(el, s)
    sc = np.repeat(np.exp2(s.astype(np.float64)), 32, axis=-1)
    normal = np.abs(a) >= 2.0 ** -6 * sc
    err = np.abs(q - a)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(a[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * sc[~normal])


def test_matmul_exact_for_representable_operands():
    rng = np.random.default_rng(5)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 448.0])
    a = rng.choice(grid, (6, 64)) * np.exp2(rng.integers(-3, 3, (6, 1)))
    a[:, 0] = a[:, 32] = 448.0 * np.exp2(rng.integers(-3, 3, 6))
    w = rng.choice(grid, (64, 5)) * 2.0 ** -7
    w[0, :] = w[32, :] = 448.0 * 2.0 ** -7
    np.testing.assert_array_equal(mx.mx_matmul(a, w), a @ w)


def _tiny(seed):
    lay = Layout(1, 3, 8, 4, 2, 32, 1, 1, True, True)
    rng = np.random.default_rng(seed)
    B, N, H, D, hid = 1, 24, 2, 32, 64
    inp = {"x": rng.standard_normal((B, N, hid)), "q": rng.standard_normal((B, N, H, D)) * 0.4,
           "k": rng.standard_normal((B, N, H, D)) * 0.4, "v": rng.standard_normal((B, N, H, D)),
           "text_k": rng.standard_normal((B, 4, H, D)) * 0.4, "text_v": rng.standard_normal((B, 4, H, D)),
           "rms_w": 1 + 0.1 * rng.standard_normal(hid)}
    for k in ("w_gs", "w_gl", "w_os", "w_ol"):
        inp[k] = rng.standard_normal((hid, hid)) * 0.05
    return lay, inp


def test_layer_special_cases():
    lay, inp = _tiny(6)
    # W_o = 0: y = x exactly, whatever the quantisation
    z = dict(inp, w_os=np.zeros_like(inp["w_os"]), w_ol=np.zeros_like(inp["w_ol"]))
    out = mx.hybrid_forward_mx(z, lay)
    np.testing.assert_array_equal(out["y"], np.asarray(inp["x"], np.float64))
    # representable x and gate weights: the MX gates equal the exact gates
    x = mx.mx_round(inp["x"], -1)
    wg = mx.mx_round(inp["w_gs"], 0), mx.mx_round(inp["w_gl"], 0)
    ref = oracle.hybrid.epilogue(x, out["o_s"], out["o_l"], wg[0], wg[1], inp["w_os"], inp["w_ol"], inp["rms_w"])
    ep = mx.epilogue_mx(x, out["o_s"], out["o_l"], wg[0], wg[1], inp["w_os"], inp["w_ol"], inp["rms_w"])
    np.testing.assert_allclose(ep["g_s"], ref["g_s"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(ep["g_l"], ref["g_l"], rtol=1e-15, atol=0)
    # ... and the output GEMM's error stays within the format's bound:
    # |delta_mx - delta| <= sum_k |A'_k W_k| (2^-4 + 2^-4 + 2^-8) + subnormal terms
    bound = (np.abs(ep["a_p"]) @ np.abs(np.concatenate([inp["w_os"], inp["w_ol"]]))) * (2 * 2.0 ** -4 + 2.0 ** -8)
    assert np.all(np.abs(ep["delta"] - ref["delta"]) <= bound + 1e-12)


def test_mutations_are_caught():
    """Plausible mistakes fail a pin: the floor-only exponent (saturating
    blocks), and blocks along the output axis of the weights."""
    orig = mx.mx_exponent
    try:
        mx.mx_exponent = lambda a: np.where(np.asarray(a) > 0, np.floor(np.log2(np.maximum(a, 1e-300))) - 8,
                                            -127).astype(np.int64)
        with pytest.raises(AssertionError):
            test_exponent_is_minimal_by_brute_force()
    finally:
        mx.mx_exponent = orig
    orig_round = mx.mx_round
    try:
        mx.mx_round = lambda a, axis=-1: orig_round(a, -1 if axis == 0 else axis)
        with pytest.raises(AssertionError):
            test_block_extent_and_axis()
    finally:
        mx.mx_round = orig_round


def test_ffn_mx():
    """W_2 = 0 gives y exactly; otherwise the MX feed-forward stays within the
    format's bound of the exact one (oracle/dit.ffn) for representable-free
    random data: each MX product is within (2 2^-4 + 2^-8) sum|a||w| of the
    exact product of its inputs, and GELU is 1.13-Lipschitz."""
    from oracle import dit
    rng = np.random.default_rng(8)
    y = rng.standard_normal((2, 10, 64))
    w_n = 1 + 0.1 * rng.standard_normal(64)
    w_1 = rng.standard_normal((64, 256)) * 0.05
    w_2 = rng.standard_normal((256, 64)) * 0.05
    np.testing.assert_array_equal(mx.ffn_mx(y, w_n, w_1, np.zeros_like(w_2)), y)
    z = mx.ffn_mx(y, w_n, w_1, w_2)
    ref = dit.ffn(y, w_n, w_1, w_2)
    h = dit.rmsnorm(y, w_n)
    c = 2 * 2.0 ** -4 + 2.0 ** -8
    e1 = (np.abs(h) @ np.abs(w_1)) * c + np.abs(h - mx.round_bf16(h)) @ np.abs(w_1)  # first product
    u = dit.gelu_tanh(h @ w_1)
    bound = 1.13 * e1 @ np.abs(w_2) + ((np.abs(u) + 1.13 * e1) @ np.abs(w_2)) * c
    assert np.all(np.abs(z - ref) <= bound + 1e-12)
    assert np.abs(z - ref).max() > 0  # quantisation is visible
