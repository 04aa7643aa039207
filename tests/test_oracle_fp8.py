"""Pins of the fp8 (e4m3) emulation in the oracle (CPU).

The rounding is pinned by torch's float8_e4m3fn conversion and the format's
closed forms.  The softmax branch on quantised inputs is pinned by
  * uniform scores: every probability is 1, so the output is the plain mean
    of the dequantised values over the key set;
  * inputs built so that every scaled probability lies on the e4m3 grid and
    the running maximum rises across tiles: the emulation then equals the
    unquantised softmax branch (itself pinned by brute force) on the
    dequantised inputs;
  * unrounded probabilities on random data: again the unquantised branch on
    the dequantised inputs, to float32 accuracy;
  * hand-derived probability codes for a walk over two frames of 96 keys
    (tiles of 64 + 32 per frame), a maximum that rises inside one tile, and
    a probability in e4m3's subnormal range.
Planted mistakes in each step (source mutations of the emulation) fail one
of these pins (``test_planted_fp8_mistake_is_caught``)."""
import inspect
import math

import numpy as np
import pytest
import torch

import oracle.hybrid as H
from oracle import fp8
from oracle.layout import Layout, frame_sets

TAU2 = float(np.float32(2 * math.log(2)))   # float32 tau with tau log2(e) == 2 exactly in float32


def _torch_e4m3(x):
    t = torch.from_numpy(np.asarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_round_e4m3_matches_torch_float8_e4m3fn():
    g = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([g.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(fp8.round_e4m3(x), _torch_e4m3(x))


def test_round_e4m3_closed_forms():
    # largest finite, smallest subnormal, ties to even, saturation
    assert fp8.round_e4m3(448.0) == 448.0 and fp8.round_e4m3(1000.0) == 448.0
    assert fp8.round_e4m3(-1e9) == -448.0
    assert fp8.round_e4m3(2.0 ** -9) == 2.0 ** -9
    assert fp8.round_e4m3(2.0 ** -10) == 0.0          # tie between 0 and 2^-9 -> even (0)
    assert fp8.round_e4m3(3 * 2.0 ** -10) == 2.0 ** -8  # tie 1 vs 2 (x 2^-9) -> even (2)
    assert fp8.round_e4m3(1.0625) == 1.0              # 1 + 1/16 is halfway 1 .. 1.125 -> even
    assert fp8.round_e4m3(1.1875) == 1.25             # halfway 1.125 .. 1.25 -> even mantissa
    assert fp8.round_e4m3(17.0) == 16.0 and fp8.round_e4m3(19.0) == 20.0
    # every e4m3 value is a fixed point
    vals = [m * 2.0 ** -9 for m in range(8)] + [(1 + m / 8) * 2.0 ** e for e in range(-6, 9) for m in range(8)]
    vals = [v for v in vals if v <= 448]
    assert np.array_equal(fp8.round_e4m3(vals), vals)


def test_quantise_per_head_scale_and_range():
    g = np.random.Generator(np.random.PCG64(6))
    x = g.standard_normal((2, 50, 3, 8)).astype(np.float32)
    x[1, 7, 2, 3] = 40.0
    dq, s = fp8.quantise(x)
    assert s.shape == (2, 3) and s.dtype == np.float32
    assert s[1, 2] == np.float32(40.0) / np.float32(448.0)
    # the absmax element maps to the code 448 exactly
    assert dq[1, 7, 2, 3] == pytest.approx(40.0, rel=1e-7)
    # relative error of a 3-bit mantissa is at most 2^-4 for normal codes
    big = np.abs(x) > 0.05 * np.abs(x).max(axis=(1, 3), keepdims=True)
    rel = np.abs(dq - x) / np.abs(x)
    assert np.all(rel[big] <= 2.0 ** -4 + 1e-6)


def _rand(shape, rng, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _branch(inp, lay, **kw):
    return fp8.softmax_branch_fp8(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, **kw)


def _dequantised(inp):
    return {n: fp8.quantise(inp[n])[0] for n in ("q", "k", "v", "text_k", "text_v")}


def test_uniform_scores_give_the_mean_of_the_quantised_values():
    """Q = 0: every score is 0, every probability 1 (code 2^8 exactly), so
    O_s is the plain mean of the dequantised V over S(f)'s tokens and the
    text; the text values carry their own scale."""
    lay = Layout(1, 5, 70, 10, 2, 16)
    rng = np.random.default_rng(11)
    inp = {"q": np.zeros((1, 350, 2, 16), np.float32), "k": _rand((1, 350, 2, 16), rng),
           "v": _rand((1, 350, 2, 16), rng), "text_k": _rand((1, 10, 2, 16), rng),
           "text_v": _rand((1, 10, 2, 16), rng, 7.0)}
    out = _branch(inp, lay)
    dq = _dequantised(inp)
    sets = frame_sets(5, 1, 1)
    for f in range(5):
        keys = np.concatenate([np.arange(g * 70, (g + 1) * 70) for g in sorted(sets[f][0])])
        allv = np.concatenate([dq["v"][0, keys], dq["text_v"][0]], axis=0)   # [keys, H, D]
        want = allv.mean(axis=0)
        np.testing.assert_allclose(out[0, f * 70:(f + 1) * 70], np.broadcast_to(want, (70, 2, 16)),
                                   rtol=1e-12, atol=1e-15)


def _grid_inputs(rng, lay):
    """Codes on a grid: scales 2^-7 (absmax 3.5), q one-hot +1 per row, video
    keys in {-1, -0.5, 0}, text keys in {0.5, 1}: with tau log2(e) = 2 every
    log2-score is an integer in [-2, 2], the text raises the running maximum,
    and every scaled probability 2^(8 + k), k in [-4, 0], is an e4m3 value."""
    B, N, L, Hh, D = lay.batch, lay.n_video, lay.text_tokens, lay.heads, lay.head_dim
    q = np.zeros((B, N, Hh, D), np.float32)
    cols = rng.integers(0, D - 2, size=(B, N, Hh))
    np.put_along_axis(q, cols[..., None], 1.0, axis=3)
    q[:, 0, :, D - 1] = 3.5                       # absmax on a column where every key is 0
    k = rng.choice([-1.0, -0.5, 0.0], size=(B, N, Hh, D)).astype(np.float32)
    k[..., D - 2:] = 0.0
    k[:, 1, :, D - 2] = 3.5                       # absmax on a column where every query is 0
    tk = rng.choice([0.5, 1.0], size=(B, L, Hh, D)).astype(np.float32)
    tk[..., D - 2:] = 0.0
    tk[:, 0, :, D - 2] = 3.5
    return {"q": q, "k": k, "v": _rand((B, N, Hh, D), rng), "text_k": tk,
            "text_v": _rand((B, L, Hh, D), rng, 3.0)}


def test_probabilities_on_the_grid_equal_the_unquantised_branch():
    lay = Layout(2, 6, 96, 40, 2, 32)
    inp = _grid_inputs(np.random.default_rng(12), lay)
    assert fp8.scale_log2(32, TAU2) == np.float32(2.0)
    dq = _dequantised(inp)
    for n in ("q", "k", "text_k"):               # the construction quantises exactly
        assert np.array_equal(dq[n], inp[n])
    out = _branch(inp, lay, scale=TAU2)
    ref = H.softmax_branch(dq["q"], dq["k"], dq["v"], dq["text_k"], dq["text_v"], lay, scale=TAU2)
    # tau = TAU2 in float64 differs from 2 ln 2 by 3e-8 relative
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_unrounded_probabilities_equal_the_unquantised_branch():
    """round_p=False: the walk, the lazy maximum and the rescales are exact
    rewrites of softmax, so the result is the unquantised branch on the
    dequantised inputs up to float32 probabilities (ragged frames and text,
    2-frame chunks, two batches, outliers, a sharp scale)."""
    lay = Layout(2, 7, 100, 70, 2, 32, chunk_frames=2)
    rng = np.random.default_rng(13)
    inp = {n: _rand((2, 700 if n in ("q", "k", "v") else 70, 2, 32), rng) for n in ("q", "k", "v", "text_k", "text_v")}
    inp["v"][0, 5, 1, 3] = 9.0
    inp["text_k"] *= np.float32(1.7)
    inp["text_v"] *= np.float32(0.3)
    out = _branch(inp, lay, scale=0.6, round_p=False)
    dq = _dequantised(inp)
    ref = H.softmax_branch(dq["q"], dq["k"], dq["v"], dq["text_k"], dq["text_v"], lay, scale=0.6)
    err = np.abs(out - ref)
    assert err.max() <= 1e-6 * np.abs(ref).max()
    assert err.sum() <= 1e-6 * np.abs(ref).sum()


def _coded_case(T, n, groups, sl2_target):
    """One head, D = 8, no text.  Query rows e_0 * 1.75 (code 448, scale 2^-8);
    key j has k_j0 = code_j * 2^-8 (its log2-score is 448 code_j 2^-16 tau
    log2 e); value rows are one-hot 1.75 on the dimension of the key's group.
    groups: list of (first key, key count, key code)."""
    N, D = T * n, 8
    q = np.zeros((1, N, 1, D), np.float32)
    q[..., 0] = 1.75
    k = np.zeros((1, N, 1, D), np.float32)
    v = np.zeros((1, N, 1, D), np.float32)
    k[0, 0, 0, 7] = 1.75                     # fixes the key scale at 2^-8 (column unused by q)
    for gi, (j0, cnt, code) in enumerate(groups):
        k[0, j0:j0 + cnt, 0, 0] = code / 256.0
        v[0, j0:j0 + cnt, 0, gi] = 1.75
    tau = sl2_target / fp8.LOG2E
    empty = np.zeros((1, 0, 1, D), np.float32)
    return {"q": q, "k": k, "v": v, "text_k": empty, "text_v": empty}, Layout(1, T, n, 0, 1, D), tau


def test_codes_of_a_frame_tiled_walk():
    """Two frames of 96 keys (tiles f0[0:64], f0[64:96], f1[0:64], f1[64:96]).
    log2-scores: 0 on f0[0:64], t1 = 0.9*256/448 on f0[64:96], t2 = 0.9 on
    f1[0:32], 0 elsewhere.  The maximum stays 0 through f0 (t1 < 0.75) and
    moves to t2 at f1's first tile (alpha = 2^-t2).  Codes of P*2^8:
    f0[0:64] 256 (then x alpha), f0[64:96] 256*2^t1 = 366.5 -> 352 (then x
    alpha), f1[0:32] 256, f1[32:96] 256*2^-t2 = 137.2 -> 144."""
    t2 = 0.9
    t1 = t2 * 256 / 448
    groups = [(0, 64, 0), (64, 32, 256), (96, 32, 448), (128, 32, 0), (160, 32, 0)]
    inp, lay, tau = _coded_case(2, 96, groups, t2 * 65536 / 448 ** 2)
    out = _branch(inp, lay, scale=tau)
    a = 2.0 ** -t2
    w = [a, 352 / 256 * a, 1.0, 144 / 256, 144 / 256]
    l = 64 * a + 32 * 2.0 ** t1 * a + 32 + 32 * a + 32 * a
    want = np.zeros(8)
    for gi, (_, cnt, _) in enumerate(groups):
        want[gi] = cnt * w[gi] * 1.75 / l
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(want, (192, 8)), rtol=2e-6, atol=1e-12)


def test_codes_when_the_maximum_rises_inside_a_tile():
    """One tile of 64 keys: log2-score 0 on keys 0..31, t1 = 0.5143 on keys
    32..63, so the maximum is t1 from the first tile on: codes 256*2^-t1 =
    179.3 -> 176 and 256."""
    t1 = 0.9 * 256 / 448
    groups = [(0, 32, 0), (32, 32, 256)]
    inp, lay, tau = _coded_case(1, 64, groups, 0.9 * 65536 / 448 ** 2)
    out = _branch(inp, lay, scale=tau)
    l = 32 * 2.0 ** -t1 + 32
    want = np.array([32 * 176 / 256 * 1.75 / l, 32 * 1.75 / l, 0, 0, 0, 0, 0, 0])
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(want, (64, 8)), rtol=2e-6, atol=1e-12)


def test_subnormal_probability_code():
    """log2-score 0 on keys 0..31 and -15.3 on keys 32..63: P*2^8 = 2^-7.3 =
    3.25 * 2^-9 rounds to the subnormal code 3 * 2^-9."""
    groups = [(0, 32, 0), (32, 32, -448)]
    inp, lay, tau = _coded_case(1, 64, groups, 15.3 * 65536 / 448 ** 2)
    out = _branch(inp, lay, scale=tau)
    l = 32 + 32 * 2.0 ** -15.3
    want = np.array([32 * 1.75 / l, 32 * 3 * 2.0 ** -9 / 256 * 1.75 / l, 0, 0, 0, 0, 0, 0])
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(want, (64, 8)), rtol=2e-6, atol=1e-15)


PINS = (test_uniform_scores_give_the_mean_of_the_quantised_values,
        test_probabilities_on_the_grid_equal_the_unquantised_branch,
        test_unrounded_probabilities_equal_the_unquantised_branch,
        test_codes_of_a_frame_tiled_walk,
        test_codes_when_the_maximum_rises_inside_a_tile,
        test_subnormal_probability_code)


def _all_fp8_pins():
    for pin in PINS:
        pin()


def _source_mutant(fn_name, old, new):
    src = inspect.getsource(getattr(fp8, fn_name))
    assert src.count(old) == 1, (fn_name, old)
    ns = dict(fp8.__dict__)
    exec(compile(src.replace(old, new), "<mutant %s>" % fn_name, "exec"), ns)
    return ns[fn_name]


def _final_max_rows(qc, tiles, round_p=True, mfma_prec=0.0, perturb=None):
    """The earlier reading: every probability rounded against the row's final
    maximum."""
    s = np.concatenate([(qc @ kc.T) * np.float64(dq) for kc, _, dq in tiles], axis=1)
    vd = np.concatenate([v for _, v, _ in tiles], axis=0)
    p = np.exp2(s - s.max(axis=1, keepdims=True) + fp8.P_SCALE_LOG2)
    out = ((fp8.round_e4m3(p) if round_p else p) @ vd) / p.sum(axis=1, keepdims=True)
    return out, np.full(qc.shape[0], np.inf), None


def _tiles_across_frames(frames, n, L):
    keys = [g * n + j for g in sorted(frames) for j in range(n)]
    out = []
    for i in range(0, len(keys), fp8.KEY_TILE):
        chunk = keys[i:i + fp8.KEY_TILE]
        if chunk[-1] - chunk[0] + 1 != len(chunk):   # straddles a gap in S(f): split there
            cut = next(j for j in range(1, len(chunk)) if chunk[j] != chunk[j - 1] + 1)
            out += [("v", chunk[0], cut), ("v", chunk[cut], len(chunk) - cut)]
        else:
            out.append(("v", chunk[0], len(chunk)))
    out += [("t", t0, min(fp8.KEY_TILE, L - t0)) for t0 in range(0, L, fp8.KEY_TILE)]
    return out


def _scaled_output(*a, **kw):
    return ORIG_BRANCH(*a, **kw) / 1.05


ORIG_BRANCH = fp8.softmax_branch_fp8

FP8_MUTANTS = {
    "normaliser scaled by 1.05": lambda: [("softmax_branch_fp8", _scaled_output)],
    "normaliser sums the rounded probabilities": lambda: [(
        "online_rows", _source_mutant("online_rows", "l += p.sum(axis=1)", "l += pw.sum(axis=1)"))],
    "no rescale of the output when the maximum moves": lambda: [(
        "online_rows", _source_mutant("online_rows", "acc *= alpha[:, None]", "acc *= 1.0"))],
    "rescale factor inverted": lambda: [(
        "online_rows", _source_mutant("online_rows", "m.astype(np.float64) - m_new.astype(np.float64)",
                                      "m_new.astype(np.float64) - m.astype(np.float64)"))],
    "probabilities rounded against the final maximum": lambda: [("online_rows", _final_max_rows)],
    "no slack on the running maximum": lambda: [("P_SLACK", 0.0)],
    "32-key tiles": lambda: [("KEY_TILE", 32)],
    "tiles run across frame boundaries": lambda: [("key_tiles", _tiles_across_frames)],
    "probabilities scaled by 2^7": lambda: [("P_SCALE_LOG2", 7.0)],
    "text values dequantised with the video scale": lambda: [(
        "softmax_branch_fp8", _source_mutant("softmax_branch_fp8", "tvc[b, t0:t0 + cnt, h] * np.float64(stv[b, h])",
                                             "tvc[b, t0:t0 + cnt, h] * np.float64(sv[b, h])"))],
    "text logits with the video key scale": lambda: [(
        "softmax_branch_fp8", _source_mutant("softmax_branch_fp8", "np.float32(sq[b, h] * stk[b, h])",
                                             "np.float32(sq[b, h] * sk[b, h])"))],
}


def test_fp8_pins_pass_on_unmodified_emulation():
    _all_fp8_pins()


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_planted_fp8_mistake_is_caught(name, monkeypatch):
    for attr, val in FP8_MUTANTS[name]():
        monkeypatch.setattr(fp8, attr, val)
    with pytest.raises(AssertionError):
        _all_fp8_pins()


def test_fp8_reading_gap_on_the_fp8_workload():
    """The gap that the fp8 reading itself leaves on O_s at the fp8 workload
    (per-head absmax with 1% x8 outliers), on 16 sampled tokens per frame:
    within the limit the GPU tests assume (tests/gpu_util.FP8_READING_LIMIT);
    its largest element error comes from the Q/K/V quantisation (the
    unrounded-probability emulation shows it too), the probability rounding
    adds ~2-3% in the mean."""
    from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, make_inputs, sample_tokens
    from tests.gpu_util import FP8_READING_LIMIT, errors, oracle_layout
    w = WORKLOADS[5]
    inp = make_inputs(w)
    tok = sample_tokens(w, per_frame=16)
    lay = oracle_layout(w)
    emu = _branch(inp, lay, tokens=tok)
    qkv_only = _branch(inp, lay, tokens=tok, round_p=False)
    ref = H.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, tokens=tok)
    gap, gap_qkv, gap_p = errors(emu, ref), errors(qkv_only, ref), errors(emu, qkv_only)
    print("emulation vs unquantised", gap, "Q/K/V only", gap_qkv, "P rounding only", gap_p)
    assert gap[0] <= FP8_READING_LIMIT[0] and gap[1] <= FP8_READING_LIMIT[1], gap
    assert gap_qkv[0] >= 0.9 * gap[0]
    assert gap_p[0] <= 0.03 and 0.01 <= gap_p[1] <= 0.04, gap_p


def test_decision_margins():
    """margins=True: inf for a one-tile walk; the frame-tiled walk's rows
    decide at tile maxima t1 = 0.514 (against 0 + 0.75), t2 = 0.9 (against
    0.75) and 0 (against t2 + 0.75): smallest margin 0.15."""
    groups = [(0, 32, 0), (32, 32, 256)]
    inp, lay, tau = _coded_case(1, 64, groups, 0.9 * 65536 / 448 ** 2)
    _, marg = _branch(inp, lay, scale=tau, margins=True)
    assert np.all(np.isinf(marg))
    groups = [(0, 64, 0), (64, 32, 256), (96, 32, 448), (128, 32, 0), (160, 32, 0)]
    inp, lay, tau = _coded_case(2, 96, groups, 0.9 * 65536 / 448 ** 2)
    out, marg = _branch(inp, lay, scale=tau, margins=True)
    np.testing.assert_allclose(marg, 0.15, rtol=1e-5)
    np.testing.assert_array_equal(out, _branch(inp, lay, scale=tau))


def test_deviation_bound_covers_the_summation_model():
    """mfma_prec > 0: with every score, probability and product step moved at
    random inside the model (perturb), each output element stays within the
    bound -- on random data with outliers and sharp rows, text and ragged
    frames, at D = 64 (one step per score) and D = 128 (two), for the rows
    whose decisions cannot flip (margin > 0).  The bound is not vacuous: a
    16x smaller one is exceeded."""
    for D, seed in ((64, 14), (128, 15)):
        lay = Layout(2, 6, 150, 70, 2, D)
        rng = np.random.default_rng(seed)
        inp = {n: _rand((2, 900 if n in ("q", "k", "v") else 70, 2, D), rng, D ** -0.25) for n in
               ("q", "k", "v", "text_k", "text_v")}
        for n in ("q", "k", "v", "text_k", "text_v"):
            mask = rng.random(inp[n].shape) < 0.01
            inp[n][mask] *= np.float32(8.0)
        prec = 2.0 ** -10.5
        out, marg, bnd = _branch(inp, lay, mfma_prec=prec)
        np.testing.assert_array_equal(out, _branch(inp, lay))
        ok = marg > 0
        assert ok.mean() > 0.97, ok.mean()
        worst = 0.0
        for s in range(3):
            pert, _, _ = _branch(inp, lay, mfma_prec=prec, perturb=np.random.default_rng(100 + s))
            diff = np.abs(pert - out)[ok]
            assert np.all(diff <= bnd[ok]), (D, (diff / bnd[ok]).max())
            worst = max(worst, float((diff / np.maximum(bnd[ok] / 16, 1e-300)).max()))
        assert worst > 1.0, worst
