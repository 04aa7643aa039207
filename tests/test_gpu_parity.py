"""GPU parity: the HIP layer through the C ABI against the fp64 oracle.

Small workloads are compared element by element on every output; the
768p-shaped workloads on a seeded sample of 64 tokens per frame plus each
frame's first and last (all heads, all batches), which the oracle evaluates
with full states.  Further cases: attention sharp enough that the softmax
kernel's running maximum moves mid-walk, a non-default softmax scale, the
symmetries of the definition (tokens permuted inside a frame, text order), a
NaN-filled workspace, and the fp16 range of the branch outputs."""
import numpy as np
import pytest

from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, Workload, make_inputs, sample_tokens
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _run_and_check(w, tokens=None, keys=("y", "delta", "o_s", "o_l", "g"), tol=None):
    inp = make_inputs(w)
    print("case", w, flush=True)
    g = gu.run_gpu(w, inp)
    ref = gu.run_oracle(w, inp, tokens=tokens)
    report, bad = gu.compare(w, g, ref, tokens=tokens, keys=keys, tol=tol)
    print(w.name, {k: "max %.2e mean %.2e" % v for k, v in report.items()}, flush=True)
    assert not bad, bad
    return g, ref, inp


@pytest.mark.parametrize("wid", [1, 2])
def test_small_workloads_full(wid):
    _run_and_check(WORKLOADS[wid])


@pytest.mark.parametrize("w", [WORKLOADS[5], WORKLOADS[5].with_(name="fp8-d128-ragged", batch=1, frames=6,
                                                                  tokens_per_frame=200, text_tokens=40,
                                                                  heads=2, head_dim=128, seed=51)],
                         ids=["fp8-softmax", "fp8-d128-ragged"])
def test_fp8_softmax(w):
    """fp8 e4m3 softmax branch: layer output and delta within 4e-2 max|ref|
    of the unquantised oracle; the bf16 parts (linear branch, gates) within
    the bf16 bounds; dequantisation scales bit-exact; softmax output against
    the e4m3 emulation within its per-element deviation bound; the gap the
    reading itself leaves against the unquantised oracle (the emulation's)
    within FP8_READING_LIMIT."""
    from oracle import fp8
    inp = make_inputs(w)
    g = gu.run_gpu(w, inp)
    ref = gu.run_oracle(w, inp)
    rep1, bad1 = gu.compare(w, g, ref, keys=("y", "delta"))
    rep2, bad2 = gu.compare(w, g, ref, keys=("o_l", "g"), tol=gu.TOL["bf16"])
    e_raw = gu.errors(g["o_soft"], ref["o_s"])
    print(w.name, rep1, rep2, "o_s vs unquantised", e_raw, flush=True)
    assert not bad1, bad1
    assert not bad2, bad2
    assert np.array_equal(g["scales"].astype(np.float32), fp8.scales(inp))
    # the emulation with its bound on 128 sampled tokens per frame, every head and batch
    tok = sample_tokens(w, per_frame=128)
    emu, marg, bnd = gu.fp8_emulation(inp, w, tokens=tok)
    gap = gu.errors(emu, ref["o_s"][:, tok])
    print(w.name, "reading gap (emulation vs unquantised)", gap, flush=True)
    gu.assert_fp8_emulation(g["o_soft"][:, tok], emu, marg, bnd, w.name)
    assert gap[0] <= gu.FP8_READING_LIMIT[0] and gap[1] <= gu.FP8_READING_LIMIT[1], gap


@pytest.mark.parametrize("wid", [3, 4])
def test_768p_workloads_sampled(wid):
    w = WORKLOADS[wid]
    _run_and_check(w, tokens=sample_tokens(w, per_frame=64))


EDGE = [
    Workload("ragged-bf16", 1, 5, 100, 37, 2, 64, seed=31),
    Workload("ragged-d128", 2, 4, 70, 0, 2, 128, seed=32),
    Workload("no-anchor-r0", 1, 6, 64, 20, 2, 64, chunk_frames=2, chunk_radius=0, anchor_first=False,
             anchor_last=False, seed=33),
    Workload("first-anchor-only", 1, 7, 96, 64, 1, 128, chunk_frames=3, anchor_last=False, seed=34),
    Workload("one-frame", 1, 1, 130, 5, 3, 64, seed=35),
    Workload("two-frames", 1, 2, 64, 3, 1, 64, seed=36),
    Workload("ragged-f32", 1, 5, 50, 7, 2, 64, act="f32", soft="f32", seed=37),
    Workload("f32-d128", 1, 4, 33, 9, 1, 128, act="f32", soft="f32", chunk_frames=2, seed=38),
    # frame counts past the scan's 16- and 32-lane forms, and past 64 (the
    # per-thread form)
    Workload("frames-40-chunk3", 1, 40, 32, 16, 2, 64, chunk_frames=3, seed=39),
    Workload("frames-70", 1, 70, 16, 8, 2, 128, seed=40),
    # hidden 256 (the 256 x 256 GEMM tiles and their row epilogue) with one
    # token, and with one token past a whole tile
    Workload("one-token-d128", 1, 1, 1, 3, 2, 128, seed=42),
    Workload("tile-plus-one", 1, 1, 257, 5, 2, 128, seed=43),
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_edge_cases(w):
    _run_and_check(w)


def test_zero_output_weights_give_identity_bit_exact():
    w = WORKLOADS[2].with_(frames=5, seed=41)
    inp = make_inputs(w)
    inp["w_os"][:] = 0
    inp["w_ol"][:] = 0
    g = gu.run_gpu(w, inp)
    assert np.array_equal(g["y"], inp["x"].astype(np.float64))


def test_zero_gate_weights_give_half():
    w = WORKLOADS[2].with_(frames=4, seed=42)
    inp = make_inputs(w)
    inp["w_gs"][:] = 0
    inp["w_gl"][:] = 0
    g = gu.run_gpu(w, inp)
    assert np.all(g["gates"] == 0.5)


def test_head_major_strides_and_in_place_residual():
    import torch
    w = WORKLOADS[2].with_(frames=6, seed=43)
    inp = make_inputs(w)
    dev = gu.to_device(inp, w.act)
    # q/k/v stored head-major [B, H, N, D] and viewed as [B, N, H, D]
    for nm in ("q", "k", "v"):
        dev[nm] = dev[nm].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    ref = gu.run_gpu(w, inp)
    x_copy = dev["x"].clone()
    out = gu.run_gpu(w, inp, dev=dev, y=dev["x"])  # y aliases x
    assert np.array_equal(out["y"], ref["y"])
    assert not torch.equal(dev["x"], x_copy)


def sharp_inputs(w):
    """Inputs whose rows' running maximum must move by more than the softmax
    kernel's 8-log2-unit slack partway through the key walk, so that its
    rescale of the partial output and row sum runs: the keys of the last
    frame (an anchor, the last video frame of every walk) and the text keys
    are scaled by 4 (exact in bf16), so the largest scores of a row come
    late in its walk and exceed its first tile's maximum by ~10-15 log2
    units.  (A shared offset along one dimension would do it too, but leaves
    dL/dq as a near-cancelling sum that bf16 rounding of dS cannot resolve
    to the bound.)"""
    inp = make_inputs(w)
    n = w.tokens_per_frame
    k = inp["k"].copy()
    k[:, (w.frames - 1) * n:] *= np.float32(4.0)
    inp.update(k=k, text_k=inp["text_k"] * np.float32(4.0))
    return inp


def rescale_fraction(w, inp):
    """Fraction of (row, head) pairs whose largest log2-score exceeds the
    largest one of their first 64-key tile by more than 8: each of them
    moves the kernel's running maximum at least once after its first tile."""
    from oracle.layout import frame_sets
    n, tau = w.tokens_per_frame, w.head_dim ** -0.5
    sets = frame_sets(w.frames, w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)
    hits = total = 0
    for f in range(w.frames):
        keys = np.concatenate([np.arange(g * n, (g + 1) * n) for g in sorted(sets[f][0])])
        for h in range(w.heads):
            Q = inp["q"][0, f * n:(f + 1) * n, h].astype(np.float64)
            K = np.concatenate([inp["k"][0, keys, h], inp["text_k"][0, :, h]]).astype(np.float64)
            t = tau * np.log2(np.e) * (Q @ K.T)
            hits += int(np.sum(t.max(axis=1) - t[:, :64].max(axis=1) > 8.0))
            total += t.shape[0]
    return hits / total


SHARP = [Workload("sharp-d64", 1, 6, 256, 96, 2, 64, seed=81),
         Workload("sharp-d128", 1, 5, 192, 130, 2, 128, seed=82)]


@pytest.mark.parametrize("w", SHARP, ids=[w.name for w in SHARP])
def test_sharp_attention_moves_the_running_maximum(w):
    """y, delta, O_s, O_l and the gates element by element at the bf16 bounds
    on inputs where most rows rescale their partial output mid-walk."""
    inp = sharp_inputs(w)
    frac = rescale_fraction(w, inp)
    print(w.name, "rows that rescale after their first tile: %.3f" % frac, flush=True)
    assert frac >= 0.5, frac
    g = gu.run_gpu(w, inp)
    ref = gu.run_oracle(w, inp)
    report, bad = gu.compare(w, g, ref)
    print(w.name, {k: "max %.2e mean %.2e" % v for k, v in report.items()}, flush=True)
    assert not bad, bad


SCALED = [WORKLOADS[2].with_(name="scale-bf16", frames=5, tokens_per_frame=300, text_tokens=40, seed=83),
          WORKLOADS[5].with_(name="scale-fp8", frames=5, tokens_per_frame=300, text_tokens=40, seed=84),
          WORKLOADS[1].with_(name="scale-f32", frames=6, seed=85)]


@pytest.mark.parametrize("w", SCALED, ids=[w.name for w in SCALED])
def test_softmax_scale_argument(w):
    """A non-zero softmax_scale through the C ABI replaces 1/sqrt(D): bf16,
    fp8 (O_s against the emulation at the same scale) and float32."""
    scale = 0.6 / np.sqrt(w.head_dim) if w.soft != "f32" else 0.37
    inp = make_inputs(w)
    g = gu.run_gpu(w, inp, softmax_scale=float(scale))
    ref = gu.run_oracle(w, inp, scale=float(scale))
    if w.soft == "fp8":
        report, bad = gu.compare(w, g, ref, keys=("y", "delta"))
        emu, marg, bnd = gu.fp8_emulation(inp, w, scale=float(scale))
        gu.assert_fp8_emulation(g["o_soft"], emu, marg, bnd, w.name)
    else:
        report, bad = gu.compare(w, g, ref)
    print(w.name, {k: "max %.2e mean %.2e" % v for k, v in report.items()}, flush=True)
    assert not bad, bad
    # and it is not the default scale
    base = gu.run_gpu(w, inp)
    assert gu.errors(base["o_soft"], ref["o_s"])[1] > 10 * gu.TOL[w.act][1]


def test_permutation_symmetries():
    """The definition is equivariant under a permutation of the tokens inside
    each frame (applied to x, q, k, v) and invariant under a permutation of
    the text tokens: the GPU's outputs follow within the bf16 bounds."""
    w = WORKLOADS[2].with_(name="perm", frames=5, tokens_per_frame=320, seed=86)
    inp = make_inputs(w)
    base = gu.run_gpu(w, inp)
    rng = np.random.default_rng(86)
    n = w.tokens_per_frame
    perm = np.concatenate([f * n + rng.permutation(n) for f in range(w.frames)])
    pin = dict(inp)
    for name in ("x", "q", "k", "v"):
        pin[name] = np.ascontiguousarray(inp[name][:, perm])
    tperm = rng.permutation(w.text_tokens)
    for name in ("text_k", "text_v"):
        pin[name] = np.ascontiguousarray(inp[name][:, tperm])
    got = gu.run_gpu(w, pin)
    for key in ("y", "delta_f32", "o_soft", "o_lin", "gates"):
        e = gu.errors(got[key], base[key][:, perm])
        print("perm", key, "max %.2e mean %.2e" % e, flush=True)
        assert e[0] <= gu.TOL["bf16"][0] and e[1] <= gu.TOL["bf16"][1], (key, e)


POISON = [WORKLOADS[2].with_(name="poison-bf16", frames=4, tokens_per_frame=200, text_tokens=30, seed=87),
          WORKLOADS[5].with_(name="poison-fp8", frames=4, tokens_per_frame=200, text_tokens=30, seed=88),
          WORKLOADS[5].with_(name="poison-fp8-mx", batch=1, frames=4, tokens_per_frame=130, text_tokens=0,
                             heads=4, soft="fp8_mx", seed=89),
          WORKLOADS[1].with_(name="poison-f32", frames=4, seed=90)]


@pytest.mark.parametrize("w", POISON, ids=[w.name for w in POISON])
def test_workspace_contents_are_never_read_before_written(w):
    """A workspace filled with NaN (every byte 0xFF) gives the same outputs,
    bit for bit, as a zeroed one: no kernel reads scratch it did not write
    in the same call."""
    import torch
    from hybrid_softmax_linear_block_amd import api
    inp = make_inputs(w)
    soft = w.soft if w.soft in ("fp8", "fp8_mx") else None
    size = api.workspace_size(gu.api_layout(w), w.act, soft)
    outs = []
    for fill in (0, 255):
        ws = torch.full((size,), fill, dtype=torch.uint8, device="cuda")
        outs.append(gu.run_gpu(w, inp, workspace=ws))
    for key in outs[0]:
        if key == "scales" and not soft:
            continue               # written by the fp8 paths only
        assert np.array_equal(outs[0][key], outs[1][key]), key
    assert np.all(np.isfinite(outs[1]["y"]))


def test_fp16_branch_outputs_saturate():
    """The bf16 path carries O_s and O_l in fp16 between kernels.  Both are
    convex combinations of value rows, so they leave fp16's range only when
    |v| does: a head whose values are all 2^17 (exact in bf16) gives
    O_s = O_l = 2^17 in exact arithmetic, and the library stores 65504 (the
    largest fp16 value), not inf or NaN; the other head is unaffected."""
    w = WORKLOADS[2].with_(name="fp16-range", frames=4, tokens_per_frame=128, text_tokens=16, heads=2, seed=91)
    inp = make_inputs(w)
    inp["v"][:, :, 1] = 2.0 ** 17
    inp["text_v"][:, :, 1] = 2.0 ** 17
    g = gu.run_gpu(w, inp)
    ref = gu.run_oracle(w, inp)
    assert np.all(g["o_soft"][:, :, 1] == 65504.0)
    ol = g["o_lin"][:, :, 1]
    ref_ol = ref["o_l"][:, :, 1]
    assert np.all(ol[ref_ol > 65504.0] == 65504.0)
    assert np.all(np.isfinite(g["y"]))
    e = gu.errors(g["o_soft"][:, :, 0], ref["o_s"][:, :, 0])
    assert e[0] <= gu.TOL["bf16"][0] and e[1] <= gu.TOL["bf16"][1], e
