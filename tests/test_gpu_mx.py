"""GPU parity of the fp8 version with MX e4m3 GEMMs (soft = "fp8_mx")
through the C ABI, against oracle/mx.py.

The gate GEMM is checked against its exact MX definition (both sides take
the same e4m3 codes and block exponents of x and W_g; only the kernel's fp32
accumulation differs).  The output GEMM is checked from the kernel's own
branch outputs and gates: the oracle forms A' from them in float64 and
quantises it.  The kernel quantises its fp32 A', whose RMS factor comes from
its own sum of squares, so an element whose value lies within ~1e-5 of an
e4m3 rounding boundary can take the neighbouring code (one step, 2^-4
relative, of one of 2 hid terms); a wrong exponent or block (factor-2 or
larger errors) fails the bounds by far.
The layer output is checked against the unquantised oracle with the fp8
bound.  (Bounds and their derivation at GATE_ATOL and MX_DELTA_TOL.)  The projection of the block call is checked through the linear
branch, which reads q, k, v exactly as the projection stored them."""
import numpy as np
import pytest

from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, Workload, make_inputs, make_projection_weights
from oracle import mx
from oracle import projection as oproj
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# Gates: the scaled f8f6f4 matrix instruction returns each step of 64
# products only to within 2^-11.07 of the step's largest |product| (the
# register-only probe of tests/gpu_util.FP8_MFMA_PREC, which takes 2^-10.5),
# and the steps are summed in float32.  So with MX values x, w:
#   |dz| <= FP8_MFMA_PREC * sum_steps max_{k in step} |x_k w_k|
#           + (K / 64) 2^-24 sum_k |x_k w_k|,
# the largest product of a step bounded by max|x| max|w| over the step, and
# |dg| <= sigma' |dz| <= |dz| / 4, plus the fp32 sigmoid.  For ordinary
# tokens that is ~1-2e-4 (measured errors 1-2e-5); a wrong block exponent
# moves gates by far more (0.46 measured with a mis-mapped operand).
GATE_ATOL = 1e-6
# Output GEMM from the kernel's own A' inputs: mean at the bf16 bound; max at
# the fp8 bound, since an A' element within ~1e-5 of an e4m3 rounding
# boundary can round the other way on the two sides (one 2^-4 step of one of
# 2 hid terms; measured max 1.0e-2, mean 2e-4; a wrong exponent gives mean 0.38).
MX_DELTA_TOL = (4e-2, 2e-3)
MX_CASES = [WORKLOADS[2].with_(name="mx-workload2", soft="fp8_mx"),
            Workload("mx-ragged-b2-d128", 2, 5, 100, 37, 2, 128, soft="fp8_mx", seed=61),
            Workload("mx-notext-d64", 1, 4, 130, 0, 4, 64, soft="fp8_mx", seed=62),
            Workload("mx-one-partial-tile", 1, 2, 50, 3, 2, 128, soft="fp8_mx", seed=65)]  # 100 tokens


def _hid(a, w):
    return np.asarray(a).reshape(w.batch, w.n_video, w.hidden)


def _check_gemms(w, inp, g):
    """Gate GEMM against its MX definition; output GEMM from the kernel's own
    branch outputs and gates."""
    x = np.asarray(inp["x"], np.float64)
    wg = np.concatenate([inp["w_gs"], inp["w_gl"]], axis=1)
    z = mx.mx_matmul(x, wg)
    gates_ref = 0.5 * (1.0 + np.tanh(0.5 * z))
    xm, wm = np.abs(mx.mx_round(x, -1)), np.abs(mx.mx_round(wg, 0))
    K = xm.shape[-1]
    steps = [slice(k0, min(K, k0 + 64)) for k0 in range(0, K, 64)]
    big = sum(xm[..., st].max(axis=-1, keepdims=True) * wm[st].max(axis=0, keepdims=True) for st in steps)
    dz = gu.FP8_MFMA_PREC * big + len(steps) * 2.0 ** -24 * (xm @ wm)
    # largest error as a fraction of its bound (<= 1 passes)
    gerr = (np.abs(g["gates"] - gates_ref) / (0.25 * dz + GATE_ATOL)).max()
    hid = w.hidden
    gs, gl = g["gates"][..., :hid], g["gates"][..., hid:]
    ol = _hid(g["o_lin"], w)
    r = ol * np.asarray(inp["rms_w"], np.float64) / np.sqrt(np.mean(ol * ol, axis=-1, keepdims=True) + 1e-6)
    a_p = np.concatenate([gs * _hid(g["o_soft"], w), gl * r], axis=-1)
    delta_ref = mx.mx_matmul(a_p, np.concatenate([inp["w_os"], inp["w_ol"]], axis=0))
    derr = gu.errors(g["delta_f32"], delta_ref)
    return gerr, derr


@pytest.mark.parametrize("w", MX_CASES, ids=[w.name for w in MX_CASES])
def test_mx_layer(w):
    inp = make_inputs(w)
    print("case", w.name, flush=True)
    g = gu.run_gpu(w, inp)
    gerr, derr = _check_gemms(w, inp, g)
    ref = gu.run_oracle(w, inp)
    rep_y, bad_y = gu.compare(w, g, ref, keys=("y",), tol=gu.TOL["fp8"])
    rep_l, bad_l = gu.compare(w, g, ref, keys=("o_l",), tol=gu.TOL["bf16"])
    print(w.name, "gates err/bound %.3f" % gerr, "delta vs MX(A') W_o max %.2e mean %.2e" % derr, rep_y, rep_l,
          flush=True)
    assert gerr <= 1.0, gerr
    assert derr[0] <= MX_DELTA_TOL[0] and derr[1] <= MX_DELTA_TOL[1], derr
    assert not bad_y, bad_y
    assert not bad_l, bad_l


@pytest.mark.parametrize("w", MX_CASES[:2], ids=[w.name for w in MX_CASES[:2]])
def test_mx_block(w):
    """hyb_block_forward with MX: the projection's stored q, k, v (seen
    through the linear branch, against the oracle's MX projection rounded to
    bf16), the gates from the x codes the projection wrote, and the output
    GEMM as above."""
    import torch
    inp = make_inputs(w)
    wts = make_projection_weights(w)
    print("case", w.name, flush=True)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(torch.bfloat16) for k, v in inp.items()}
    wd = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(torch.bfloat16) for k, v in wts.items()}
    f32 = dict(dtype=torch.float32, device="cuda")
    B, N, H, D, hid = w.batch, w.n_video, w.heads, w.head_dim, w.hidden
    dbg = {"o_soft": torch.empty(B, N, H, D, **f32), "o_lin": torch.empty(B, N, H, D, **f32),
           "delta_f32": torch.empty(B, N, hid, **f32), "gates": torch.empty(B, N, 2 * hid, **f32)}
    y = api.block_forward(gu.api_layout(w), dev["x"], wd["w_q"], wd["w_k"], wd["w_v"], dev["text_k"],
                          dev["text_v"], dev["w_gs"], dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"],
                          soft="fp8_mx", debug=dbg)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy().astype(np.float64) for k, v in dbg.items()}
    g["y"] = y.float().cpu().numpy().astype(np.float64)
    q, k, v = mx.qkv_projection_mx(inp["x"], wts["w_q"], wts["w_k"], wts["w_v"], w.heads)
    ref_inp = dict(inp, q=oproj.round_bf16(q), k=oproj.round_bf16(k), v=oproj.round_bf16(v))
    ref = gu.run_oracle(w, ref_inp)
    gerr, derr = _check_gemms(w, inp, g)
    rep_l, bad_l = gu.compare(w, g, ref, keys=("o_l",), tol=gu.TOL["bf16"])
    rep_y, bad_y = gu.compare(w, g, ref, keys=("y",), tol=gu.TOL["fp8"])
    print(w.name, "gates err/bound %.3f" % gerr, "delta max %.2e mean %.2e" % derr, rep_l, rep_y, flush=True)
    assert gerr <= 1.0, gerr
    assert derr[0] <= MX_DELTA_TOL[0] and derr[1] <= MX_DELTA_TOL[1], derr
    assert not bad_l, bad_l
    assert not bad_y, bad_y


def test_mx_768p_sampled():
    """768p shape in the bench's launch configuration: both MX GEMMs on a
    sample of tokens (MX blocks lie within a token row, so a row of the
    reference needs only that token)."""
    import torch
    w = WORKLOADS[3].with_(soft="fp8_mx")
    inp = make_inputs(w)
    print("case", w.name, "fp8_mx", flush=True)
    g = gu.run_gpu(w, inp)
    rng = np.random.default_rng(7)
    tok = np.sort(rng.choice(w.n_video, 256, replace=False))
    sub = dict(inp, x=np.asarray(inp["x"])[:, tok])
    gs = {"gates": g["gates"][:, tok], "o_soft": g["o_soft"][:, tok], "o_lin": g["o_lin"][:, tok],
          "delta_f32": g["delta_f32"][:, tok]}
    ws = w.with_(frames=1, tokens_per_frame=tok.size)
    gerr, derr = _check_gemms(ws, sub, gs)
    print("768p mx gates err/bound %.3f" % gerr, "delta max %.2e mean %.2e" % derr, flush=True)
    assert gerr <= 1.0, gerr
    assert derr[0] <= MX_DELTA_TOL[0] and derr[1] <= MX_DELTA_TOL[1], derr
    del g
    torch.cuda.empty_cache()



def test_mx_zero_and_outlier_blocks():
    """Exponent edge cases: all-zero 32-feature blocks and a whole zero token
    (exponent -127, codes 0, gates exactly 1/2 for the zero token), a token
    whose blocks are scaled by 1e4 (exponents 6-7) and a block scaled by
    1e-30 (exponent -107), against the MX definition."""
    w = Workload("mx-edge", 1, 3, 64, 8, 2, 128, soft="fp8_mx", seed=64)  # hid 256, 192 tokens
    inp = make_inputs(w)
    x = np.array(inp["x"], np.float64)
    x[0, 5, :] = 0.0                       # zero token
    x[0, 7, 32:96] = 0.0                   # two zero blocks
    x[0, 9, :] *= 1e4                      # large block exponents
    x[0, 11, 64:96] *= 1e-30               # tiny block (bf16 keeps it): exponent -107
    inp["x"] = oproj.round_bf16(x)
    print("case", w.name, flush=True)
    g = gu.run_gpu(w, inp)
    gerr, derr = _check_gemms(w, inp, g)
    print(w.name, "gates err/bound %.3f" % gerr, "delta max %.2e mean %.2e" % derr, flush=True)
    assert gerr <= 1.0, gerr
    assert derr[0] <= MX_DELTA_TOL[0] and derr[1] <= MX_DELTA_TOL[1], derr
    assert np.all(g["gates"][0, 5] == 0.5)
    assert np.all(np.isfinite(g["y"]))




def test_fp8_version_768p_sampled():
    """The fp8 version at the 768p shape, in the bench's launch configuration
    (soft = fp8_mx): the e4m3 softmax branch at D = 128 against the e4m3
    emulation within its deviation bound (every 4th head), the reading's own
    gap against the unquantised oracle, and y against the unquantised
    oracle, on 16 sampled tokens per frame (plus each frame's first and last)
    evaluated one by one with full states."""
    from hybrid_softmax_linear_block_amd.inputs import sample_tokens
    w = WORKLOADS[3].with_(soft="fp8_mx")
    inp = make_inputs(w)
    print("case", w.name, "fp8_mx 768p sampled", flush=True)
    g = gu.run_gpu(w, inp)
    tok = sample_tokens(w, per_frame=16)
    heads = list(range(0, w.heads, 4))          # the emulation with its bound on every 4th head
    emu, marg, bnd = gu.fp8_emulation(inp, w, tokens=tok, heads=heads)
    ref = gu.run_oracle(w, inp, tokens=tok)
    rep_y, bad_y = gu.compare(w, g, ref, tokens=tok, keys=("y",), tol=gu.TOL["fp8"])
    rep_l, bad_l = gu.compare(w, g, ref, tokens=tok, keys=("o_l",), tol=gu.TOL["bf16"])
    gap = gu.errors(emu, ref["o_s"][:, :, heads])
    e_raw = gu.errors(g["o_soft"][:, tok], ref["o_s"])
    print("768p fp8 version: o_s vs unquantised", e_raw, "reading gap", gap, rep_y, rep_l, flush=True)
    gu.assert_fp8_emulation(g["o_soft"][:, tok][:, :, heads], emu, marg, bnd, "768p fp8 version")
    assert gap[0] <= gu.FP8_READING_LIMIT[0] and gap[1] <= gu.FP8_READING_LIMIT[1], gap
    assert not bad_y, bad_y
    assert not bad_l, bad_l
