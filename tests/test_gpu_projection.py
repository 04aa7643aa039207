"""GPU parity of the Q/K/V input projection and of the layer with its
projection (hyb_qkv_project, hyb_block_forward) against the fp64 oracle.

The projection's outputs are compared with the oracle's fp64 product; its
absmax must equal, bit for bit, the maximum |value| of the q/k/v tensors it
wrote (the quantity the fp8 scales are defined on).  The block call must give
exactly the output of the layer fed with the projection's q, k, v (the same
kernels run), and match the oracle layer on the bf16-stored projections."""
import numpy as np
import pytest

from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import (WORKLOADS, Workload, make_inputs, make_projection_weights,
                                                    sample_tokens)
from oracle import projection as oproj
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    WORKLOADS[2],                                                   # hid 512: 256-column tiles
    Workload("proj-ragged-b2", 2, 3, 100, 16, 2, 64, seed=61),      # hid 128, waves straddle batches
    Workload("proj-hid192", 1, 2, 96, 8, 3, 64, seed=62),           # hid 192: 64-column tiles
    Workload("proj-d128", 2, 2, 70, 0, 2, 128, seed=63),            # hid 256, no text
]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)


def _project(w, inp, wts):
    import torch
    lay = gu.api_layout(w)
    amax = torch.zeros(3 * w.batch * w.heads, dtype=torch.int32, device="cuda")
    q, k, v = api.qkv_project(lay, _dev(inp["x"]), _dev(wts["w_q"]), _dev(wts["w_k"]), _dev(wts["w_v"]),
                              absmax=amax)
    torch.cuda.synchronize()
    return q, k, v, amax


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_projection_matches_oracle_and_absmax_is_exact(w):
    import torch
    inp = make_inputs(w)
    wts = make_projection_weights(w)
    print("case", w.name, flush=True)
    q, k, v, amax = _project(w, inp, wts)
    ref = oproj.qkv_projection(inp["x"], wts["w_q"], wts["w_k"], wts["w_v"], w.heads)
    got_amax = amax.cpu().numpy().astype(np.uint32).view(np.float32).reshape(3, w.batch, w.heads)
    for t, (g, r) in enumerate(zip((q, k, v), ref)):
        gn = g.float().cpu().numpy().astype(np.float64)
        e = gu.errors(gn, r)
        print(w.name, "qkv"[t], "max %.2e mean %.2e" % e, flush=True)
        assert e[0] <= 1e-2 and e[1] <= 2e-3, e
        # absmax of the stored bf16 values, bit-exact
        own = g.float().abs().amax(dim=(1, 3)).cpu().numpy().astype(np.float32)
        assert np.array_equal(got_amax[t], own), (t, got_amax[t], own)
        # and the oracle's absmax of its bf16-rounded projection, within one bf16 step
        oref = oproj.absmax_per_head(oproj.round_bf16(r))
        assert np.allclose(got_amax[t], oref, rtol=2 ** -7, atol=0), (t, got_amax[t], oref)
    torch.cuda.synchronize()


def test_projection_768p_sampled():
    """768p shape, the bench's launch configuration: sampled tokens against the
    oracle's product, absmax exact against the full outputs."""
    import torch
    w = WORKLOADS[3]
    inp = make_inputs(w)
    wts = make_projection_weights(w)
    q, k, v, amax = _project(w, inp, wts)
    tok = sample_tokens(w, per_frame=8)
    xs = inp["x"][:, tok]
    got_amax = amax.cpu().numpy().astype(np.uint32).view(np.float32).reshape(3, w.batch, w.heads)
    for t, (g, wname) in enumerate(zip((q, k, v), ("w_q", "w_k", "w_v"))):
        r = oproj.project(xs, wts[wname], w.heads)
        gn = g[:, torch.from_numpy(tok).to("cuda")].float().cpu().numpy().astype(np.float64)
        e = gu.errors(gn, r)
        print("768p", "qkv"[t], "max %.2e mean %.2e" % e, flush=True)
        assert e[0] <= 1e-2 and e[1] <= 2e-3, e
        own = g.float().abs().amax(dim=(1, 3)).cpu().numpy().astype(np.float32)
        assert np.array_equal(got_amax[t], own)


BLOCK_CASES = [WORKLOADS[2], WORKLOADS[5],
               Workload("block-ragged-b2", 2, 3, 100, 16, 2, 64, seed=64),
               Workload("block-fp8-d128", 1, 4, 90, 24, 2, 128, soft="fp8", outlier_frac=0.01, seed=65)]


def _block(w, inp, wts, debug=False):
    import torch
    lay = gu.api_layout(w)
    d = {k: _dev(v) for k, v in inp.items()}
    dbg = None
    if debug:
        f32 = dict(dtype=torch.float32, device="cuda")
        dbg = {"scales": torch.empty(5, w.batch, w.heads, **f32)}
    y = api.block_forward(lay, d["x"], _dev(wts["w_q"]), _dev(wts["w_k"]), _dev(wts["w_v"]), d["text_k"],
                          d["text_v"], d["w_gs"], d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"],
                          soft="fp8" if w.soft == "fp8" else None, debug=dbg)
    torch.cuda.synchronize()
    return y, dbg


@pytest.mark.parametrize("w", BLOCK_CASES, ids=[w.name for w in BLOCK_CASES])
def test_block_forward_is_layer_on_projected_inputs(w):
    """Bit-exact: the block call equals the layer called on the projection's
    q, k, v; with fp8 the fused absmax gives the same scales as the layer's own
    absmax pass."""
    import torch
    inp = make_inputs(w)
    wts = make_projection_weights(w)
    print("case", w.name, flush=True)
    yb, dbg = _block(w, inp, wts, debug=True)
    q, k, v, _ = _project(w, inp, wts)
    d = {kk: _dev(vv) for kk, vv in inp.items()}
    f32 = dict(dtype=torch.float32, device="cuda")
    dbg2 = {"scales": torch.empty(5, w.batch, w.heads, **f32)}
    yl = api.forward(gu.api_layout(w), d["x"], q, k, v, d["text_k"], d["text_v"], d["w_gs"], d["w_gl"],
                     d["w_os"], d["w_ol"], d["rms_w"], soft="fp8" if w.soft == "fp8" else None, debug=dbg2)
    torch.cuda.synchronize()
    assert torch.equal(yb, yl)
    if w.soft == "fp8":
        assert torch.equal(dbg["scales"], dbg2["scales"])


@pytest.mark.parametrize("w", BLOCK_CASES, ids=[w.name for w in BLOCK_CASES])
def test_block_forward_matches_oracle(w):
    """The block output against the oracle layer run on the oracle's
    projections rounded to bf16 (the stored q, k, v)."""
    import oracle
    inp = make_inputs(w)
    wts = make_projection_weights(w)
    yb, _ = _block(w, inp, wts)
    q, k, v = oproj.qkv_projection(inp["x"], wts["w_q"], wts["w_k"], wts["w_v"], w.heads)
    ref_inp = dict(inp, q=oproj.round_bf16(q), k=oproj.round_bf16(k), v=oproj.round_bf16(v))
    ref = oracle.hybrid_forward(ref_inp, gu.oracle_layout(w))
    e = gu.errors(yb.float().cpu().numpy().astype(np.float64), ref["y"])
    ed = gu.errors(yb.float().cpu().numpy().astype(np.float64) - inp["x"], ref["delta"])
    tmax, tmean = gu.TOL["fp8" if w.soft == "fp8" else "bf16"]
    print(w.name, "y max %.2e mean %.2e" % e, "delta max %.2e mean %.2e" % ed, flush=True)
    assert e[0] <= tmax and e[1] <= tmean, e
    # delta carries the bf16 rounding of y; bound it like y's own error relative to delta
    assert ed[0] <= max(tmax, 4e-2), ed
