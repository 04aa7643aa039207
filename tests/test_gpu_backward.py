"""GPU parity of the backward pass (hyb_attn_backward) against the fp64
oracle's chain-rule gradients (oracle/backward.py, pinned by finite
differences), through the C ABI.

Bounds.  Every gradient is compared as max |gpu - ref| / max |ref| and
sum |gpu - ref| / sum |ref|.  The HIP path rounds some operands to bf16
(relative step 2^-8): dO_s, dZ and dR leave the output GEMM's epilogue in
bf16; P and dS enter the softmax products in bf16; every output is bf16.
One such rounding gives a mean relative error of about 1.4e-3 (measured on
dL/dO_s, which passes through exactly one).  The computed operands of the
linear branch (the states, phi(q), phi(k), and dnum where it multiplies the
states) are split into bf16 hi + lo and add nothing at this level; the copy
of dnum summed into the state gradients is bf16, averaged over a frame.  The longest paths (dq, dk, dtext_k: dO_s or
dR, then dS, then the output) pass through three roundings, so their mean
error is at most about 3 x 1.4e-3 = 4.2e-3: bound 5e-3.  The max bound is the
forward's, 1e-2.  Measured: mean 1.4e-3 to 3.2e-3, max at most 5.1e-3.
"""
import numpy as np
import pytest

import oracle.backward as obw
from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, Workload, make_grad_output, make_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL_GRAD = (1e-2, 5e-3)

CASES = [
    WORKLOADS[2],                                                          # D 64, 15 x 1024, text 128
    Workload("bwd-ragged-b2", 2, 5, 100, 20, 2, 64, qkv_scale=0.5, seed=71),  # ragged tiles, 2 batches
    Workload("bwd-d128-notext", 1, 6, 70, 0, 2, 128, qkv_scale=0.5, seed=72),  # linear states without text
    Workload("bwd-chunked", 1, 9, 40, 36, 2, 64, chunk_frames=2, qkv_scale=0.5, seed=73),
    Workload("bwd-no-anchor-r0", 1, 6, 64, 8, 2, 128, chunk_radius=0, anchor_first=False, anchor_last=False,
             qkv_scale=0.5, seed=74),
    Workload("bwd-tiny-frames-hid192", 2, 4, 5, 3, 3, 64, qkv_scale=0.5, seed=76),   # 5 tokens/frame, hid 192
    Workload("bwd-one-frame", 1, 1, 90, 10, 2, 64, qkv_scale=0.5, seed=77),
]

NAMES = [("dx", "dx"), ("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dtext_k", "dtext_k"),
         ("dtext_v", "dtext_v"), ("dw_gate_soft", "dw_gs"), ("dw_gate_lin", "dw_gl"), ("dw_out_soft", "dw_os"),
         ("dw_out_lin", "dw_ol"), ("drms_weight", "drms_w")]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)


def run_backward(w, inp, dy, weight_grads=api.WEIGHT_GRADS, **kw):
    import torch
    d = {k: _dev(v) for k, v in inp.items()}
    B, N, H, D = w.batch, w.n_video, w.heads, w.head_dim
    f32 = dict(dtype=torch.float32, device="cuda")
    dbg = {"d_os": torch.empty(B, N, H, D, **f32), "d_ol": torch.empty(B, N, H, D, **f32),
           "lse2": torch.empty(B, H, N, **f32)}
    g = api.backward(gu.api_layout(w), d["x"], d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["w_gs"],
                     d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], _dev(dy), weight_grads=weight_grads, debug=dbg,
                     **kw)
    torch.cuda.synchronize()
    out = {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items()}
    out.update({k: v.cpu().numpy().astype(np.float64) for k, v in dbg.items()})
    return out


def check_backward(w, inp, dy, scale=None):
    print("case", w.name, flush=True)
    got = run_backward(w, inp, dy, softmax_scale=scale or 0.0)
    ref = obw.hybrid_backward(inp, gu.oracle_layout(w), dy, scale=scale)
    B, N, H = w.batch, w.n_video, w.heads
    # intermediates: dL/dO_s, dL/dO_l and the softmax row statistics
    e = gu.errors(got["d_os"], ref["d_os"])
    print(w.name, "d_os max %.2e mean %.2e" % e, flush=True)
    assert e[0] <= 1e-2 and e[1] <= 2e-3, e
    e = gu.errors(got["d_ol"], ref["d_ol"])
    print(w.name, "d_ol max %.2e mean %.2e" % e, flush=True)
    assert e[0] <= 1e-2 and e[1] <= 2e-3, e
    lse = got["lse2"] * np.log(2.0)                                   # [B, H, N] -> natural log
    ref_lse = ref["lse"].transpose(0, 2, 1)
    assert np.max(np.abs(lse - ref_lse)) <= 2e-2, np.max(np.abs(lse - ref_lse))
    failed = []
    for gname, rname in NAMES:
        g = got[gname]
        r = ref[rname]
        if r.size == 0:
            assert g.size == 0
            continue
        e = gu.errors(g.reshape(r.shape), r)
        print(w.name, gname, "max %.2e mean %.2e" % e, flush=True)
        if not (e[0] <= TOL_GRAD[0] and e[1] <= TOL_GRAD[1]):
            failed.append((gname, e))
    assert not failed, failed


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_matches_oracle(w):
    check_backward(w, make_inputs(w), make_grad_output(w))


def test_backward_sharp_attention():
    """Inputs on which the forward kernel's running maximum moves mid-walk
    (tests/test_gpu_parity.sharp_inputs): the saved row statistics and every
    gradient that recomputes P from them."""
    from tests.test_gpu_parity import SHARP, rescale_fraction, sharp_inputs
    for w in SHARP:
        inp = sharp_inputs(w)
        assert rescale_fraction(w, inp) >= 0.5
        check_backward(w, inp, make_grad_output(w))


def test_backward_softmax_scale():
    """A non-zero softmax_scale through the backward's C ABI."""
    w = Workload("bwd-scale", 1, 5, 96, 24, 2, 64, qkv_scale=0.7, seed=78)
    check_backward(w, make_inputs(w), make_grad_output(w), scale=0.21)


def test_frozen_weights_are_not_written_and_rest_unchanged():
    """Null weight-gradient pointers (frozen weights, stage A2's softmax
    side) skip those gradients; the activation gradients are bit-identical
    to the full call."""
    import torch
    w = CASES[1]
    inp = make_inputs(w)
    dy = make_grad_output(w)
    full = run_backward(w, inp, dy)
    part = run_backward(w, inp, dy, weight_grads=("w_gate_lin", "w_out_lin", "rms_weight"))
    for k in ("dx", "dq", "dk", "dv", "dtext_k", "dtext_v", "dw_gate_lin", "dw_out_lin", "drms_weight"):
        assert np.array_equal(full[k], part[k]), k
    assert "dw_gate_soft" not in part and "dw_out_soft" not in part
    torch.cuda.synchronize()


def test_backward_head_major_strides_bit_identical():
    """q, k, v, text_k, text_v as head-major [B, H, tokens, D] storage viewed
    as [B, tokens, H, D]: the same gradients bit for bit."""
    import torch
    w = CASES[1]
    inp = make_inputs(w)
    dy = make_grad_output(w)
    base = run_backward(w, inp, dy)
    d = {k: _dev(v) for k, v in inp.items()}
    for name in ("q", "k", "v", "text_k", "text_v"):
        d[name] = d[name].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # strided view
    g = api.backward(gu.api_layout(w), d["x"], d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["w_gs"],
                     d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], _dev(dy))
    torch.cuda.synchronize()
    for k_, v_ in g.items():
        assert np.array_equal(v_.float().cpu().numpy().astype(np.float64), base[k_]), k_


def test_backward_768p_sampled():
    """768p shape, the bench's launch configuration: dq and dx on sampled
    tokens against the oracle evaluated one token at a time (full states);
    the key-side gradients are checked by test_backward_768p_key_side."""
    import torch
    from hybrid_softmax_linear_block_amd.inputs import sample_tokens
    w = WORKLOADS[3]
    inp = make_inputs(w)
    dy = make_grad_output(w)
    d = {k: _dev(v) for k, v in inp.items()}
    g = api.backward(gu.api_layout(w), d["x"], d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["w_gs"],
                     d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], _dev(dy), weight_grads=())
    torch.cuda.synchronize()
    tok = sample_tokens(w, per_frame=6)
    t = torch.from_numpy(tok).to("cuda")
    dq = g["dq"][:, t].float().cpu().numpy().astype(np.float64)
    dx = g["dx"][:, t].float().cpu().numpy().astype(np.float64)
    del g
    rq, rx = obw.dq_dx_at(inp, gu.oracle_layout(w), dy, tok)
    for name, got, ref in (("dq", dq, rq), ("dx", dx, rx)):
        e = gu.errors(got, ref)
        print("768p", name, "max %.2e mean %.2e" % e, flush=True)
        assert e[0] <= TOL_GRAD[0] and e[1] <= TOL_GRAD[1], (name, e)


def test_backward_768p_key_side():
    """768p shape, the bench's launch configuration: the key-side gradients
    of the dK/dV kernel and the linear branch (dk, dv, dtext_k, dtext_v) for
    every key of two heads, and the weight gradients dW_gate_lin,
    dW_out_lin and drms_weight in full.  Oracle: dL/dO_s and dL/dO_l from the
    epilogue's reverse step (row blocks; neither depends on O_s), then the
    softmax and linear branches' reverse steps on the two heads alone (the
    branches are independent per head)."""
    import torch
    w = WORKLOADS[3]
    heads = [0, 13]
    inp = make_inputs(w)
    dy = make_grad_output(w)
    d = {k: _dev(v) for k, v in inp.items()}
    g = api.backward(gu.api_layout(w), d["x"], d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["w_gs"],
                     d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], _dev(dy),
                     weight_grads=("w_gate_lin", "w_out_lin", "rms_weight"))
    torch.cuda.synchronize()
    got = {k: g[k][:, :, heads].float().cpu().numpy().astype(np.float64) for k in ("dk", "dv", "dtext_k", "dtext_v")}
    for k in ("dw_gate_lin", "dw_out_lin", "drms_weight"):
        got[k] = g[k].float().cpu().numpy().astype(np.float64)
    del g
    torch.cuda.empty_cache()
    print("768p key side: GPU done, oracle", flush=True)
    ref = obw.key_side_grads(inp, gu.oracle_layout(w), dy, heads, log=lambda m: print("oracle:", m, flush=True))
    failed = []
    for gname, rname in (("dk", "dk"), ("dv", "dv"), ("dtext_k", "dtext_k"), ("dtext_v", "dtext_v"),
                         ("dw_gate_lin", "dw_gl"), ("dw_out_lin", "dw_ol"), ("drms_weight", "drms_w")):
        e = gu.errors(got[gname].reshape(ref[rname].shape), ref[rname])
        print("768p", gname, "max %.2e mean %.2e" % e, flush=True)
        if not (e[0] <= TOL_GRAD[0] and e[1] <= TOL_GRAD[1]):
            failed.append((gname, e))
    assert not failed, failed


def test_backward_from_training_forward_bit_identical():
    """forward_train's y equals forward's y, and the backward that reads its
    saved values (no recompute) gives the recomputing backward's gradients,
    bit for bit."""
    import torch
    w = CASES[3]
    inp = make_inputs(w)
    dy = make_grad_output(w)
    base = run_backward(w, inp, dy)
    d = {k: _dev(v) for k, v in inp.items()}
    lay = gu.api_layout(w)
    args = (lay, d["x"], d["q"], d["k"], d["v"], d["text_k"], d["text_v"], d["w_gs"], d["w_gl"], d["w_os"],
            d["w_ol"], d["rms_w"])
    y_plain = api.forward(*args)
    y_train, saved = api.forward_train(*args)
    g = api.backward(*args, _dev(dy), saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(y_plain, y_train)
    for k_, v_ in g.items():
        assert np.array_equal(v_.float().cpu().numpy().astype(np.float64), base[k_]), k_


BLOCK_CASES = [CASES[1], Workload("bwd-block-d128", 1, 5, 60, 16, 2, 128, qkv_scale=0.5, seed=75)]


@pytest.mark.parametrize("w", BLOCK_CASES, ids=[w.name for w in BLOCK_CASES])
def test_block_backward_matches_oracle(w):
    """Through the Q/K/V projection: dx, dtext_k/v and every weight gradient
    (the projection's included) against the oracle's block backward, which
    takes the library's bf16 rounding of q, k, v as its reading of the stored
    projections (the gradient is evaluated at the stored values)."""
    import torch
    from hybrid_softmax_linear_block_amd.inputs import make_projection_weights
    from oracle.projection import qkv_projection, round_bf16
    inp = make_inputs(w)
    dy = make_grad_output(w)
    pw = make_projection_weights(w)
    d = {k: _dev(v) for k, v in inp.items()}
    p = {k: _dev(v) for k, v in pw.items()}
    g = api.block_backward(gu.api_layout(w), d["x"], p["w_q"], p["w_k"], p["w_v"], d["text_k"], d["text_v"],
                           d["w_gs"], d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], _dev(dy))
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items()}
    # oracle: layer gradients at the bf16-stored projections, then through the projection
    q, k, v = (round_bf16(t) for t in qkv_projection(inp["x"], pw["w_q"], pw["w_k"], pw["w_v"], w.heads))
    ref = obw.hybrid_backward(dict(inp, q=q, k=k, v=v), gu.oracle_layout(w), dy)
    M, hid = w.batch * w.n_video, w.hidden
    xf = np.asarray(inp["x"], np.float64).reshape(M, hid)
    dx = ref["dx"].reshape(M, hid)
    for name, dname in (("w_q", "dq"), ("w_k", "dk"), ("w_v", "dv")):
        dd = ref[dname].reshape(M, hid)
        dx = dx + dd @ np.asarray(pw[name], np.float64).T
        ref["d" + name] = xf.T @ dd
    ref["dx"] = dx.reshape(w.batch, w.n_video, hid)
    failed = []
    for gname, rname in (("dx", "dx"), ("dtext_k", "dtext_k"), ("dtext_v", "dtext_v"), ("dw_q", "dw_q"),
                         ("dw_k", "dw_k"), ("dw_v", "dw_v"), ("dw_gate_soft", "dw_gs"), ("dw_out_lin", "dw_ol"),
                         ("drms_weight", "drms_w")):
        r = ref[rname]
        if r.size == 0:
            continue
        e = gu.errors(got[gname].reshape(r.shape), r)
        print(w.name, gname, "max %.2e mean %.2e" % e, flush=True)
        if not (e[0] <= TOL_GRAD[0] and e[1] <= TOL_GRAD[1]):
            failed.append((gname, e))
    assert not failed, failed
