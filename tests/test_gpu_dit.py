"""GPU parity of one DiT block (hyb_dit_block_forward: projection, layer,
residual RMSNorm + tanh-GELU feed-forward) against the fp64 oracle
(oracle/dit.py), through the C ABI.

The oracle rounds q, k, v and the layer output y to bf16 where the library
stores them.  Bound on z: max 1e-2 of max |z|, mean 5e-3.  One bf16
rounding gives a mean relative error of about 1.4e-3; the feed-forward path
passes three (the normalised input, the GELU output, z itself), so its mean
error is at most about 3 x 1.4e-3 = 4.2e-3, on top of the layer's (measured
<= 1.6e-3 on y).  The feed-forward alone is also checked from the library's
own layer output, on every case and at the 768p shape on sampled tokens."""
TOL_BLOCK = (1e-2, 5e-3)
import numpy as np
import pytest

from oracle import dit as odit
from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import (WORKLOADS, Workload, make_ffn_weights, make_inputs,
                                                    make_projection_weights, sample_tokens)
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [WORKLOADS[2],                                                     # hid 512, F 2048
         Workload("dit-ragged-b2", 2, 3, 100, 16, 2, 64, seed=81),          # hid 128, F 512
         Workload("dit-d128", 1, 4, 70, 24, 2, 128, seed=82)]               # hid 256, F 1024


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)


def _run(w, inp, pw, fw, block_only=False, soft=None):
    import torch
    d = {k: _dev(v) for k, v in inp.items()}
    p = {k: _dev(v) for k, v in pw.items()}
    f = {k: _dev(v) for k, v in fw.items()}
    lay = gu.api_layout(w)
    if block_only:
        out = api.block_forward(lay, d["x"], p["w_q"], p["w_k"], p["w_v"], d["text_k"], d["text_v"], d["w_gs"],
                                d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], soft=soft)
    else:
        out = api.dit_block_forward(lay, d["x"], p["w_q"], p["w_k"], p["w_v"], d["text_k"], d["text_v"],
                                    d["w_gs"], d["w_gl"], d["w_os"], d["w_ol"], d["rms_w"], f["w_n"], f["w_1"],
                                    f["w_2"], soft=soft)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_dit_block_matches_oracle(w):
    inp = make_inputs(w)
    pw = make_projection_weights(w)
    fw = make_ffn_weights(w)
    print("case", w.name, flush=True)
    z = _run(w, inp, pw, fw)
    ref = odit.dit_block(inp, gu.oracle_layout(w), pw, fw)
    e = gu.errors(z, ref["z"])
    print(w.name, "z max %.2e mean %.2e" % e, flush=True)
    assert e[0] <= TOL_BLOCK[0] and e[1] <= TOL_BLOCK[1], e
    # the feed-forward alone, from the library's own layer output
    y = _run(w, inp, pw, fw, block_only=True)
    e = gu.errors(z, odit.ffn(y, fw["w_n"], fw["w_1"], fw["w_2"]))
    print(w.name, "z from gpu y max %.2e mean %.2e" % e, flush=True)
    assert e[0] <= TOL_BLOCK[0] and e[1] <= TOL_BLOCK[1], e


def test_dit_block_zero_ffn_is_block_bit_exact():
    w = CASES[1]
    inp = make_inputs(w)
    pw = make_projection_weights(w)
    fw = make_ffn_weights(w)
    fw["w_2"] = np.zeros_like(fw["w_2"])
    assert np.array_equal(_run(w, inp, pw, fw), _run(w, inp, pw, fw, block_only=True))


# The MX feed-forward against oracle/mx.ffn_mx from the library's own layer
# output: both quantise the same bf16 normalised input (codes differ only
# where the fp32 and fp64 RMSNorm round to different bf16 values) and the
# GELU output (fp32 against fp64: an element within ~1e-6 of an e4m3
# rounding boundary can round the other way, one 2^-4 step of one of F
# terms), then z is rounded to bf16, whose own mean relative error is about
# 2^-10 ~ 1e-3 (measured mean 1.4e-3 in all).  Max at the fp8 bound; a wrong
# exponent or block gives mean errors near 0.4.
TOL_FFN_MX = (4e-2, 3e-3)


def test_dit_block_fp8_mx():
    """The DiT block in the fp8 version (MX projection, layer and
    feed-forward GEMMs): W_2 = 0 gives the block output bit for bit, and the
    feed-forward matches the MX oracle from the library's own layer output."""
    from oracle import mx
    for w in (CASES[2], Workload("dit-mx-ragged-b2", 2, 3, 100, 16, 4, 64, seed=83)):  # hid 256, F 1024
        inp = make_inputs(w)
        pw = make_projection_weights(w)
        fw = make_ffn_weights(w)
        y = _run(w, inp, pw, fw, block_only=True, soft="fp8_mx")
        z = _run(w, inp, pw, fw, soft="fp8_mx")
        e = gu.errors(z, mx.ffn_mx(y, fw["w_n"], fw["w_1"], fw["w_2"]))
        e_bf = gu.errors(z, odit.ffn(y, fw["w_n"], fw["w_1"], fw["w_2"]))
        print(w.name, "fp8_mx z vs MX oracle max %.2e mean %.2e" % e, "vs bf16 oracle max %.2e mean %.2e" % e_bf,
              flush=True)
        assert e[0] <= TOL_FFN_MX[0] and e[1] <= TOL_FFN_MX[1], e
    fz = dict(fw, w_2=np.zeros_like(fw["w_2"]))
    assert np.array_equal(_run(w, inp, pw, fz, soft="fp8_mx"), y)


def test_dit_block_768p_ffn_sampled():
    """Bench shape and launch configuration: the feed-forward on sampled
    tokens against the oracle applied to the library's own layer output."""
    w = WORKLOADS[3]
    inp = make_inputs(w)
    pw = make_projection_weights(w)
    fw = make_ffn_weights(w)
    z = _run(w, inp, pw, fw)
    y = _run(w, inp, pw, fw, block_only=True)
    tok = sample_tokens(w, per_frame=8)
    ys = y[:, tok]
    e = gu.errors(z[:, tok], odit.ffn(ys, fw["w_n"], fw["w_1"], fw["w_2"]))
    print("768p z max %.2e mean %.2e" % e, flush=True)
    assert e[0] <= TOL_BLOCK[0] and e[1] <= TOL_BLOCK[1], e
