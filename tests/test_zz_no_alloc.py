"""hyb_attn_forward_noalloc (the layer with the library's built-in scratch
instead of a workspace) against hyb_attn_forward on the same inputs: both
run the same kernels, so every output is compared bit for bit.  Calls run
back to back, each later one smaller than the one before, so that they run
on scratch an earlier call left behind; a call that needs more scratch than
the library holds is rejected before any launch."""
import numpy as np
import pytest

from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, make_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CALLS = [
    WORKLOADS[5],                                             # fp8 softmax, B2: 191 MiB of scratch
    WORKLOADS[2].with_(name="bf16-6-frames", frames=6, seed=71),
    WORKLOADS[5].with_(name="fp8-mx-small", batch=1, frames=4, tokens_per_frame=300, text_tokens=30,
                       heads=4, soft="fp8_mx", seed=72),
    WORKLOADS[1].with_(name="f32-small", frames=5, seed=73),
]


def _debug(w):
    import torch
    f32 = dict(dtype=torch.float32, device="cuda")
    B, N, H, D, hid = w.batch, w.n_video, w.heads, w.head_dim, w.hidden
    return {"o_soft": torch.empty(B, N, H, D, **f32), "o_lin": torch.empty(B, N, H, D, **f32),
            "delta_f32": torch.empty(B, N, hid, **f32), "gates": torch.empty(B, N, 2 * hid, **f32)}


def test_noalloc_matches_the_workspace_entry_point():
    import torch
    sizes = [api.workspace_size(gu.api_layout(w), w.act, w.soft if w.soft in ("fp8", "fp8_mx") else None)
             for w in CALLS]
    assert all(s <= api.NOALLOC_SCRATCH_BYTES for s in sizes)
    assert sizes == sorted(sizes, reverse=True)
    for w in CALLS:
        print("case", w.name, flush=True)
        inp = make_inputs(w)
        dev = gu.to_device(inp, w.act)
        lay = gu.api_layout(w)
        soft = w.soft if w.soft in ("fp8", "fp8_mx") else None
        args = (lay, dev["x"], dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["w_gs"],
                dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"])
        d_ref, d_new = _debug(w), _debug(w)
        y_ref = api.forward(*args, soft=soft, debug=d_ref)
        y_new = torch.empty_like(dev["x"])
        api.forward_noalloc(*args, y_new, soft=soft, debug=d_new)
        torch.cuda.synchronize()
        assert torch.equal(y_new, y_ref), w.name
        for k in d_ref:
            assert torch.equal(d_new[k], d_ref[k]), (w.name, k)
        # and it is the layer: y against the oracle at the workload's bound
        ref = gu.run_oracle(w, inp)
        tol = gu.TOL["fp8"] if soft else gu.TOL[w.act]
        e = gu.errors(y_new.float().cpu().numpy(), ref["y"])
        assert e[0] <= tol[0] and e[1] <= tol[1], (w.name, e)


def test_noalloc_rejects_calls_beyond_its_scratch():
    w = WORKLOADS[3]
    lay = gu.api_layout(w)
    assert api.workspace_size(lay, "bf16") > api.NOALLOC_SCRATCH_BYTES
    import torch
    x = torch.zeros(1, 16, dtype=torch.bfloat16, device="cuda")
    t = torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.HybError) as e:
        api.forward_noalloc(lay, x, t, t, t, t, t, x, x, x, x, x, x)
    assert e.value.status == api.HYB_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in api.load().hyb_last_error()
