"""Out-of-bounds checks of the kernels' index math, by guard bands.

Every tensor the library reads sits inside a larger device buffer whose
margins hold NaN; Q, K, V and the text keys and values also carry one
16-byte granule of NaN between consecutive token rows (a token stride of
H*D + 8 elements).  A read past a tensor's rows, heads or batches, or into
that padding, turns some output into NaN or changes it: 0 x NaN is NaN, so
even a masked key shows through its value row.  Every buffer the library
writes (the outputs, the float32 debug copies, the gradients and the
workspace) sits between margins that hold a fixed bit pattern, so a write
outside it changes a margin.

Each case must give, bit for bit, the outputs of the same call on plain
contiguous tensors (the arithmetic does not depend on the strides), leave
every input buffer unchanged and every output margin as it was.  The cases
are small and ragged (partial key tiles, partial query tiles, partial
256-token GEMM tiles, empty text) on every forward path and on the
backward."""
import numpy as np
import pytest

from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import WORKLOADS, Workload, make_grad_output, make_inputs
from tests import gpu_util as gu

MARGIN_BYTES = 1 << 18   # each side of every buffer
ROW_PAD = 8              # elements of NaN after each token row of Q, K, V and the text


class Guarded:
    """A device tensor of ``shape`` inside a buffer with ``MARGIN_BYTES`` of
    ``fill`` on each side (and ``row_pad`` elements of ``fill`` after each
    token row of a [B, tokens, H, D] tensor)."""

    def __init__(self, shape, dtype, fill, host=None, row_pad=0, device="cuda"):
        import torch
        es = torch.empty((), dtype=dtype).element_size()
        m = MARGIN_BYTES // es
        shape = tuple(int(s) for s in shape)
        if row_pad:
            b, t, h, d = shape
            row = h * d + row_pad
            inner = b * t * row
            stride = (t * row, row, d, 1)
        else:
            inner = int(np.prod(shape))
            stride = tuple(int(np.prod(shape[i + 1:])) for i in range(len(shape)))
        self.buf = torch.full((m + inner + m,), fill, dtype=dtype, device=device)
        self.t = self.buf.as_strided(shape, stride, m)
        if host is not None:
            self.t.copy_(torch.from_numpy(np.ascontiguousarray(host)).to(dtype).to(device))
        outside = torch.ones(self.buf.numel(), dtype=torch.bool, device=device)
        outside.as_strided(shape, stride, m).fill_(False)
        self.outside = outside
        self.before = self._bits().clone()

    def _bits(self):
        import torch
        es = self.buf.element_size()
        return self.buf.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[es])

    def unchanged(self):
        """Every element of the buffer as it was (inputs)."""
        import torch
        return bool(torch.equal(self._bits(), self.before))

    def margins_intact(self):
        """Every element outside the tensor as it was (outputs)."""
        import torch
        return bool(torch.equal(self._bits()[self.outside], self.before[self.outside]))


def test_guard_helper_sees_writes_outside_the_tensor():
    """The helper on the host: writes into the tensor leave the margins
    intact; a write into either margin or into the padding after a token row
    does not; NaN fills compare by their bits."""
    import torch
    host = np.arange(2 * 3 * 2 * 8, dtype=np.float32).reshape(2, 3, 2, 8)
    for dt, fill in ((torch.bfloat16, float("nan")), (torch.float32, 1234.0)):
        g = Guarded(host.shape, dt, fill, host=host, row_pad=ROW_PAD, device="cpu")
        assert g.unchanged() and g.margins_intact()
        assert np.array_equal(g.t.float().numpy(), host)
        g.t.fill_(3.0)
        assert g.margins_intact() and not g.unchanged()
        for pos in (0, g.buf.numel() - 1, MARGIN_BYTES // g.buf.element_size() + 2 * 8):  # margins, row padding
            h = Guarded(host.shape, dt, fill, host=host, row_pad=ROW_PAD, device="cpu")
            h.buf[pos] = 5.0
            assert not h.margins_intact(), pos
    w = Guarded((5,), torch.uint8, 0xA5, device="cpu")
    w.buf[w.buf.numel() - 1] = 0
    assert not w.margins_intact()


def _dtype(act):
    import torch
    return torch.float32 if act == "f32" else torch.bfloat16


def _guard_inputs(w, inp):
    import torch
    dt = _dtype(w.act)
    nan = float("nan")
    g = {}
    for name, a in inp.items():
        if a.size == 0:
            g[name] = None
            continue
        pad = ROW_PAD if name in ("q", "k", "v", "text_k", "text_v") else 0
        g[name] = Guarded(a.shape, dt, nan, host=a, row_pad=pad)
    return g


def _tensor(g, w, name):
    import torch
    if g[name] is not None:
        return g[name].t
    B, H, D = w.batch, w.heads, w.head_dim
    return torch.empty((B, 0, H, D), dtype=_dtype(w.act), device="cuda")


FORWARD = [
    WORKLOADS[2].with_(name="guard-bf16-d64", frames=4, tokens_per_frame=200, text_tokens=30, seed=101),
    WORKLOADS[2].with_(name="guard-bf16-d128-chunked", batch=2, frames=7, tokens_per_frame=70, text_tokens=17,
                       heads=2, head_dim=128, chunk_frames=2, seed=102),
    WORKLOADS[2].with_(name="guard-bf16-notext-noanchor", frames=5, tokens_per_frame=96, text_tokens=0,
                       anchor_first=False, anchor_last=False, seed=103),
    WORKLOADS[5].with_(name="guard-fp8", frames=4, tokens_per_frame=200, text_tokens=30, seed=104),
    WORKLOADS[5].with_(name="guard-fp8-mx", batch=1, frames=4, tokens_per_frame=130, text_tokens=0, heads=4,
                       soft="fp8_mx", seed=105),
    WORKLOADS[1].with_(name="guard-f32", frames=4, seed=106),
]


@pytest.mark.gpu
@pytest.mark.parametrize("w", FORWARD, ids=[w.name for w in FORWARD])
def test_forward_stays_inside_its_buffers(w):
    import torch
    print("case", w.name, flush=True)
    inp = make_inputs(w)
    soft = w.soft if w.soft in ("fp8", "fp8_mx") else None
    base = gu.run_gpu(w, inp)

    gin = _guard_inputs(w, inp)
    B, N, H, D, hid = w.batch, w.n_video, w.heads, w.head_dim, w.hidden
    sentinel = 1234.0
    y = Guarded((B, N, hid), _dtype(w.act), sentinel)
    dbg = {"o_soft": Guarded((B, N, H, D), torch.float32, sentinel),
           "o_lin": Guarded((B, N, H, D), torch.float32, sentinel),
           "delta_f32": Guarded((B, N, hid), torch.float32, sentinel),
           "gates": Guarded((B, N, 2 * hid), torch.float32, sentinel),
           "scales": Guarded((5, B, H), torch.float32, sentinel)}
    size = api.workspace_size(gu.api_layout(w), w.act, soft)
    ws = Guarded((size,), torch.uint8, 0xA5)
    api.forward(gu.api_layout(w), gin["x"].t, gin["q"].t, gin["k"].t, gin["v"].t, _tensor(gin, w, "text_k"),
                _tensor(gin, w, "text_v"), gin["w_gs"].t, gin["w_gl"].t, gin["w_os"].t, gin["w_ol"].t,
                gin["rms_w"].t, soft=soft, y=y.t, workspace=ws.t, debug={k: v.t for k, v in dbg.items()})
    torch.cuda.synchronize()

    for name, g in gin.items():
        assert g is None or g.unchanged(), "input %s or its margins were written" % name
    assert y.margins_intact(), "write outside y"
    assert ws.margins_intact(), "write outside the workspace"
    for name, g in dbg.items():
        assert g.margins_intact(), "write outside %s" % name
    got = {"y": y.t.float().cpu().numpy().astype(np.float64)}
    got.update({k: v.t.cpu().numpy().astype(np.float64) for k, v in dbg.items()})
    for key in base:
        if key == "scales" and not soft:
            continue
        assert np.all(np.isfinite(got[key])), key
        assert np.array_equal(got[key], base[key]), key


BACKWARD = [
    Workload("guard-bwd-ragged-b2", 2, 5, 100, 20, 2, 64, qkv_scale=0.5, seed=111),
    Workload("guard-bwd-d128-chunked", 1, 7, 70, 17, 2, 128, chunk_frames=2, qkv_scale=0.5, seed=112),
]


@pytest.mark.gpu
@pytest.mark.parametrize("w", BACKWARD, ids=[w.name for w in BACKWARD])
def test_backward_stays_inside_its_buffers(w):
    import torch
    print("case", w.name, flush=True)
    inp = make_inputs(w)
    dy = make_grad_output(w)
    lay = gu.api_layout(w)
    bf = torch.bfloat16
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(bf) for k, v in inp.items()}
    dyd = torch.from_numpy(np.ascontiguousarray(dy)).to("cuda").to(bf)
    base = api.backward(lay, dev["x"], dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["w_gs"],
                        dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"], dyd)
    torch.cuda.synchronize()
    base = {k: v.float().cpu().numpy() for k, v in base.items()}

    gin = _guard_inputs(w, inp)
    gdy = Guarded(dy.shape, bf, float("nan"), host=dy)
    B, N, L, H, D, hid = w.batch, w.n_video, w.text_tokens, w.heads, w.head_dim, w.hidden
    sentinel = -77.0
    shapes = {"dx": ((B, N, hid), bf), "dq": ((B, N, H, D), bf), "dk": ((B, N, H, D), bf),
              "dv": ((B, N, H, D), bf), "dtext_k": ((B, L, H, D), bf), "dtext_v": ((B, L, H, D), bf),
              "dw_gate_soft": ((hid, hid), torch.float32), "dw_gate_lin": ((hid, hid), torch.float32),
              "dw_out_soft": ((hid, hid), torch.float32), "dw_out_lin": ((hid, hid), torch.float32),
              "drms_weight": ((hid,), torch.float32)}
    gout = {k: Guarded(s, dt, sentinel) for k, (s, dt) in shapes.items()}
    ws = Guarded((api.backward_workspace_size(lay),), torch.uint8, 0x5A)
    api.backward(lay, gin["x"].t, gin["q"].t, gin["k"].t, gin["v"].t, gin["text_k"].t, gin["text_v"].t,
                 gin["w_gs"].t, gin["w_gl"].t, gin["w_os"].t, gin["w_ol"].t, gin["rms_w"].t, gdy.t,
                 grads={k: v.t for k, v in gout.items()}, workspace=ws.t)
    torch.cuda.synchronize()

    for name, g in list(gin.items()) + [("dy", gdy)]:
        assert g is None or g.unchanged(), "input %s or its margins were written" % name
    assert ws.margins_intact(), "write outside the workspace"
    for name, g in gout.items():
        assert g.margins_intact(), "write outside %s" % name
        got = g.t.float().cpu().numpy()
        assert np.all(np.isfinite(got)), name
        assert np.array_equal(got, base[name]), name


BLOCKS = [
    (Workload("guard-block-ragged-b2", 2, 3, 100, 16, 2, 64, seed=121), None),
    (Workload("guard-block-d128-fp8", 1, 4, 70, 24, 2, 128, seed=122), "fp8"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("w,soft", BLOCKS, ids=[w.name for w, _ in BLOCKS])
def test_projection_block_and_dit_block_stay_inside_their_buffers(w, soft):
    """hyb_qkv_project, hyb_block_forward and hyb_dit_block_forward (the
    projection GEMM, its absmax epilogue and the feed-forward GEMMs) with
    guarded inputs, outputs and workspaces."""
    import torch
    from hybrid_softmax_linear_block_amd.inputs import make_ffn_weights, make_projection_weights
    print("case", w.name, soft, flush=True)
    inp, pw, fw = make_inputs(w), make_projection_weights(w), make_ffn_weights(w)
    lay = gu.api_layout(w)
    bf = torch.bfloat16
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(bf) for k, v in {**inp, **pw, **fw}.items()}
    B, N, H, D, hid = w.batch, w.n_video, w.heads, w.head_dim, w.hidden
    args = ("w_gs", "w_gl", "w_os", "w_ol", "rms_w")
    base_q = [t.float().cpu().numpy() for t in api.qkv_project(lay, dev["x"], dev["w_q"], dev["w_k"], dev["w_v"])]
    base_y = api.block_forward(lay, dev["x"], dev["w_q"], dev["w_k"], dev["w_v"], dev["text_k"], dev["text_v"],
                               *[dev[a] for a in args], soft=soft).float().cpu().numpy()
    base_z = api.dit_block_forward(lay, dev["x"], dev["w_q"], dev["w_k"], dev["w_v"], dev["text_k"], dev["text_v"],
                                   *[dev[a] for a in args], dev["w_n"], dev["w_1"], dev["w_2"],
                                   soft=soft).float().cpu().numpy()
    torch.cuda.synchronize()

    gin = _guard_inputs(w, {**inp, **pw, **fw})
    t = {k: v.t for k, v in gin.items()}
    sentinel = 1234.0
    gq = [Guarded((B, N, H, D), bf, sentinel) for _ in range(3)]
    gam = Guarded((3 * B * H,), torch.int32, 0x5A5A5A5A)
    ws = Guarded((api.qkv_workspace_size(lay),), torch.uint8, 0xA5)
    api.qkv_project(lay, t["x"], t["w_q"], t["w_k"], t["w_v"], q=gq[0].t, k=gq[1].t, v=gq[2].t, absmax=gam.t,
                    workspace=ws.t)
    gy = Guarded((B, N, hid), bf, sentinel)
    wsb = Guarded((api.block_workspace_size(lay, soft),), torch.uint8, 0xA5)
    api.block_forward(lay, t["x"], t["w_q"], t["w_k"], t["w_v"], t["text_k"], t["text_v"], *[t[a] for a in args],
                      soft=soft, y=gy.t, workspace=wsb.t)
    gz = Guarded((B, N, hid), bf, sentinel)
    F = fw["w_1"].shape[1]
    wsd = Guarded((api.dit_block_workspace_size(lay, F, soft),), torch.uint8, 0xA5)
    api.dit_block_forward(lay, t["x"], t["w_q"], t["w_k"], t["w_v"], t["text_k"], t["text_v"],
                          *[t[a] for a in args], t["w_n"], t["w_1"], t["w_2"], soft=soft, z=gz.t, workspace=wsd.t)
    torch.cuda.synchronize()

    for name, g in gin.items():
        assert g.unchanged(), "input %s or its margins were written" % name
    for name, g in [("q", gq[0]), ("k", gq[1]), ("v", gq[2]), ("absmax", gam), ("qkv workspace", ws), ("y", gy),
                    ("block workspace", wsb), ("z", gz), ("dit workspace", wsd)]:
        assert g.margins_intact(), "write outside %s" % name
    for i in range(3):
        assert np.array_equal(gq[i].t.float().cpu().numpy(), base_q[i]), "qkv"[i]
    for name, g, ref in (("y", gy, base_y), ("z", gz, base_z)):
        got = g.t.float().cpu().numpy()
        assert np.all(np.isfinite(got)), name
        assert np.array_equal(got, ref), name


@pytest.mark.gpu
def test_noalloc_entry_point_stays_inside_its_buffers():
    """hyb_attn_forward_noalloc (the library's own scratch) with guarded
    inputs and outputs."""
    import torch
    w = WORKLOADS[2].with_(name="guard-noalloc", frames=4, tokens_per_frame=200, text_tokens=30, seed=131)
    print("case", w.name, flush=True)
    inp = make_inputs(w)
    base = gu.run_gpu(w, inp, debug=False)
    gin = _guard_inputs(w, inp)
    y = Guarded((w.batch, w.n_video, w.hidden), torch.bfloat16, 1234.0)
    api.forward_noalloc(gu.api_layout(w), gin["x"].t, gin["q"].t, gin["k"].t, gin["v"].t, gin["text_k"].t,
                        gin["text_v"].t, gin["w_gs"].t, gin["w_gl"].t, gin["w_os"].t, gin["w_ol"].t, gin["rms_w"].t,
                        y.t)
    torch.cuda.synchronize()
    for name, g in gin.items():
        assert g.unchanged(), "input %s or its margins were written" % name
    assert y.margins_intact(), "write outside y"
    got = y.t.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, base["y"])


@pytest.mark.gpu
def test_training_forward_saved_backward_and_block_backward_stay_inside_their_buffers():
    """hyb_attn_forward_train writing its saved buffer, hyb_attn_backward
    reading it, and hyb_block_backward, with guarded inputs, outputs, saved
    buffer and workspaces."""
    import torch
    from hybrid_softmax_linear_block_amd.inputs import make_projection_weights
    w = Workload("guard-train-ragged-b2", 2, 5, 100, 20, 2, 64, qkv_scale=0.5, seed=141)
    print("case", w.name, flush=True)
    inp, pw, dy = make_inputs(w), make_projection_weights(w), make_grad_output(w)
    lay = gu.api_layout(w)
    bf = torch.bfloat16
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(bf) for k, v in {**inp, **pw}.items()}
    dyd = torch.from_numpy(np.ascontiguousarray(dy)).to("cuda").to(bf)
    layer = lambda t: (t["x"], t["q"], t["k"], t["v"], t["text_k"], t["text_v"], t["w_gs"], t["w_gl"], t["w_os"],
                       t["w_ol"], t["rms_w"])
    block = lambda t: (t["x"], t["w_q"], t["w_k"], t["w_v"], t["text_k"], t["text_v"], t["w_gs"], t["w_gl"],
                       t["w_os"], t["w_ol"], t["rms_w"])
    y0, saved0 = api.forward_train(lay, *layer(dev))
    g0 = api.backward(lay, *layer(dev), dyd, saved=saved0)
    b0 = api.block_backward(lay, *block(dev), dyd)
    torch.cuda.synchronize()
    g0 = {k: v.float().cpu().numpy() for k, v in g0.items()}
    b0 = {k: v.float().cpu().numpy() for k, v in b0.items()}

    gin = _guard_inputs(w, {**inp, **pw})
    gdy = Guarded(dy.shape, bf, float("nan"), host=dy)
    t = {k: v.t for k, v in gin.items()}
    B, N, L, H, D, hid = w.batch, w.n_video, w.text_tokens, w.heads, w.head_dim, w.hidden
    sentinel = -77.0
    gy = Guarded((B, N, hid), bf, sentinel)
    gsaved = Guarded((api.saved_size(lay),), torch.uint8, 0x3C)
    wsf = Guarded((api.workspace_size(lay, "bf16"),), torch.uint8, 0xA5)
    api.forward_train(lay, *layer(t), y=gy.t, saved=gsaved.t, workspace=wsf.t)
    shapes = {"dx": ((B, N, hid), bf), "dq": ((B, N, H, D), bf), "dk": ((B, N, H, D), bf),
              "dv": ((B, N, H, D), bf), "dtext_k": ((B, L, H, D), bf), "dtext_v": ((B, L, H, D), bf),
              "dw_gate_soft": ((hid, hid), torch.float32), "dw_gate_lin": ((hid, hid), torch.float32),
              "dw_out_soft": ((hid, hid), torch.float32), "dw_out_lin": ((hid, hid), torch.float32),
              "drms_weight": ((hid,), torch.float32)}
    gout = {k: Guarded(s, dt, sentinel) for k, (s, dt) in shapes.items()}
    wsb = Guarded((api.backward_workspace_size(lay),), torch.uint8, 0x5A)
    api.backward(lay, *layer(t), gdy.t, saved=gsaved.t, grads={k: v.t for k, v in gout.items()}, workspace=wsb.t)
    wsk = Guarded((api.block_backward_workspace_size(lay),), torch.uint8, 0x5A)
    b1 = api.block_backward(lay, *block(t), gdy.t, workspace=wsk.t)
    torch.cuda.synchronize()

    for name, g in list(gin.items()) + [("dy", gdy)]:
        assert g.unchanged(), "input %s or its margins were written" % name
    for name, g in [("y", gy), ("saved", gsaved), ("forward workspace", wsf), ("backward workspace", wsb),
                    ("block backward workspace", wsk)] + list(gout.items()):
        assert g.margins_intact(), "write outside %s" % name
    assert np.array_equal(gy.t.float().cpu().numpy(), y0.float().cpu().numpy()), "y"
    for name, g in gout.items():
        got = g.t.float().cpu().numpy()
        assert np.all(np.isfinite(got)), name
        assert np.array_equal(got, g0[name]), name
    for name, v in b1.items():
        got = v.float().cpu().numpy()
        assert np.all(np.isfinite(got)), name
        assert np.array_equal(got, b0[name]), name
