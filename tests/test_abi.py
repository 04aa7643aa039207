"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, fills the frame tables exactly as the oracle does, and
rejects bad arguments before launching anything."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import oracle
from hybrid_softmax_linear_block_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyb_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(api.LIB_PATH), reason="libhybattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hyb_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = api.load()
    names = declared_functions()
    assert names == sorted(["hyb_attn_forward", "hyb_last_error", "hyb_layout_tables",
                            "hyb_status_string", "hyb_workspace_size", "hyb_qkv_workspace_size",
                            "hyb_qkv_project", "hyb_block_workspace_size", "hyb_block_forward",
                            "hyb_backward_workspace_size", "hyb_attn_backward",
                            "hyb_dit_block_workspace_size", "hyb_dit_block_forward", "hyb_saved_size",
                            "hyb_attn_forward_train", "hyb_block_backward_workspace_size", "hyb_block_backward",
                            "hyb_attn_forward_noalloc"])
    for n in names:
        assert hasattr(lib, n), n


def test_layout_tables_bit_exact_against_oracle():
    for T, C, R, af, al in itertools.product(range(1, 36), (1, 2, 3, 5), (0, 1, 2), (0, 1), (0, 1)):
        lay = api.Layout(1, T, 1, 0, 1, 64, C, R, bool(af), bool(al))
        sf, sc, fw, bw = api.layout_tables(lay)
        osf, osc, ofw, obw = oracle.tables(T, C, R, af, al)
        assert np.array_equal(sf, np.array(osf, np.int32)), (T, C, R, af, al)
        assert np.array_equal(sc, np.array(osc, np.int32))
        assert np.array_equal(fw, np.array(ofw, np.int32)), (T, C, R, af, al, fw, ofw)
        assert np.array_equal(bw, np.array(obw, np.int32))


def test_worked_example_tables():
    sf, sc, fw, bw = api.layout_tables(api.Layout(1, 15, 4032, 512, 24, 128))
    assert list(sf[7][:sc[7]]) == [0, 6, 7, 8, 14]
    assert list(fw[7]) == [1, 6] and list(bw[7]) == [9, 14]


def test_table_validation():
    with pytest.raises(api.HybError) as e:
        api.layout_tables(api.Layout(1, 0, 1, 0, 1, 64))
    assert e.value.status == api.HYB_ERR_INVALID_ARGUMENT
    with pytest.raises(api.HybError):
        api.layout_tables(api.Layout(1, 5, 1, 0, 1, 64, chunk_frames=0))
    with pytest.raises(api.HybError):
        api.layout_tables(api.Layout(1, 5, 1, 0, 1, 64, chunk_radius=-1))


def test_workspace_size_and_dtype_rules():
    lay = api.Layout(1, 15, 4032, 512, 24, 128)
    n = api.workspace_size(lay, "bf16")
    # fp16 branch outputs (2 x 372 MB) + fp16 A' (743 MB) dominate
    assert 1.5e9 < n < 2.0e9
    assert api.workspace_size(lay, "bf16", "fp8") > n
    with pytest.raises(api.HybError) as e:
        api.workspace_size(lay, "f32", "fp8")
    assert e.value.status == api.HYB_ERR_UNSUPPORTED
    with pytest.raises(api.HybError) as e:
        api.workspace_size(api.Layout(1, 15, 64, 16, 2, 32), "bf16")
    assert e.value.status == api.HYB_ERR_UNSUPPORTED
    assert api.workspace_size(api.Layout(1, 15, 64, 16, 2, 32), "f32") > 0
    with pytest.raises(api.HybError) as e:
        api.workspace_size(api.Layout(1, 15, 64, 16, 2, 48), "f32")
    assert e.value.status == api.HYB_ERR_UNSUPPORTED


def _call(lay, **over):
    """Call hyb_attn_forward with fake but aligned addresses; every case here
    must fail validation before any HIP call is made."""
    lib = api.load()
    c = lay.c()
    base = 1 << 40
    T4 = api._Tensor
    H, D = lay.heads, lay.head_dim
    st = (lay.n_video * H * D, H * D, D)
    args = dict(act=1, soft=1, x=base, q=T4(base + (1 << 34), *st), k=T4(base + (2 << 34), *st),
                v=T4(base + (3 << 34), *st), tk=T4(base + (4 << 34), *st), tv=T4(base + (5 << 34), *st),
                wgs=base + (6 << 34), wgl=base + (7 << 34), wos=base + (8 << 34), wol=base + (9 << 34),
                rms=base + (10 << 34), scale=0.0, eps=1e-6, y=base + (11 << 34), ws=base + (12 << 34),
                wsb=1 << 40, stream=None)
    args.update(over)
    r = lib.hyb_attn_forward(ctypes.byref(c), args["act"], args["soft"], args["x"], args["q"], args["k"],
                             args["v"], args["tk"], args["tv"], args["wgs"], args["wgl"], args["wos"],
                             args["wol"], args["rms"], args["scale"], args["eps"], args["y"], args["ws"],
                             args["wsb"], args["stream"], None)
    return r, lib.hyb_last_error().decode()


def test_forward_validation_errors():
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    T4 = api._Tensor
    assert _call(lay, x=None)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(lay, q=T4(None, 0, 0, 0))[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(lay, wgs=(1 << 40) + 2)[0] == api.HYB_ERR_INVALID_ARGUMENT       # misaligned
    assert _call(lay, ws=(1 << 40) + 16)[0] == api.HYB_ERR_INVALID_ARGUMENT       # workspace not 256-aligned
    assert _call(lay, k=T4(1 << 41, 1024 * 512, 512 + 4, 64))[0] == api.HYB_ERR_INVALID_ARGUMENT  # stride
    assert _call(lay, eps=0.0)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(lay, eps=float("nan"))[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(lay, scale=-1.0)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(lay, act=0, soft=2)[0] == api.HYB_ERR_UNSUPPORTED
    assert _call(lay, act=2, soft=2)[0] == api.HYB_ERR_UNSUPPORTED
    r, msg = _call(lay, wsb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL and "needs" in msg
    # y overlapping q is rejected
    r, msg = _call(lay, y=(1 << 40) + (1 << 34) + 4096)
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlaps" in msg
    # text tensors may be NULL only without text
    assert _call(lay, tk=T4(None, 0, 0, 0))[0] == api.HYB_ERR_INVALID_ARGUMENT
    bad = api.Layout(1, 15, 1024, 128, 8, 64, chunk_frames=0)
    assert _call(bad)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _call(api.Layout(0, 15, 1024, 128, 8, 64))[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert api.load().hyb_status_string(3) == b"workspace too small"


def _qkv_call(lay, **over):
    """hyb_qkv_project with fake aligned addresses; must fail validation."""
    lib = api.load()
    c = lay.c()
    base = 1 << 40
    args = dict(x=base, wq=base + (1 << 34), wk=base + (2 << 34), wv=base + (3 << 34), q=base + (4 << 34),
                k=base + (5 << 34), v=base + (6 << 34), amax=None, ws=base + (7 << 34), wsb=1 << 40)
    args.update(over)
    r = lib.hyb_qkv_project(ctypes.byref(c), args["x"], args["wq"], args["wk"], args["wv"], args["q"], args["k"],
                            args["v"], args["amax"], args["ws"], args["wsb"], None)
    return r, lib.hyb_last_error().decode()


def test_qkv_project_validation_errors():
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    assert _qkv_call(lay, x=None)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert _qkv_call(lay, wk=(1 << 40) + 8)[0] == api.HYB_ERR_INVALID_ARGUMENT      # misaligned
    assert _qkv_call(lay, ws=(1 << 40) + 16)[0] == api.HYB_ERR_INVALID_ARGUMENT     # workspace alignment
    assert _qkv_call(lay, amax=(1 << 40) + 2)[0] == api.HYB_ERR_INVALID_ARGUMENT
    r, msg = _qkv_call(lay, k=(1 << 40) + (4 << 34) + 4096)                         # k overlaps q
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlap" in msg
    r, msg = _qkv_call(lay, wsb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL and "needs" in msg
    assert _qkv_call(api.Layout(1, 15, 64, 16, 2, 32))[0] == api.HYB_ERR_UNSUPPORTED   # head_dim 32
    hid = 8 * 64
    assert api.qkv_workspace_size(lay) == 3 * hid * hid * 2


def test_block_forward_validation_errors():
    lib = api.load()
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    c = lay.c()
    base = 1 << 40
    T4 = api._Tensor
    st = (128 * 512, 512, 64)

    def call(**over):
        a = dict(soft=1, x=base, wq=base + (1 << 34), wk=base + (2 << 34), wv=base + (3 << 34),
                 tk=T4(base + (4 << 34), *st), tv=T4(base + (5 << 34), *st), wgs=base + (6 << 34),
                 wgl=base + (7 << 34), wos=base + (8 << 34), wol=base + (9 << 34), rms=base + (10 << 34),
                 scale=0.0, eps=1e-6, y=base + (11 << 34), ws=base + (12 << 34), wsb=1 << 40)
        a.update(over)
        return lib.hyb_block_forward(ctypes.byref(c), a["soft"], a["x"], a["wq"], a["wk"], a["wv"], a["tk"],
                                     a["tv"], a["wgs"], a["wgl"], a["wos"], a["wol"], a["rms"], a["scale"],
                                     a["eps"], a["y"], a["ws"], a["wsb"], None, None)

    assert call(wq=None) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(wgs=None) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(tk=T4(None, 0, 0, 0)) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(eps=0.0) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(soft=0) == api.HYB_ERR_UNSUPPORTED                  # float32 softmax with bf16 activations
    assert call(wsb=1000) == api.HYB_ERR_WORKSPACE_TOO_SMALL
    n = api.block_workspace_size(lay)
    assert n > api.workspace_size(lay, "bf16") + 3 * 15 * 1024 * 512 * 2
    assert api.block_workspace_size(lay, "fp8") > n


def test_backward_validation_errors():
    """hyb_attn_backward with fake aligned addresses: every bad argument is
    rejected before anything is launched."""
    lib = api.load()
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    c = lay.c()
    base = 1 << 40
    T4 = api._Tensor
    st = (15 * 1024 * 512, 512, 64)
    tst = (128 * 512, 512, 64)
    slot = iter(range(1, 64))

    def nxt():
        return base + (next(slot) << 34)
    a0 = dict(x=nxt(), q=T4(nxt(), *st), k=T4(nxt(), *st), v=T4(nxt(), *st), tk=T4(nxt(), *tst),
              tv=T4(nxt(), *tst), wgs=nxt(), wgl=nxt(), wos=nxt(), wol=nxt(), rms=nxt(), scale=0.0, eps=1e-6,
              dy=nxt(), dx=nxt(), dq=nxt(), dk=nxt(), dv=nxt(), dtk=nxt(), dtv=nxt(), dwgs=nxt(), dwgl=nxt(),
              dwos=nxt(), dwol=nxt(), drms=nxt(), sv=None, svb=0, ws=nxt(), wsb=1 << 40)

    def call(lay_c=c, **over):
        a = dict(a0)
        a.update(over)
        r = lib.hyb_attn_backward(ctypes.byref(lay_c), a["x"], a["q"], a["k"], a["v"], a["tk"], a["tv"], a["wgs"],
                                  a["wgl"], a["wos"], a["wol"], a["rms"], a["scale"], a["eps"], a["dy"], a["dx"],
                                  a["dq"], a["dk"], a["dv"], a["dtk"], a["dtv"], a["dwgs"], a["dwgl"], a["dwos"],
                                  a["dwol"], a["drms"], a["sv"], a["svb"], a["ws"], a["wsb"], None, None)
        return r, lib.hyb_last_error().decode()

    assert call(dy=None)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert call(dq=None)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert call(dtk=None)[0] == api.HYB_ERR_INVALID_ARGUMENT                 # text present, dtext_k needed
    assert call(dx=a0["dx"] + 8)[0] == api.HYB_ERR_INVALID_ARGUMENT           # misaligned
    assert call(dwgs=a0["dwgs"] + 4)[0] == api.HYB_ERR_INVALID_ARGUMENT       # misaligned weight gradient
    assert call(ws=a0["ws"] + 16)[0] == api.HYB_ERR_INVALID_ARGUMENT          # workspace alignment
    assert call(eps=float("nan"))[0] == api.HYB_ERR_INVALID_ARGUMENT
    r, msg = call(dk=a0["dq"] + 4096)                                         # dk overlaps dq
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlaps" in msg
    r, msg = call(dv=a0["q"].ptr + 1024)                                      # output over an input
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlaps input" in msg
    r, msg = call(wsb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL and "needs" in msg
    # frozen weights: null gradient pointers are accepted (the call then reaches the
    # workspace check with the fake sizes)
    r, msg = call(dwgs=None, dwos=None, drms=None, wsb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL
    sv = nxt()
    assert call(sv=sv + 64, svb=1 << 40)[0] == api.HYB_ERR_INVALID_ARGUMENT          # saved alignment
    r, msg = call(sv=sv, svb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL and "saved" in msg
    r, msg = call(sv=sv, svb=1 << 40, dq=sv + 4096, wsb=1 << 34)                    # output over saved
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "saved" in msg
    n = api.saved_size(lay)
    M, hid = 15 * 1024, 512
    assert n >= M * hid * 2 * 6 + 8 * 15 * 1024 * 4
    bad = api.Layout(1, 15, 64, 16, 2, 32).c()
    assert call(lay_c=bad)[0] == api.HYB_ERR_UNSUPPORTED                      # head_dim 32
    big = api.Layout(1, 2, 64, 0, 160, 128).c()
    assert call(lay_c=big)[0] == api.HYB_ERR_UNSUPPORTED                      # hidden 20480
    n = api.backward_workspace_size(lay)
    assert n > api.workspace_size(lay, "bf16")


def test_dit_block_validation_errors():
    lib = api.load()
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    c = lay.c()
    base = 1 << 40
    T4 = api._Tensor
    st = (128 * 512, 512, 64)

    def call(**over):
        a = dict(soft=1, x=base, wq=base + (1 << 34), wk=base + (2 << 34), wv=base + (3 << 34),
                 tk=T4(base + (4 << 34), *st), tv=T4(base + (5 << 34), *st), wgs=base + (6 << 34),
                 wgl=base + (7 << 34), wos=base + (8 << 34), wol=base + (9 << 34), rms=base + (10 << 34),
                 wn=base + (11 << 34), w1=base + (12 << 34), w2=base + (13 << 34), F=2048, scale=0.0, eps=1e-6,
                 z=base + (14 << 34), ws=base + (15 << 34), wsb=1 << 40)
        a.update(over)
        return lib.hyb_dit_block_forward(ctypes.byref(c), a["soft"], a["x"], a["wq"], a["wk"], a["wv"], a["tk"],
                                         a["tv"], a["wgs"], a["wgl"], a["wos"], a["wol"], a["rms"], a["wn"],
                                         a["w1"], a["w2"], a["F"], a["scale"], a["eps"], a["z"], a["ws"],
                                         a["wsb"], None, None)

    assert call(w1=None) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(wn=base + 2) == api.HYB_ERR_INVALID_ARGUMENT              # misaligned
    assert call(F=100) == api.HYB_ERR_INVALID_ARGUMENT                    # not a multiple of 64
    assert call(F=0) == api.HYB_ERR_INVALID_ARGUMENT
    assert call(wsb=1000) == api.HYB_ERR_WORKSPACE_TOO_SMALL
    assert call(wq=None) == api.HYB_ERR_INVALID_ARGUMENT                  # checked by the block call, pre-launch
    n = api.dit_block_workspace_size(lay, 2048)
    M, hid = 15 * 1024, 512
    assert n >= api.block_workspace_size(lay) + 2 * M * hid * 2 + M * 2048 * 2 + 2 * 2048 * hid * 2


def test_block_backward_validation_errors():
    lib = api.load()
    lay = api.Layout(1, 15, 1024, 128, 8, 64)
    c = lay.c()
    base = 1 << 40
    T4 = api._Tensor
    st = (128 * 512, 512, 64)
    slot = iter(range(1, 64))

    def nxt():
        return base + (next(slot) << 34)
    a0 = dict(x=nxt(), wq=nxt(), wk=nxt(), wv=nxt(), tk=T4(nxt(), *st), tv=T4(nxt(), *st), wgs=nxt(), wgl=nxt(),
              wos=nxt(), wol=nxt(), rms=nxt(), scale=0.0, eps=1e-6, dy=nxt(), dx=nxt(), dtk=nxt(), dtv=nxt(),
              dwq=nxt(), dwk=nxt(), dwv=nxt(), dwgs=nxt(), dwgl=nxt(), dwos=nxt(), dwol=nxt(), drms=nxt(),
              ws=nxt(), wsb=1 << 34)

    def call(**over):
        a = dict(a0)
        a.update(over)
        r = lib.hyb_block_backward(ctypes.byref(c), a["x"], a["wq"], a["wk"], a["wv"], a["tk"], a["tv"], a["wgs"],
                                   a["wgl"], a["wos"], a["wol"], a["rms"], a["scale"], a["eps"], a["dy"], a["dx"],
                                   a["dtk"], a["dtv"], a["dwq"], a["dwk"], a["dwv"], a["dwgs"], a["dwgl"], a["dwos"],
                                   a["dwol"], a["drms"], a["ws"], a["wsb"], None, None)
        return r, lib.hyb_last_error().decode()

    assert call(wq=None)[0] == api.HYB_ERR_INVALID_ARGUMENT
    assert call(dwk=a0["dwk"] + 4)[0] == api.HYB_ERR_INVALID_ARGUMENT
    r, msg = call(dx=a0["x"] + 1024)
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlaps" in msg
    r, msg = call(dwq=a0["dwk"])
    assert r == api.HYB_ERR_INVALID_ARGUMENT and "overlaps" in msg
    r, msg = call(wsb=1000)
    assert r == api.HYB_ERR_WORKSPACE_TOO_SMALL
    assert api.block_backward_workspace_size(lay) > api.backward_workspace_size(lay)


def test_fp8_mx_mode_validation():
    """HYB_FP8_MX needs bf16 activations and a hidden size that is a multiple
    of 256; its workspace adds the e4m3 GEMM operands to the fp8 one."""
    from hybrid_softmax_linear_block_amd import api
    bad = api.Layout(1, 2, 64, 0, 3, 64)      # hid 192
    with pytest.raises(api.HybError) as e:
        api.workspace_size(bad, "bf16", "fp8_mx")
    assert "256" in str(e.value)
    with pytest.raises(api.HybError):
        api.workspace_size(api.Layout(1, 2, 64, 0, 4, 64), "f32", "fp8_mx")
    ok = api.Layout(2, 3, 100, 16, 4, 64)     # hid 256, 600 tokens -> 768 exponent rows
    w8 = api.workspace_size(ok, "bf16", "fp8")
    wmx = api.workspace_size(ok, "bf16", "fp8_mx")
    M, hid, mpad = 600, 256, 768
    assert wmx - w8 >= M * hid + (hid // 32) * mpad * 3 + (hid // 32) * 2 * hid * 2
    assert api.block_workspace_size(ok, "fp8_mx") > api.block_workspace_size(ok, "fp8")
    # the DiT block's MX feed-forward needs ffn_hidden % 256 == 0
    with pytest.raises(api.HybError) as e:
        api.dit_block_workspace_size(ok, 320, "fp8_mx")
    assert "256" in str(e.value)
    assert api.dit_block_workspace_size(ok, 320, "fp8") > 0
    assert api.dit_block_workspace_size(ok, 1024, "fp8_mx") > api.dit_block_workspace_size(ok, 1024, "fp8")


def test_noalloc_size_limit_is_checked_on_the_host():
    """hyb_attn_forward_noalloc rejects a layout whose workspace exceeds its
    built-in scratch before any HIP call (so no GPU is needed here); the
    header's limit and the binding's agree."""
    text = open(HEADER).read()
    m = re.search(r"#define HYB_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u \* (\d+)u\)", text)
    assert m and int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == api.NOALLOC_SCRATCH_BYTES
    lib = api.load()
    lay = api.Layout(1, 15, 4032, 512, 24, 128).c()
    t = api._Tensor(16, 0, 0, 0)
    st = lib.hyb_attn_forward_noalloc(ctypes.byref(lay), 1, 1, 16, t, t, t, t, t, 16, 16, 16, 16, 16,
                                      0.0, 1e-6, 16, None, None)
    assert st == api.HYB_ERR_WORKSPACE_TOO_SMALL
    assert b"built-in scratch" in lib.hyb_last_error()
    small = api.Layout(1, 0, 64, 0, 1, 64).c()   # invalid layout: reported first
    assert lib.hyb_attn_forward_noalloc(ctypes.byref(small), 1, 1, 16, t, t, t, t, t, 16, 16, 16, 16, 16,
                                        0.0, 1e-6, 16, None, None) == api.HYB_ERR_INVALID_ARGUMENT
