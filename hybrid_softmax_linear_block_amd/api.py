"""ctypes binding of libhybattn.so (C ABI in include/hyb_attn.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and the current stream.  If the library is
missing, ``load()`` raises -- there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# HYB_ATTN_LIB selects another build of the same library (the host-sanitized
# one of build_lib.build(sanitize=True)).
LIB_PATH = os.environ.get("HYB_ATTN_LIB") or os.path.join(_PKG, "libhybattn.so")

HYB_OK, HYB_ERR_INVALID_ARGUMENT, HYB_ERR_UNSUPPORTED, HYB_ERR_WORKSPACE_TOO_SMALL, HYB_ERR_HIP = range(5)
DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "fp8_mx": 3}  # fp8_mx: fp8 softmax branch + MX e4m3 GEMMs


class HybError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("hyb status %d: %s" % (status, msg))
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "frames", "tokens_per_frame", "text_tokens", "heads", "head_dim",
        "chunk_frames", "chunk_radius", "anchor_first", "anchor_last")]


class _Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_tok", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class _Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales",
                                                "stage_events")]


STAGES = ("weights", "quant", "softmax", "states", "scan", "readout", "gate", "out", "qkv", "ffn")
BWD_STAGES = ("forward", "epilogue", "wgrad", "rms", "softmax", "linear")


class _BwdDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("d_os", "d_ol", "lse2", "stage_events")]


@dataclass(frozen=True)
class Layout:
    batch: int
    frames: int
    tokens_per_frame: int
    text_tokens: int
    heads: int
    head_dim: int
    chunk_frames: int = 1
    chunk_radius: int = 1
    anchor_first: bool = True
    anchor_last: bool = True

    def c(self):
        return _Layout(self.batch, self.frames, self.tokens_per_frame, self.text_tokens, self.heads,
                       self.head_dim, self.chunk_frames, self.chunk_radius, int(self.anchor_first),
                       int(self.anchor_last))

    @property
    def n_video(self):
        return self.frames * self.tokens_per_frame

    @property
    def hidden(self):
        return self.heads * self.head_dim


_lib = None


def load(path=None):
    """Load the HIP library (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libhybattn.so not found at %s; build it with "
                           "python -m hybrid_softmax_linear_block_amd.build_lib" % p)
    lib = ctypes.CDLL(p)
    lib.hyb_layout_tables.restype = ctypes.c_int
    lib.hyb_layout_tables.argtypes = [ctypes.POINTER(_Layout)] + [ctypes.POINTER(ctypes.c_int32)] * 4
    lib.hyb_workspace_size.restype = ctypes.c_int
    lib.hyb_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_attn_forward.restype = ctypes.c_int
    lib.hyb_attn_forward.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        + [_Tensor] * 5 + [ctypes.c_void_p] * 5 + [ctypes.c_float, ctypes.c_float]
        + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_Debug)])
    lib.hyb_attn_forward_noalloc.restype = ctypes.c_int
    lib.hyb_attn_forward_noalloc.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        + [_Tensor] * 5 + [ctypes.c_void_p] * 5 + [ctypes.c_float, ctypes.c_float]
        + [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Debug)])
    lib.hyb_qkv_workspace_size.restype = ctypes.c_int
    lib.hyb_qkv_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_qkv_project.restype = ctypes.c_int
    lib.hyb_qkv_project.argtypes = ([ctypes.POINTER(_Layout)] + [ctypes.c_void_p] * 8
                                    + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
    lib.hyb_block_workspace_size.restype = ctypes.c_int
    lib.hyb_block_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_block_forward.restype = ctypes.c_int
    lib.hyb_block_forward.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_int] + [ctypes.c_void_p] * 4 + [_Tensor] * 2 + [ctypes.c_void_p] * 5
        + [ctypes.c_float, ctypes.c_float]
        + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_Debug)])
    lib.hyb_dit_block_workspace_size.restype = ctypes.c_int
    lib.hyb_dit_block_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.c_int, ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_dit_block_forward.restype = ctypes.c_int
    lib.hyb_dit_block_forward.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_int] + [ctypes.c_void_p] * 4 + [_Tensor] * 2 + [ctypes.c_void_p] * 8
        + [ctypes.c_int32, ctypes.c_float, ctypes.c_float]
        + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_Debug)])
    lib.hyb_backward_workspace_size.restype = ctypes.c_int
    lib.hyb_backward_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_attn_backward.restype = ctypes.c_int
    lib.hyb_attn_backward.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_void_p] + [_Tensor] * 5 + [ctypes.c_void_p] * 5
        + [ctypes.c_float, ctypes.c_float] + [ctypes.c_void_p] * 7 + [ctypes.c_void_p] * 5
        + [ctypes.c_void_p, ctypes.c_size_t]
        + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_BwdDebug)])
    lib.hyb_block_backward_workspace_size.restype = ctypes.c_int
    lib.hyb_block_backward_workspace_size.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_block_backward.restype = ctypes.c_int
    lib.hyb_block_backward.argtypes = (
        [ctypes.POINTER(_Layout)] + [ctypes.c_void_p] * 4 + [_Tensor] * 2 + [ctypes.c_void_p] * 5
        + [ctypes.c_float, ctypes.c_float] + [ctypes.c_void_p] * 4 + [ctypes.c_void_p] * 8
        + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_BwdDebug)])
    lib.hyb_saved_size.restype = ctypes.c_int
    lib.hyb_saved_size.argtypes = [ctypes.POINTER(_Layout), ctypes.POINTER(ctypes.c_size_t)]
    lib.hyb_attn_forward_train.restype = ctypes.c_int
    lib.hyb_attn_forward_train.argtypes = (
        [ctypes.POINTER(_Layout), ctypes.c_void_p] + [_Tensor] * 5 + [ctypes.c_void_p] * 5
        + [ctypes.c_float, ctypes.c_float] + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
        + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.POINTER(_Debug)])
    lib.hyb_status_string.restype = ctypes.c_char_p
    lib.hyb_status_string.argtypes = [ctypes.c_int]
    lib.hyb_last_error.restype = ctypes.c_char_p
    lib.hyb_last_error.argtypes = []
    _lib = lib
    return lib


def _check(st):
    if st != HYB_OK:
        raise HybError(st, load().hyb_last_error().decode())


def layout_tables(lay: Layout):
    """Host-side frame tables: (soft_frames [T,T], soft_count [T], fwd [T,2], bwd [T,2])."""
    lib = load()
    T = lay.frames
    sf = np.zeros(T * T, np.int32)
    sc = np.zeros(T, np.int32)
    fw = np.zeros(2 * T, np.int32)
    bw = np.zeros(2 * T, np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    c = lay.c()
    _check(lib.hyb_layout_tables(ctypes.byref(c), sf.ctypes.data_as(P), sc.ctypes.data_as(P),
                                 fw.ctypes.data_as(P), bw.ctypes.data_as(P)))
    return sf.reshape(T, T), sc, fw.reshape(T, 2), bw.reshape(T, 2)


def workspace_size(lay: Layout, act="bf16", soft=None):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_workspace_size(ctypes.byref(c), DTYPES[act], DTYPES[soft or act], ctypes.byref(n)))
    return n.value


def _tensor4(t):
    if t is None or t.numel() == 0:
        return _Tensor(None, 0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, tokens, H, D] tensor with contiguous D")
    return _Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else t.data_ptr()


def forward(lay: Layout, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
            rms_weight, soft=None, softmax_scale=0.0, eps=1e-6, y=None, workspace=None, debug=None,
            stream=None):
    """y = x + delta for the hybrid layer, computed by libhybattn on the GPU.

    Tensors are torch device tensors in the activation dtype (float32 or
    bfloat16): x [B, N, hid]; q, k, v [B, N, H, D]; text_k, text_v
    [B, L, H, D]; weights [hid, hid] ([in][out]); rms_weight [hid].  ``soft``
    is None (same as the activations), "fp8" (e4m3 softmax branch) or
    "fp8_mx" (the fp8 version: also the gate and output GEMMs on MX e4m3
    operands; bf16 activations, hid % 256 == 0).  ``debug`` may map any of
    o_soft, o_lin, delta_f32, gates, scales to float32 device tensors, and
    "stage_events" to the address of an array of 2 * len(STAGES) hipEvent_t
    (see ``StageTimer``).
    """
    import torch
    lib = load()
    act = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(x.dtype)
    if act is None:
        raise ValueError("activations must be float32 or bfloat16")
    for t in (x, q, k, v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight):
        if t.dtype != x.dtype or not t.is_cuda:
            raise ValueError("all tensors must be device tensors of the activation dtype")
    for t in (x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight):
        if not t.is_contiguous():
            raise ValueError("x, weights and rms_weight must be contiguous")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(workspace_size(lay, act, soft), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _Debug(*([_ptr(debug.get(n)) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales")]
                       + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    st = lib.hyb_attn_forward(
        ctypes.byref(c), DTYPES[act], DTYPES[soft or act], x.data_ptr(),
        _tensor4(q), _tensor4(k), _tensor4(v), _tensor4(text_k), _tensor4(text_v),
        w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(), w_out_lin.data_ptr(),
        rms_weight.data_ptr(), float(softmax_scale), float(eps), y.data_ptr(), workspace.data_ptr(),
        workspace.numel(), stream, ctypes.byref(dbg) if dbg is not None else None)
    _check(st)
    return y


NOALLOC_SCRATCH_BYTES = 256 * 1024 * 1024  # HYB_NOALLOC_SCRATCH_BYTES in include/hyb_attn.h


def forward_noalloc(lay: Layout, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
                    rms_weight, y, soft=None, softmax_scale=0.0, eps=1e-6, debug=None, stream=None):
    """hyb_attn_forward_noalloc: the layer of ``forward`` with the library's
    built-in scratch instead of a workspace.  ``y`` must be given (this call
    allocates nothing, not even its output); the other arguments are those of
    ``forward``.  Calls on one GPU share the scratch: do not overlap them."""
    lib = load()
    act = _act_of(x, (x, q, k, v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, y),
                  (x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, y))
    dbg = None
    if debug:
        dbg = _Debug(*([_ptr(debug.get(n)) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales")]
                       + [debug.get("stage_events")]))
    if stream is None:
        import torch
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    st = lib.hyb_attn_forward_noalloc(
        ctypes.byref(c), DTYPES[act], DTYPES[soft or act], x.data_ptr(),
        _tensor4(q), _tensor4(k), _tensor4(v), _tensor4(text_k), _tensor4(text_v),
        w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(), w_out_lin.data_ptr(),
        rms_weight.data_ptr(), float(softmax_scale), float(eps), y.data_ptr(), stream,
        ctypes.byref(dbg) if dbg is not None else None)
    _check(st)
    return y


def _act_of(x, same_dtype, contiguous):
    import torch
    act = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(x.dtype)
    if act is None:
        raise ValueError("activations must be float32 or bfloat16")
    for t in same_dtype:
        if t.dtype != x.dtype or not t.is_cuda:
            raise ValueError("all tensors must be device tensors of the activation dtype")
    for t in contiguous:
        if not t.is_contiguous():
            raise ValueError("x, y, weights and rms_weight must be contiguous")
    return act


def qkv_workspace_size(lay: Layout):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_qkv_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return n.value


def qkv_project(lay: Layout, x, w_q, w_k, w_v, q=None, k=None, v=None, absmax=None, workspace=None,
                stream=None):
    """q, k, v = x W_q, x W_k, x W_v (bf16) by libhybattn, plus optionally the
    per-(tensor, batch, head) absmax of the outputs into ``absmax`` (an int32
    device tensor [3, B, H] receiving float32 bit patterns).  Returns
    (q, k, v) as [B, N, H, D] tensors."""
    import torch
    lib = load()
    for t in (x, w_q, w_k, w_v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x and the weights must be contiguous bfloat16 device tensors")
    B, N, H, D = lay.batch, lay.frames * lay.tokens_per_frame, lay.heads, lay.head_dim
    outs = []
    for t in (q, k, v):
        if t is None:
            t = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=x.device)
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.numel() != B * N * H * D:
            raise ValueError("q, k, v must be contiguous bfloat16 [B, N, H, D]")
        outs.append(t)
    if absmax is not None and (absmax.dtype != torch.int32 or absmax.numel() != 3 * B * H):
        raise ValueError("absmax must be an int32 tensor of 3*B*H elements")
    if workspace is None:
        workspace = torch.empty(qkv_workspace_size(lay), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    _check(lib.hyb_qkv_project(ctypes.byref(c), x.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
                               outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), _ptr(absmax),
                               workspace.data_ptr(), workspace.numel(), stream))
    return tuple(outs)


def block_workspace_size(lay: Layout, soft=None):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_block_workspace_size(ctypes.byref(c), DTYPES[soft or "bf16"], ctypes.byref(n)))
    return n.value


def block_forward(lay: Layout, x, w_q, w_k, w_v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft,
                  w_out_lin, rms_weight, soft=None, softmax_scale=0.0, eps=1e-6, y=None, workspace=None,
                  debug=None, stream=None):
    """The layer with its Q/K/V projection (bf16 activations): y = x + delta
    with q, k, v = x W_q, x W_k, x W_v computed on the GPU.  Arguments as in
    ``forward`` plus the projection weights [hid, hid] ([in][out])."""
    import torch
    lib = load()
    for t in (x, w_q, w_k, w_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, weights and rms_weight must be contiguous bfloat16 device tensors")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(block_workspace_size(lay, soft), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _Debug(*([_ptr(debug.get(n)) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales")]
                       + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    _check(lib.hyb_block_forward(
        ctypes.byref(c), DTYPES[soft or "bf16"], x.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
        _tensor4(text_k), _tensor4(text_v), w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(),
        w_out_lin.data_ptr(), rms_weight.data_ptr(), float(softmax_scale), float(eps), y.data_ptr(),
        workspace.data_ptr(), workspace.numel(), stream, ctypes.byref(dbg) if dbg is not None else None))
    return y


class StageTimer:
    """2 HIP events per stage, recorded by the library around each stage on
    the call's stream; ``elapsed_ms()`` returns per-stage milliseconds of the
    last recorded call.  ``stages`` is STAGES (forward and block calls) or
    BWD_STAGES (backward calls); ``span_ms`` runs from the start of stage
    ``first`` to the end of stage ``last``."""

    def __init__(self, stages=STAGES, first="qkv", last="out"):
        import torch
        self.stages, self.first, self.last = stages, first, last
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        n = 2 * len(stages)
        self.events = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev
        torch.cuda.synchronize()

    @property
    def address(self):
        return ctypes.addressof(self.events)

    def elapsed_ms(self):
        out = {}
        for i, name in enumerate(self.stages):
            a, b = self.events[2 * i], self.events[2 * i + 1]
            self._hip.hipEventSynchronize(b)
            ms = ctypes.c_float(0)
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def span_ms(self):
        """Milliseconds from the start of stage ``first`` to the end of stage
        ``last``: the whole call on the GPU (for forward calls the projection
        stage is recorded first, empty unless the call projects)."""
        a, b = self.events[2 * self.stages.index(self.first)], self.events[2 * self.stages.index(self.last) + 1]
        self._hip.hipEventSynchronize(b)
        ms = ctypes.c_float(0)
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for ev in self.events:
            if ev:
                self._hip.hipEventDestroy(ev)
        self.events = None


def backward_workspace_size(lay: Layout):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_backward_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return n.value


WEIGHT_GRADS = ("w_gate_soft", "w_gate_lin", "w_out_soft", "w_out_lin", "rms_weight")


def saved_size(lay: Layout):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_saved_size(ctypes.byref(c), ctypes.byref(n)))
    return n.value


def forward_train(lay: Layout, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
                  rms_weight, softmax_scale=0.0, eps=1e-6, y=None, saved=None, workspace=None, debug=None,
                  stream=None):
    """Training forward (bf16): returns (y, saved) where ``saved`` is the
    uint8 device buffer of forward values that ``backward(..., saved=saved)``
    reads instead of recomputing the forward."""
    import torch
    lib = load()
    for t in (x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, weights and rms_weight must be contiguous bfloat16 device tensors")
    if y is None:
        y = torch.empty_like(x)
    if saved is None:
        saved = torch.empty(saved_size(lay), dtype=torch.uint8, device=x.device)
    if workspace is None:
        workspace = torch.empty(workspace_size(lay, "bf16"), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _Debug(*([_ptr(debug.get(n)) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales")]
                       + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    _check(lib.hyb_attn_forward_train(
        ctypes.byref(c), x.data_ptr(), _tensor4(q), _tensor4(k), _tensor4(v), _tensor4(text_k), _tensor4(text_v),
        w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(), w_out_lin.data_ptr(),
        rms_weight.data_ptr(), float(softmax_scale), float(eps), y.data_ptr(), saved.data_ptr(), saved.numel(),
        workspace.data_ptr(), workspace.numel(), stream, ctypes.byref(dbg) if dbg is not None else None))
    return y, saved


def backward(lay: Layout, x, q, k, v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
             rms_weight, dy, softmax_scale=0.0, eps=1e-6, weight_grads=WEIGHT_GRADS, grads=None,
             workspace=None, debug=None, stream=None, saved=None):
    """Gradients of sum(dy * y) for the layer (bf16 activations), by libhybattn.

    Returns a dict: dx, dq, dk, dv, dtext_k, dtext_v (bf16, contiguous
    [B, tokens, H, D] / [B, N, hid]) and, for the names in ``weight_grads``,
    "d" + name as float32 tensors (weights [hid, hid], rms_weight [hid]).
    ``grads`` may pre-supply any of those output tensors.  ``debug`` may map
    "d_os", "d_ol" (float32 [B, N, H, D]), "lse2" (float32 [B, H, N]) and
    "stage_events" (address of 2 * len(BWD_STAGES) hipEvent_t, see
    ``StageTimer``).  ``saved``: the buffer of ``forward_train`` on the same
    inputs (then no forward recompute runs)."""
    import torch
    lib = load()
    for t in (x, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, dy):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, weights, rms_weight and dy must be contiguous bfloat16 device tensors")
    B, N, H, D = lay.batch, lay.n_video, lay.heads, lay.head_dim
    L, hid = lay.text_tokens, lay.hidden
    out = dict(grads or {})
    bf = dict(dtype=torch.bfloat16, device=x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    for name, shape in (("dx", (B, N, hid)), ("dq", (B, N, H, D)), ("dk", (B, N, H, D)), ("dv", (B, N, H, D)),
                        ("dtext_k", (B, L, H, D)), ("dtext_v", (B, L, H, D))):
        if name not in out:
            out[name] = torch.empty(shape, **bf)
    wptr = []
    for name in WEIGHT_GRADS:
        key = "d" + name
        if name in weight_grads:
            if key not in out:
                out[key] = torch.empty((hid,) if name == "rms_weight" else (hid, hid), **f32)
            wptr.append(out[key].data_ptr())
        else:
            wptr.append(None)
    if workspace is None:
        workspace = torch.empty(backward_workspace_size(lay), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _BwdDebug(*([_ptr(debug.get(n)) for n in ("d_os", "d_ol", "lse2")] + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    tptr = [out[n].data_ptr() if out[n].numel() else None for n in ("dtext_k", "dtext_v")]
    _check(lib.hyb_attn_backward(
        ctypes.byref(c), x.data_ptr(), _tensor4(q), _tensor4(k), _tensor4(v), _tensor4(text_k), _tensor4(text_v),
        w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(), w_out_lin.data_ptr(),
        rms_weight.data_ptr(), float(softmax_scale), float(eps), dy.data_ptr(), out["dx"].data_ptr(),
        out["dq"].data_ptr(), out["dk"].data_ptr(), out["dv"].data_ptr(), tptr[0], tptr[1], *wptr,
        saved.data_ptr() if saved is not None else None, saved.numel() if saved is not None else 0,
        workspace.data_ptr(), workspace.numel(), stream, ctypes.byref(dbg) if dbg is not None else None))
    return out


def dit_block_workspace_size(lay: Layout, ffn_hidden, soft=None):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_dit_block_workspace_size(ctypes.byref(c), DTYPES[soft or "bf16"], int(ffn_hidden),
                                            ctypes.byref(n)))
    return n.value


def dit_block_forward(lay: Layout, x, w_q, w_k, w_v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft,
                      w_out_lin, rms_weight, ffn_norm_weight, w_ff1, w_ff2, soft=None, softmax_scale=0.0,
                      eps=1e-6, z=None, workspace=None, debug=None, stream=None):
    """One block: z = y + GELU_tanh(RMSNorm(y) W_1) W_2 with y the layer with
    its Q/K/V projection (bf16).  Arguments as in ``block_forward`` plus the
    feed-forward weights ffn_norm_weight [hid], w_ff1 [hid, F], w_ff2 [F, hid]."""
    import torch
    lib = load()
    for t in (x, w_q, w_k, w_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, ffn_norm_weight,
              w_ff1, w_ff2):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, weights and norm weights must be contiguous bfloat16 device tensors")
    F = w_ff1.shape[1]
    if tuple(w_ff1.shape) != (lay.hidden, F) or tuple(w_ff2.shape) != (F, lay.hidden):
        raise ValueError("w_ff1 must be [hid, F] and w_ff2 [F, hid]")
    if z is None:
        z = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(dit_block_workspace_size(lay, F, soft), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _Debug(*([_ptr(debug.get(n)) for n in ("o_soft", "o_lin", "delta_f32", "gates", "scales")]
                       + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    _check(lib.hyb_dit_block_forward(
        ctypes.byref(c), DTYPES[soft or "bf16"], x.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(),
        _tensor4(text_k), _tensor4(text_v), w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(),
        w_out_lin.data_ptr(), rms_weight.data_ptr(), ffn_norm_weight.data_ptr(), w_ff1.data_ptr(),
        w_ff2.data_ptr(), int(F), float(softmax_scale), float(eps), z.data_ptr(), workspace.data_ptr(),
        workspace.numel(), stream, ctypes.byref(dbg) if dbg is not None else None))
    return z


def block_backward_workspace_size(lay: Layout):
    lib = load()
    n = ctypes.c_size_t(0)
    c = lay.c()
    _check(lib.hyb_block_backward_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return n.value


BLOCK_WEIGHT_GRADS = ("w_q", "w_k", "w_v") + WEIGHT_GRADS


def block_backward(lay: Layout, x, w_q, w_k, w_v, text_k, text_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin,
                   rms_weight, dy, softmax_scale=0.0, eps=1e-6, weight_grads=BLOCK_WEIGHT_GRADS, workspace=None,
                   debug=None, stream=None):
    """Gradients of sum(dy * y) for the layer with its Q/K/V projection
    (bf16).  Returns dx, dtext_k, dtext_v and "d" + name (float32) for the
    weights named in ``weight_grads``."""
    import torch
    lib = load()
    for t in (x, w_q, w_k, w_v, w_gate_soft, w_gate_lin, w_out_soft, w_out_lin, rms_weight, dy):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, weights, rms_weight and dy must be contiguous bfloat16 device tensors")
    B, N, H, D, L, hid = lay.batch, lay.n_video, lay.heads, lay.head_dim, lay.text_tokens, lay.hidden
    bf = dict(dtype=torch.bfloat16, device=x.device)
    out = {"dx": torch.empty((B, N, hid), **bf), "dtext_k": torch.empty((B, L, H, D), **bf),
           "dtext_v": torch.empty((B, L, H, D), **bf)}
    wptr = []
    for name in BLOCK_WEIGHT_GRADS:
        if name in weight_grads:
            out["d" + name] = torch.empty((hid,) if name == "rms_weight" else (hid, hid), dtype=torch.float32,
                                          device=x.device)
            wptr.append(out["d" + name].data_ptr())
        else:
            wptr.append(None)
    if workspace is None:
        workspace = torch.empty(block_backward_workspace_size(lay), dtype=torch.uint8, device=x.device)
    dbg = None
    if debug:
        dbg = _BwdDebug(*([_ptr(debug.get(n)) for n in ("d_os", "d_ol", "lse2")] + [debug.get("stage_events")]))
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    c = lay.c()
    tptr = [out[n].data_ptr() if out[n].numel() else None for n in ("dtext_k", "dtext_v")]
    _check(lib.hyb_block_backward(
        ctypes.byref(c), x.data_ptr(), w_q.data_ptr(), w_k.data_ptr(), w_v.data_ptr(), _tensor4(text_k),
        _tensor4(text_v), w_gate_soft.data_ptr(), w_gate_lin.data_ptr(), w_out_soft.data_ptr(),
        w_out_lin.data_ptr(), rms_weight.data_ptr(), float(softmax_scale), float(eps), dy.data_ptr(),
        out["dx"].data_ptr(), tptr[0], tptr[1], *wptr, workspace.data_ptr(), workspace.numel(), stream,
        ctypes.byref(dbg) if dbg is not None else None))
    return out
