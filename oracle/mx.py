"""MX (OCP microscaling) e4m3 emulation of the fp8 GEMMs (oracle, test
infrastructure only).

Source: VDN-H3 article (tahou.com, article 216474224916730885), section
"性能实测表现" (measured performance): the fp8 version of the model is the
one timed against the dense baseline; the article does not say which
products it quantises.  The library's reading of the whole fp8 version: the
softmax branch as in oracle/fp8.py, and the Q/K/V projection, the gate GEMM
and the output GEMM on microscaling e4m3 operands.

Block format (OCP Microscaling Formats (MX) specification v1.0, block size
32, element type E4M3, shared scale E8M0): a block of 32 consecutive
elements along the contraction axis stores one power of two 2^s
(-127 <= s <= 127) and 32 e4m3 elements; the block's values are 2^s times
the elements.

Readings taken where the pages are silent (the library implements the same):
  * the block exponent is the smallest s >= -127 with max|block| <= 448 * 2^s,
    so no element saturates (the specification's example conversion, which
    takes floor(log2 max|block|) - 8 and clamps, can clip the largest element
    by up to 1/8);
  * elements are round-to-nearest-even e4m3 of the block's values / 2^s
    (oracle/fp8.round_e4m3; exact scaling in float64);
  * activations (x, and A' of the gated epilogue) are blocked along the
    features of each token; weights ([in][out], y = x W) along the input
    axis of each output column; products are exact and summed exactly here
    (the kernel accumulates in fp32);
  * A' = [g_s * O_s | g_l * RMSNorm(O_l)] is quantised as computed (in the
    library, from its fp32 value in the gate GEMM's epilogue); the gates
    themselves are not quantised;
  * in the DiT block's feed-forward, the normalised input is quantised from
    its stored bf16 value and the GELU output as computed (in the library,
    in the first GEMM's epilogue).

Pinned by tests/test_oracle_mx.py: the exponent's closed forms and its
minimality by brute force, element rounding against torch's float8_e4m3fn
conversion, exact round trips of representable blocks, the block extent and
axis, the format's error bound, exact products of representable operands,
and the fp8-version layer against the unquantised layer in the W_o = 0 and
exactly-representable special cases.
"""
import numpy as np

from .dit import gelu_tanh, rmsnorm
from .fp8 import round_e4m3, softmax_branch_fp8
from .hybrid import _rows, linear_branch, linear_states, sigmoid
from .projection import project, round_bf16

BLOCK = 32
E4M3_MAX = 448.0


def mx_exponent(amax):
    """Smallest integer s >= -127 with amax <= 448 * 2^s (amax >= 0, exact)."""
    a = np.asarray(amax, np.float64)
    m, e = np.frexp(a)                      # a = m 2^e, m in [0.5, 1) (0 for a = 0)
    # a = (2m) 2^(e-1) with 2m in [1, 2): s = e - 1 - 8, plus one when 2m > 1.75
    s = (e - 9) + (m > 0.875)
    s = np.where(a > 0, s, -127)
    return np.maximum(s, -127).astype(np.int64)


def mx_quantise(a, axis=-1):
    """Blocks of 32 along ``axis`` (its length a multiple of 32).  Returns
    (elements, exponents): elements are the e4m3 values (float64, same shape
    as a), exponents the int block exponents (axis length / 32 along axis)."""
    a = np.moveaxis(np.asarray(a, np.float64), axis, -1)
    K = a.shape[-1]
    assert K % BLOCK == 0, "contraction length must be a multiple of 32"
    blk = a.reshape(a.shape[:-1] + (K // BLOCK, BLOCK))
    s = mx_exponent(np.max(np.abs(blk), axis=-1))
    el = round_e4m3(blk * np.exp2(-s.astype(np.float64))[..., None])
    return np.moveaxis(el.reshape(a.shape), -1, axis), np.moveaxis(s, -1, axis)


def mx_dequantise(el, s, axis=-1):
    el = np.moveaxis(np.asarray(el, np.float64), axis, -1)
    s = np.moveaxis(np.asarray(s), axis, -1)
    K = el.shape[-1]
    v = el.reshape(el.shape[:-1] + (K // BLOCK, BLOCK)) * np.exp2(s.astype(np.float64))[..., None]
    return np.moveaxis(v.reshape(el.shape), -1, axis)


def mx_round(a, axis=-1):
    """The value the MX encoding of ``a`` represents."""
    el, s = mx_quantise(a, axis)
    return mx_dequantise(el, s, axis)


def mx_matmul(a, w):
    """a [..., K] (blocks along K) times w [K, N] ([in][out], blocks along
    K of each column), both MX-quantised, product exact."""
    return mx_round(a, -1) @ mx_round(w, 0)


def qkv_projection_mx(x, w_q, w_k, w_v, heads):
    """q, k, v = MX(x) MX(W) in float64 ([B, N, H, D]; the library then
    rounds them to bf16)."""
    xm = mx_round(x, -1)
    return tuple(project(xm, mx_round(w, 0), heads) for w in (w_q, w_k, w_v))


def epilogue_mx(x, o_s, o_l, w_gs, w_gl, w_os, w_ol, rms_w, eps=1e-6):
    """Gated fusion with MX gate and output GEMMs; same outputs as
    hybrid.epilogue plus a_p (A' before quantisation)."""
    x = np.asarray(x, np.float64)
    B, M, hid = x.shape
    os_ = np.asarray(o_s, np.float64).reshape(B, M, hid)
    ol_ = np.asarray(o_l, np.float64).reshape(B, M, hid)
    g_s = sigmoid(mx_matmul(x, w_gs))
    g_l = sigmoid(mx_matmul(x, w_gl))
    ms = np.mean(ol_ * ol_, axis=-1, keepdims=True)
    r = ol_ * np.asarray(rms_w, np.float64) / np.sqrt(ms + eps)
    a_p = np.concatenate([g_s * os_, g_l * r], axis=-1)
    w_o = np.concatenate([np.asarray(w_os, np.float64), np.asarray(w_ol, np.float64)], axis=0)
    delta = mx_matmul(a_p, w_o)
    return {"g_s": g_s, "g_l": g_l, "r": r, "a_p": a_p, "delta": delta, "y": x + delta}


def hybrid_forward_mx(inp, lay, scale=None, eps=1e-6, tokens=None):
    """The fp8 version of the layer: e4m3 softmax branch (oracle/fp8.py),
    linear branch in float64, MX gate and output GEMMs."""
    rows = _rows(lay, tokens)
    o_s = softmax_branch_fp8(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, scale=scale,
                             tokens=rows)
    st = linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
    o_l = linear_branch(inp["q"], st, lay, eps=eps, tokens=rows)
    ep = epilogue_mx(np.asarray(inp["x"])[:, rows], o_s, o_l, inp["w_gs"], inp["w_gl"], inp["w_os"], inp["w_ol"],
                     inp["rms_w"], eps=eps)
    ep.update({"o_s": o_s, "o_l": o_l, "tokens": rows})
    return ep


def ffn_mx(y, w_n, w_1, w_2, eps=1e-6):
    """The feed-forward of oracle/dit.py with MX GEMMs:
    z = y + MX(GELU(MX(bf16(RMSNorm(y))) MX(W_1))) MX(W_2)."""
    y = np.asarray(y, np.float64)
    h = round_bf16(rmsnorm(y, w_n, eps))
    u = gelu_tanh(mx_matmul(h, w_1))
    return y + mx_matmul(u, w_2)
