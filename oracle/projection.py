"""fp64 definition of the Q/K/V input projection that feeds the hybrid layer
(oracle, test infrastructure only).

Source: VDN-H3 article (tahou.com, article 216474224916730885), section
"分阶段适配预训练模型" (staged adaptation): stages A2 and B keep one set of
Q/K/V projections shared by both attention branches (frozen in A1/A2, LoRA
in B), so the layer's q, k and v come from a single projection of the block
input.  The performance section's fp8 version (section "性能实测表现")
quantises the softmax branch's inputs; the library's reading of that
quantisation (per (tensor, batch, head) absmax / 448) is in oracle/fp8.py.

Readings taken where the article is silent (the library implements the same):
  * q = x W_q, k = x W_k, v = x W_v with [in][out] row-major weights and no
    bias, the hidden axis split into heads as hid = H * D, head-major within
    a token (feature h * D + d is head h, dim d);
  * the projections are stored in the activation dtype (bf16, round to
    nearest even) before the layer reads them; the absmax that sets the fp8
    scale is taken over those stored values.

Pinned by tests/test_oracle_projection.py (one-hot and diagonal weights,
head split, absmax of constructed inputs).
"""
import numpy as np


def project(x, w, heads):
    """x [B, N, hid], w [hid, hid] ([in][out]) -> [B, N, H, D] float64."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, N, hid = x.shape
    if w.shape != (hid, hid) or hid % heads:
        raise ValueError("weight must be [hid, hid] with hid divisible by heads")
    y = (x.reshape(B * N, hid) @ w).reshape(B, N, heads, hid // heads)
    return y


def qkv_projection(x, w_q, w_k, w_v, heads):
    """The three projections of the block input: (q, k, v), each [B, N, H, D]."""
    return project(x, w_q, heads), project(x, w_k, heads), project(x, w_v, heads)


def round_bf16(a):
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    The value is first rounded to float32 (nearest even), then to bf16; for
    the projections this is the single rounding the stored tensor carries up
    to the rare double-rounding tie, which the parity bounds absorb."""
    u = np.ascontiguousarray(np.asarray(a, np.float32)).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def absmax_per_head(t):
    """max |t| over tokens and head dims of a [B, tokens, H, D] tensor -> [B, H]."""
    return np.max(np.abs(np.asarray(t, np.float64)), axis=(1, 3))
