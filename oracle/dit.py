"""fp64 definition of one DiT block around the hybrid layer (oracle, test
infrastructure only).

Source: VDN-H3 article (tahou.com, article 216474224916730885), section
"分阶段适配预训练模型" (staged adaptation): each block of the denoiser has
Q/K/V/O projections (here: the shared Q/K/V projection of the block input,
and the layer's two output projections) and a feed-forward network, frozen
in stages A1 and A2.  The article says nothing else about the block.

Readings taken where the article is silent (the library implements the same):
  * block(x) = z with
        y = layer(x; q, k, v = x W_q, x W_k, x W_v)     (oracle/hybrid.py,
                                                          oracle/projection.py)
        z = y + GELU(RMSNorm(y) W_1) W_2
  * the feed-forward input is normalised with RMSNorm over the hidden size
    (the only normalisation the article names), weight w_n, the layer's eps;
  * GELU is the tanh form, 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)));
  * no biases, [in][out] weights: W_1 [hid][F], W_2 [F][hid], F = 4 hid;
  * the stored intermediates follow the activation dtype: q, k, v and y are
    rounded to bf16 before the next step reads them (the FFN's own
    intermediates are not: the oracle keeps them in fp64).
  * timestep modulation (adaLN) and cross-attention are not in the article
    and are not part of the block.

Pinned by tests/test_oracle_dit.py: GELU against torch's tanh GELU and its
limits, RMSNorm scale invariance and a hand example, one-hot / zero FFN
weights, and the composition with the layer oracle.
"""
import math

import numpy as np

from .hybrid import hybrid_forward
from .projection import qkv_projection, round_bf16


def gelu_tanh(u):
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def rmsnorm(y, w, eps=1e-6):
    """y [..., hid] -> y w / sqrt(mean(y^2) + eps) over the last axis."""
    y = np.asarray(y, np.float64)
    return y * np.asarray(w, np.float64) / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)


def ffn(y, w_n, w_1, w_2, eps=1e-6):
    """Residual feed-forward: y + GELU(RMSNorm(y) W_1) W_2."""
    y = np.asarray(y, np.float64)
    h = rmsnorm(y, w_n, eps)
    u = gelu_tanh(h @ np.asarray(w_1, np.float64))
    return y + u @ np.asarray(w_2, np.float64)


def dit_block(inp, lay, proj, ffn_w, eps=1e-6, round_between=True):
    """One block: projection, hybrid layer, feed-forward.

    inp: the layer inputs of hybrid.hybrid_forward (its q, k, v are ignored);
    proj: w_q, w_k, w_v; ffn_w: w_n, w_1, w_2.  With round_between the
    projections and the layer output are rounded to bf16 before the next step
    (the library's storage).  Returns dict with q, k, v, y (layer output) and
    z (block output)."""
    q, k, v = qkv_projection(inp["x"], proj["w_q"], proj["w_k"], proj["w_v"], lay.heads)
    if round_between:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    layer_in = dict(inp, q=q, k=k, v=v)
    y = hybrid_forward(layer_in, lay, eps=eps)["y"]
    if round_between:
        y = round_bf16(y)
    z = ffn(y, ffn_w["w_n"], ffn_w["w_1"], ffn_w["w_2"], eps)
    return {"q": q, "k": k, "v": v, "y": y, "z": z}
