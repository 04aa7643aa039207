"""fp64 CPU oracle for the VDN-H3 dual-branch hybrid attention layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library and imports nothing from
``hybrid_softmax_linear_block_amd``.

Source: the VDN-H3 open-source article (tahou.com, article 216474224916730885),
section "技术核心设计 / 双分支混合注意力机制" (dual-branch hybrid attention) and
section "自适应门控融合双分支输出" (adaptive gated fusion of the branch outputs).

Every function is a plain definition evaluated in float64 with NumPy; no
blocking, fusion or reordering beyond what the definition states.  Readings
the article leaves open are listed in the module docstrings of ``layout``
and ``hybrid`` and are the same as the ones the HIP library implements.

Parity status per function (what pins it, in ``tests/test_oracle_*.py``):
  layout.frame_sets / layout.tables   pinned: the article's worked example
                                      (frame 7 of 0..14), closed form for the
                                      per-frame window, partition invariant.
  hybrid.softmax_branch               pinned: dense token-mask brute force,
                                      torch SDPA special case, constant-V.
  hybrid.linear_states / linear_branch pinned: exact integer text-once
                                      invariant, quadratic masked brute force,
                                      constant-V closed form, phi closed forms.
  hybrid.epilogue                     pinned: zero/one-hot weight closed forms,
                                      RMSNorm scope closed form.
  projection.project / qkv_projection pinned: one-hot (non-symmetric
                                      permutation) and diagonal weights, head
                                      split, a hand-computed example.
  projection.absmax_per_head          pinned: constructed tensors.
  projection.round_bf16               pinned: torch bfloat16 conversion.
  backward.hybrid_backward and its    pinned: central finite differences of
  reverse steps (softmax_backward,    the forward oracle along random
  linear_backward, epilogue_backward) directions for every input, per step
                                      and for the whole layer, on three frame
                                      layouts; planted mistakes are caught.
  backward.softmax_lse                pinned: closed forms (q = 0, constant keys).
  dit.gelu_tanh / rmsnorm / ffn /     pinned: torch's tanh GELU and its limits,
  dit_block                           RMSNorm hand example and scale
                                      invariance, zero / identity / one-hot
                                      feed-forward weights, composition with
                                      the layer oracle.
  fp8.round_e4m3 / quantise           pinned: torch's float8_e4m3fn conversion,
                                      the format's closed forms.
  fp8.softmax_branch_fp8              pinned: uniform scores (mean of the
                                      quantised values), probabilities on the
                                      e4m3 grid and unrounded probabilities
                                      (both equal to softmax_branch on the
                                      dequantised inputs), hand-derived codes
                                      of a frame-tiled walk, a maximum rising
                                      inside a tile, a subnormal code; planted
                                      mistakes are caught.
  mx.mx_exponent / mx_quantise /      pinned: closed forms and brute-force
  mx_matmul / epilogue_mx /           minimality of the block exponent,
  hybrid_forward_mx                   torch's float8_e4m3fn rounding, exact
                                      round trips, block extent and axis, the
                                      format's error bound, exact products of
                                      representable operands, W_o = 0.
  Anchor frames as queries (they attend to every frame, their linear rows
  hold text only) are a reading the article cannot confirm: it says only
  that the anchors interact with the other frames.  The oracle's form of
  that reading is pinned like every other frame's (hand-written frame sets,
  the per-frame closed form, dense-mask brute force, text-only linear rows).
"""
from .layout import Layout, frame_sets, tables  # noqa: F401
from .hybrid import (phi, softmax_branch, linear_states, linear_branch,  # noqa: F401
                     epilogue, hybrid_forward)
from . import projection  # noqa: F401
from . import backward  # noqa: F401
from . import dit  # noqa: F401
from . import mx  # noqa: F401
