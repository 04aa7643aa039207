"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP layer
through the C ABI binding, compare with the fp64 oracle."""
import numpy as np

import oracle
from oracle.layout import Layout as OLayout
from hybrid_softmax_linear_block_amd import api
from hybrid_softmax_linear_block_amd.inputs import make_inputs

TOL = {  # (max |err| / max |ref|, mean relative error)
    "f32": (1e-4, 1e-4),
    "bf16": (1e-2, 2e-3),
    "fp8": (4e-2, 4e-2),
}

# fp8 softmax output against the e4m3 emulation (oracle/fp8.py), which takes
# every code and every move of the running maximum in float32 as the kernel
# does.  What is left between the two: the fp16 storage of O_s (at most 2^-11
# relative per element), float32 accumulation of up to ~25,000 products in
# the matrix cores and of the normaliser, and rare codes that flip where
# v_exp_f32 (1 ulp) puts a scaled probability on the other side of an e4m3
# rounding boundary (one key's weight moves by at most 2^-3 relative).  Each
# is well below the bf16 bounds, which are used here; a probability rounded
# against another maximum moves O_s by ~3% mean, a wrong code or scale by
# 100%.
FP8_EMU_TOL = (1e-2, 2e-3)

# Limit of the fp8 reading itself: what per-(tensor, batch, head) absmax
# quantisation of Q, K, V (with the 1% x8 outliers of the fp8 workload) and
# e4m3 probabilities leave on O_s against the unquantised oracle.  The
# emulation gives max 0.184 / mean 0.057 on the fp8 workload (every token;
# 0.210 / 0.058 on 64 sampled tokens per frame), Q/K/V quantisation alone
# 0.184 / 0.048, probability rounding alone 0.010 / 0.023.  The layer output
# stays within the fp8 bound (TOL["fp8"]).
FP8_READING_LIMIT = (0.25, 0.065)


def oracle_layout(w):
    return OLayout(w.batch, w.frames, w.tokens_per_frame, w.text_tokens, w.heads, w.head_dim,
                   w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)


def api_layout(w):
    return api.Layout(w.batch, w.frames, w.tokens_per_frame, w.text_tokens, w.heads, w.head_dim,
                      w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)


def to_device(inp, act):
    import torch
    dt = torch.float32 if act == "f32" else torch.bfloat16
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(dt) for k, v in inp.items()}


def run_gpu(w, inp, debug=True, dev=None, **kw):
    """Run the layer on cuda:0.  Returns numpy float64 outputs."""
    import torch
    dev = dev or to_device(inp, w.act)
    B, N, H, D, hid = w.batch, w.n_video, w.heads, w.head_dim, w.hidden
    dbg = None
    if debug:
        f32 = dict(dtype=torch.float32, device="cuda")
        dbg = {"o_soft": torch.empty(B, N, H, D, **f32), "o_lin": torch.empty(B, N, H, D, **f32),
               "delta_f32": torch.empty(B, N, hid, **f32), "gates": torch.empty(B, N, 2 * hid, **f32),
               "scales": torch.empty(5, B, H, **f32)}
    y = api.forward(api_layout(w), dev["x"], dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"],
                    dev["w_gs"], dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"],
                    soft=w.soft if w.soft in ("fp8", "fp8_mx") else None, debug=dbg, **kw)
    torch.cuda.synchronize()
    out = {"y": y.float().cpu().numpy().astype(np.float64)}
    if dbg:
        for k, v in dbg.items():
            out[k] = v.cpu().numpy().astype(np.float64)
    return out


def run_oracle(w, inp, tokens=None):
    return oracle.hybrid_forward(inp, oracle_layout(w), tokens=tokens)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    mx = float(err.max() / max(np.abs(ref).max(), 1e-30))
    mean_rel = float(err.sum() / max(np.abs(ref).sum(), 1e-30))
    return mx, mean_rel


def compare(w, g, ref, tokens=None, keys=("y", "delta", "o_s", "o_l", "g"), tol=None):
    """Compare GPU outputs g (full arrays) with oracle outputs ref (at tokens)."""
    tmax, tmean = tol or TOL[w.soft if w.soft == "fp8" else w.act]
    hid = w.hidden
    B = w.batch
    pick = (lambda a: a) if tokens is None else (lambda a: a[:, tokens])
    pairs = {
        "y": (pick(g["y"]), ref["y"]),
        "delta": (pick(g["delta_f32"]), ref["delta"]),
        "o_s": (pick(g["o_soft"]).reshape(B, -1, hid), ref["o_s"].reshape(B, -1, hid)),
        "o_l": (pick(g["o_lin"]).reshape(B, -1, hid), ref["o_l"].reshape(B, -1, hid)),
        "g": (pick(g["gates"]), np.concatenate([ref["g_s"], ref["g_l"]], axis=-1)),
    }
    report = {}
    for k in keys:
        a, b = pairs[k]
        report[k] = errors(a, b)
    bad = {k: v for k, v in report.items() if not (v[0] <= tmax and v[1] <= tmean)}
    return report, bad
