"""Throughput of the hybrid attention layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline] [--block]

One step = one full forward of the layer (softmax branch, state build, scan,
readout, gate GEMM + epilogue, output GEMM + residual) over one batch of
seeded synthetic inputs already resident in HBM.  Prints one JSON line.
With --block a step starts one stage earlier, at the layer input x: the
Q/K/V projection (one GEMM with the fp8 absmax in its epilogue) and then the
layer, and the line carries that metric instead.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from hybrid_softmax_linear_block_amd import api  # noqa: E402
from hybrid_softmax_linear_block_amd.inputs import (WORKLOADS, make_ffn_weights, make_grad_output,  # noqa: E402
                                                    make_inputs, make_projection_weights, sample_tokens)

WORKLOADS_ID = {w.name: i for i, w in WORKLOADS.items()}

METRIC = "hybrid-attn layer Mtokens/s + softmax-branch TFLOP/s (768p-shaped, bf16)"
METRIC_BLOCK = "hybrid-attn layer with its Q/K/V projection Mtokens/s (768p-shaped, bf16)"
METRIC_DIT = "DiT block (Q/K/V projection + hybrid layer + feed-forward) Mtokens/s (768p-shaped, bf16)"
METRIC_TRAIN = "hybrid-attn layer training step (forward keeping its values + backward) Mtokens/s (768p-shaped, bf16)"
METRIC_BLOCK_BWD = ("hybrid-attn layer with its Q/K/V projection, backward (recompute + all gradients) Mtokens/s "
                    "(768p-shaped, bf16)")
METRIC_BWD = "hybrid-attn layer backward (forward recompute + all gradients) Mtokens/s (768p-shaped, bf16)"
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense MFMA TFLOP/s, MI355X published
PEAK_HBM_GBS = 8000.0  # HBM3E, MI355X published
HBM_PEAK_GBS = 8000.0
# source files whose text determines each measured kernel (hashed together)
KERNEL_SOURCES = {"softmax": ("attn_softmax.hip", "attn_tiles.h", "mfma_common.h", "work_items.h"),
                  "softmax_fp8": ("fp8_softmax.hip", "mfma_common.h", "work_items.h")}


def sources_sha256(kernel_key):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel_key]:
        h.update(open(os.path.join(ROOT, "hybrid_softmax_linear_block_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def layout_of(w):
    return api.Layout(w.batch, w.frames, w.tokens_per_frame, w.text_tokens, w.heads, w.head_dim,
                      w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)


def softmax_pairs(w):
    """Visible (query, key) pairs per (batch, head), from the library's tables."""
    _, sc, _, _ = api.layout_tables(layout_of(w))
    n = w.tokens_per_frame
    return int(sum(n * (int(c) * n + w.text_tokens) for c in sc))


def work_counts(w):
    pairs = softmax_pairs(w)
    B, H, D, N, T, L, hid = w.batch, w.heads, w.head_dim, w.n_video, w.frames, w.text_tokens, w.hidden
    soft = 4.0 * D * pairs * B * H
    states = 2.0 * (N + L) * D * (D + 1) * B * H
    readout = 2.0 * N * D * (D + 1) * B * H
    gemm = 2 * (2.0 * B * N * hid * 2 * hid)
    return {"pairs_per_bh": pairs, "softmax_flop": soft, "linear_flop": states + readout, "gemm_flop": gemm,
            "layer_flop": soft + states + readout + gemm}


def stage_work(w, soft, block=False, ffn_hidden=0):
    """Algorithmic work per stage of the bf16 path: FLOP for the MFMA
    kernels, the HBM bytes each kernel must move for the others (inputs read
    once, outputs written once, intermediates in the formats the path uses)."""
    B, H, D, N, T, L, hid = w.batch, w.heads, w.head_dim, w.n_video, w.frames, w.text_tokens, w.hidden
    es = 2
    st = (D * D + D) * 4
    wc = work_counts(w)
    gemm_flop = 2.0 * B * N * hid * 2 * hid
    work = {
        "weights": ("hbm", 2 * 2 * (2 * hid * hid * 2)),
        "softmax": ("mfma", wc["softmax_flop"]),
        "states": ("hbm", 2 * B * (N + L) * hid * es + B * H * (T + 1) * st),
        "scan": ("hbm", B * H * (T + 1) * st + B * H * T * (2 * D * D * 2 + D * 4)),
        # reads q and the combined states, writes O_l (fp16) and the per-head sums of squares
        "readout": ("hbm", B * N * hid * es + B * H * T * (2 * D * D * 2 + D * 4) + B * N * hid * 2 + B * N * H * 4),
        "gate": ("mfma", gemm_flop),
        "out": ("mfma", gemm_flop),
    }
    if soft:
        work["quant"] = ("hbm", (3 * B * N + 2 * B * L) * hid * (es + 1))
    if soft == "fp8_mx":
        # gate and output weights read in bf16, written as codes + exponents;
        # x read in bf16, written as codes + exponents (in the projection's
        # stage when there is one)
        work["weights"] = ("hbm", 2 * (2 * hid * hid) * (2 + 1 + 1.0 / 32)
                           + (0 if block else B * N * hid * (2 + 1 + 1.0 / 32)))
    if block:
        # x [B*N][hid] @ [hid][3 hid]: 2 * B*N * hid * 3 hid
        work["qkv"] = ("mfma", 2.0 * B * N * hid * 3 * hid)
    if ffn_hidden:
        # two GEMMs, [B*N][hid] @ [hid][F] and [B*N][F] @ [F][hid]
        work["ffn"] = ("mfma", 2 * 2.0 * B * N * hid * ffn_hidden)
    return work


def backward_work(w):
    """Algorithmic work of the backward stages: FLOP of the MFMA products
    (softmax: S, dP, dQ in the query-centric kernel and S, dP, dV, dK in the
    key-centric one, 2 D each per visible pair; epilogue: dA' and dx GEMMs;
    weight gradients: the two token-contraction GEMMs) and the forward
    recompute (the forward without its output GEMM)."""
    wc = work_counts(w)
    B, N, hid = w.batch, w.n_video, w.hidden
    gemm = 2.0 * B * N * hid * 2 * hid
    return {"forward": ("mfma", wc["softmax_flop"] + wc["linear_flop"] + gemm),
            "epilogue": ("mfma", 2 * gemm), "wgrad": ("mfma", 2 * gemm),
            "softmax": ("mfma", wc["softmax_flop"] * 14.0 / 4.0)}


def stage_roofline(w, soft, stage_ms, block=False, ffn_hidden=0):
    out = {}
    for k, (bound, amount) in stage_work(w, soft, block, ffn_hidden).items():
        t = stage_ms.get(k, 0.0)
        if t <= 0:
            continue
        if bound == "mfma":
            fp8 = soft and (k == "softmax" or (soft == "fp8_mx" and k in ("gate", "out", "qkv", "ffn")))
            peak = PEAK["fp8" if fp8 else w.act]
            ach = amount / (t * 1e-3) / 1e12
            out[k] = {"bound": "mfma", "algorithmic": amount, "unit": "TFLOP/s", "achieved": round(ach, 2),
                      "peak": peak, "frac": round(ach / peak, 4)}
        else:
            ach = amount / (t * 1e-3) / 1e9
            out[k] = {"bound": "hbm", "algorithmic": amount, "unit": "GB/s", "achieved": round(ach, 1),
                      "peak": PEAK_HBM_GBS, "frac": round(ach / PEAK_HBM_GBS, 4)}
    return out


def describe(w):
    return ("%s: batch %d, %d latent frames x %d tokens/frame, %d heads x dim %d (hidden %d), %d text tokens, "
            "chunk %d frame(s) radius %d, anchors %s, %s%s" % (
                w.name, w.batch, w.frames, w.tokens_per_frame, w.heads, w.head_dim, w.hidden, w.text_tokens,
                w.chunk_frames, w.chunk_radius,
                "/".join(str(a) for a, on in ((0, w.anchor_first), (w.frames - 1, w.anchor_last)) if on) or "none",
                w.act, {"fp8": " (softmax fp8)", "fp8_mx": " (fp8 version: e4m3 softmax branch, MX e4m3 GEMMs)"}.get(
                    w.soft, "")))


def traffic_for(kernel_key, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if the summary
    under profiles/ was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel_key, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != sources_sha256(kernel_key):
        return None
    return rec.get("bytes_per_launch")


def _counter_sum(csv_path, kernel_substr, counter):
    import csv
    tot, disp = 0.0, set()
    for r in csv.DictReader(open(csv_path)):
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            tot += float(r["Counter_Value"])
            disp.add(r["Dispatch_Id"])
    return tot, len(disp)


def write_traffic(pmc_dir, w):
    """HBM bytes per launch of the softmax kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reports for the
    plain 1 GiB copy of --calibrate-copy (runtime copy kernel)."""
    import glob

    def find(sub):
        return glob.glob(os.path.join(pmc_dir, sub, "*counter_collection.csv"))[0]
    fetch, nf = _counter_sum(find("fetch"), "k_attn_bf16", "FETCH_SIZE")
    write, nw = _counter_sum(find("write"), "k_attn_bf16", "WRITE_SIZE")
    cf, ncf = _counter_sum(find("cfetch"), "copyBuffer", "FETCH_SIZE")
    cw, ncw = _counter_sum(find("cwrite"), "copyBuffer", "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024.0
    f_scale = copy_kib * ncf / cf if cf else None
    w_scale = copy_kib * ncw / cw if cw else None
    rd = fetch / nf * 1024 * f_scale
    wr = write / nw * 1024 * w_scale
    rec = {"kernel": "k_attn_bf16_sp", "workload": w.name, "bytes_per_launch": rd + wr,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "sources": list(KERNEL_SOURCES["softmax"]),
           "source_sha256": sources_sha256("softmax"),
           "commands": ["rocprofv3 --pmc FETCH_SIZE --kernel-include-regex k_attn_bf16 --output-format csv "
                        "-d PMC_DIR/fetch -o fetch -- python3 bench.py --workload %d --steps 1 --warmup 0 "
                        "--no-cpu-baseline" % WORKLOADS_ID[w.name],
                        "(same with WRITE_SIZE -> PMC_DIR/write)",
                        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d PMC_DIR/cfetch -o cfetch -- "
                        "python3 bench.py --calibrate-copy",
                        "(same with WRITE_SIZE -> PMC_DIR/cwrite)",
                        "python3 bench.py --workload %d --write-traffic PMC_DIR" % WORKLOADS_ID[w.name]]}
    out = os.path.join(ROOT, "profiles", "traffic_softmax_%s.json" % w.name)
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def host_info():
    """CPU model, usable cores and NumPy's BLAS build (for the oracle timings)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        b = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = "%s %s" % (b.get("name"), b.get("version"))
    except Exception:  # pragma: no cover - older NumPy
        pass
    return {"cpu_model": model, "cores": len(os.sched_getaffinity(0)), "blas": blas}


def oracle_full(w):
    """Wall time of the fp64 oracle over every token of a workload (no
    sampling), in the same units as the bench."""
    import oracle
    from oracle.layout import Layout as OLayout
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    info = host_info()
    ctx = threadpool_limits(limits=info["cores"]) if threadpool_limits else None
    inp = make_inputs(w)
    lay = OLayout(w.batch, w.frames, w.tokens_per_frame, w.text_tokens, w.heads, w.head_dim,
                  w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)
    try:
        t0 = time.perf_counter()
        oracle.hybrid_forward(inp, lay)
        wall = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return dict(info, workload=describe(w), kind="oracle, every token (fp64 NumPy)", wall_s=round(wall, 2),
                value=w.batch * w.n_video / wall / 1e6, unit="Mtokens/s")


def cpu_baseline(w, inp):
    """Time the fp64 oracle on the host on a bounded sample and scale to
    Mtokens/s: the full-state build over all tokens, then the softmax
    branch, readout and epilogue over every token of one query frame per
    distinct key-set size (the work of a frame depends only on that size),
    each scaled by the number of frames of its size.  Timing whole frames
    keeps the oracle's per-frame set-up in the sample at its real share."""
    import oracle
    from oracle.layout import Layout as OLayout, frame_sets
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    lay = OLayout(w.batch, w.frames, w.tokens_per_frame, w.text_tokens, w.heads, w.head_dim,
                  w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)
    sets = frame_sets(w.frames, w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)
    classes = {}
    for f in range(w.frames):
        classes.setdefault(len(sets[f][0]), []).append(f)
    n = w.tokens_per_frame
    timed = []
    try:
        t0 = time.perf_counter()
        st = oracle.linear_states(inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay)
        t_states = time.perf_counter() - t0
        t_frames = 0.0
        for size, frames in sorted(classes.items(), reverse=True):
            f = frames[len(frames) // 2]
            tok = np.arange(f * n, (f + 1) * n)
            t0 = time.perf_counter()
            o_s = oracle.softmax_branch(inp["q"], inp["k"], inp["v"], inp["text_k"], inp["text_v"], lay, tokens=tok)
            o_l = oracle.linear_branch(inp["q"], st, lay, tokens=tok)
            oracle.epilogue(inp["x"][:, tok], o_s, o_l, inp["w_gs"], inp["w_gl"], inp["w_os"], inp["w_ol"],
                            inp["rms_w"])
            dt = time.perf_counter() - t0
            t_frames += dt * len(frames)
            timed.append((f, size, len(frames), dt))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    full = t_states + t_frames
    info = host_info()
    parts = ", ".join("frame %d (%d key frames, stands for %d frames): %.1f s" % t for t in timed)
    return {"value": w.batch * w.n_video / full / 1e6, "unit": "Mtokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": info["cpu_model"], "blas": info["blas"],
            "sample": ("fp64 NumPy oracle: state build over all %d tokens (%.1f s), then softmax branch, readout "
                       "and epilogue over every token of one frame per key-set size (%s), each scaled by the "
                       "number of frames of that size: %.0f s for the whole layer"
                       % (w.n_video, t_states, parts, full)),
            "wall_s": round(t_states + sum(t[3] for t in timed), 2)}


def library_gemms(w, torch, step, api, rounds=6, reps=4):
    """torch (hipBLASLt) on the shapes of the gate GEMM (x [M, hid] @ [hid, 2 hid], bf16) and the output
    GEMM ([M, 2 hid] @ [2 hid, hid], fp16), random normal operands: the plain products (gate, out), and
    each with its epilogue as a library-based layer would run it (gate_epi: sigmoid of the bf16 product
    times a bf16 copy of the branch outputs, to fp16 -- the RMS factors left out; out_epi: addmm with the
    residual as C in fp16, one hipBLASLt call).  Each round enqueues one timed forward of the layer (its
    gate / out stage times, ours_*) and, right behind it on the same stream, one launch of each library
    form, so that both run at the clocks the softmax kernel leaves; alone_* are the plain products, reps
    launches back to back after an idle synchronisation.  Medians over the rounds."""
    M, hid = w.batch * w.n_video, w.heads * w.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    ops = {}
    for name, (k, n, dt) in {"gate": (hid, 2 * hid, torch.bfloat16), "out": (2 * hid, hid, torch.float16)}.items():
        a = torch.randn(M, k, device="cuda", generator=g).to(dt)
        b = (torch.randn(k, n, device="cuda", generator=g) * 0.02).to(dt).contiguous()
        ops[name] = (a, b)
    o = torch.randn(M, 2 * hid, device="cuda", generator=g).to(torch.bfloat16)  # branch outputs [O_s | O_l]
    res16 = torch.randn(M, hid, device="cuda", generator=g).to(torch.float16)  # residual rows
    forms = {
        "gate": lambda: torch.matmul(*ops["gate"]),
        "out": lambda: torch.matmul(*ops["out"]),
        "gate_epi": lambda: (torch.sigmoid(torch.matmul(*ops["gate"])) * o).to(torch.float16),
        "out_epi": lambda: torch.addmm(res16, *ops["out"]),
    }
    for f in forms.values():
        f()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    lib = {k: [] for k in forms}
    alone, ours = {"gate": [], "out": []}, {"gate": [], "out": []}
    for _ in range(rounds):
        torch.cuda.synchronize()
        t = api.StageTimer(last="out")
        step(t)
        e = [ev() for _ in range(len(forms) + 1)]
        e[0].record()
        for i, f in enumerate(forms.values()):
            f()
            e[i + 1].record()
        torch.cuda.synchronize()
        el = t.elapsed_ms()
        t.close()
        for name in ("gate", "out"):
            ours[name].append(el[name])
        for i, name in enumerate(forms):
            lib[name].append(e[i].elapsed_time(e[i + 1]))
        for name in ("gate", "out"):
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                forms[name]()
            e1.record()
            torch.cuda.synchronize()
            alone[name].append(e0.elapsed_time(e1) / reps)
    med = lambda v: round(float(np.median(v)), 4)  # noqa: E731
    res = {name: med(v) for name, v in lib.items()}
    for name in ("gate", "out"):
        res["ours_" + name] = med(ours[name])
        res["alone_" + name] = med(alone[name])
    res["note"] = ("torch (hipBLASLt) on the same shapes and dtypes: gate / out plain products, gate_epi / out_epi "
                   "with their epilogues as separate library calls, launched right behind a forward of the layer on "
                   "its stream; alone_* the plain products, %d launches back to back after an idle sync; ours_* "
                   "are this layer's fused GEMMs with their epilogues in that forward; medians of %d rounds"
                   % (reps, rounds))
    return res


def device_info(torch):
    """Name, CU count and peak shader clock of device 0 (the peaks above are
    MI355X's published figures: 256 CUs at 2.4 GHz)."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    clock_khz = ctypes.c_int(0)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    ok = hip.hipDeviceGetAttribute(ctypes.byref(clock_khz), 5, 0) == 0  # hipDeviceAttributeClockRate
    return {"name": props.name, "arch": props.gcnArchName, "compute_units": props.multi_processor_count,
            "peak_clock_mhz": clock_khz.value / 1000.0 if ok else None,
            "peak_basis": "published MI355X dense peaks (256 CUs, 2.4 GHz)"}


def bench_backward(args, w, lay, dev, torch):
    """Time hyb_attn_backward (forward recompute + every gradient, all weight
    gradients requested) and print one JSON line."""
    if w.act != "bf16" or w.soft != "bf16":
        print("--backward runs the bf16 path", file=sys.stderr)
        sys.exit(2)
    dy = torch.from_numpy(make_grad_output(w)).to("cuda").to(torch.bfloat16)
    ws = torch.empty(api.backward_workspace_size(lay), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lay_args = (lay, dev["x"], dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["w_gs"], dev["w_gl"],
                dev["w_os"], dev["w_ol"], dev["rms_w"])
    saved = y = fws = None
    fwd_timers = []
    if args.train:
        saved = torch.empty(api.saved_size(lay), dtype=torch.uint8, device="cuda")
        fws = torch.empty(api.workspace_size(lay, "bf16"), dtype=torch.uint8, device="cuda")
        y = torch.empty_like(dev["x"])
    if args.block:
        pw = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in make_projection_weights(w).items()}
        ws = torch.empty(api.block_backward_workspace_size(lay), dtype=torch.uint8, device="cuda")
        blk_args = (lay, dev["x"], pw["w_q"], pw["w_k"], pw["w_v"], dev["text_k"], dev["text_v"], dev["w_gs"],
                    dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"], dy)
    else:
        grads = api.backward(*lay_args, dy, workspace=ws, stream=stream)

    def step(timer=None, ftimer=None):
        if args.block:
            api.block_backward(*blk_args, workspace=ws, stream=stream,
                               debug={"stage_events": timer.address} if timer else None)
            return
        if args.train:
            api.forward_train(*lay_args, y=y, saved=saved, workspace=fws, stream=stream,
                              debug={"stage_events": ftimer.address} if ftimer else None)
        api.backward(*lay_args, dy, grads=grads, workspace=ws, stream=stream, saved=saved,
                     debug={"stage_events": timer.address} if timer else None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = [api.StageTimer(api.BWD_STAGES, "forward", "linear") for _ in range(args.steps)]
    if args.train:
        fwd_timers = [api.StageTimer() for _ in range(args.steps)]
    print("bench: timing %d %s steps" % (args.steps, "training" if args.train else "backward"), file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(timers[i], fwd_timers[i] if args.train else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {k: [] for k in api.BWD_STAGES}
    for t in timers:
        for k, v in t.elapsed_ms().items():
            stage[k].append(v)
        t.close()
    stage_ms = {k: float(np.mean(v)) for k, v in stage.items()}
    if args.train:
        fstage = {k: [] for k in api.STAGES}
        for t in fwd_timers:
            for k, v in t.elapsed_ms().items():
                fstage[k].append(v)
            t.close()
        stage_ms = dict({"fwd_" + k: float(np.mean(v)) for k, v in fstage.items() if k not in ("qkv", "ffn")},
                        **{"bwd_" + k: v for k, v in stage_ms.items()})
    ms = wall * 1e3 / args.steps
    work = backward_work(w)
    roof = {}
    for k, (bound, flop) in work.items():
        t = stage_ms.get(("bwd_" if args.train else "") + k, 0.0)
        if t > 0.05:
            ach = flop / (t * 1e-3) / 1e12
            roof[k] = {"bound": bound, "algorithmic": flop, "unit": "TFLOP/s", "achieved": round(ach, 2),
                       "peak": PEAK["bf16"], "frac": round(ach / PEAK["bf16"], 4)}
    out = {
        "metric": METRIC_TRAIN if args.train else (METRIC_BLOCK_BWD if args.block else METRIC_BWD),
        "value": round(w.batch * w.n_video / (ms * 1e-3) / 1e6, 4), "unit": "Mtokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act, "data": "synthetic",
        "config": {"workload": describe(w), "batch": w.batch, "video_tokens": w.n_video,
                   "text_tokens": w.text_tokens, "heads": w.heads, "head_dim": w.head_dim,
                   "parallelism": "none (1 GPU)", "weight_gradients": "all"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_roofline": roof,
        "device": device_info(torch),
        "roofline": dict(roof.get("softmax", {}), kernel="softmax-branch backward (k_attn_bwd_dq + k_attn_bwd_dkv)",
                         traffic=None),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block", action="store_true",
                    help="time the layer with its Q/K/V projection (x -> q, k, v -> y) instead of the layer")
    ap.add_argument("--dit", action="store_true",
                    help="time one DiT block: projection, layer and the feed-forward (4 x hid)")
    ap.add_argument("--fp8-mx", action="store_true",
                    help="the fp8 version: e4m3 softmax branch and MX e4m3 GEMMs (hidden size a multiple of 256)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (forward recompute + every gradient) instead of the forward")
    ap.add_argument("--train", action="store_true",
                    help="time a training step: forward keeping its values, then the backward reading them")
    ap.add_argument("--oracle-full", action="store_true",
                    help="only time the fp64 oracle over every token of --workload (host only) and print JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--library-gemms", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the gate and output GEMM shapes, without "
                         "epilogues, in the same process (reported as library_gemm_ms)")
    ap.add_argument("--write-traffic", metavar="PMC_DIR",
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE passes under PMC_DIR (subdirectories fetch, "
                         "write, cfetch, cwrite) into profiles/traffic_<kernel>_<workload>.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic, WORKLOADS[args.workload])
        return
    if args.oracle_full:
        print(json.dumps(oracle_full(WORKLOADS[args.workload])), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the layer shards by heads; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return
    w = WORKLOADS[args.workload]
    print("bench: generating %s" % w.name, file=sys.stderr, flush=True)
    inp = make_inputs(w)
    dt = torch.float32 if w.act == "f32" else torch.bfloat16
    dev = {k: torch.from_numpy(v).to("cuda").to(dt) for k, v in inp.items()}
    lay = layout_of(w)
    soft = "fp8_mx" if args.fp8_mx else ("fp8" if w.soft == "fp8" else None)
    if args.fp8_mx:
        w = w.with_(soft="fp8_mx")
    if args.backward or args.train:
        bench_backward(args, w, lay, dev, torch)
        return
    ffn_hidden = 4 * w.hidden if args.dit else 0
    if args.dit:
        args.block = True
    if args.block:
        if w.act != "bf16":
            print("--block and --dit run the bf16 path", file=sys.stderr)
            sys.exit(2)
        pw = {k: torch.from_numpy(v).to("cuda").to(dt) for k, v in make_projection_weights(w).items()}
        ws_bytes = api.block_workspace_size(lay, soft)
        if args.dit:
            fw = {k: torch.from_numpy(v).to("cuda").to(dt) for k, v in make_ffn_weights(w).items()}
            ws_bytes = api.dit_block_workspace_size(lay, ffn_hidden, soft)
    else:
        ws_bytes = api.workspace_size(lay, "f32" if w.act == "f32" else "bf16", soft)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(dev["x"])
    stream = torch.cuda.current_stream().cuda_stream

    def step(timer=None):
        dbg = {"stage_events": timer.address} if timer else None
        if args.dit:
            api.dit_block_forward(lay, dev["x"], pw["w_q"], pw["w_k"], pw["w_v"], dev["text_k"], dev["text_v"],
                                  dev["w_gs"], dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"], fw["w_n"],
                                  fw["w_1"], fw["w_2"], soft=soft, z=y, workspace=ws, stream=stream, debug=dbg)
        elif args.block:
            api.block_forward(lay, dev["x"], pw["w_q"], pw["w_k"], pw["w_v"], dev["text_k"], dev["text_v"],
                              dev["w_gs"], dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"], soft=soft, y=y,
                              workspace=ws, stream=stream, debug=dbg)
        else:
            api.forward(lay, dev["x"], dev["q"], dev["k"], dev["v"], dev["text_k"], dev["text_v"], dev["w_gs"],
                        dev["w_gl"], dev["w_os"], dev["w_ol"], dev["rms_w"], soft=soft, y=y, workspace=ws,
                        stream=stream, debug=dbg)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = [api.StageTimer(last="ffn" if args.dit else "out") for _ in range(args.steps)]
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(timers[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {k: [] for k in api.STAGES}
    span = []
    for t in timers:
        for k, v in t.elapsed_ms().items():
            stage[k].append(v)
        span.append(t.span_ms())
    for t in timers:
        t.close()

    def pct(v):
        p10, p50, p90 = np.percentile(np.asarray(v), [10, 50, 90])
        return {"p10": round(float(p10), 4), "p50": round(float(p50), 4), "p90": round(float(p90), 4)}
    stage_ms = {k: float(np.mean(v)) for k, v in stage.items()
                if (args.block or k != "qkv") and (args.dit or k != "ffn")}
    ms = wall * 1e3 / args.steps
    wc = work_counts(w)
    soft_key = "softmax_fp8" if soft else "softmax"
    soft_ms = stage_ms["softmax"]
    soft_tflops = wc["softmax_flop"] / (soft_ms * 1e-3) / 1e12
    peak = PEAK["fp8" if soft else w.act]
    value = w.batch * w.n_video / (ms * 1e-3) / 1e6
    sw = stage_work(w, soft, True, ffn_hidden)
    layer_flop = wc["layer_flop"] + (sw["qkv"][1] if args.block else 0.0) + (sw["ffn"][1] if args.dit else 0.0)
    metric = METRIC_DIT if args.dit else (METRIC_BLOCK if args.block else METRIC)
    if soft == "fp8_mx":
        metric = metric.replace("bf16)", "fp8 version: e4m3 softmax branch, MX e4m3 GEMMs)")
    out = {
        "metric": metric, "value": round(value, 4), "unit": "Mtokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 + e4m3 (MX GEMMs, fp8 softmax)" if soft == "fp8_mx" else w.act,
        "data": "synthetic",
        "config": {"workload": describe(w), "batch": w.batch, "video_tokens": w.n_video,
                   "text_tokens": w.text_tokens, "heads": w.heads, "head_dim": w.head_dim,
                   "parallelism": "none (1 GPU)"},
        "softmax_tflops": round(soft_tflops, 2),
        "layer_tflops": round(layer_flop / (ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "gpu_ms_percentiles": {"forward": pct(span), "softmax": pct(stage["softmax"])},
        "stage_roofline": stage_roofline(w, soft, stage_ms, args.block, ffn_hidden) if w.act != "f32" else None,
        "device": device_info(torch),
        "roofline": {"kernel": "k_attn_bf16_sp (softmax branch)" if not soft else "softmax branch fp8",
                     "bound": "mfma", "achieved": round(soft_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(soft_tflops / peak, 4), "traffic": traffic_for(soft_key, w.name),
                     "flop_per_launch": wc["softmax_flop"]},
    }
    if args.library_gemms and w.act != "f32" and not (args.block or args.dit):
        out["library_gemm_ms"] = library_gemms(w, torch, step, api)
    if not args.no_cpu_baseline and w.act != "f32":
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
