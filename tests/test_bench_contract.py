"""The bench's algorithmic work counts (the numerator of every roofline
figure it prints) against an independent count, and its one-GPU contract.
Host only."""
import os
import subprocess
import sys

import numpy as np

import bench
from hybrid_softmax_linear_block_amd.inputs import WORKLOADS
from oracle.layout import frame_sets

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _pairs_by_sets(w):
    """Visible (query, key) pairs per (batch, head) from the oracle's frame
    sets: each query of frame f sees n keys per frame of S(f) plus the text."""
    sets = frame_sets(w.frames, w.chunk_frames, w.chunk_radius, w.anchor_first, w.anchor_last)
    n = w.tokens_per_frame
    return sum(n * (len(sets[f][0]) * n + w.text_tokens) for f in range(w.frames))


def test_pairs_match_the_frame_sets():
    for wid in (1, 2, 3, 4, 5):
        w = WORKLOADS[wid]
        assert bench.softmax_pairs(w) == _pairs_by_sets(w), w.name


def test_768p_counts():
    """768p: 1.5429e9 visible pairs per (b, h), 25,510 keys per query on
    average, 4 D pairs B H = 1.8959e13 softmax FLOP, GEMMs 2 x 2 M hid 2 hid."""
    w = WORKLOADS[3]
    wc = bench.work_counts(w)
    assert abs(wc["pairs_per_bh"] / 1.5429e9 - 1) < 1e-4
    assert round(wc["pairs_per_bh"] / w.n_video) == 25510
    assert abs(wc["softmax_flop"] / 1.8959e13 - 1) < 1e-4
    assert wc["gemm_flop"] == 4.0 * 60480 * 3072 * 6144
    # the per-frame window with anchors: frame 7 sees frames {0, 6, 7, 8, 14}
    sets = frame_sets(15, 1, 1, True, True)
    assert sorted(sets[7][0]) == [0, 6, 7, 8, 14]


def test_backward_work_is_14_over_4_of_the_forward_softmax():
    w = WORKLOADS[3]
    bw = bench.backward_work(w)
    assert np.isclose(bw["softmax"][1], bench.work_counts(w)["softmax_flop"] * 14.0 / 4.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
