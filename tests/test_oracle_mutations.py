"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that at least one pin catches each.  Shows the pins are not vacuous."""
import math
import os

import numpy as np
import pytest

import oracle
import oracle.hybrid as H
import oracle.layout as LY
from oracle.layout import Layout
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAY = Layout(1, 7, 3, 4, 2, 4)
LAYC = Layout(1, 9, 2, 3, 1, 3, chunk_frames=2)


def _all_pins():
    pins.pin_worked_example(os.path.join(GOLDEN, "worked_example_frame7.txt"))
    pins.pin_worked_example(os.path.join(GOLDEN, "chunked_T31.txt"))
    for lay in (LAY, LAYC):
        pins.pin_text_once(lay, 1)
        pins.pin_softmax_bruteforce(lay, 2)
        pins.pin_linear_bruteforce(lay, 3)
    pins.pin_sdpa(Layout(1, 5, 3, 2, 1, 4, chunk_radius=5), 4)
    pins.pin_onehot_gate()
    pins.pin_onehot_out()
    pins.pin_rms_scope()


def test_pins_pass_on_unmodified_oracle():
    _all_pins()


def _full_text_each_side(states, lay):
    S, z, ST, zT = states
    Sf, zf, Sb, zb = ORIG_DIR(states, lay)
    return Sf + 0.5 * ST[:, :, None], zf + 0.5 * zT[:, :, None], Sb + 0.5 * ST[:, :, None], zb + 0.5 * zT[:, :, None]


def _window_in_forward(states, lay):
    S, z, ST, zT = states
    Sf, zf, Sb, zb = ORIG_DIR(states, lay)
    Sf = Sf.copy()
    zf = zf.copy()
    for f in range(1, lay.frames):
        Sf[:, :, f] += S[:, :, f - 1]
        zf[:, :, f] += z[:, :, f - 1]
    return Sf, zf, Sb, zb


ORIG_DIR = H.directional_states
ORIG_SOFT = H.softmax_branch
ORIG_EPI = H.epilogue
ORIG_SETS = LY.frame_sets


def _epi_transposed(x, o_s, o_l, w_gs, w_gl, w_os, w_ol, rms_w, eps=1e-6):
    return ORIG_EPI(x, o_s, o_l, np.asarray(w_gs).T, np.asarray(w_gl).T, np.asarray(w_os).T,
                    np.asarray(w_ol).T, rms_w, eps)


def _epi_rms_per_head(x, o_s, o_l, w_gs, w_gl, w_os, w_ol, rms_w, eps=1e-6):
    o = np.asarray(o_l, np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    o2 = o / np.sqrt(ms + eps) * np.sqrt(np.mean(ms, axis=-2, keepdims=True) + eps)
    return ORIG_EPI(x, o_s, o2, w_gs, w_gl, w_os, w_ol, rms_w, eps)


def _sets_radius_plus_one(T, C, R, af=True, al=True):
    return ORIG_SETS(T, C, R + 1, af, al)


def _phi_no_plus_one(u):
    u = np.asarray(u, np.float64)
    return np.where(u > 0, u, np.exp(np.minimum(u, 0.0)) - 1.0)


def _soft_unscaled(q, k, v, tk, tv, lay, scale=None, tokens=None):
    return ORIG_SOFT(q, k, v, tk, tv, lay, scale=1.0, tokens=tokens)


def _soft_no_text(q, k, v, tk, tv, lay, scale=None, tokens=None):
    return ORIG_SOFT(q, k, v, tk[:, :0], tv[:, :0], lay, scale=scale, tokens=tokens)


MUTANTS = {
    "text added in full to both states": [(H, "directional_states", _full_text_each_side)],
    "window frame leaks into forward state": [(H, "directional_states", _window_in_forward)],
    "weights used transposed": [(H, "epilogue", _epi_transposed), (oracle, "epilogue", _epi_transposed)],
    "RMSNorm per head": [(H, "epilogue", _epi_rms_per_head), (oracle, "epilogue", _epi_rms_per_head)],
    "window radius off by one": [(LY, "frame_sets", _sets_radius_plus_one), (H, "frame_sets", _sets_radius_plus_one),
                                 (oracle, "frame_sets", _sets_radius_plus_one)],
    "phi = elu (no +1)": [(H, "phi", _phi_no_plus_one)],
    "softmax without 1/sqrt(D)": [(H, "softmax_branch", _soft_unscaled), (oracle, "softmax_branch", _soft_unscaled)],
    "softmax drops text keys": [(H, "softmax_branch", _soft_no_text), (oracle, "softmax_branch", _soft_no_text)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, fn)
    with pytest.raises(AssertionError):
        _all_pins()
