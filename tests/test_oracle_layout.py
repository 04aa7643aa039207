"""Pins of the oracle's frame sets (CPU only)."""
import itertools
import os

import pytest

import oracle
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_frame7():
    pins.pin_worked_example(os.path.join(GOLDEN, "worked_example_frame7.txt"))


def test_chunked_hand_written_sets():
    pins.pin_worked_example(os.path.join(GOLDEN, "chunked_T31.txt"))


def test_closed_form_per_frame_window():
    # C=1, R=1, T=15, anchors 0/14: interior f in 2..12 keeps {0, f-1, f, f+1, 14},
    # forward [1, f-2], backward [f+2, 13]; the anchors see every frame.
    sets = oracle.frame_sets(15, 1, 1)
    for f in range(2, 13):
        assert sets[f] == ({0, f - 1, f, f + 1, 14}, set(range(1, f - 1)), set(range(f + 2, 14)))
    assert sets[1] == ({0, 1, 2, 14}, set(), set(range(3, 14)))
    assert sets[13] == ({0, 12, 13, 14}, set(range(1, 12)), set())
    for f in (0, 14):
        assert sets[f] == (set(range(15)), set(), set())


@pytest.mark.parametrize("af,al", [(1, 1), (1, 0), (0, 1), (0, 0)])
def test_partition_invariant(af, al):
    # every frame is in exactly one of S(f), F(f), B(f); F lies wholly before
    # the query's window and B wholly after it
    for T, C, R in itertools.product(range(1, 34), range(1, 7), range(0, 4)):
        sets = oracle.frame_sets(T, C, R, af, al)
        for f, (S, F, B) in enumerate(sets):
            assert S | F | B == set(range(T))
            assert not (S & F) and not (S & B) and not (F & B)
            assert f in S
            win = S - ({0} if af else set()) - ({T - 1} if al else set())
            if F and win:
                assert max(F) < min(win)
            if B and win:
                assert min(B) > max(win)


def test_tables_format():
    sf, sc, fw, bw = oracle.tables(15, 1, 1)
    assert sf[7] == [0, 6, 7, 8, 14] + [-1] * 10
    assert sc[7] == 5 and fw[7] == [1, 6] and bw[7] == [9, 14]
    assert sf[0] == list(range(15)) and fw[0] == [0, 0] and bw[0] == [0, 0]
    assert fw[1] == [0, 0] and bw[13] == [0, 0]


def test_degenerate_layouts():
    assert oracle.frame_sets(1, 1, 1) == [({0}, set(), set())]
    assert oracle.frame_sets(2, 1, 1) == [({0, 1}, set(), set()), ({0, 1}, set(), set())]
    # no anchors, radius 0: each frame alone in softmax, everything else linear
    s = oracle.frame_sets(4, 1, 0, 0, 0)
    assert s[2] == ({2}, {0, 1}, {3})
    with pytest.raises(ValueError):
        oracle.frame_sets(0, 1, 1)
