"""The binning statement (oracle/binning.py) pinned at its class boundaries.

Rows with degrees exactly at, below and above both thresholds (short_max, seg_len), with the plan
tables written out by hand from the class definitions: short deg <= short_max, long
short_max < deg <= seg_len (one segment), hub deg > seg_len (ceil(deg / seg_len) segments of seg_len
edges, the last shorter; hub segments first, then long rows, both in row order).  Planted mistakes
in a copy of the module (a strict comparison for <=, a floor for the ceiling, the segment end
off by one, long rows before hubs) must each fail the pin.
"""
import os
import types

import numpy as np
import pytest

import oracle.binning as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SHORT_MAX, SEG_LEN = 4, 10
#            row: 0  1  2  3   4   5   6   7  8
DEGREES = np.array([0, 4, 5, 10, 11, 20, 21, 3, 9])
ROW_PTR = np.concatenate([[0], np.cumsum(DEGREES)]).astype(np.int32)
# edge offsets: row 0 [0,0) 1 [0,4) 2 [4,9) 3 [9,19) 4 [19,30) 5 [30,50) 6 [50,71) 7 [71,74) 8 [74,83)
EXPECT_CLASS = [0, 0, 1, 1, 2, 2, 2, 0, 1]
EXPECT_SEGS = [
    # hub row 4 (deg 11 = seg_len + 1): two segments, 10 + 1
    (4, 19, 29, 0), (4, 29, 30, 1),
    # hub row 5 (deg 20 = 2 seg_len): two full segments
    (5, 30, 40, 2), (5, 40, 50, 3),
    # hub row 6 (deg 21): three segments, 10 + 10 + 1
    (6, 50, 60, 4), (6, 60, 70, 5), (6, 70, 71, 6),
    # long rows (short_max + 1 = 5, seg_len = 10, 9), slot -1
    (2, 4, 9, -1), (3, 9, 19, -1), (8, 74, 83, -1),
]
EXPECT_HUBS = [(4, 0, 2), (5, 2, 2), (6, 4, 3)]


def _pin(mod):
    assert list(mod.classify(ROW_PTR, SHORT_MAX, SEG_LEN)) == EXPECT_CLASS
    segs, hubs, nhs = mod.plan(ROW_PTR, SHORT_MAX, SEG_LEN)
    assert [tuple(int(v) for v in s) for s in segs] == EXPECT_SEGS
    assert [tuple(int(v) for v in h) for h in hubs] == EXPECT_HUBS
    assert nhs == 7


def test_binning_boundaries():
    _pin(B)


def test_binning_degenerate_thresholds():
    """short_max = 0: every row with an edge is binned; seg_len = 1: every row of two or more edges
    is a hub with one segment per edge."""
    assert list(B.classify(ROW_PTR, 0, 1)) == [0, 2, 2, 2, 2, 2, 2, 2, 2]
    segs, hubs, nhs = B.plan(ROW_PTR, 0, 1)
    assert nhs == int(DEGREES[DEGREES > 1].sum())
    assert all(e - b == 1 for _, b, e, _ in segs[:nhs])


MUTANTS = [
    ("short_strict", "if d <= short_max:", "if d < short_max:"),
    ("long_strict", "elif d <= seg_len:", "elif d < seg_len:"),
    ("floor_segments", "n = (e - b + seg_len - 1) // seg_len", "n = (e - b) // seg_len"),
    ("segment_end_off_by_one", "min(e, b + (k + 1) * seg_len)", "min(e, b + (k + 1) * seg_len - 1)"),
    ("hub_segments_reversed", "    n_hub_segs = len(segs)\n", "    n_hub_segs = len(segs)\n    segs.reverse()\n"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_binning_mistake_fails_the_pin(name, old, new):
    src = open(B.__file__).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mod = types.ModuleType(f"binning_{name}")
    exec(compile(src.replace(old, new), f"binning_{name}.py", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        _pin(mod)
