"""Plain CPU statement of the degree-binning plan -- TEST INFRASTRUCTURE ONLY.

The GPU binner must reproduce these integers exactly.  The pages size their
per-row work by a host-computed maximum degree (POPCORNBENCH l2_p37, the
passages on copying row_ptr to the host to find max_degree); the binning below
replaces that with three degree classes computed once per graph:

* short: deg <= short_max                 -> one lane group per row
* long:  short_max < deg <= seg_len       -> one workgroup per row (one segment)
* hub:   deg > max(short_max, seg_len)    -> split into ceil(deg / seg_len) segments
                                             of seg_len edges (the last one shorter)

Segment table order: every hub segment first (hub rows in increasing row id,
segments in edge order), then every long row (increasing row id).  A hub
segment's partial-state slot is its index in the table; a long row has slot -1.
Hub table: (row, first segment, number of segments) in increasing row id.
"""
from __future__ import annotations

import numpy as np


def classify(row_ptr: np.ndarray, short_max: int, seg_len: int) -> np.ndarray:
    """0 = short, 1 = long, 2 = hub, per row."""
    deg = np.diff(np.asarray(row_ptr, dtype=np.int64))
    cls = np.zeros(deg.size, dtype=np.int32)
    for i, d in enumerate(deg):
        if d <= short_max:
            cls[i] = 0
        elif d <= seg_len:
            cls[i] = 1
        else:
            cls[i] = 2
    return cls


def plan(row_ptr: np.ndarray, short_max: int, seg_len: int):
    """Returns (segments int32 [S,4] = (row, e_begin, e_end, slot), hubs int32 [Hb,3], n_hub_segments)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    cls = classify(row_ptr, short_max, seg_len)
    segs = []
    hubs = []
    for i in np.flatnonzero(cls == 2):
        b, e = int(row_ptr[i]), int(row_ptr[i + 1])
        n = (e - b + seg_len - 1) // seg_len
        hubs.append((int(i), len(segs), n))
        for k in range(n):
            segs.append((int(i), b + k * seg_len, min(e, b + (k + 1) * seg_len), len(segs)))
    n_hub_segs = len(segs)
    for i in np.flatnonzero(cls == 1):
        segs.append((int(i), int(row_ptr[i]), int(row_ptr[i + 1]), -1))
    seg_arr = np.array(segs, dtype=np.int32).reshape(-1, 4)
    hub_arr = np.array(hubs, dtype=np.int32).reshape(-1, 3)
    return seg_arr, hub_arr, n_hub_segs
