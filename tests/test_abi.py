"""C-ABI checks that need no GPU: the library loads, exports every function that
include/gat.h declares, the ctypes mirror of gat_plan matches, and every
host-side argument check returns its status before anything touches the device.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
import oracle.binning as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gat.h")

OK, NULL, SIZE, UNSUP, WS, ARGS, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6, 7


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gat.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return gat.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gat_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("gat_sddmm", "gat_edge_softmax", "gat_aggregate", "gat_fused_layer", "gat_plan_build"):
        assert op in names


def test_library_exports_every_declared_symbol(L):
    nm = subprocess.run(["nm", "-D", "--defined-only", gat.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (gat_\w+)$", nm.stdout, flags=re.M))
    declared = set(declared_functions())
    assert declared <= exported, f"missing exports: {declared - exported}"
    assert set(gat.EXPORTED) == declared
    for name in declared:
        assert hasattr(L, name)


def test_plan_struct_layout(L):
    assert L.gat_plan_sizeof() == ctypes.sizeof(gat.GatPlanStruct)


def test_status_strings(L):
    for s in range(8):
        assert L.gat_status_str(s) and L.gat_status_str(s) != b"unknown status"
    assert L.gat_status_str(99) == b"unknown status"


def test_supported_shapes(L):
    ok = [(h, d) for h in (1, 2, 4, 8, 16) for d in (16, 32, 64, 128) if h * d <= 1024]
    for h in range(0, 20):
        for d in (0, 8, 16, 24, 32, 64, 128, 256):
            assert L.gat_shape_supported(h, d) == int((h, d) in ok)


def test_workspace_bytes(L):
    assert L.gat_plan_workspace_bytes(-1, 10, 4, 64, -1, 0) == 0
    assert L.gat_plan_workspace_bytes(10, 2**31, 4, 64, -1, 0) == 0
    assert L.gat_plan_workspace_bytes(10, 10, 3, 64, -1, 0) == 0
    a = L.gat_plan_workspace_bytes(2**20, 2**24, 4, 64, -1, 0)
    b = L.gat_plan_workspace_bytes(2**20, 2**24, 4, 64, 0, 1)
    assert 0 < a < b and a % 256 == 0
    assert L.gat_plan_workspace_bytes(0, 0, 1, 16, -1, 0) > 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails a host check first


def test_sddmm_host_checks(L):
    f = L.gat_sddmm
    assert f(FAKE, FAKE, -1, FAKE, 4, FAKE, 4, 0, 1, 64, 1.0, FAKE, None) == SIZE
    assert f(FAKE, FAKE, 10, FAKE, 2**31, FAKE, 4, 0, 1, 64, 1.0, FAKE, None) == SIZE
    assert f(FAKE, FAKE, 10, FAKE, 4, FAKE, 4, 0, 3, 64, 1.0, FAKE, None) == UNSUP
    assert f(FAKE, FAKE, 10, FAKE, 4, FAKE, 4, 0, 16, 128, 1.0, FAKE, None) == UNSUP
    assert f(FAKE, FAKE, 10, FAKE, 4, FAKE, 4, 7, 1, 64, 1.0, FAKE, None) == UNSUP
    assert f(None, FAKE, 10, FAKE, 4, FAKE, 4, 0, 1, 64, 1.0, FAKE, None) == NULL
    assert f(FAKE, FAKE, 10, FAKE, 4, FAKE, 4, 0, 1, 64, 1.0, None, None) == NULL
    assert f(FAKE, FAKE, 10, FAKE, 0, FAKE, 4, 0, 1, 64, 1.0, FAKE, None) == ARGS
    assert f(None, None, 0, None, 0, None, 0, 0, 1, 64, 1.0, None, None) == OK   # nothing to do


def test_softmax_host_checks(L):
    f = L.gat_edge_softmax
    assert f(FAKE, -1, 5, 1, FAKE, FAKE, None, None) == SIZE
    assert f(FAKE, 4, 5, 3, FAKE, FAKE, None, None) == UNSUP
    assert f(None, 4, 5, 1, FAKE, FAKE, None, None) == NULL
    assert f(FAKE, 4, 5, 1, None, FAKE, None, None) == NULL
    assert f(None, 0, 0, 1, None, None, None, None) == OK
    bad = gat.GatPlanStruct()   # magic not set
    assert f(FAKE, 4, 5, 1, FAKE, FAKE, ctypes.byref(bad), None) == ARGS


def test_aggregate_host_checks(L):
    f = L.gat_aggregate
    assert f(FAKE, FAKE, 4, 4, -2, FAKE, FAKE, 0, 1, 64, FAKE, None, None) == SIZE
    assert f(FAKE, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 48, FAKE, None, None) == UNSUP
    assert f(FAKE, FAKE, 4, 4, 5, FAKE, FAKE, 2, 1, 64, FAKE, None, None) == UNSUP
    assert f(None, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 64, FAKE, None, None) == NULL
    assert f(FAKE, FAKE, 4, 4, 5, None, FAKE, 0, 1, 64, FAKE, None, None) == NULL
    assert f(FAKE, FAKE, 4, 0, 5, FAKE, FAKE, 0, 1, 64, FAKE, None, None) == ARGS
    assert f(None, None, 0, 0, 0, None, None, 0, 1, 64, None, None, None) == OK


def test_fused_layer_host_checks(L):
    f = L.gat_fused_layer
    args = lambda sc, q, k: (FAKE, FAKE, 4, 4, 5, 4, 64, 0, sc, q, k, 1.0, FAKE, FAKE, None, None)  # noqa: E731
    assert f(*args(FAKE, FAKE, FAKE)) == ARGS      # both scores and q,k
    assert f(*args(None, None, None)) == ARGS      # neither
    assert f(*args(None, FAKE, None)) == ARGS      # q without k
    assert f(*args(None, None, FAKE)) == ARGS      # k without q
    assert f(FAKE, FAKE, 4, 4, 5, 4, 64, 0, FAKE, None, None, 1.0, None, FAKE, None, None) == NULL   # v missing
    assert f(FAKE, FAKE, 4, 4, 5, 5, 64, 0, FAKE, None, None, 1.0, FAKE, FAKE, None, None) == UNSUP
    assert f(FAKE, FAKE, -4, 4, 5, 4, 64, 0, FAKE, None, None, 1.0, FAKE, FAKE, None, None) == SIZE


def test_noalloc_host_checks(L):
    """The allocation-free fused layer: the same argument checks as gat_fused_layer, and a graph
    whose plan exceeds the library's fixed array is refused before anything is enqueued."""
    f = L.gat_fused_layer_noalloc
    args = lambda sc, q, k: (FAKE, FAKE, 4, 4, 5, 4, 64, 0, sc, q, k, 1.0, FAKE, FAKE, None)  # noqa: E731
    assert f(*args(FAKE, FAKE, FAKE)) == ARGS
    assert f(*args(None, None, None)) == ARGS
    assert f(*args(None, FAKE, None)) == ARGS
    assert f(FAKE, FAKE, 4, 4, 5, 4, 64, 0, FAKE, None, None, 1.0, None, FAKE, None) == NULL
    assert f(FAKE, FAKE, 4, 4, 5, 5, 64, 0, FAKE, None, None, 1.0, FAKE, FAKE, None) == UNSUP
    assert f(FAKE, FAKE, -4, 4, 5, 4, 64, 0, FAKE, None, None, 1.0, FAKE, FAKE, None) == SIZE
    assert f(None, None, 0, 0, 0, 4, 64, 0, None, None, None, 1.0, None, None, None) == OK
    # 2^22 rows, 2^26 edges, 8 x 16: the plan needs ~94 MB, the array holds 64 MiB
    need = L.gat_fused_layer_noalloc_bytes(2**22, 2**26, 8, 16)
    assert need > gat.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, FAKE, 2**22, 2**22, 2**26, 8, 16, 0, FAKE, None, None, 1.0, FAKE, FAKE, None) == SCRATCH
    # the metric workload (2^20 rows, 2^24 edges, 4 x 64) fits, and the sizes are the planned call's
    need4 = L.gat_fused_layer_noalloc_bytes(2**20, 2**24, 4, 64)
    assert 0 < need4 <= gat.NOALLOC_SCRATCH_BYTES
    assert need4 == L.gat_plan_workspace_bytes(2**20, 2**24, 4, 64, -1, 0)
    assert L.gat_fused_layer_noalloc_bytes(-1, 5, 4, 64) == 0
    assert L.gat_fused_layer_noalloc_bytes(4, 5, 3, 64) == 0


def test_sddmm_backward_host_checks(L):
    """COO SDDMM backward: every argument check fails on the host, before anything is enqueued."""
    f, wsb = L.gat_sddmm_backward, L.gat_sddmm_backward_workspace_bytes
    need = wsb(16384, 1024, 768, 1, 128)
    # at least: the two radix key/value buffers, the grouping's columns and the scaled gradient
    assert need >= 16384 * 4 * 5 + 16384 * 1 * 4
    assert wsb(-1, 4, 4, 1, 64) == 0 and wsb(5, 2**31, 4, 1, 64) == 0 and wsb(5, 4, 4, 3, 64) == 0
    assert wsb(0, 0, 0, 1, 64) > 0

    def call(E=10, ns=4, nd=4, dt=0, H=1, D=64, src=FAKE, dst=FAKE, sf=FAKE, df=FAKE, g=FAKE, ds=FAKE, dd=FAKE,
             ws=FAKE, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = wsb(max(E, 0), max(ns, 0), max(nd, 0), H, D) if wsb(E, ns, nd, H, D) else 1 << 30
        return f(src, dst, E, sf, ns, df, nd, dt, H, D, 1.0, g, ds, dd, ws, ws_bytes, None)

    assert call(E=-1) == SIZE and call(ns=2**31) == SIZE and call(nd=-3) == SIZE
    assert call(H=3) == UNSUP and call(D=48) == UNSUP and call(H=16, D=128) == UNSUP and call(dt=7) == UNSUP
    assert call(ws=None) == NULL
    assert call(ws=ctypes.c_void_p(0x1010)) == ARGS                 # not 256-byte aligned
    assert call(ws_bytes=wsb(10, 4, 4, 1, 64) - 1) == WS
    assert call(ns=0) == ARGS and call(nd=0) == ARGS                # an edge needs both endpoints
    assert call(src=None) == NULL and call(dst=None) == NULL and call(g=None) == NULL
    assert call(df=None) == NULL                                    # d_src gathers dst_feat
    assert call(sf=None) == NULL                                    # d_dst gathers src_feat
    # nothing asked for, or no rows on either side: nothing to enqueue
    assert call(E=0, ns=0, nd=0, src=None, dst=None, g=None) == OK
    assert call(E=0, ds=None, dd=None, src=None, dst=None, g=None, sf=None, df=None) == OK


def test_plan_refused_for_another_row_ptr(L):
    """A plan is tied to the row_ptr array it was built from: a call with another array of the same
    sizes is refused on the host (it would leave the rows the plan does not cover unwritten)."""
    p = gat.GatPlanStruct()
    p.magic, p.ws, p.n_rows, p.n_edges = 0x47415450, 0x2000, 4, 5
    p.state_floats, p.row_ptr = 4 * 66, 0x3000
    other = ctypes.c_void_p(0x4000)
    assert L.gat_edge_softmax(other, 4, 5, 1, FAKE, FAKE, ctypes.byref(p), None) == WS
    assert L.gat_aggregate(other, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 64, FAKE, ctypes.byref(p), None) == WS
    assert L.gat_fused_layer(other, FAKE, 4, 4, 5, 4, 64, 0, FAKE, None, None, 1.0, FAKE, FAKE,
                             ctypes.byref(p), None) == WS
    assert L.gat_edge_softmax_backward(other, 4, 5, 1, FAKE, FAKE, FAKE, ctypes.byref(p), None) == WS


def test_plan_build_host_checks(L):
    f = L.gat_plan_build
    p = gat.GatPlanStruct()
    need = L.gat_plan_workspace_bytes(100, 1000, 4, 64, -1, 0)
    assert f(FAKE, 100, 1000, 4, 64, -1, 0, FAKE, need, None, None) == NULL
    assert f(None, 100, 1000, 4, 64, -1, 0, FAKE, need, ctypes.byref(p), None) == NULL
    assert f(FAKE, 100, 1000, 4, 64, -1, 0, ctypes.c_void_p(0x1010), need, ctypes.byref(p), None) == ARGS
    assert f(FAKE, 100, 1000, 4, 64, -1, 0, FAKE, need - 1, ctypes.byref(p), None) == WS
    assert f(FAKE, 100, 1000, 5, 64, -1, 0, FAKE, need, ctypes.byref(p), None) == UNSUP
    assert f(FAKE, -100, 1000, 4, 64, -1, 0, FAKE, need, ctypes.byref(p), None) == SIZE


def test_binning_reference_tiles_rows():
    """The CPU binning statement: classes partition the rows; hub segments tile each hub row once."""
    r = np.random.default_rng(0)
    deg = np.concatenate([r.integers(0, 40, 500), [5000, 2049, 2048, 33, 32, 0, 12000]])
    rp = G.row_ptr_from_degrees(deg)
    for short_max, seg_len in [(32, 2048), (0, 1), (0, 7), (100, 64), (2**31 - 1, 2048)]:
        segs, hubs, nhs = B.plan(rp, short_max, seg_len)
        cls = B.classify(rp, short_max, seg_len)
        covered = np.zeros(rp[-1], np.int32)
        for row, b, e, slot in segs:
            assert rp[row] <= b < e <= rp[row + 1] and e - b <= max(seg_len, short_max + 1, 1) + seg_len
            covered[b:e] += 1
        nonshort = np.flatnonzero(cls > 0)
        for i in nonshort:
            assert np.all(covered[rp[i]:rp[i + 1]] == 1)
        assert covered.sum() == sum(deg[i] for i in nonshort)
        assert nhs == sum(-(-deg[i] // seg_len) for i in np.flatnonzero(cls == 2))
        assert np.all(segs[:nhs, 3] == np.arange(nhs)) and np.all(segs[nhs:, 3] == -1)


def test_csc_struct_layout_and_workspace(L):
    assert L.gat_csc_sizeof() == ctypes.sizeof(gat.GatCscStruct)
    assert L.gat_csc_workspace_bytes(-1, 4, 4, 4, 64) == 0
    assert L.gat_csc_workspace_bytes(4, 4, 2**31, 4, 64) == 0
    assert L.gat_csc_workspace_bytes(4, 4, 4, 3, 64) == 0
    a = L.gat_csc_workspace_bytes(2**20, 2**20, 2**24, 4, 64)
    assert a > 6 * 4 * 2**24 and a % 256 == 0
    assert L.gat_csc_workspace_bytes(0, 0, 0, 1, 16) > 0
    assert L.gat_layer_backward_workspace_bytes(-1, 4) == 0
    assert L.gat_layer_backward_workspace_bytes(4, 3) == 0
    assert L.gat_layer_backward_workspace_bytes(2**24, 4) >= 3 * 4 * 4 * 2**24
    assert L.gat_layer_backward_workspace_bytes(0, 4) > 0


def test_csc_build_host_checks(L):
    f = L.gat_csc_build
    c = gat.GatCscStruct()
    need = L.gat_csc_workspace_bytes(100, 80, 1000, 4, 64)
    assert f(FAKE, FAKE, 100, 80, 1000, 4, 64, FAKE, need, None, None) == NULL
    assert f(None, FAKE, 100, 80, 1000, 4, 64, FAKE, need, ctypes.byref(c), None) == NULL
    assert f(FAKE, None, 100, 80, 1000, 4, 64, FAKE, need, ctypes.byref(c), None) == NULL
    assert f(FAKE, FAKE, 100, 0, 1000, 4, 64, FAKE, need, ctypes.byref(c), None) == ARGS
    assert f(FAKE, FAKE, 100, 80, 1000, 4, 64, ctypes.c_void_p(0x1010), need, ctypes.byref(c), None) == ARGS
    assert f(FAKE, FAKE, 100, 80, 1000, 4, 64, FAKE, need - 1, ctypes.byref(c), None) == WS
    assert f(FAKE, FAKE, 100, 80, 1000, 3, 64, FAKE, need, ctypes.byref(c), None) == UNSUP
    assert f(FAKE, FAKE, 100, -80, 1000, 4, 64, FAKE, need, ctypes.byref(c), None) == SIZE


def test_backward_host_checks(L):
    bad_plan, bad_csc = gat.GatPlanStruct(), gat.GatCscStruct()   # magic not set
    f = L.gat_edge_softmax_backward
    assert f(FAKE, -1, 5, 1, FAKE, FAKE, FAKE, None, None) == SIZE
    assert f(FAKE, 4, 5, 3, FAKE, FAKE, FAKE, None, None) == UNSUP
    assert f(FAKE, 4, 5, 1, None, FAKE, FAKE, None, None) == NULL
    assert f(FAKE, 4, 5, 1, FAKE, FAKE, None, None, None) == NULL
    assert f(FAKE, 4, 5, 1, FAKE, FAKE, FAKE, ctypes.byref(bad_plan), None) == ARGS
    assert f(None, 0, 0, 1, None, None, None, None, None) == OK
    g = L.gat_aggregate_backward
    assert g(FAKE, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 64, FAKE, FAKE, FAKE, None, None) == NULL        # no csc
    assert g(FAKE, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 64, FAKE, FAKE, FAKE, ctypes.byref(bad_csc), None) == ARGS
    assert g(FAKE, FAKE, 4, 4, 5, FAKE, FAKE, 0, 1, 48, FAKE, FAKE, FAKE, ctypes.byref(bad_csc), None) == UNSUP
    assert g(FAKE, FAKE, 4, 4, -5, FAKE, FAKE, 0, 1, 64, FAKE, FAKE, FAKE, ctypes.byref(bad_csc), None) == SIZE
    h = L.gat_fused_layer_backward

    def hargs(sc, q, k, plan, csc, heads=4):
        return (FAKE, FAKE, 4, 4, 5, heads, 64, 0, sc, q, k, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                plan, csc, FAKE, 1 << 20, None)
    pr, cr = ctypes.byref(bad_plan), ctypes.byref(bad_csc)
    assert h(*hargs(FAKE, FAKE, FAKE, pr, cr)) == ARGS          # both modes
    assert h(*hargs(None, None, None, pr, cr)) == ARGS          # neither
    assert h(*hargs(FAKE, None, None, None, cr)) == NULL        # plan required
    assert h(*hargs(FAKE, None, None, pr, None)) == NULL        # csc required
    assert h(*hargs(FAKE, None, None, pr, cr)) == ARGS          # plan not built
    assert h(*hargs(FAKE, None, None, pr, cr, heads=3)) == UNSUP


def test_batch_csr_host_checks(L):
    f = L.gat_batch_csr
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 5, FAKE, FAKE, None) == SIZE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, -4, 5, FAKE, FAKE, None) == SIZE
    assert f(None, FAKE, FAKE, FAKE, FAKE, 2, 4, 5, FAKE, FAKE, None) == NULL
    assert f(FAKE, None, FAKE, FAKE, FAKE, 2, 4, 5, FAKE, FAKE, None) == NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 5, None, FAKE, None) == NULL


def test_block_diagonal_reference():
    """The numpy batch statement: each graph's rows keep their degrees and shifted sources."""
    r = np.random.default_rng(3)
    gs = [G.random_csr(n, ns, 5, r) for n, ns in [(4, 3), (0, 2), (6, 1), (3, 0 + 5)]]
    gs.append(G.csr_from_degrees(np.zeros(3, int), 4, r))
    bd = G.block_diagonal(gs)
    assert bd.n_rows == sum(g.n_rows for g in gs) and bd.n_src == sum(g.n_src for g in gs)
    assert np.array_equal(bd.degrees(), np.concatenate([g.degrees() for g in gs]))
    lrp, lcol, ro, eo, so = G.batch_arrays(gs)
    for b, g in enumerate(gs):
        assert np.array_equal(bd.col_idx[eo[b]:eo[b + 1]] - so[b], g.col_idx)
        assert np.array_equal(bd.row_ptr[ro[b]:ro[b + 1] + 1] - eo[b], g.row_ptr)
        assert np.array_equal(lrp[ro[b] + b:ro[b + 1] + b + 1], g.row_ptr)


def test_relation_block_host_checks(L):
    f = L.gat_relation_block
    args = lambda B, N, D, H, P, nodes=FAKE, out=FAKE: (nodes, FAKE, FAKE, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE,  # noqa: E731
                                                        FAKE, FAKE, FAKE, FAKE, B, N, D, H, P, out, None)
    assert f(*args(-1, 24, 96, 4, 16)) == SIZE
    assert f(*args(4, 24, 96, 5, 16)) == UNSUP
    assert f(*args(4, 64, 128, 8, 16)) == UNSUP
    assert f(*args(4, 24, 96, 4, 0)) == UNSUP
    assert f(*args(4, 24, 96, 4, 16, nodes=None)) == NULL
    assert f(*args(4, 24, 96, 4, 16, out=ctypes.c_void_p(0x1004))) == ARGS
    assert f(*args(0, 24, 96, 4, 16, nodes=None, out=None)) == OK
    up = lambda v: (v + 3) // 4 * 4  # noqa: E731
    assert L.gat_relation_block_lds_bytes(24, 96, 4, 16) == 4 * (up(24 * 96) + 3 * up(24 * 97) + up(4 * 576) + up(576)
                                                                 + up(16 * 16 + 16 + 64 + 4) + 2 * 16 * 100)
    assert L.gat_relation_block_lds_bytes(4, 260, 4, 16) == 0
    assert L.gat_relation_block_lds_bytes(24, 96, 4, 65) == 0


def test_linear_host_checks(L):
    f = L.gat_linear
    outs = (ctypes.c_void_p * 3)(0x1000, 0x2000, 0x3000)

    def call(M=10, K=64, N=96, n_out=1, x=FAKE, w=FAKE, out=outs, xd=0, yd=0):
        return f(x, xd, w, None, M, K, N, out, n_out, yd, None)

    assert call(M=-1) == SIZE
    assert call(M=2**31) == SIZE
    assert call(M=2**31 - 1, N=65536) == SIZE          # more than 2^24 tiles
    assert call(K=12) == UNSUP
    assert call(K=-8) == UNSUP
    assert call(K=65544) == UNSUP
    assert call(N=0) == UNSUP
    assert call(N=97, n_out=3) == UNSUP
    assert call(n_out=0) == UNSUP and call(n_out=4) == UNSUP
    assert call(xd=2) == UNSUP and call(yd=7) == UNSUP
    assert call(out=None) == NULL
    assert call(N=96, n_out=3, out=(ctypes.c_void_p * 3)(0x1000, None, 0x3000)) == NULL
    assert call(x=None) == NULL and call(w=None) == NULL
    assert call(x=ctypes.c_void_p(0x1002)) == ARGS
    assert call(w=ctypes.c_void_p(0x1008)) == ARGS
    assert call(M=0) == OK                              # nothing to do: returns before any launch
