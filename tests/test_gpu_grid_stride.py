"""The grid-stride loop of the edge-parallel kernels (SDDMM, the backward's edge dot products).
Their grids reach the stride only past 2^29 edges, so the tests lower the workgroup cap through
the library's testing hook and require bitwise the results of the default grid, and the oracle's
within tolerance, on the 16384-edge COO workload, the 2^24-edge power-law graph and a graph with
every degree class."""
import numpy as np
import pytest
import torch

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import abs_feat, assert_close, assert_close_sum, mixed_graph, to_dev, to_np

pytestmark = pytest.mark.gpu


def _with_cap(cap, fn):
    L = gat.lib()
    prev = L.gat_testing_edge_grid_cap(cap)
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        L.gat_testing_edge_grid_cap(prev)


def test_cap_hook_round_trip():
    L = gat.lib()
    default = L.gat_testing_edge_grid_cap(7)
    assert default == 1 << 23
    assert L.gat_testing_edge_grid_cap(0) == 7
    assert L.gat_testing_edge_grid_cap(-1) == default
    assert L.gat_testing_edge_grid_cap(1 << 40) == default
    assert L.gat_testing_edge_grid_cap(0) == default


@pytest.mark.parametrize("cap", [1, 3, 64])
def test_c2_sddmm_grid_stride(cap):
    w = G.WORKLOADS["c2"]
    si, di, sf, df = (to_dev(a) for a in G.make_coo(w, 0))
    ref = gat.gat_sddmm(si, di, sf, df)
    got = _with_cap(cap, lambda: gat.gat_sddmm(si, di, sf, df))
    assert torch.equal(got, ref)
    a, b, c, d = G.make_coo(w, 0)
    assert_close(to_np(got), oracle.get().sddmm(a, b, c, d), "f32", f"c2 sddmm, {cap} workgroups")


def test_c4_sddmm_grid_stride():
    """The SDDMM the benchmark times (q row of every edge, k gathered), 2^24 edges on 512 workgroups."""
    w = G.WORKLOADS["c4"]
    g = G.make_graph(w, 0)
    q, k = to_dev(G.make_features(w, g.n_rows, 0, "q")), to_dev(G.make_features(w, g.n_src, 0, "k"))
    col, dst = to_dev(g.col_idx), to_dev(G.row_of_edge(g.row_ptr))
    ref = gat.gat_sddmm(col, dst, k, q)
    got = _with_cap(512, lambda: gat.gat_sddmm(col, dst, k, q))
    assert torch.equal(got, ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_edge_dot_grid_stride(dt):
    """dweights of the aggregation backward (the edge dot kernel) at 2 and 37 workgroups."""
    g = mixed_graph(61)
    H, D = 4, 64
    r = np.random.default_rng(62)
    wts = (r.standard_normal((g.n_edges, H)) * 0.1).astype(np.float32)
    x = r.standard_normal((g.n_src, H, D)).astype(np.float32)
    x = G.f32_to_bf16_bits(x) if dt == "bf16" else x
    go = r.standard_normal((g.n_rows, H, D)).astype(np.float32)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    args = (rp, col, to_dev(wts), to_dev(x), to_dev(go), csc)
    ref, _ = gat.gat_aggregate_backward(*args, dfeat=False)
    orc = oracle.get()
    want = orc.aggregate_backward(g.row_ptr, g.col_idx, wts, x, go)[0]
    mag = orc.aggregate_backward(g.row_ptr, g.col_idx, wts, abs_feat(x), np.abs(go))[0]
    for cap in (2, 37):
        got, _ = _with_cap(cap, lambda: gat.gat_aggregate_backward(*args, dfeat=False))
        assert torch.equal(got, ref)
        assert_close_sum(to_np(got), want, mag, dt, f"dweights, {cap} workgroups")
