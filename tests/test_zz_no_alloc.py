"""The allocation-free fused layer (gat_fused_layer_noalloc) against gat_fused_layer with a plan
built by gat_plan_build (default thresholds): the same kernels on the same tables, so the outputs
must be bitwise equal.  Calls follow each other on one stream, each smaller than the one before,
so a call that read the previous call's tables left in the library's array would show."""
import numpy as np
import pytest
import torch

from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import mixed_graph, to_dev, to_np

pytestmark = pytest.mark.gpu


def _feat(r, n, H, D, bf16):
    x = r.standard_normal((n, H, D)).astype(np.float32)
    return G.f32_to_bf16_bits(x) if bf16 else x


def _pair(rp, col, v, n_rows, H, D, E, **kw):
    """(library-array call, planned call) on the same inputs; the library-array call runs first
    into an output filled with NaN, so an unwritten element would show."""
    out = torch.full((n_rows, H, D), float("nan"), dtype=torch.float32, device=v.device)
    gat.gat_fused_layer_noalloc(rp, col, v, out, **kw)
    got = to_np(out)
    plan = gat.gat_plan_build(rp, E, H, D)
    want = to_np(gat.gat_fused_layer(rp, col, v, plan=plan, **kw))
    return got, want


def test_noalloc_equals_planned_call_on_shrinking_inputs():
    print("\nno-alloc: c4 graph, then a mixed graph with hubs, then a small graph", flush=True)
    # 1) the metric workload's graph: 2^20 rows, 2^24 edges, 4 x 64 bf16, scores N(0, 1)
    w = G.WORKLOADS["c4"]
    g = G.make_graph(w, 0)
    r = np.random.default_rng(7)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    s = to_dev(r.standard_normal((g.n_edges, 4)).astype(np.float32))
    v = to_dev(_feat(r, g.n_src, 4, 64, True))
    got, want = _pair(rp, col, v, g.n_rows, 4, 64, g.n_edges, scores=s)
    assert np.array_equal(got, want)
    del rp, col, s, v
    # 2) fewer rows, hubs split over several segments, full layer (q . k on the fly), bf16
    g = mixed_graph(3, n_rows=2000, n_src=3000, hubs=(2500, 4100, 9000))
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    q, k, v = (to_dev(_feat(r, n, 2, 64, True)) for n in (g.n_rows, g.n_src, g.n_src))
    got, want = _pair(rp, col, v, g.n_rows, 2, 64, g.n_edges, q=q, k=k, scale=0.125)
    assert np.array_equal(got, want)
    # 3) smaller still, fp32 scores, one hub
    g = mixed_graph(4, n_rows=200, n_src=300, hubs=(1500,))
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    s = to_dev(r.standard_normal((g.n_edges, 8)).astype(np.float32))
    v = to_dev(_feat(r, g.n_src, 8, 16, False))
    got, want = _pair(rp, col, v, g.n_rows, 8, 16, g.n_edges, scores=s)
    assert np.array_equal(got, want)
    deg = np.diff(g.row_ptr)
    assert np.all(got[deg == 0] == 0.0) and not np.any(np.signbit(got[deg == 0]))


def test_noalloc_refuses_graphs_beyond_its_array():
    """2^22 rows and 2^26 edges at 8 x 16 need ~94 MB of plan: refused before anything runs
    (the tensors below are small; the call never reads them)."""
    dev = torch.device("cuda:0")
    rp = torch.zeros(2**22 + 1, dtype=torch.int32, device=dev)
    col = torch.zeros(16, dtype=torch.int32, device=dev)
    lib = gat.lib()
    st = lib.gat_fused_layer_noalloc(rp.data_ptr(), col.data_ptr(), 2**22, 2**22, 2**26, 8, 16, 0, col.data_ptr(),
                                     None, None, 1.0, col.data_ptr(), col.data_ptr(), None)
    assert st == 7   # GAT_ERR_SCRATCH
