"""Launch-bound sizes: a batch of small graphs as one block-diagonal CSR (assembled on the device,
bit-exact against the numpy statement; batched outputs bitwise equal to per-graph outputs and within
tolerance of the oracle), and the path captured in a HIP graph and replayed (every replay equal to
the eager result on the inputs current at that replay)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import assert_close, mixed_graph, to_dev, to_np

pytestmark = pytest.mark.gpu


def _batch():
    w = G.WORKLOADS["c1"]
    r = np.random.default_rng(31)
    gs = [G.make_graph(w, seed) for seed in range(5)]
    gs.insert(2, G.csr_from_degrees(np.zeros(0, int), 3, r))      # a graph without rows
    gs.insert(4, G.csr_from_degrees(np.zeros(7, int), 5, r))      # rows without edges
    gs.append(mixed_graph(32, n_rows=300, n_src=200))              # long rows and hubs
    return gs


def _device_batch(gs):
    lrp, lcol, ro, eo, so = (to_dev(a) for a in G.batch_arrays(gs))
    return gat.gat_batch_csr(lrp, lcol, ro, eo, so)


def test_batch_csr_bit_exact():
    gs = _batch()
    rp, col = _device_batch(gs)
    bd = G.block_diagonal(gs)
    assert np.array_equal(to_np(rp), bd.row_ptr)
    assert np.array_equal(to_np(col), bd.col_idx)


@pytest.mark.parametrize("plan_on", [False, True], ids=["no_plan", "plan"])
def test_batched_outputs_equal_per_graph_outputs(plan_on):
    gs = _batch()
    H, D = 1, 64
    r = np.random.default_rng(33)
    scores = [r.standard_normal((g.n_edges, H)).astype(np.float32) for g in gs]
    feats = [r.standard_normal((g.n_src, H, D)).astype(np.float32) for g in gs]
    qs = [r.standard_normal((g.n_rows, H, D)).astype(np.float32) for g in gs]
    ks = [r.standard_normal((g.n_src, H, D)).astype(np.float32) for g in gs]
    rp, col = _device_batch(gs)
    E = col.numel()
    sc = to_dev(np.concatenate(scores))
    x, q, k = (to_dev(np.concatenate(a)) for a in (feats, qs, ks))
    plan = gat.gat_plan_build(rp, E, H, D) if plan_on else None
    fused = to_np(gat.gat_fused_layer(rp, col, x, scores=sc, plan=plan))
    layer = to_np(gat.gat_fused_layer(rp, col, x, q=q, k=k, plan=plan))
    soft = to_np(gat.gat_edge_softmax(rp, sc, plan=plan))
    ro = np.concatenate([[0], np.cumsum([g.n_rows for g in gs])])
    eo = np.concatenate([[0], np.cumsum([g.n_edges for g in gs])])
    for b, g in enumerate(gs):
        if g.n_rows == 0:
            continue
        grp, gcol = to_dev(g.row_ptr), to_dev(g.col_idx)
        gplan = gat.gat_plan_build(grp, g.n_edges, H, D) if plan_on else None
        gx, gq, gk = to_dev(feats[b]), to_dev(qs[b]), to_dev(ks[b])
        if g.n_edges == 0:
            assert np.all(fused[ro[b]:ro[b + 1]] == 0.0) and np.all(layer[ro[b]:ro[b + 1]] == 0.0)
            continue
        gs_ = to_dev(scores[b])
        assert np.array_equal(fused[ro[b]:ro[b + 1]], to_np(gat.gat_fused_layer(grp, gcol, gx, scores=gs_, plan=gplan)))
        assert np.array_equal(layer[ro[b]:ro[b + 1]], to_np(gat.gat_fused_layer(grp, gcol, gx, q=gq, k=gk, plan=gplan)))
        assert np.array_equal(soft[eo[b]:eo[b + 1]], to_np(gat.gat_edge_softmax(grp, gs_, plan=gplan)))
    bd = G.block_diagonal(gs)
    orc = oracle.get()
    assert_close(fused, orc.softmax_aggregate(bd.row_ptr, bd.col_idx, np.concatenate(scores), np.concatenate(feats)),
                 "f32", "batched fused")


def test_hip_graph_replay_matches_eager():
    """plan + SDDMM + fused softmax/aggregate on the c1 graph captured once; three replays, each after
    new inputs are written in place (with eager library calls in between), each equal to the eager
    path on those inputs."""
    w = G.WORKLOADS["c1"]
    g = G.make_graph(w, 0)
    H, D = w.heads, w.head_dim
    r = np.random.default_rng(34)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    dst = to_dev(G.row_of_edge(g.row_ptr).astype(np.int32))
    q = to_dev(r.standard_normal((g.n_rows, H, D)).astype(np.float32))
    k = to_dev(r.standard_normal((g.n_src, H, D)).astype(np.float32))
    v = to_dev(r.standard_normal((g.n_src, H, D)).astype(np.float32))
    E = g.n_edges
    ws = torch.empty(gat.gat_plan_workspace_bytes(g.n_rows, E, H, D), dtype=torch.uint8, device=q.device)
    scores = torch.empty((E, H), dtype=torch.float32, device=q.device)
    out = torch.empty((g.n_rows, H, D), dtype=torch.float32, device=q.device)

    def step(s_buf, o_buf):
        plan = gat.gat_plan_build(rp, E, H, D, ws=ws)
        gat.gat_sddmm(col, dst, k, q, out=s_buf)
        gat.gat_fused_layer(rp, col, v, scores=s_buf, out=o_buf, plan=plan)

    step(scores, out)                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(scores, out)
    torch.cuda.synchronize()
    s_ref = torch.empty_like(scores)
    o_ref = torch.empty_like(out)
    for it in range(3):
        q.copy_(torch.from_numpy(r.standard_normal((g.n_rows, H, D)).astype(np.float32)).to(q.device))
        v.copy_(torch.from_numpy(r.standard_normal((g.n_src, H, D)).astype(np.float32)).to(v.device))
        step(s_ref, o_ref)                 # eager, on the same plan workspace, before the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(scores), to_np(s_ref)), f"replay {it}: scores"
        assert np.array_equal(to_np(out), to_np(o_ref)), f"replay {it}: output"
