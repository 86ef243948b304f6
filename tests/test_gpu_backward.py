"""Backward pass on the GPU against the oracle's backward: the transposed graph (bit-exact against a
stable numpy argsort), edge-softmax backward, aggregation backward and the fused / full-layer
backward, at small sizes over every degree class and at the full 2^20-row power-law size on
sampled rows and sources."""
import numpy as np
import pytest

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import (assert_close, assert_close_sum, assert_positive_zero_rows, mixed_graph, to_dev,
                               to_np)

pytestmark = pytest.mark.gpu


def _f64(a):
    return (G.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _softmax_bwd_mag(row_ptr, alpha, g_abs):
    """alpha * (|g| + sum_row alpha * |g|): the magnitude of the softmax-backward terms."""
    rows = G.row_of_edge(row_ptr)
    n = row_ptr.size - 1
    tot = np.stack([np.bincount(rows, weights=alpha[:, h] * g_abs[:, h], minlength=n) for h in range(alpha.shape[1])], 1)
    return alpha * (g_abs + tot[rows])

SHAPES = [(1, 64, "f32"), (8, 32, "f32"), (4, 64, "bf16"), (8, 16, "f32"), (2, 16, "bf16"), (16, 64, "f32"),
          (8, 128, "bf16")]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _feat(r, n, H, D, dt, scale=1.0):
    x = r.standard_normal((n, H, D)).astype(np.float32) * np.float32(scale)
    return G.f32_to_bf16_bits(x) if dt == "bf16" else x


def popular_graph(seed: int):
    """mixed_graph with a third of the edges redirected to three sources, so the transposed graph
    has short, long and hub rows too."""
    g = mixed_graph(seed)
    r = np.random.default_rng(seed + 100)
    col = g.col_idx.copy()
    pick = r.random(g.n_edges) < 0.33
    col[pick] = r.choice([7, 500, 999], pick.sum(), p=[0.6, 0.3, 0.1]).astype(np.int32)
    return G.CsrGraph(g.row_ptr, col, g.n_src)


def _csc_reference(g):
    perm = np.argsort(g.col_idx, kind="stable").astype(np.int32)
    col_ptr = np.searchsorted(g.col_idx[perm], np.arange(g.n_src + 1), side="left").astype(np.int32)
    rows = G.row_of_edge(g.row_ptr).astype(np.int32)
    return col_ptr, rows[perm], perm, rows


def _graphs():
    r = np.random.default_rng(9)
    wide = G.random_csr(300, (1 << 21) + 5, 40, r, zero_frac=0.1, duplicates=True)
    single = G.random_csr(50, 1, 9, r, zero_frac=0.2, duplicates=True)
    edgeless = G.csr_from_degrees(np.zeros(17, int), 11, r)
    return {"mixed": mixed_graph(11), "popular": popular_graph(12), "wide_22bit": wide, "single_source": single,
            "edgeless": edgeless}


@pytest.mark.parametrize("name", ["mixed", "popular", "wide_22bit", "single_source", "edgeless"])
def test_csc_bit_exact(name):
    g = _graphs()[name]
    csc = gat.gat_csc_build(to_dev(g.row_ptr), to_dev(g.col_idx), g.n_src, 4, 64)
    col_ptr, row_idx, perm, rows = _csc_reference(g)
    assert np.array_equal(to_np(csc.table("col_ptr")), col_ptr)
    assert np.array_equal(to_np(csc.table("perm")), perm)
    assert np.array_equal(to_np(csc.table("row_idx")), row_idx)
    assert np.array_equal(to_np(csc.table("rows")), rows)


@pytest.mark.parametrize("H", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("sched", [None, (-1, 0), (0, 3), (5, 64)], ids=str)
def test_edge_softmax_backward(orc, H, sched):
    g = mixed_graph(13)
    r = np.random.default_rng(14)
    s = (r.standard_normal((g.n_edges, H)) * 2).astype(np.float32)
    alpha = orc.edge_softmax(g.row_ptr, s).astype(np.float32)
    grad = r.standard_normal((g.n_edges, H)).astype(np.float32)
    rp = to_dev(g.row_ptr)
    plan = None if sched is None else gat.gat_plan_build(rp, g.n_edges, H, 64, short_max=sched[0], seg_len=sched[1])
    got = to_np(gat.gat_edge_softmax_backward(rp, to_dev(alpha), to_dev(grad), plan=plan))
    want = orc.edge_softmax_backward(g.row_ptr, alpha, grad)
    assert_close(got, want, "f32", "edge softmax backward")


@pytest.mark.parametrize("H", [1, 4, 8, 16])
@pytest.mark.parametrize("seg_len", [5000, 1024, 129])
def test_edge_softmax_backward_chunk_boundaries(orc, H, seg_len):
    """Long rows and hub segments whose alpha/grad runs end on, just before and just past the
    1024-float chunks the backward segment kernel streams (a one-chunk row is written from
    registers, longer ones are read again), out of place and in place."""
    degs = []
    for n in (1024, 2048, 3072):
        degs += [max(1, n // H - 1), n // H, n // H + 1]
    degs = np.array(degs + [0, 1, 3, 0, 7], dtype=np.int64)
    r = np.random.default_rng(41 + H)
    r.shuffle(degs)
    g = G.csr_from_degrees(degs, 600, r)
    alpha = orc.edge_softmax(g.row_ptr, r.standard_normal((g.n_edges, H)) * 2).astype(np.float32)
    grad = r.standard_normal((g.n_edges, H)).astype(np.float32)
    rp = to_dev(g.row_ptr)
    plan = gat.gat_plan_build(rp, g.n_edges, H, 64, short_max=0, seg_len=seg_len)
    want = orc.edge_softmax_backward(g.row_ptr, alpha, grad)
    got = gat.gat_edge_softmax_backward(rp, to_dev(alpha), to_dev(grad), plan=plan)
    assert_close(to_np(got), want, "f32", f"edge softmax backward, seg_len {seg_len}")
    gd = to_dev(grad)
    gat.gat_edge_softmax_backward(rp, to_dev(alpha), gd, out=gd, plan=plan)
    assert np.array_equal(to_np(gd), to_np(got))


def test_edge_softmax_backward_in_place(orc):
    g = mixed_graph(15)
    r = np.random.default_rng(16)
    H = 4
    alpha = orc.edge_softmax(g.row_ptr, r.standard_normal((g.n_edges, H))).astype(np.float32)
    grad = r.standard_normal((g.n_edges, H)).astype(np.float32)
    rp = to_dev(g.row_ptr)
    gd = to_dev(grad)
    gat.gat_edge_softmax_backward(rp, to_dev(alpha), gd, out=gd, plan=gat.gat_plan_build(rp, g.n_edges, H, 64))
    assert_close(to_np(gd), orc.edge_softmax_backward(g.row_ptr, alpha, grad), "f32", "in place")


@pytest.mark.parametrize("H,D,dt", SHAPES)
def test_aggregate_backward(orc, H, D, dt):
    g = popular_graph(17)
    r = np.random.default_rng(18)
    w = (r.standard_normal((g.n_edges, H)) * 0.1).astype(np.float32)
    x = _feat(r, g.n_src, H, D, dt)
    go = r.standard_normal((g.n_rows, H, D)).astype(np.float32)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    dw, dx = gat.gat_aggregate_backward(rp, col, to_dev(w), to_dev(x), to_dev(go), csc)
    want_dw, want_dx = orc.aggregate_backward(g.row_ptr, g.col_idx, w, x, go)
    mag_dw = orc.aggregate_backward(g.row_ptr, g.col_idx, w, np.abs(_f64(x)), np.abs(go))[0]
    mag_dx = orc.aggregate_backward(g.row_ptr, g.col_idx, np.abs(w), x, np.abs(go))[1]
    assert_close_sum(to_np(dw), want_dw, mag_dw, dt, "dweights")
    assert_close_sum(to_np(dx), want_dx, mag_dx, "f32", "dfeat")
    assert_positive_zero_rows(to_np(dx), np.bincount(g.col_idx, minlength=g.n_src), "dfeat of unread sources")


@pytest.mark.parametrize("H,D,dt", SHAPES)
def test_fused_softmax_aggregate_backward(orc, H, D, dt):
    g = popular_graph(19)
    r = np.random.default_rng(20)
    s = (r.standard_normal((g.n_edges, H)) * 2).astype(np.float32)
    v = _feat(r, g.n_src, H, D, dt)
    go = r.standard_normal((g.n_rows, H, D)).astype(np.float32)
    rp, col, vd, sd = to_dev(g.row_ptr), to_dev(g.col_idx), to_dev(v), to_dev(s)
    plan = gat.gat_plan_build(rp, g.n_edges, H, D)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    out = gat.gat_fused_layer(rp, col, vd, scores=sd, plan=plan)
    ds, dq, dk, dv = gat.gat_fused_layer_backward(rp, col, vd, to_dev(go), plan, csc, scores=sd)
    assert dq is None and dk is None
    want_ds, want_dv = orc.softmax_aggregate_backward(g.row_ptr, g.col_idx, s, v, go)
    alpha = orc.edge_softmax(g.row_ptr, s)
    g_abs = orc.aggregate_backward(g.row_ptr, g.col_idx, alpha, np.abs(_f64(v)), np.abs(go))[0]
    mag_dv = orc.aggregate_backward(g.row_ptr, g.col_idx, alpha, v, np.abs(go))[1]
    assert_close_sum(to_np(ds), want_ds, _softmax_bwd_mag(g.row_ptr, alpha, g_abs), dt, "dscores")
    assert_close_sum(to_np(dv), want_dv, mag_dv, "f32", "dv")


def _layer_mags(orc, row_ptr, col_idx, q, k, v, go, scale):
    """Term magnitudes of dq, dk, dv: the same sums over |g_s| |k|, |g_s| |q| and alpha |grad_out|."""
    rows = G.row_of_edge(row_ptr).astype(np.int32)
    s = orc.sddmm(col_idx, rows, k, q, scale=scale)
    alpha = orc.edge_softmax(row_ptr, s)
    ga = orc.aggregate_backward(row_ptr, col_idx, alpha, v, go)[0]
    gs = np.abs(orc.edge_softmax_backward(row_ptr, alpha, ga)) * abs(scale)
    g_abs = orc.aggregate_backward(row_ptr, col_idx, alpha, np.abs(_f64(v)), np.abs(go))[0]
    gs_mag = _softmax_bwd_mag(row_ptr, alpha, g_abs) * abs(scale)
    kq = np.abs(_f64(k))
    mq = orc.aggregate(row_ptr, col_idx, gs + gs_mag, kq)
    mk = orc.aggregate_backward(row_ptr, col_idx, gs + gs_mag, kq, np.abs(_f64(q)))[1]
    mv = orc.aggregate_backward(row_ptr, col_idx, alpha, v, np.abs(go))[1]
    return mq, mk, mv


@pytest.mark.parametrize("H,D,dt", SHAPES)
def test_layer_backward(orc, H, D, dt):
    g = popular_graph(21)
    r = np.random.default_rng(22)
    qs = 1.0 / np.sqrt(D)
    q, k, v = _feat(r, g.n_rows, H, D, dt), _feat(r, g.n_src, H, D, dt), _feat(r, g.n_src, H, D, dt)
    go = r.standard_normal((g.n_rows, H, D)).astype(np.float32)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    plan = gat.gat_plan_build(rp, g.n_edges, H, D)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    out = gat.gat_fused_layer(rp, col, vd, q=qd, k=kd, scale=qs, plan=plan)
    ds, dq, dk, dv = gat.gat_fused_layer_backward(rp, col, vd, to_dev(go), plan, csc, q=qd, k=kd, scale=qs)
    assert ds is None
    want = orc.layer_backward(g.row_ptr, g.col_idx, q, k, v, go, scale=qs)
    mags = _layer_mags(orc, g.row_ptr, g.col_idx, q, k, v, go, qs)
    for name, got, w, m in zip(("dq", "dk", "dv"), (dq, dk, dv), want, mags):
        assert_close_sum(to_np(got), w, m, dt, name)
    assert_positive_zero_rows(to_np(dq), g.degrees(), "dq of rows without edges")


def test_layer_backward_edgeless():
    g = G.csr_from_degrees(np.zeros(9, int), 6, np.random.default_rng(0))
    H, D = 4, 32
    r = np.random.default_rng(1)
    q, k, v = (to_dev(_feat(r, n, H, D, "f32")) for n in (9, 6, 6))
    go = to_dev(r.standard_normal((9, H, D)).astype(np.float32))
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    plan = gat.gat_plan_build(rp, 0, H, D)
    csc = gat.gat_csc_build(rp, col, 6, H, D)
    out = gat.gat_fused_layer(rp, col, v, q=q, k=k, plan=plan)
    _, dq, dk, dv = gat.gat_fused_layer_backward(rp, col, v, go, plan, csc, q=q, k=k)
    for t in (dq, dk, dv):
        a = to_np(t)
        assert np.all(a == 0.0) and not np.any(np.signbit(a))


def test_layer_backward_deterministic():
    g = popular_graph(23)
    H, D = 4, 64
    r = np.random.default_rng(24)
    q, k, v = (to_dev(_feat(r, n, H, D, "bf16")) for n in (g.n_rows, g.n_src, g.n_src))
    go = to_dev(r.standard_normal((g.n_rows, H, D)).astype(np.float32))
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    plan = gat.gat_plan_build(rp, g.n_edges, H, D)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    out = gat.gat_fused_layer(rp, col, v, q=q, k=k, plan=plan)
    a = [to_np(t) for t in gat.gat_fused_layer_backward(rp, col, v, go, plan, csc, q=q, k=k)[1:]]
    b = [to_np(t) for t in gat.gat_fused_layer_backward(rp, col, v, go, plan, csc, q=q, k=k)[1:]]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_layer_backward_c4_sampled(orc):
    """2^20-row power-law graph, 4 x 64 bf16, in the configuration the benchmark times: dq on sampled
    rows and dk, dv on sampled sources, each against the oracle on the sub-graph of every row with
    an edge into the sampled sources (which holds every edge those gradients sum over)."""
    w = G.WORKLOADS["c4"]
    g = G.make_graph(w, 0)
    H, D = w.heads, w.head_dim
    q = G.make_features(w, g.n_rows, 0, "q")
    k = G.make_features(w, g.n_src, 0, "k")
    v = G.make_features(w, g.n_src, 0, "v")
    r = np.random.default_rng(25)
    go = r.standard_normal((g.n_rows, H, D)).astype(np.float32)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    plan = gat.gat_plan_build(rp, g.n_edges, H, D)
    csc = gat.gat_csc_build(rp, col, g.n_src, H, D)
    out = gat.gat_fused_layer(rp, col, vd, q=qd, k=kd, plan=plan)
    _, dq, dk, dv = gat.gat_fused_layer_backward(rp, col, vd, to_dev(go), plan, csc, q=qd, k=kd)
    dq, dk, dv = to_np(dq), to_np(dk), to_np(dv)
    srcs = r.choice(g.n_src, 48, replace=False)
    rows_of_edges = G.row_of_edge(g.row_ptr)
    hit = np.isin(g.col_idx, srcs)
    rows = np.unique(rows_of_edges[hit])
    deg = g.degrees()
    rows = np.union1d(rows, [int(np.argmax(deg))])         # and the largest hub row
    sub_rp, sub_col, _ = G.take_rows(g, rows)
    want_dq, want_dk, want_dv = orc.layer_backward(sub_rp, sub_col, q[rows], k, v, go[rows])
    mq, mk, mv = _layer_mags(orc, sub_rp, sub_col, q[rows], k, v, go[rows], 1.0)
    assert_close_sum(dq[rows], want_dq, mq, "bf16", "dq (sampled rows)")
    assert_close_sum(dk[srcs], want_dk[srcs], mk[srcs], "bf16", "dk (sampled sources)")
    assert_close_sum(dv[srcs], want_dv[srcs], mv[srcs], "f32", "dv (sampled sources)")
