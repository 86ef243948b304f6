"""Every output of every entry point written between two bands of canary elements: nothing outside
the output range changes and every element inside it is written (the canary is a NaN pattern no
kernel produces).  Caller workspaces (plan, transposed graph, layer backward, SDDMM backward) are
checked the same way past their stated size.  The values themselves are checked against the oracle
by the parity tests."""
import numpy as np
import pytest
import torch

from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import assert_guard, guarded, mixed_graph, to_dev, to_np

pytestmark = pytest.mark.gpu

SCHEDULES = [None, (-1, 0), (3, 100)]     # no plan, default thresholds, small thresholds (many hub segments)


def _feat(r, n, H, D, dt):
    x = r.standard_normal((n, H, D)).astype(np.float32)
    return G.f32_to_bf16_bits(x) if dt == "bf16" else x


def _ws(nbytes):
    """A workspace of exactly nbytes (a multiple of 256) followed by a canary band."""
    buf, view = guarded((nbytes // 4,), torch.int32)
    return buf, view.view(torch.uint8)


def _ws_bands(buf, what):
    b = to_np(buf)
    assert np.all(b[:4096] == 0x7FC0DEAD) and np.all(b[-4096:] == 0x7FC0DEAD), f"{what}: write past the workspace"


@pytest.fixture(scope="module")
def problem():
    g = mixed_graph(12)
    r = np.random.default_rng(13)
    H, D = 4, 32
    p = dict(g=g, H=H, D=D, rp=to_dev(g.row_ptr), col=to_dev(g.col_idx),
             rows=to_dev(G.row_of_edge(g.row_ptr)),
             s=to_dev((r.standard_normal((g.n_edges, H)) * 2).astype(np.float32)),
             w=to_dev((r.standard_normal((g.n_edges, H)) * 0.1).astype(np.float32)),
             go=to_dev(r.standard_normal((g.n_rows, H, D)).astype(np.float32)))
    for dt in ("f32", "bf16"):
        p["q_" + dt] = to_dev(_feat(r, g.n_rows, H, D, dt))
        p["k_" + dt] = to_dev(_feat(r, g.n_src, H, D, dt))
        p["v_" + dt] = to_dev(_feat(r, g.n_src, H, D, dt))
    return p


def _plan(p, sched):
    if sched is None:
        return None
    g = p["g"]
    need = gat.gat_plan_workspace_bytes(g.n_rows, g.n_edges, p["H"], p["D"], *sched)
    buf, ws = _ws(need)
    plan = gat.gat_plan_build(p["rp"], g.n_edges, p["H"], p["D"], short_max=sched[0], seg_len=sched[1], ws=ws)
    plan.guard = buf
    return plan


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("sched", SCHEDULES, ids=str)
def test_forward_outputs(problem, dt, sched):
    p = problem
    g, H, D = p["g"], p["H"], p["D"]
    plan = _plan(p, sched)
    q, k, v = p["q_" + dt], p["k_" + dt], p["v_" + dt]
    buf, out = guarded((g.n_edges, H))
    gat.gat_sddmm(p["col"], p["rows"], k, q, scale=0.5, out=out)
    assert_guard(buf, "sddmm")
    buf, out = guarded((g.n_edges, H))
    gat.gat_edge_softmax(p["rp"], p["s"], out=out, plan=plan)
    assert_guard(buf, "edge softmax")
    buf, out = guarded((g.n_rows, H, D))
    gat.gat_aggregate(p["rp"], p["col"], p["w"], v, out=out, plan=plan)
    assert_guard(buf, "aggregate")
    buf, out = guarded((g.n_rows, H, D))
    gat.gat_fused_layer(p["rp"], p["col"], v, scores=p["s"], out=out, plan=plan)
    assert_guard(buf, "fused softmax+aggregate")
    buf, out = guarded((g.n_rows, H, D))
    gat.gat_fused_layer(p["rp"], p["col"], v, q=q, k=k, scale=0.25, out=out, plan=plan)
    assert_guard(buf, "full layer")
    if plan is not None:
        _ws_bands(plan.guard, "plan")


def test_noalloc_output(problem):
    p = problem
    g, H, D = p["g"], p["H"], p["D"]
    buf, out = guarded((g.n_rows, H, D))
    gat.gat_fused_layer_noalloc(p["rp"], p["col"], p["v_bf16"], out, q=p["q_bf16"], k=p["k_bf16"], scale=0.25)
    assert_guard(buf, "allocation-free layer")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_outputs(problem, dt):
    p = problem
    g, H, D = p["g"], p["H"], p["D"]
    q, k, v = p["q_" + dt], p["k_" + dt], p["v_" + dt]
    plan = _plan(p, (-1, 0))
    cbuf, cws = _ws(gat.gat_csc_workspace_bytes(g.n_rows, g.n_src, g.n_edges, H, D))
    csc = gat.gat_csc_build(p["rp"], p["col"], g.n_src, H, D, ws=cws)

    buf, out = guarded((g.n_edges, H))
    alpha = gat.gat_edge_softmax(p["rp"], p["s"], plan=plan)
    gat.gat_edge_softmax_backward(p["rp"], alpha, p["w"], out=out, plan=plan)
    assert_guard(buf, "edge softmax backward")

    bw, dw = guarded((g.n_edges, H))
    bf, df = guarded((g.n_src, H, D))
    gat.gat_aggregate_backward(p["rp"], p["col"], p["w"], v, p["go"], csc, dweights=dw, dfeat=df)
    assert_guard(bw, "dweights")
    assert_guard(bf, "dfeat")

    lbuf, lws = _ws(gat.gat_layer_backward_workspace_bytes(g.n_edges, H))
    bs, ds = guarded((g.n_edges, H))
    bv, dv = guarded((g.n_src, H, D))
    gat.gat_fused_layer_backward(p["rp"], p["col"], v, p["go"], plan, csc, scores=p["s"], ws=lws, dscores=ds, dv=dv)
    assert_guard(bs, "dscores")
    assert_guard(bv, "dv (scores mode)")

    bq, dq = guarded((g.n_rows, H, D))
    bk, dk = guarded((g.n_src, H, D))
    bv, dv = guarded((g.n_src, H, D))
    gat.gat_fused_layer_backward(p["rp"], p["col"], v, p["go"], plan, csc, q=q, k=k, scale=0.25, ws=lws, dq=dq,
                                 dk=dk, dv=dv)
    for b, name in ((bq, "dq"), (bk, "dk"), (bv, "dv")):
        assert_guard(b, name)
    _ws_bands(plan.guard, "plan")
    _ws_bands(cbuf, "transposed graph")
    _ws_bands(lbuf, "layer backward")

    # COO SDDMM backward over the same edges (src = column, dst = row)
    sbuf, sws = _ws(gat.gat_sddmm_backward_workspace_bytes(g.n_edges, g.n_src, g.n_rows, H, D))
    bsrc, dsrc = guarded((g.n_src, H, D))
    bdst, ddst = guarded((g.n_rows, H, D))
    gat.gat_sddmm_backward(p["col"], p["rows"], k, q, p["w"], ws=sws, d_src=dsrc, d_dst=ddst)
    assert_guard(bsrc, "sddmm backward d_src")
    assert_guard(bdst, "sddmm backward d_dst")
    _ws_bands(sbuf, "sddmm backward")


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_linear_outputs(x_dtype):
    M, K, N = 333, 136, 384
    x, w, b = G.make_linear(M, K, N, seed=3, x_dtype=x_dtype, bias=True)
    bufs, outs = zip(*(guarded((M, N // 3), torch.bfloat16) for _ in range(3)))
    gat.gat_linear(to_dev(x), to_dev(w), to_dev(b), n_out=3, y_dtype=torch.bfloat16, out=list(outs))
    for i, bb in enumerate(bufs):
        assert_guard(bb, f"linear bf16 output {i}")
    buf, out = guarded((M, N))
    gat.gat_linear(to_dev(x), to_dev(w), to_dev(b), out=[out])
    assert_guard(buf, "linear fp32 output")


@pytest.mark.parametrize("mask", ["ones", "random_empty"])
def test_relation_block_output(mask):
    R = G.RELATION_BLOCK
    nodes, pair, m, prm = G.make_relation_block(R["B"], R["N"], R["D"], R["H"], R["P"], 5, mask=mask)
    buf, out = guarded(nodes.shape)
    gat.gat_relation_block(to_dev(nodes), to_dev(pair), to_dev(m), {k: to_dev(v) for k, v in prm.items()}, out=out)
    assert_guard(buf, f"relation block ({mask})")


def test_batch_csr_outputs():
    r = np.random.default_rng(7)
    gs = [G.random_csr(30, 50, 9, r), G.csr_from_degrees(np.zeros(0, int), 3, r), G.random_csr(17, 20, 9, r),
          G.csr_from_degrees(np.zeros(7, int), 5, r), mixed_graph(8, n_rows=300, n_src=200)]
    bd = G.block_diagonal(gs)
    brp, rp = guarded((bd.n_rows + 1,), torch.int32)
    bcol, col = guarded((bd.n_edges,), torch.int32)
    gat.gat_batch_csr(*(to_dev(a) for a in G.batch_arrays(gs)), row_ptr=rp, col=col)
    assert_guard(brp, "batched row_ptr")
    assert_guard(bcol, "batched col_idx")
    assert np.array_equal(to_np(rp), bd.row_ptr) and np.array_equal(to_np(col), bd.col_idx)
