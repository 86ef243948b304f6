"""COO SDDMM backward on the GPU against the oracle: d_src and d_dst element by element, at small
sizes with every grouping class (unread rows, short, long and hub keys, repeated pairs), at the
16384-edge 1024 x 768 fp32 workload, and at 2^24 edges over two 2^18-row 4 x 32 bf16 tables; the
empty graph, one side only, integer inputs (bit-exact), repeat runs (bitwise) and guard bands."""
import numpy as np
import pytest
import torch

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import assert_close_sum, to_dev, to_np

pytestmark = pytest.mark.gpu

SHAPES = [(1, 64, "f32"), (8, 32, "f32"), (4, 64, "bf16"), (8, 16, "f32"), (2, 16, "bf16"), (16, 64, "f32"),
          (8, 128, "bf16"), (1, 128, "f32")]
CANARY = 0x7FC0DEAD


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _feat(r, n, H, D, dt):
    x = r.standard_normal((n, H, D)).astype(np.float32)
    return G.f32_to_bf16_bits(x) if dt == "bf16" else x


def _abs(a):
    return np.abs(G.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float32)


def skewed_coo(seed, ns=301, nd=257, E=5003):
    """Uniform edges plus a source hub (3000 edges on src 7), a destination hub (2500 edges on one
    dst, just over two 1024-edge segments), a long source key (300 edges on src 11), 40 copies of one
    (src, dst) pair, and the top ten rows of each side never read."""
    assert ns > 20 and nd > 20
    r = np.random.default_rng(seed)
    si = r.integers(0, ns - 10, E)
    di = r.integers(0, nd - 10, E)
    hub_d = min(100, nd - 11)
    si = np.concatenate([si, np.full(3000, 7), r.integers(0, ns - 10, 2500), np.full(300, 11), np.full(40, 5)])
    di = np.concatenate([di, r.integers(0, nd - 10, 3000), np.full(2500, hub_d), r.integers(0, nd - 10, 300),
                         np.full(40, 9)])
    assert si.max() < ns - 10 and di.max() < nd - 10
    p = r.permutation(si.size)
    return si[p].astype(np.int32), di[p].astype(np.int32), ns, nd


def _check(orc, si, di, sf, df, grad, scale, got_src, got_dst, what):
    want_src, want_dst = orc.sddmm_backward(si, di, sf, df, grad, scale=scale)
    mag_src, mag_dst = orc.sddmm_backward(si, di, _abs(sf), _abs(df), np.abs(grad), scale=abs(scale))
    # bf16 inputs are exact in fp32: both gradients are fp32 sums of fp32 products
    if got_src is not None:
        assert_close_sum(got_src, want_src, mag_src, "f32", f"{what}: d_src")
        unread = np.bincount(si, minlength=sf.shape[0]) == 0
        assert np.all(got_src[unread] == 0.0) and not np.any(np.signbit(got_src[unread])), f"{what}: unread d_src"
    if got_dst is not None:
        assert_close_sum(got_dst, want_dst, mag_dst, "f32", f"{what}: d_dst")
        unread = np.bincount(di, minlength=df.shape[0]) == 0
        assert np.all(got_dst[unread] == 0.0) and not np.any(np.signbit(got_dst[unread])), f"{what}: unread d_dst"


@pytest.mark.parametrize("H,D,dt", SHAPES)
def test_sddmm_backward(orc, H, D, dt):
    si, di, ns, nd = skewed_coo(31)
    r = np.random.default_rng(32)
    sf, df = _feat(r, ns, H, D, dt), _feat(r, nd, H, D, dt)
    grad = r.standard_normal((si.size, H)).astype(np.float32)
    d_src, d_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df), to_dev(grad), scale=0.375)
    _check(orc, si, di, sf, df, grad, 0.375, to_np(d_src), to_np(d_dst), f"H{H} D{D} {dt}")


def test_c2_sddmm_backward(orc):
    """The 16384-edge COO workload (1024 x 128 sources, 768 x 128 destinations, fp32)."""
    w = G.WORKLOADS["c2"]
    si, di, sf, df = G.make_coo(w, 0)
    grad = np.random.default_rng(33).standard_normal((w.n_edges, w.heads)).astype(np.float32)
    d_src, d_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df), to_dev(grad))
    _check(orc, si, di, sf, df, grad, 1.0, to_np(d_src), to_np(d_dst), "c2")


def test_sddmm_backward_2e24_edges(orc):
    """2^24 uniform edges between two 2^18-row tables of 4 x 32 bf16 (about 64 edges per row on
    each side), the inputs the benchmark times, every element against the oracle."""
    w = G.WORKLOADS["coo24"]
    si, di, sf, df = G.make_coo(w, 0)
    grad = np.random.default_rng(1).standard_normal((w.n_edges, w.heads)).astype(np.float32)
    d_src, d_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df), to_dev(grad))
    _check(orc, si, di, sf, df, grad, 1.0, to_np(d_src), to_np(d_dst), "2^24 edges")


def test_sddmm_backward_one_side_and_repeat(orc):
    """Asking for one gradient gives the bits of the two-sided call; repeat calls are bitwise equal."""
    si, di, ns, nd = skewed_coo(35)
    H, D = 4, 64
    r = np.random.default_rng(36)
    sf, df = (to_dev(_feat(r, n, H, D, "bf16")) for n in (ns, nd))
    grad = to_dev(r.standard_normal((si.size, H)).astype(np.float32))
    a_src, a_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), sf, df, grad)
    b_src, b_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), sf, df, grad)
    o_src, none1 = gat.gat_sddmm_backward(to_dev(si), to_dev(di), sf, df, grad, need_dst=False)
    none2, o_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), sf, df, grad, need_src=False)
    assert none1 is None and none2 is None
    for x, y in ((a_src, b_src), (a_dst, b_dst), (a_src, o_src), (a_dst, o_dst)):
        assert np.array_equal(to_np(x), to_np(y))


def test_sddmm_backward_integers_bit_exact(orc):
    """Small integers: every product and partial sum is exact in fp32, so the result is the
    oracle's bit for bit, whatever the summation order."""
    si, di, ns, nd = skewed_coo(37)
    H, D = 8, 32
    r = np.random.default_rng(38)
    sf = G.f32_to_bf16_bits(r.integers(-4, 5, (ns, H, D)).astype(np.float32))
    df = r.integers(-4, 5, (nd, H, D)).astype(np.float32)
    df_b = G.f32_to_bf16_bits(df)
    grad = r.integers(-3, 4, (si.size, H)).astype(np.float32)
    d_src, d_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df_b), to_dev(grad), scale=2.0)
    want_src, want_dst = orc.sddmm_backward(si, di, sf, df_b, grad, scale=2.0)
    assert np.array_equal(to_np(d_src), want_src.astype(np.float32))
    assert np.array_equal(to_np(d_dst), want_dst.astype(np.float32))


def test_sddmm_backward_empty_and_guard_bands(orc):
    """No edges: both gradients +0.0.  Outputs embedded between canary regions: nothing outside
    them changes, and every element inside is written."""
    H, D, pad = 2, 64, 4096
    r = np.random.default_rng(39)
    for si, di, ns, nd in ((np.zeros(0, np.int32), np.zeros(0, np.int32), 13, 6), skewed_coo(40)):
        sf, df = _feat(r, ns, H, D, "f32"), _feat(r, nd, H, D, "f32")
        grad = r.standard_normal((si.size, H)).astype(np.float32)
        bufs, views = [], []
        for n in (ns, nd):
            b = torch.full((pad + n * H * D + pad,), CANARY, dtype=torch.int32, device="cuda")
            bufs.append(b)
            views.append(b.view(torch.float32)[pad:pad + n * H * D].view(n, H, D))
        gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df), to_dev(grad), d_src=views[0],
                               d_dst=views[1])
        for b in bufs:
            a = to_np(b)
            assert np.all(a[:pad] == CANARY) and np.all(a[-pad:] == CANARY)
            assert not np.any(a[pad:-pad] == CANARY)
        if si.size == 0:
            for v in views:
                a = to_np(v)
                assert np.all(a == 0.0) and not np.any(np.signbit(a))
        else:
            _check(orc, si, di, sf, df, grad, 1.0, to_np(views[0]), to_np(views[1]), "guarded")


def test_sddmm_backward_matches_autograd_of_the_forward():
    """Against torch autograd (fp64, CPU) of the forward definition gathered with index_select."""
    si, di, ns, nd = skewed_coo(41, ns=97, nd=83, E=2000)
    H, D = 4, 16
    r = np.random.default_rng(42)
    sf, df = _feat(r, ns, H, D, "f32"), _feat(r, nd, H, D, "f32")
    grad = r.standard_normal((si.size, H)).astype(np.float32)
    a = torch.from_numpy(sf).double().requires_grad_()
    b = torch.from_numpy(df).double().requires_grad_()
    out = 0.5 * (a.index_select(0, torch.from_numpy(si).long()) * b.index_select(0, torch.from_numpy(di).long())).sum(-1)
    out.backward(torch.from_numpy(grad).double())
    d_src, d_dst = gat.gat_sddmm_backward(to_dev(si), to_dev(di), to_dev(sf), to_dev(df), to_dev(grad), scale=0.5)
    np.testing.assert_allclose(to_np(d_src), a.grad.numpy(), rtol=1e-4, atol=1e-3)
    np.testing.assert_allclose(to_np(d_dst), b.grad.numpy(), rtol=1e-4, atol=1e-3)
