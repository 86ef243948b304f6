"""Node projections on the matrix cores against the oracle's nn.Linear: several 128 x 128 tiles with
ragged row, column and K tails, fp32 and bf16 inputs and outputs, with and without bias, y split
into three arrays (q, k, v), the in-kernel bf16 rounding of fp32 inputs (bitwise against inputs
rounded beforehand, ties included), degenerate sizes, the full 2^20-row projections around the
power-law layer on sampled rows, and the projected layer (q/k/v projection, attention layer,
output projection) end to end.

The kernel multiplies bf16 operands exactly and sums in fp32, so the oracle is given the bf16
values of x and w and the bound is the one for an fp32 sum of K terms:
|y - ref| <= atol + rtol * (|ref| + sum_k |x_k w_k| + |b|)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import assert_close_sum, mixed_graph, to_dev, to_np

pytestmark = pytest.mark.gpu


def _f64(a):
    return (G.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _bf16(x):
    """The operand the kernel multiplies: bf16 inputs as they are, fp32 inputs rounded (nearest even)."""
    return x if x.dtype == np.uint16 else G.f32_to_bf16_bits(x)


def _nan_outs(M, N, n_out, y_dtype):
    return [torch.full((M, N // n_out), float("nan"), dtype=y_dtype, device="cuda") for _ in range(n_out)]


def _run(x, w, b, n_out=1, y_dtype=torch.float32):
    M, N = x.shape[0], w.shape[0]
    outs = _nan_outs(M, N, n_out, y_dtype)
    ys = gat.gat_linear(to_dev(x), to_dev(w), None if b is None else to_dev(b), n_out=n_out, y_dtype=y_dtype,
                        out=outs)
    return np.concatenate([to_np(y.float()) for y in ys], axis=1)


def _check(got, x, w, b, kind, what, rows=None):
    orc = oracle.get()
    xb = _bf16(x if rows is None else x[rows])
    b64 = None if b is None else b.astype(np.float64)
    want = orc.linear(xb, w, b64)
    mag = orc.linear(np.abs(_f64(xb)), np.abs(_f64(w)), None if b is None else np.abs(b64))
    assert_close_sum(got, want, mag, kind, what)


CASES = [  # (M, K, N, n_out)
    (300, 256, 768, 3),     # q/k/v of a 4 x 64 layer, ragged rows
    (129, 64, 130, 1),      # one row and two columns past a tile
    (1, 8, 1, 1),           # a single element
    (1000, 200, 256, 1),    # K not a multiple of the 64-wide K step
    (257, 136, 384, 3),     # three 128-column arrays, ragged K
    (64, 520, 96, 2),       # nine K steps, a two-way split inside one tile
]


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16], ids=["y_f32", "y_bf16"])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_linear_matches_oracle(case, x_dtype, y_dtype):
    M, K, N, n_out = case
    x, w, b = G.make_linear(M, K, N, seed=M + K + N, x_dtype=x_dtype, bias=M % 2 == 0)
    got = _run(x, w, b, n_out, y_dtype)
    _check(got, x, w, b, "f32" if y_dtype == torch.float32 else "bf16_out", f"linear {case} {x_dtype}")


def test_bf16_output_is_the_rounded_fp32_output():
    x, w, b = G.make_linear(333, 192, 200, seed=5)
    y32 = gat.gat_linear(to_dev(x), to_dev(w), to_dev(b))[0]
    y16 = gat.gat_linear(to_dev(x), to_dev(w), to_dev(b), y_dtype=torch.bfloat16)[0]
    want = G.f32_to_bf16_bits(to_np(y32))
    assert np.array_equal(to_np(y16.view(torch.int16)).view(np.uint16), want)


def test_fp32_input_rounds_to_nearest_even():
    """fp32 x with planted ties (low half 0x8000, both parities of the kept bit) and near-ties gives
    bitwise the result of the same x rounded beforehand and passed as bf16."""
    M, K, N = 200, 128, 160
    x, w, b = G.make_linear(M, K, N, seed=7, x_dtype="f32")
    r = np.random.default_rng(8)
    u = x.view(np.uint32).copy()
    pick = r.random(u.shape) < 0.5
    low = r.choice(np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], np.uint32), size=u.shape)
    u[pick] = (u[pick] & np.uint32(0xFFFF0000)) | low[pick]
    xf = u.view(np.float32)
    assert np.any((u & 0x1FFFF) == 0x18000) and np.any((u & 0x1FFFF) == 0x08000)
    y_round_in_kernel = gat.gat_linear(to_dev(xf), to_dev(w), to_dev(b))[0]
    y_rounded_before = gat.gat_linear(to_dev(G.f32_to_bf16_bits(xf)), to_dev(w), to_dev(b))[0]
    assert torch.equal(y_round_in_kernel, y_rounded_before)


def test_split_outputs_are_column_blocks():
    x, w, b = G.make_linear(300, 256, 768, seed=9)
    X, W, B = to_dev(x), to_dev(w), to_dev(b)
    one = gat.gat_linear(X, W, B)[0]
    q, k, v = gat.gat_linear(X, W, B, n_out=3)
    assert torch.equal(torch.cat([q, k, v], 1), one)


def test_deterministic_and_launch_independent():
    x, w, b = G.make_linear(700, 256, 384, seed=10)
    X, W, B = to_dev(x), to_dev(w), to_dev(b)
    a = gat.gat_linear(X, W, B)[0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c = gat.gat_linear(X, W, B, stream=s)[0]
    s.synchronize()
    assert torch.equal(a, c)


def test_degenerate_sizes():
    dev = torch.device("cuda")
    # no rows: nothing is launched, the (empty) arrays come back
    ys = gat.gat_linear(torch.empty((0, 64), dtype=torch.bfloat16, device=dev),
                        torch.zeros((96, 64), dtype=torch.bfloat16, device=dev), n_out=3)
    assert [tuple(y.shape) for y in ys] == [(0, 32)] * 3
    # in_dim 0: y is the bias on every row, or +0.0 without one
    b = torch.arange(40, dtype=torch.float32, device=dev) - 7.5
    x0 = torch.empty((5, 0), dtype=torch.bfloat16, device=dev)
    w0 = torch.empty((40, 0), dtype=torch.bfloat16, device=dev)
    outs = _nan_outs(5, 40, 1, torch.float32)
    y = gat.gat_linear(x0, w0, b, out=outs)[0]
    assert torch.equal(y, b.expand(5, 40))
    z = gat.gat_linear(x0, w0, out=_nan_outs(5, 40, 1, torch.float32))[0]
    assert torch.equal(z, torch.zeros_like(z)) and not torch.signbit(z).any()
    # zero weights give exactly the bias
    x, w, bb = G.make_linear(130, 64, 129, seed=11)
    yz = gat.gat_linear(to_dev(x), torch.zeros((129, 64), dtype=torch.bfloat16, device=dev), to_dev(bb))[0]
    assert np.array_equal(to_np(yz), np.broadcast_to(bb, (130, 129)))


def test_input_checks_raise():
    dev = torch.device("cuda")
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device=dev)
    with pytest.raises(gat.GatError):
        gat.gat_linear(x, torch.zeros((8, 12), dtype=torch.bfloat16, device=dev))      # K % 8 != 0
    flat = torch.zeros(4 * 16 + 1, dtype=torch.bfloat16, device=dev)
    with pytest.raises(gat.GatError):
        gat.gat_linear(flat[1:].view(4, 16), torch.zeros((8, 16), dtype=torch.bfloat16, device=dev))  # misaligned


def _sample_rows(M, k, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(64), M - 64 + np.arange(64), r.integers(0, M, k)]))


@pytest.mark.parametrize("which", ["qkv", "out"])
def test_full_size_projections_sampled(which):
    """The projections around the 2^20-row power-law layer (model dimension 4 x 64 = 256), in the
    launch configuration the benchmark times: q/k/v from bf16 node rows into three bf16 arrays, and
    the output projection from the layer's fp32 output to fp32; every element written, sampled rows
    against the oracle."""
    p = G.PROJECTION
    M, K = p["M"], p["K"]
    if which == "qkv":
        x, w, b = G.make_linear(M, K, 3 * K, seed=12, x_dtype="bf16", bias=False)
        n_out, y_dtype, kind = 3, torch.bfloat16, "bf16_out"
    else:
        x, w, b = G.make_linear(M, K, K, seed=13, x_dtype="f32", bias=True)
        n_out, y_dtype, kind = 1, torch.float32, "f32"
    outs = _nan_outs(M, w.shape[0], n_out, y_dtype)
    ys = gat.gat_linear(to_dev(x), to_dev(w), None if b is None else to_dev(b), n_out=n_out, y_dtype=y_dtype,
                        out=outs)
    y = torch.cat(ys, 1)
    assert bool(torch.isfinite(y).all())
    rows = _sample_rows(M, 3000, 14)
    got = to_np(y[torch.from_numpy(rows).to(y.device)].float())
    _check(got, x, w, b, kind, f"full-size {which}", rows=rows)


def test_projected_layer_end_to_end():
    """q, k, v = x Wqkv^T (bf16, the layer's input dtype); o = graph attention layer; y = o Wo^T + bo,
    on a graph with every degree class (and rows without edges, whose y is the bias); against the
    oracle's projections and layer in fp64.  q/k/v are rounded to bf16 mid-path on the GPU and
    not in the oracle, a quantisation the exp of the softmax amplifies: the contract bound only."""
    H, D = 4, 64
    F = H * D
    g = mixed_graph(41, n_rows=400, n_src=400, hubs=(2500,))
    n = g.n_rows
    x, wqkv, _ = G.make_linear(n, F, 3 * F, seed=15, x_dtype="bf16", bias=False)
    _, wo, bo = G.make_linear(1, F, F, seed=16)
    scale = 1.0 / np.sqrt(D)
    q, k, v = gat.gat_linear(to_dev(x), to_dev(wqkv), n_out=3, y_dtype=torch.bfloat16)
    rp, col = to_dev(g.row_ptr), to_dev(g.col_idx)
    o = gat.gat_fused_layer(rp, col, v.view(n, H, D), q=q.view(n, H, D), k=k.view(n, H, D), scale=scale)
    y = to_np(gat.gat_linear(o.view(n, F), to_dev(wo), to_dev(bo))[0])

    orc = oracle.get()
    qkv = orc.linear(x, wqkv)
    q64, k64, v64 = (a.reshape(n, H, D) for a in np.split(qkv, 3, axis=1))
    o64 = orc.layer(g.row_ptr, g.col_idx, q64, k64, v64, scale).reshape(n, F)
    want = orc.linear(o64, wo, bo.astype(np.float64))
    mag = orc.linear(np.abs(o64), np.abs(_f64(wo)), np.abs(bo.astype(np.float64)))
    assert_close_sum(y, want, mag, "bf16_chain", "projected layer")
    empty = g.degrees() == 0
    assert empty.any() and np.array_equal(y[empty], np.broadcast_to(bo, (int(empty.sum()), F)))
