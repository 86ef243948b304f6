"""The dense relation-biased attention block (the l2_p4 page) on the GPU against the oracle: the
page's shapes with every pair attending, random masks, rows with no pair kept (which return the
node row), other shapes up to the LDS limit (widths that are and are not whole 16-column blocks,
head widths that are and are not multiples of 4, node counts that are not), the 4096-element
batch the benchmark times, and in place."""
import numpy as np
import pytest
import torch

import oracle
from sparse_graph_attention_degree_amd import gat
from sparse_graph_attention_degree_amd import graphs as G
from tests.gpu_helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu

PAGE = G.RELATION_BLOCK


def _run(B, N, D, H, P, seed, mask, in_place=False):
    nodes, pair, m, prm = G.make_relation_block(B, N, D, H, P, seed, mask=mask)
    nd = to_dev(nodes)
    out = gat.gat_relation_block(nd, to_dev(pair), to_dev(m), {k: to_dev(v) for k, v in prm.items()},
                                 out=nd if in_place else None)
    return to_np(out), oracle.get().relation_attention(nodes, pair, m, prm), nodes, m


@pytest.mark.parametrize("mask", ["ones", "random", "random_empty"])
def test_page_shapes(mask):
    got, want, nodes, m = _run(PAGE["B"], PAGE["N"], PAGE["D"], PAGE["H"], PAGE["P"], 51, mask)
    assert_close(got, want, "f32", f"relation block ({mask})")
    empty = m.sum(-1) == 0
    if empty.any():   # no pair kept: the node row comes back unchanged
        assert np.array_equal(got[empty], nodes[empty])


# (batch, nodes, dim, heads, pair_dim).  pair_dim 16 with dim a multiple of 16 up to 128 and up to 64
# nodes runs the matrix-core kernel; the other shapes the general one.
@pytest.mark.parametrize("shape", [(2, 7, 32, 2, 8), (1, 1, 16, 1, 4), (3, 33, 64, 8, 5), (2, 40, 128, 8, 16),
                                   (1, 17, 48, 16, 3), (256, 24, 96, 4, 16), (3, 64, 64, 2, 16),
                                   (5, 1, 32, 1, 16), (2, 17, 48, 3, 16), (7, 33, 64, 8, 16), (2, 65, 64, 4, 16),
                                   (2, 20, 160, 4, 16), (3, 48, 80, 4, 16), (2, 30, 112, 8, 16),
                                   (4, 26, 128, 4, 16)], ids=str)
def test_other_shapes(shape):
    got, want, _, _ = _run(*shape, 52, "random")
    assert_close(got, want, "f32", f"relation block {shape}")


def test_benchmark_batch_every_element():
    """The 4096-element batch the benchmark times (the page's shape, every pair attending), every
    element against the oracle."""
    got, want, _, _ = _run(4096, PAGE["N"], PAGE["D"], PAGE["H"], PAGE["P"], 0, "ones")
    assert_close(got, want, "f32", "relation block, 4096 elements")


@pytest.mark.parametrize("mask", ["ones", "random_empty"])
def test_misaligned_pair_features_take_the_general_kernel(mask):
    """pair_feats (not required to be 16-byte aligned) one float past an aligned address: the
    matrix-core kernel's 16-byte loads do not apply, the general kernel gives the same result."""
    B, N, D, H, P = PAGE["B"], PAGE["N"], PAGE["D"], PAGE["H"], PAGE["P"]
    nodes, pair, m, prm = G.make_relation_block(B, N, D, H, P, 54, mask=mask)
    flat = torch.empty(pair.size + 1, dtype=torch.float32, device="cuda")
    shifted = flat[1:].view(pair.shape)
    shifted.copy_(torch.from_numpy(pair).cuda())
    assert shifted.data_ptr() % 16 != 0
    params = {k: to_dev(v) for k, v in prm.items()}
    got = to_np(gat.gat_relation_block(to_dev(nodes), shifted, to_dev(m), params))
    want = oracle.get().relation_attention(nodes, pair, m, prm)
    assert_close(got, want, "f32", f"relation block, misaligned pair features ({mask})")
    aligned = to_np(gat.gat_relation_block(to_dev(nodes), to_dev(pair), to_dev(m), params))
    assert_close(aligned, want, "f32", f"relation block, aligned ({mask})")


def test_in_place():
    got, want, _, _ = _run(PAGE["B"], PAGE["N"], PAGE["D"], PAGE["H"], PAGE["P"], 53, "random", in_place=True)
    assert_close(got, want, "f32", "relation block in place")


def test_unsupported_shapes_raise():
    L = gat.lib()
    assert L.gat_relation_block_lds_bytes(64, 128, 8, 16) == 0        # 256 KB of LDS
    assert L.gat_relation_block_lds_bytes(24, 96, 5, 16) == 0         # dim not a multiple of heads
    assert L.gat_relation_block_lds_bytes(24, 96, 32, 16) == 0        # more than 16 heads
    assert L.gat_relation_block_lds_bytes(24, 98, 2, 16) == 0         # dim not a multiple of 4
    nodes, pair, m, prm = G.make_relation_block(1, 64, 128, 8, 16, 0, mask="ones")
    with pytest.raises(gat.GatError):
        gat.gat_relation_block(to_dev(nodes), to_dev(pair), to_dev(m), {k: to_dev(v) for k, v in prm.items()})
