"""Seeded synthetic inputs for the CSR graph-attention path.

This module is the one place both sides of every parity check take their inputs
from: the HIP library and the CPU oracle.  It holds none of the method's
arithmetic (no dot products, no softmax, no aggregation) -- only graph structure,
random values and slicing.

Workloads (sizes and distributions as the five workload descriptions state them;
the readings of loosely stated ones are listed with each generator):

* ``c1``  CSR neighbourhood softmax+aggregate, 1 head: 384 rows, Poisson(18)
  in-degrees with forced zero-degree rows, uniform col_idx over 384 sources,
  scores fp32 N(0,1) [E,1], values fp32 N(0,1) [384,1,64].  The problem shape is
  the one of POPCORNBENCH task l2_p37 (Kimi-K2.6, CSR graph-attention
  neighbourhood softmax + aggregation), its reference-model passage.
* ``c2``  COO SDDMM: src_feat [1024,1,128], dst_feat [768,1,128] fp32 N(0,1),
  16384 edges with uniform src/dst indices.  Shape of POPCORNBENCH task l1_p10
  (edge-only SDDMM), its reference-model passage.
* ``c3``  16384 rows, Poisson(18), scores fp32 N(0, sd=2) [E,8], features fp32
  N(0,1) [16384,8,32].  Multi-head layout of POPCORNBENCH task l1_p18
  (multi-head sparse aggregation).
* ``c4``  2^20 rows, power-law in-degree (pdf exponent 2.1, mean 16, cap 10000),
  E = 2^24, 4 heads x 64, q/k/v bf16 from fp32 N(0,1) with round-to-nearest-even.
* ``c5``  2^22 rows, E = 2^26, Zipf rank-frequency in-degrees (exponent 1.5,
  cap 200000), exactly 5 % zero-degree rows, 8 heads x 16, fp32 N(0,1).

Every array is a deterministic function of (workload, seed).  Independent
streams come from ``numpy.random.SeedSequence(seed).spawn``.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# stream indices inside SeedSequence(seed).spawn(NSTREAMS)
_S_DEG, _S_COL, _S_SCORE, _S_FEAT, _S_ZERO, _S_Q, _S_K, _S_V, _S_COO = range(9)
_NSTREAMS = 9


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(_NSTREAMS)[stream]))


# ----------------------------------------------------------------------------- dtypes
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs are finite N(0,1) samples, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(shape, std: float, rng: np.random.Generator, dtype: str = "f32") -> np.ndarray:
    """N(0, std^2) samples: float32 array, or bf16 bit patterns (uint16) for dtype 'bf16'."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- degrees
def row_ptr_from_degrees(deg: np.ndarray) -> np.ndarray:
    deg = np.asarray(deg, dtype=np.int64)
    rp = np.zeros(deg.size + 1, dtype=np.int64)
    np.cumsum(deg, out=rp[1:])
    if rp[-1] >= 2**31:
        raise ValueError("edge count does not fit int32")
    return rp.astype(np.int32)


def degrees_poisson(n: int, mean: float, rng: np.random.Generator) -> np.ndarray:
    return rng.poisson(mean, size=n).astype(np.int64)


def force_zero_rows(deg: np.ndarray, frac: float, rng: np.random.Generator) -> np.ndarray:
    """Reading of "some zero-degree rows" for a Poisson(18) graph, where a zero
    draw has probability ~1.5e-8: rows 0 and n-1 plus a seeded ``frac`` of the
    remaining rows get degree 0."""
    deg = deg.copy()
    n = deg.size
    deg[0] = 0
    deg[n - 1] = 0
    k = int(round(frac * (n - 2)))
    if k:
        deg[1 + rng.choice(n - 2, size=k, replace=False)] = 0
    return deg


def degrees_powerlaw(n: int, n_edges: int, alpha: float, cap: int, rng: np.random.Generator) -> np.ndarray:
    """Power-law in-degrees with pdf ~ x^-alpha, capped, summing to exactly n_edges.

    Reading: continuous Pareto with tail index alpha-1, deg = min(cap, floor(xm * u^(-1/(alpha-1)))),
    u uniform in (0,1]; xm found by bisection as the largest value whose total is
    <= n_edges; the remaining few edges go +1 to seeded random rows below the cap.
    """
    u = 1.0 - rng.random(n)                     # (0, 1]
    base = u ** (-1.0 / (alpha - 1.0))          # >= 1

    def total(xm):
        return int(np.minimum(cap, np.floor(xm * base)).sum())

    lo, hi = 0.0, float(n_edges) / n
    while total(hi) <= n_edges:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) <= n_edges:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 1e-12 * hi:
            break
    deg = np.minimum(cap, np.floor(lo * base)).astype(np.int64)
    left = n_edges - int(deg.sum())
    while left > 0:
        cand = np.flatnonzero(deg < cap)
        pick = rng.choice(cand, size=min(left, cand.size), replace=False)
        deg[pick] += 1
        left -= pick.size
    return deg


def degrees_zipf(n: int, n_edges: int, exponent: float, cap: int, zero_frac: float,
                 rng_zero: np.random.Generator, rng_perm: np.random.Generator) -> np.ndarray:
    """Zipf rank-frequency in-degrees, capped, with an exact zero-row fraction.

    Reading (numpy-style Zipf sampling capped at 200k would give ~1.4e9 edges, far
    from the stated ~64M): exactly round(zero_frac*n) seeded rows get degree 0; each
    other row gets 1 base edge plus min(cap-1, floor(lam * r^-exponent)) for its rank
    r = 1, 2, ...; lam is the largest value (bisection) whose total stays <= n_edges
    (water-filling under the cap); the few leftover edges go +1 to the lowest ranks
    below the cap; a seeded permutation maps rank to row id.
    """
    n_zero = int(round(zero_frac * n))
    zero_rows = rng_zero.choice(n, size=n_zero, replace=False)
    nz = n - n_zero
    remaining = n_edges - nz
    if remaining < 0:
        raise ValueError("too few edges for the non-zero rows")
    w = np.arange(1, nz + 1, dtype=np.float64) ** (-exponent)

    def extra(lam):
        return np.minimum(cap - 1, np.floor(lam * w))

    lo, hi = 0.0, 1.0
    while extra(hi).sum() <= remaining:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if extra(mid).sum() <= remaining:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 1e-13 * hi:
            break
    ex = extra(lo).astype(np.int64)
    left = remaining - int(ex.sum())
    if left:
        below = np.flatnonzero(ex < cap - 1)[:left]
        ex[below] += 1
        left -= below.size
    assert left == 0
    rank_deg = 1 + ex
    mask = np.ones(n, dtype=bool)
    mask[zero_rows] = False
    rows = np.flatnonzero(mask)
    rows = rows[rng_perm.permutation(nz)]
    deg = np.zeros(n, dtype=np.int64)
    deg[rows] = rank_deg
    return deg


# ----------------------------------------------------------------------------- problems
@dataclass
class CsrGraph:
    row_ptr: np.ndarray         # int32 [N+1]
    col_idx: np.ndarray         # int32 [E]
    n_src: int

    @property
    def n_rows(self) -> int:
        return self.row_ptr.size - 1

    @property
    def n_edges(self) -> int:
        return int(self.col_idx.size)

    def degrees(self) -> np.ndarray:
        return np.diff(self.row_ptr.astype(np.int64))


@dataclass
class Workload:
    name: str
    kind: str                   # "csr" or "coo"
    heads: int
    head_dim: int
    dtype: str                  # feature storage: "f32" or "bf16"
    n_rows: int = 0
    n_src: int = 0
    n_edges: int = 0            # exact for power-law / zipf / coo; Poisson gives ~mean*N
    n_dst: int = 0              # coo only
    degree: str = ""            # poisson | powerlaw | zipf
    params: dict = field(default_factory=dict)
    score_std: float = 1.0
    description: str = ""


WORKLOADS = {
    "c1": Workload("c1", "csr", 1, 64, "f32", n_rows=384, n_src=384, degree="poisson",
                   params=dict(mean=18.0, zero_frac=0.02), score_std=1.0,
                   description="csr softmax+aggregate, 1 head: 384 rows, Poisson(18), 384x64 fp32"),
    "c2": Workload("c2", "coo", 1, 128, "f32", n_src=1024, n_dst=768, n_edges=16384,
                   description="coo sddmm: 1024x128 / 768x128 fp32, 16384 edges"),
    "coo24": Workload("coo24", "coo", 4, 32, "bf16", n_src=2**18, n_dst=2**18, n_edges=2**24,
                      description="coo sddmm at scale: 2^18 x 4x32 / 2^18 x 4x32 bf16, 2^24 uniform edges"),
    "c3": Workload("c3", "csr", 8, 32, "f32", n_rows=16384, n_src=16384, degree="poisson",
                   params=dict(mean=18.0), score_std=2.0,
                   description="multi-head softmax+aggregate: 16384 rows, Poisson(18), 8x32 fp32"),
    "c4": Workload("c4", "csr", 4, 64, "bf16", n_rows=2**20, n_src=2**20, n_edges=2**24, degree="powerlaw",
                   params=dict(alpha=2.1, cap=10000), score_std=1.0,
                   description="gat layer: 2^20 rows, power-law(2.1, mean 16, cap 10k), 4x64 bf16"),
    "c5": Workload("c5", "csr", 8, 16, "f32", n_rows=2**22, n_src=2**22, n_edges=2**26, degree="zipf",
                   params=dict(exponent=1.5, cap=200000, zero_frac=0.05), score_std=1.0,
                   description="skew stress: 2^22 rows, 2^26 edges, zipf(1.5) cap 200k, 5% zero rows, 8x16 fp32"),
}


def make_degrees(w: Workload, seed: int) -> np.ndarray:
    if w.degree == "poisson":
        deg = degrees_poisson(w.n_rows, w.params["mean"], _rng(seed, _S_DEG))
        if w.params.get("zero_frac"):
            deg = force_zero_rows(deg, w.params["zero_frac"], _rng(seed, _S_ZERO))
        return deg
    if w.degree == "powerlaw":
        return degrees_powerlaw(w.n_rows, w.n_edges, w.params["alpha"], w.params["cap"], _rng(seed, _S_DEG))
    if w.degree == "zipf":
        return degrees_zipf(w.n_rows, w.n_edges, w.params["exponent"], w.params["cap"], w.params["zero_frac"],
                            _rng(seed, _S_ZERO), _rng(seed, _S_DEG))
    raise ValueError(w.degree)


def make_graph(w: Workload, seed: int = 0) -> CsrGraph:
    deg = make_degrees(w, seed)
    rp = row_ptr_from_degrees(deg)
    col = _rng(seed, _S_COL).integers(0, w.n_src, size=int(rp[-1]), dtype=np.int32)
    return CsrGraph(rp, col, w.n_src)


def make_scores(w: Workload, n_edges: int, seed: int = 0) -> np.ndarray:
    """Edge scores fp32 [E, H], N(0, score_std^2)."""
    return normal((n_edges, w.heads), w.score_std, _rng(seed, _S_SCORE), "f32")


def make_features(w: Workload, n_nodes: int, seed: int = 0, stream: str = "feat") -> np.ndarray:
    """Node features [n, H, D]: fp32, or bf16 bit patterns (uint16)."""
    s = {"feat": _S_FEAT, "q": _S_Q, "k": _S_K, "v": _S_V}[stream]
    return normal((n_nodes, w.heads, w.head_dim), 1.0, _rng(seed, s), w.dtype)


def make_coo(w: Workload, seed: int = 0):
    """COO problem: (src_idx, dst_idx, src_feat [Ns,H,D], dst_feat [Nd,H,D])."""
    r = _rng(seed, _S_COO)
    src_idx = r.integers(0, w.n_src, size=w.n_edges, dtype=np.int32)
    dst_idx = r.integers(0, w.n_dst, size=w.n_edges, dtype=np.int32)
    src_feat = normal((w.n_src, w.heads, w.head_dim), 1.0, _rng(seed, _S_K), w.dtype)
    dst_feat = normal((w.n_dst, w.heads, w.head_dim), 1.0, _rng(seed, _S_Q), w.dtype)
    return src_idx, dst_idx, src_feat, dst_feat


# ----------------------------------------------------------------------------- small graphs for tests
def random_csr(n_rows: int, n_src: int, max_deg: int, rng: np.random.Generator, zero_frac: float = 0.1,
               duplicates: bool = True) -> CsrGraph:
    """Small random CSR graph: uniform degrees in [0, max_deg], a fraction forced to 0.
    Without ``duplicates`` each row's sources are distinct (requires max_deg <= n_src)."""
    deg = rng.integers(0, max_deg + 1, size=n_rows)
    deg[rng.random(n_rows) < zero_frac] = 0
    rp = row_ptr_from_degrees(deg)
    cols = []
    for d in deg:
        if duplicates:
            cols.append(rng.integers(0, n_src, size=d))
        else:
            cols.append(rng.choice(n_src, size=d, replace=False))
    col = np.concatenate(cols).astype(np.int32) if cols else np.zeros(0, np.int32)
    return CsrGraph(rp, col, n_src)


def csr_from_degrees(deg, n_src: int, rng: np.random.Generator) -> CsrGraph:
    rp = row_ptr_from_degrees(np.asarray(deg))
    col = rng.integers(0, n_src, size=int(rp[-1]), dtype=np.int32)
    return CsrGraph(rp, col, n_src)


def page_degrees_mod5(n: int, avg: int) -> np.ndarray:
    """Deterministic degrees of the CSR edge-softmax task (POPCORNBENCH l1_p6, its
    input generator): avg + (i % 5 - 2), at least 1."""
    i = np.arange(n)
    return np.maximum(1, avg + (i % 5) - 2)


def page_degrees_mod7(n: int, avg: int) -> np.ndarray:
    """Deterministic degrees of the CSR softmax+aggregate task (POPCORNBENCH l2_p37,
    its input generator): avg + (i % 7 - 3), at least 1."""
    i = np.arange(n)
    return np.maximum(1, avg + (i % 7) - 3)


# ----------------------------------------------------------------------------- helpers
def take_rows(g: CsrGraph, rows: np.ndarray):
    """Sub-CSR of the given rows (in the given order).

    Returns (row_ptr', col_idx', edge_ids) where edge_ids maps each edge of the
    sub-graph to its index in ``g`` (used to slice [E,H] scores / outputs)."""
    rows = np.asarray(rows, dtype=np.int64)
    rp = g.row_ptr.astype(np.int64)
    starts, ends = rp[rows], rp[rows + 1]
    deg = ends - starts
    sub_rp = np.zeros(rows.size + 1, dtype=np.int64)
    np.cumsum(deg, out=sub_rp[1:])
    total = int(sub_rp[-1])
    # edge_ids[k] = starts[r] + (k - sub_rp[r]) for k in segment r
    seg = np.repeat(np.arange(rows.size), deg)
    edge_ids = starts[seg] + (np.arange(total) - sub_rp[seg])
    return sub_rp.astype(np.int32), g.col_idx[edge_ids], edge_ids


# Dense relation-biased attention block (the l2_p4 page): its shapes, and seeded inputs with
# nn.Linear-style weights U(-1/sqrt(fan_in), 1/sqrt(fan_in)) and a LayerNorm affine near identity.
RELATION_BLOCK = dict(B=4, N=24, D=96, P=16, H=4)


def make_relation_block(B: int, N: int, D: int, H: int, P: int, seed: int = 0, mask: str = "ones"):
    """(nodes [B,N,D], pair [B,N,N,P], mask [B,N,N], params) as float32.  mask: "ones" (every pair
    attends, as the page's inputs), "random" (Bernoulli(0.6) with the diagonal kept), or
    "random_empty" (Bernoulli(0.4), some rows with no pair at all)."""
    r = np.random.default_rng(np.random.SeedSequence([seed, 0x5E1A]))
    f32 = lambda a: np.asarray(a, np.float32)  # noqa: E731
    nodes = f32(r.standard_normal((B, N, D)))
    pair = f32(r.standard_normal((B, N, N, P)))
    if mask == "ones":
        m = np.ones((B, N, N), np.float32)
    elif mask == "random":
        m = f32(r.random((B, N, N)) < 0.6)
        m[:, np.arange(N), np.arange(N)] = 1.0
    elif mask == "random_empty":
        m = f32(r.random((B, N, N)) < 0.4)
        m[:, ::3, :] = 0.0
    else:
        raise ValueError(mask)
    u = lambda shape, fan_in: f32(r.uniform(-1.0, 1.0, shape) / np.sqrt(fan_in))  # noqa: E731
    params = dict(gamma=f32(1.0 + 0.1 * r.standard_normal(D)), beta=f32(0.1 * r.standard_normal(D)),
                  wq=u((D, D), D), wk=u((D, D), D), wv=u((D, D), D), wo=u((D, D), D),
                  w1=u((P, P), P), b1=u((P,), P), w2=u((H, P), P), b2=u((H,), P))
    return nodes, pair, m, params


# Node projections around the c4 layer: 2^20 node rows of model dimension H*D = 256 in, the
# q/k/v projection to 3 * 256 columns (bf16 out, the layer's input dtype) and the output
# projection from the layer's fp32 output back to 256 columns.
PROJECTION = dict(M=2**20, K=256, heads=4, head_dim=64)


def make_linear(M: int, K: int, N: int, seed: int = 0, x_dtype: str = "bf16", bias: bool = True):
    """(x [M,K], w [N,K] bf16 bits, bias [N] fp32 or None).  x: N(0,1) as fp32, or bf16 bits
    (rounded to nearest even); w: nn.Linear's U(-1/sqrt(K), 1/sqrt(K)) rounded to bf16."""
    r = np.random.default_rng(np.random.SeedSequence([seed, 0x11AE]))
    x = r.standard_normal((M, K), dtype=np.float32)
    if x_dtype == "bf16":
        x = f32_to_bf16_bits(x)
    elif x_dtype != "f32":
        raise ValueError(x_dtype)
    bound = 1.0 / np.sqrt(max(K, 1))
    w = f32_to_bf16_bits(r.uniform(-bound, bound, (N, K)).astype(np.float32))
    b = r.uniform(-bound, bound, N).astype(np.float32) if bias else None
    return x, w, b

def batch_arrays(graphs):
    """The inputs of a block-diagonal batch: the graphs' row_ptr and col_idx concatenated as they
    are, and int32 prefix sums [B+1] of their rows, edges and sources."""
    local_rp = np.concatenate([g.row_ptr for g in graphs]).astype(np.int32)
    local_col = np.concatenate([g.col_idx for g in graphs] + [np.zeros(0, np.int32)]).astype(np.int32)
    off = lambda xs: np.concatenate([[0], np.cumsum(xs)]).astype(np.int32)  # noqa: E731
    return (local_rp, local_col, off([g.n_rows for g in graphs]), off([g.n_edges for g in graphs]),
            off([g.n_src for g in graphs]))


def block_diagonal(graphs) -> CsrGraph:
    """The batch as one CSR: graph b's rows, edges and sources shifted by the totals before it."""
    rp = [np.zeros(1, np.int64)]
    cols = [np.zeros(0, np.int32)]
    e0 = s0 = 0
    for g in graphs:
        rp.append(g.row_ptr[1:].astype(np.int64) + e0)
        cols.append((g.col_idx.astype(np.int64) + s0).astype(np.int32))
        e0 += g.n_edges
        s0 += g.n_src
    return CsrGraph(np.concatenate(rp).astype(np.int32), np.concatenate(cols), s0)


def row_of_edge(row_ptr: np.ndarray) -> np.ndarray:
    """Destination row id of every edge (COO expansion of a CSR row pointer)."""
    deg = np.diff(row_ptr.astype(np.int64))
    return np.repeat(np.arange(deg.size, dtype=np.int32), deg)


def sample_rows(g: CsrGraph, k: int, seed: int) -> np.ndarray:
    """Row sample for full-size parity: the k highest-degree rows, every zero row
    class representative, the first/last rows, and seeded uniform rows."""
    deg = g.degrees()
    r = np.random.default_rng(seed)
    top = np.argsort(-deg, kind="stable")[: max(1, k // 8)]
    zeros = np.flatnonzero(deg == 0)[:4]
    ends = np.array([0, g.n_rows - 1])
    uni = r.choice(g.n_rows, size=min(g.n_rows, k), replace=False)
    return np.unique(np.concatenate([top, zeros, ends, uni]).astype(np.int64))


def array_digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()
