"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import numpy as np
import torch

from sparse_graph_attention_degree_amd import graphs as G

# Tolerances from the benchmark spec: fp32 paths 1e-5 abs + 1e-4 rel; bf16 feature
# tables with fp32 accumulation 1e-5 abs + 2e-2 rel.
TOL = {"f32": (1e-5, 1e-4), "bf16": (1e-5, 2e-2)}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(a).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def dtype_name(a: np.ndarray) -> str:
    return "bf16" if a.dtype == np.uint16 else "f32"


def assert_close(got, want, kind: str, what: str = ""):
    atol, rtol = TOL[kind]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, 0)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {atol}+{rtol}*|ref|; worst at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")
    return float(err.max()) if err.size else 0.0


def assert_close_sum(got, want, mag, kind: str, what: str = ""):
    """Gradients are sums of many signed terms (a source read by thousands of edges, a softmax
    row): |got - want| <= atol + rtol * (|want| + mag), where mag is the same sum taken over the
    terms' absolute values (rtol is then the relative error of a sum, as fp32 accumulation gives)."""
    atol, rtol = TOL[kind]
    got, want, mag = (np.asarray(a, dtype=np.float64) for a in (got, want, mag))
    assert got.shape == want.shape == mag.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - want)
    bad = err > atol + rtol * (np.abs(want) + mag)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, 0)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} out of tolerance; worst at {i}: got {got[i]!r} "
                             f"want {want[i]!r} (term magnitude {mag[i]!r})")


def assert_positive_zero_rows(out: np.ndarray, deg: np.ndarray, what=""):
    z = deg == 0
    assert np.all(out[z] == 0.0) and not np.any(np.signbit(out[z])), f"{what}: zero rows not +0.0"


def mixed_graph(seed: int, n_rows=320, n_src=1000, hubs=(2500, 4100)):
    """Degrees spanning every bin: zeros, ones, short, long, and a few hubs."""
    r = np.random.default_rng(seed)
    deg = np.concatenate([np.zeros(12, int), np.ones(20, int), r.integers(2, 33, n_rows - 12 - 20 - 30 - len(hubs)),
                          r.integers(33, 400, 30), np.array(hubs, int)])
    r.shuffle(deg)
    return G.csr_from_degrees(deg, n_src, r)
