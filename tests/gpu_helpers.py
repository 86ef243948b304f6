"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
from __future__ import annotations

import numpy as np
import torch

from sparse_graph_attention_degree_amd import graphs as G

# Tolerances from the benchmark spec: fp32 paths 1e-5 abs + 1e-4 rel; bf16 feature
# tables with fp32 accumulation 1e-5 abs + 2e-2 rel.  The oracle reads the same bf16 bits the
# kernels read (widened exactly), so a bf16-input result must also meet the fp32 bound: each
# check of kind "bf16" applies both, and "bf16" alone would let an accumulation in bf16 pass.
# "bf16_out": the result itself is stored as bf16 (rounded once, at most 2^-8 relative), so the
# second bound adds that rounding.  "bf16_chain": a bf16 rounding of an intermediate (q/k/v
# projected, then used) is a quantisation both sides take in different precisions; only the
# contract bound applies.
TOL = {"f32": (1e-5, 1e-4), "bf16": (1e-5, 2e-2), "bf16_out": (1e-5, 2e-2), "bf16_chain": (1e-5, 2e-2)}
FP32_LEVEL = (1e-5, 1e-4)
BF16_ROUNDING = 2.0 ** -8


def _second_bound(kind, want, mag):
    """The fp32-level bound applied on top of the contract bound (None: no second bound)."""
    atol, rtol = FP32_LEVEL
    if kind == "bf16":
        return atol + rtol * (np.abs(want) + mag)
    if kind == "bf16_out":
        return atol + rtol * (np.abs(want) + mag) + BF16_ROUNDING * np.abs(want)
    return None


def _fail(what, bad, err, got, want, label):
    i = np.unravel_index(np.argmax(np.where(bad, err, 0)), err.shape)
    raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside the {label} bound; worst at {i}: "
                         f"got {got[i]!r} want {want[i]!r}")


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


def assert_close(got, want, kind: str, what: str = "", mag=None):
    """|got - want| <= atol + rtol |want| (the contract bound of `kind`); for bf16 kinds also the
    fp32-level bound, 1e-5 + 1e-4 (|want| + mag), mag being the same result computed over the
    terms' absolute values where the result is a sum whose terms can cancel (0 if not given)."""
    atol, rtol = TOL[kind]
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    if bad.any():
        _fail(what, bad, err, got, want, f"{atol}+{rtol}*|ref|")
    m = np.zeros_like(want) if mag is None else np.asarray(mag, dtype=np.float64)
    second = _second_bound(kind, want, m)
    if second is not None:
        bad = err > second
        if bad.any():
            _fail(what, bad, err, got, want, f"fp32-level ({kind})")
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
    second = _second_bound(kind, want, mag)
    if second is not None:
        bad = err > second
        if bad.any():
            _fail(what, bad, err, got, want, f"fp32-level ({kind})")


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


def abs_feat(a: np.ndarray) -> np.ndarray:
    """|a| in a's own type (bf16 bit patterns: the sign bit cleared, exact)."""
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


# ----------------------------------------------------------------------------- guard bands
CANARY32 = 0x7FC0DEAD      # a NaN no kernel writes
CANARY16 = 0x7FAD          # a bf16 NaN no kernel writes
GUARD = 4096               # canary elements on each side


def guarded(shape, dtype=torch.float32):
    """(buffer, view): a device output of `shape` between two bands of GUARD canary elements."""
    n = int(np.prod(shape))
    if dtype in (torch.float32, torch.int32):
        buf = torch.full((GUARD + n + GUARD,), CANARY32, dtype=torch.int32, device=dev())
    elif dtype == torch.bfloat16:
        buf = torch.full((GUARD + n + GUARD,), CANARY16, dtype=torch.int16, device=dev())
    else:
        raise TypeError(dtype)
    return buf, buf.view(dtype)[GUARD:GUARD + n].view(*shape)


def assert_guard(buf, what=""):
    """The bands are untouched and every element between them was written."""
    canary = CANARY32 if buf.dtype == torch.int32 else CANARY16
    b = to_np(buf)
    assert np.all(b[:GUARD] == canary) and np.all(b[-GUARD:] == canary), f"{what}: write outside the output"
    inner = b[GUARD:-GUARD]
    assert not np.any(inner == canary), f"{what}: {int((inner == canary).sum())} output elements not written"
