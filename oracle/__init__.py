"""CPU oracle for the CSR graph-attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never does.

``oracle.c`` holds the plain double-precision definitions (see its header for
the page passages each follows); this module compiles it with gcc and wraps it
with ctypes.  ``binning.py`` is the plain CPU statement of the degree binning.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over independent rows)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported feature dtype {a.dtype}")


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes wrapper around one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        self.path = path
        self.lib = ctypes.CDLL(path)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        L = self.lib
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = None
        L.oracle_sddmm.argtypes = [i64, vp, vp, vp, vp, i32, i32, i32, dbl, vp]
        L.oracle_edge_softmax.argtypes = [i64, vp, i32, vp, vp]
        L.oracle_aggregate.argtypes = [i64, vp, vp, i32, i32, vp, vp, i32, vp]
        L.oracle_softmax_aggregate.argtypes = [i64, vp, vp, i32, i32, vp, vp, i32, vp]
        L.oracle_layer.argtypes = [i64, vp, vp, i32, i32, vp, vp, vp, i32, dbl, vp]
        L.oracle_edge_softmax_backward.argtypes = [i64, vp, i32, vp, vp, vp]
        L.oracle_sddmm_backward.argtypes = [i64, vp, vp, vp, i64, vp, i64, i32, i32, i32, dbl, vp, vp, vp]
        L.oracle_aggregate_backward.argtypes = [i64, vp, vp, i32, i32, i64, vp, vp, i32, vp, vp, vp]
        L.oracle_softmax_aggregate_backward.argtypes = [i64, vp, vp, i32, i32, i64, vp, vp, i32, vp, vp, vp]
        L.oracle_layer_backward.argtypes = [i64, vp, vp, i32, i32, i64, vp, vp, vp, i32, dbl, vp, vp, vp, vp]
        L.oracle_relation_attention.argtypes = [i64, i64, i32, i32, i32] + [vp] * 5 + [dbl] + [vp] * 8 + [vp]
        L.oracle_linear.argtypes = [i64, i32, i32, vp, i32, vp, i32, vp, vp]
        for f in (L.oracle_sddmm, L.oracle_edge_softmax, L.oracle_aggregate,
                  L.oracle_softmax_aggregate, L.oracle_layer, L.oracle_edge_softmax_backward,
                  L.oracle_aggregate_backward, L.oracle_softmax_aggregate_backward, L.oracle_layer_backward,
                  L.oracle_relation_attention, L.oracle_linear):
            f.restype = i32

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    # --- steps -------------------------------------------------------------------------
    def sddmm(self, src_idx, dst_idx, src_feat, dst_feat, scale: float = 1.0) -> np.ndarray:
        src_idx = np.ascontiguousarray(src_idx, np.int32)
        dst_idx = np.ascontiguousarray(dst_idx, np.int32)
        src_feat = np.ascontiguousarray(src_feat)
        dst_feat = np.ascontiguousarray(dst_feat)
        assert src_feat.dtype == dst_feat.dtype and src_feat.ndim == 3 and dst_feat.ndim == 3
        H, D = src_feat.shape[1:]
        assert dst_feat.shape[1:] == (H, D)
        out = np.empty((src_idx.size, H), np.float64)
        rc = self.lib.oracle_sddmm(src_idx.size, _p(src_idx), _p(dst_idx), _p(src_feat), _p(dst_feat),
                                   _dtype_code(src_feat), H, D, float(scale), _p(out))
        assert rc == 0
        return out

    def edge_softmax(self, row_ptr, scores) -> np.ndarray:
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        scores = np.ascontiguousarray(scores, np.float64)
        E, H = scores.shape
        assert row_ptr[-1] == E
        out = np.full((E, H), np.nan, np.float64)
        rc = self.lib.oracle_edge_softmax(row_ptr.size - 1, _p(row_ptr), H, _p(scores), _p(out))
        assert rc == 0
        return out

    def aggregate(self, row_ptr, col_idx, weights, feat) -> np.ndarray:
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        weights = np.ascontiguousarray(weights, np.float64)
        feat = np.ascontiguousarray(feat)
        H, D = feat.shape[1:]
        n = row_ptr.size - 1
        out = np.full((n, H, D), np.nan, np.float64)
        rc = self.lib.oracle_aggregate(n, _p(row_ptr), _p(col_idx), H, D, _p(weights), _p(feat),
                                       _dtype_code(feat), _p(out))
        assert rc == 0
        return out

    def softmax_aggregate(self, row_ptr, col_idx, scores, feat) -> np.ndarray:
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        scores = np.ascontiguousarray(scores, np.float64)
        feat = np.ascontiguousarray(feat)
        H, D = feat.shape[1:]
        n = row_ptr.size - 1
        out = np.full((n, H, D), np.nan, np.float64)
        rc = self.lib.oracle_softmax_aggregate(n, _p(row_ptr), _p(col_idx), H, D, _p(scores), _p(feat),
                                               _dtype_code(feat), _p(out))
        assert rc == 0
        return out

    def layer(self, row_ptr, col_idx, q, k, v, scale: float = 1.0) -> np.ndarray:
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
        assert q.dtype == k.dtype == v.dtype
        H, D = v.shape[1:]
        n = row_ptr.size - 1
        assert q.shape[0] == n
        out = np.full((n, H, D), np.nan, np.float64)
        rc = self.lib.oracle_layer(n, _p(row_ptr), _p(col_idx), H, D, _p(q), _p(k), _p(v),
                                   _dtype_code(v), float(scale), _p(out))
        assert rc == 0
        return out


    # --- backward (derivatives of the steps above) --------------------------------------
    def sddmm_backward(self, src_idx, dst_idx, src_feat, dst_feat, grad, scale: float = 1.0):
        """(dL/dsrc_feat [n_src,H,D], dL/ddst_feat [n_dst,H,D]) of sddmm from dL/dout [E,H]."""
        src_idx = np.ascontiguousarray(src_idx, np.int32)
        dst_idx = np.ascontiguousarray(dst_idx, np.int32)
        src_feat = np.ascontiguousarray(src_feat)
        dst_feat = np.ascontiguousarray(dst_feat)
        grad = np.ascontiguousarray(grad, np.float64)
        assert src_feat.dtype == dst_feat.dtype and src_feat.ndim == 3 and dst_feat.ndim == 3
        ns, H, D = src_feat.shape
        nd = dst_feat.shape[0]
        assert dst_feat.shape[1:] == (H, D) and grad.shape == (src_idx.size, H) and dst_idx.size == src_idx.size
        d_src = np.full((ns, H, D), np.nan, np.float64)
        d_dst = np.full((nd, H, D), np.nan, np.float64)
        rc = self.lib.oracle_sddmm_backward(src_idx.size, _p(src_idx), _p(dst_idx), _p(src_feat), ns, _p(dst_feat),
                                            nd, _dtype_code(src_feat), H, D, float(scale), _p(grad), _p(d_src),
                                            _p(d_dst))
        assert rc == 0
        return d_src, d_dst

    def edge_softmax_backward(self, row_ptr, alpha, grad) -> np.ndarray:
        """dL/dscores from the softmax output alpha and dL/dalpha, both [E,H]."""
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        alpha = np.ascontiguousarray(alpha, np.float64)
        grad = np.ascontiguousarray(grad, np.float64)
        E, H = alpha.shape
        assert grad.shape == (E, H) and row_ptr[-1] == E
        out = np.full((E, H), np.nan, np.float64)
        rc = self.lib.oracle_edge_softmax_backward(row_ptr.size - 1, _p(row_ptr), H, _p(alpha), _p(grad), _p(out))
        assert rc == 0
        return out

    def aggregate_backward(self, row_ptr, col_idx, weights, feat, grad):
        """(dL/dweights [E,H], dL/dfeat [n_src,H,D]) from dL/dout [N,H,D]."""
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        weights = np.ascontiguousarray(weights, np.float64)
        feat = np.ascontiguousarray(feat)
        grad = np.ascontiguousarray(grad, np.float64)
        ns, H, D = feat.shape
        n = row_ptr.size - 1
        assert grad.shape == (n, H, D)
        dw = np.full(weights.shape, np.nan, np.float64)
        df = np.full((ns, H, D), np.nan, np.float64)
        rc = self.lib.oracle_aggregate_backward(n, _p(row_ptr), _p(col_idx), H, D, ns, _p(weights), _p(feat),
                                                _dtype_code(feat), _p(grad), _p(dw), _p(df))
        assert rc == 0
        return dw, df

    def softmax_aggregate_backward(self, row_ptr, col_idx, scores, feat, grad):
        """(dL/dscores [E,H], dL/dfeat [n_src,H,D]) of softmax + aggregation."""
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        scores = np.ascontiguousarray(scores, np.float64)
        feat = np.ascontiguousarray(feat)
        grad = np.ascontiguousarray(grad, np.float64)
        ns, H, D = feat.shape
        n = row_ptr.size - 1
        assert grad.shape == (n, H, D)
        ds = np.full(scores.shape, np.nan, np.float64)
        df = np.full((ns, H, D), np.nan, np.float64)
        rc = self.lib.oracle_softmax_aggregate_backward(n, _p(row_ptr), _p(col_idx), H, D, ns, _p(scores), _p(feat),
                                                        _dtype_code(feat), _p(grad), _p(ds), _p(df))
        assert rc == 0
        return ds, df

    def layer_backward(self, row_ptr, col_idx, q, k, v, grad, scale: float = 1.0):
        """(dL/dq [N,H,D], dL/dk [n_src,H,D], dL/dv [n_src,H,D]) of the full layer."""
        row_ptr = np.ascontiguousarray(row_ptr, np.int32)
        col_idx = np.ascontiguousarray(col_idx, np.int32)
        q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
        grad = np.ascontiguousarray(grad, np.float64)
        assert q.dtype == k.dtype == v.dtype
        ns, H, D = v.shape
        n = row_ptr.size - 1
        assert q.shape == (n, H, D) and k.shape == (ns, H, D) and grad.shape == (n, H, D)
        dq = np.full((n, H, D), np.nan, np.float64)
        dk = np.full((ns, H, D), np.nan, np.float64)
        dv = np.full((ns, H, D), np.nan, np.float64)
        rc = self.lib.oracle_layer_backward(n, _p(row_ptr), _p(col_idx), H, D, ns, _p(q), _p(k), _p(v),
                                            _dtype_code(v), float(scale), _p(grad), _p(dq), _p(dk), _p(dv))
        assert rc == 0
        return dq, dk, dv


    # --- dense relation-biased attention block ------------------------------------------
    def relation_attention(self, nodes, pair, mask, params: dict, eps: float = 1e-5) -> np.ndarray:
        """out [B,N,D] of the block; params: gamma, beta [D], wq, wk, wv, wo [D,D], w1 [P,P], b1 [P],
        w2 [H,P], b2 [H] (any float arrays, widened to double)."""
        f = lambda a: np.ascontiguousarray(a, np.float64)  # noqa: E731
        nodes, pair, mask = f(nodes), f(pair), f(mask)
        B, N, D = nodes.shape
        P = pair.shape[-1]
        H = params["w2"].shape[0]
        assert pair.shape == (B, N, N, P) and mask.shape == (B, N, N) and D % H == 0
        w = {k: f(v) for k, v in params.items()}
        out = np.full((B, N, D), np.nan, np.float64)
        rc = self.lib.oracle_relation_attention(B, N, D, H, P, _p(nodes), _p(pair), _p(mask), _p(w["gamma"]),
                                                _p(w["beta"]), float(eps), _p(w["wq"]), _p(w["wk"]), _p(w["wv"]),
                                                _p(w["wo"]), _p(w["w1"]), _p(w["b1"]), _p(w["w2"]), _p(w["b2"]),
                                                _p(out))
        assert rc == 0
        return out

    # --- node projections ---------------------------------------------------------------
    def linear(self, x, w, bias=None) -> np.ndarray:
        """out [M,N] = x [M,K] . w [N,K]^T + bias [N]; x and w fp32, bf16 bits (uint16) or fp64."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        assert x.ndim == 2 and w.ndim == 2 and x.shape[1] == w.shape[1]
        M, K = x.shape
        N = w.shape[0]
        b = None if bias is None else np.ascontiguousarray(bias, np.float64)
        assert b is None or b.shape == (N,)
        out = np.full((M, N), np.nan, np.float64)
        rc = self.lib.oracle_linear(M, K, N, _p(x), _dtype_code(x), _p(w), _dtype_code(w),
                                    None if b is None else _p(b), _p(out))
        assert rc == 0
        return out


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
