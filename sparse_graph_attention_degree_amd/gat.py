"""ctypes binding of libgat.so (include/gat.h).  Argument marshalling only.

Every function takes torch tensors that already live on the current HIP device,
checks dtype / shape / contiguity, and calls the C entry point of the same name
with raw device pointers and the current torch stream.  Every step of the path
runs in the library's gfx950 kernels; there is no CPU fallback -- a missing
library or a CPU tensor raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgat.so")

GAT_F32, GAT_BF16 = 0, 1
STATUS = {0: "GAT_OK", 1: "GAT_ERR_NULL", 2: "GAT_ERR_SIZE", 3: "GAT_ERR_UNSUPPORTED", 4: "GAT_ERR_WORKSPACE",
          5: "GAT_ERR_ARGS", 6: "GAT_ERR_HIP", 7: "GAT_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20
DEFAULT_SHORT_MAX = 64
DEFAULT_SEG_LEN = 1024

EXPORTED = ["gat_plan_workspace_bytes", "gat_plan_build", "gat_sddmm", "gat_edge_softmax", "gat_aggregate",
            "gat_fused_layer", "gat_status_str", "gat_shape_supported", "gat_plan_sizeof",
            "gat_csc_workspace_bytes", "gat_csc_sizeof", "gat_csc_build", "gat_edge_softmax_backward",
            "gat_aggregate_backward", "gat_layer_backward_workspace_bytes", "gat_fused_layer_backward",
            "gat_batch_csr", "gat_relation_block_lds_bytes", "gat_relation_block", "gat_linear",
            "gat_fused_layer_noalloc", "gat_fused_layer_noalloc_bytes", "gat_sddmm_backward_workspace_bytes",
            "gat_sddmm_backward", "gat_testing_edge_grid_cap"]


class GatError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({_lib().gat_status_str(status).decode()})")


class GatPlanStruct(ctypes.Structure):
    """Mirror of ``gat_plan`` (checked against gat_plan_sizeof at load)."""
    _fields_ = [("n_rows", ctypes.c_int64), ("n_edges", ctypes.c_int64),
                ("short_max", ctypes.c_int32), ("seg_len", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("state_floats", ctypes.c_int64),
                ("seg_capacity", ctypes.c_int64), ("hub_capacity", ctypes.c_int64),
                ("hubseg_capacity", ctypes.c_int64), ("n_blocks", ctypes.c_int64),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("row_ptr", ctypes.c_void_p),
                ("off_counts", ctypes.c_size_t), ("off_blocks", ctypes.c_size_t), ("off_segs", ctypes.c_size_t),
                ("off_hubs", ctypes.c_size_t), ("off_partials", ctypes.c_size_t),
                ("magic", ctypes.c_uint32)]


class GatCscStruct(ctypes.Structure):
    """Mirror of ``gat_csc`` (checked against gat_csc_sizeof at load)."""
    _fields_ = [("n_rows", ctypes.c_int64), ("n_src", ctypes.c_int64), ("n_edges", ctypes.c_int64),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("off_col_ptr", ctypes.c_size_t), ("off_row_idx", ctypes.c_size_t), ("off_perm", ctypes.c_size_t),
                ("off_rows", ctypes.c_size_t), ("off_stage", ctypes.c_size_t),
                ("plan", GatPlanStruct), ("magic", ctypes.c_uint32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, f32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.gat_plan_workspace_bytes.argtypes = [i64, i64, i32, i32, i32, i32]
    L.gat_plan_workspace_bytes.restype = sz
    L.gat_plan_build.argtypes = [vp, i64, i64, i32, i32, i32, i32, vp, sz, ctypes.POINTER(GatPlanStruct), vp]
    L.gat_sddmm.argtypes = [vp, vp, i64, vp, i64, vp, i64, i32, i32, i32, f32, vp, vp]
    L.gat_edge_softmax.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    L.gat_aggregate.argtypes = [vp, vp, i64, i64, i64, vp, vp, i32, i32, i32, vp, vp, vp]
    L.gat_fused_layer.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, f32, vp, vp, vp, vp]
    L.gat_fused_layer_noalloc.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, f32, vp, vp, vp]
    L.gat_fused_layer_noalloc_bytes.argtypes = [i64, i64, i32, i32]
    L.gat_fused_layer_noalloc_bytes.restype = sz
    L.gat_csc_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.gat_csc_workspace_bytes.restype = sz
    L.gat_csc_sizeof.restype = sz
    L.gat_csc_build.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp, sz, ctypes.POINTER(GatCscStruct), vp]
    L.gat_edge_softmax_backward.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp]
    L.gat_aggregate_backward.argtypes = [vp, vp, i64, i64, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.gat_layer_backward_workspace_bytes.argtypes = [i64, i32]
    L.gat_layer_backward_workspace_bytes.restype = sz
    L.gat_fused_layer_backward.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, f32, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gat_sddmm_backward_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    L.gat_sddmm_backward_workspace_bytes.restype = sz
    L.gat_sddmm_backward.argtypes = [vp, vp, i64, vp, i64, vp, i64, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    L.gat_testing_edge_grid_cap.argtypes = [i64]
    L.gat_testing_edge_grid_cap.restype = i64
    L.gat_batch_csr.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
    L.gat_relation_block_lds_bytes.argtypes = [i32, i32, i32, i32]
    L.gat_relation_block_lds_bytes.restype = sz
    L.gat_relation_block.argtypes = [vp, vp, vp, vp, vp, f32] + [vp] * 8 + [i64, i32, i32, i32, i32, vp, vp]
    L.gat_linear.argtypes = [vp, i32, vp, vp, i64, i32, i32, ctypes.POINTER(vp), i32, i32, vp]
    for f in (L.gat_plan_build, L.gat_sddmm, L.gat_edge_softmax, L.gat_aggregate, L.gat_fused_layer,
              L.gat_fused_layer_noalloc,
              L.gat_csc_build, L.gat_edge_softmax_backward, L.gat_aggregate_backward, L.gat_fused_layer_backward,
              L.gat_sddmm_backward,
              L.gat_batch_csr, L.gat_relation_block, L.gat_linear):
        f.restype = i32
    L.gat_status_str.argtypes = [i32]
    L.gat_status_str.restype = ctypes.c_char_p
    L.gat_shape_supported.argtypes = [i32, i32]
    L.gat_shape_supported.restype = i32
    L.gat_plan_sizeof.restype = sz
    if L.gat_plan_sizeof() != ctypes.sizeof(GatPlanStruct):
        raise RuntimeError("gat_plan layout mismatch between libgat.so and the binding")
    if L.gat_csc_sizeof() != ctypes.sizeof(GatCscStruct):
        raise RuntimeError("gat_csc layout mismatch between libgat.so and the binding")
    _LIB = L
    return L


def lib():
    """The loaded ctypes library (raises if not built)."""
    return _lib()


# ----------------------------------------------------------------------------- marshalling
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise GatError(fn, status)


def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (libgat has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _feat_dtype(t):
    if t.dtype == torch.float32:
        return GAT_F32
    if t.dtype == torch.bfloat16:
        return GAT_BF16
    raise TypeError(f"features must be float32 or bfloat16, got {t.dtype}")


# ----------------------------------------------------------------------------- plan
class Plan:
    """A degree-binning plan plus the device workspace that holds its tables."""

    def __init__(self, struct: GatPlanStruct, ws: torch.Tensor):
        self.struct = struct
        self.ws = ws

    def ref(self):
        return ctypes.byref(self.struct)

    def table(self, which: str) -> torch.Tensor:
        """View of a plan table in the workspace (int32), for inspection."""
        s = self.struct
        if which == "counts":
            off, n = s.off_counts, 8
        elif which == "segs":
            off, n = s.off_segs, 4 * s.seg_capacity
        elif which == "hubs":
            off, n = s.off_hubs, 4 * s.hub_capacity
        else:
            raise KeyError(which)
        return self.ws[off:off + 4 * n].view(torch.int32)


def gat_plan_workspace_bytes(n_rows, n_edges, heads, head_dim, short_max=-1, seg_len=0) -> int:
    return int(_lib().gat_plan_workspace_bytes(n_rows, n_edges, heads, head_dim, short_max, seg_len))


def gat_plan_build(row_ptr: torch.Tensor, n_edges: int, heads: int, head_dim: int, short_max: int = -1,
                   seg_len: int = 0, ws: torch.Tensor | None = None, stream=None) -> Plan:
    """Build a degree-binning plan on the device (no synchronisation).  Allocates the
    workspace with torch unless ``ws`` (uint8, 256-byte aligned) is given."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    n_rows = row_ptr.numel() - 1
    need = gat_plan_workspace_bytes(n_rows, n_edges, heads, head_dim, short_max, seg_len)
    if need == 0:
        raise GatError("gat_plan_workspace_bytes", 2)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=row_ptr.device)
    _dev(ws, "ws", torch.uint8, 1)
    st = GatPlanStruct()
    _check("gat_plan_build", _lib().gat_plan_build(_ptr(row_ptr), n_rows, n_edges, heads, head_dim, short_max,
                                                   seg_len, _ptr(ws), ws.numel(), ctypes.byref(st),
                                                   _stream(stream)))
    return Plan(st, ws)


# ----------------------------------------------------------------------------- operations
def gat_sddmm(src_idx, dst_idx, src_feat, dst_feat, scale: float = 1.0, out=None, stream=None):
    """out[e,h] = scale * <dst_feat[dst_idx[e],h,:], src_feat[src_idx[e],h,:]>; returns fp32 [E,H]."""
    _dev(src_idx, "src_idx", torch.int32, 1)
    _dev(dst_idx, "dst_idx", torch.int32, 1)
    _dev(src_feat, "src_feat", None, 3)
    _dev(dst_feat, "dst_feat", src_feat.dtype, 3)
    E = src_idx.numel()
    if dst_idx.numel() != E or dst_feat.shape[1:] != src_feat.shape[1:]:
        raise ValueError("inconsistent sddmm shapes")
    H, D = src_feat.shape[1:]
    if out is None:
        out = torch.empty((E, H), dtype=torch.float32, device=src_feat.device)
    _dev(out, "out", torch.float32, 2)
    _check("gat_sddmm", _lib().gat_sddmm(_ptr(src_idx), _ptr(dst_idx), E, _ptr(src_feat), src_feat.shape[0],
                                         _ptr(dst_feat), dst_feat.shape[0], _feat_dtype(src_feat), H, D,
                                         float(scale), _ptr(out), _stream(stream)))
    return out


def gat_edge_softmax(row_ptr, scores, out=None, plan: Plan | None = None, stream=None):
    """Row-wise multi-head softmax of fp32 scores [E,H]; ``out`` may be ``scores``."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(scores, "scores", torch.float32, 2)
    E, H = scores.shape
    if out is None:
        out = torch.empty_like(scores)
    _dev(out, "out", torch.float32, 2)
    _check("gat_edge_softmax", _lib().gat_edge_softmax(_ptr(row_ptr), row_ptr.numel() - 1, E, H, _ptr(scores),
                                                       _ptr(out), plan.ref() if plan else None, _stream(stream)))
    return out


def gat_aggregate(row_ptr, col_idx, weights, feat, out=None, plan: Plan | None = None, stream=None):
    """out[i,h,:] = sum_e weights[e,h] * feat[col_idx[e],h,:]; returns fp32 [N,H,D]."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col_idx, "col_idx", torch.int32, 1)
    _dev(weights, "weights", torch.float32, 2)
    _dev(feat, "feat", None, 3)
    n_rows = row_ptr.numel() - 1
    H, D = feat.shape[1:]
    if out is None:
        out = torch.empty((n_rows, H, D), dtype=torch.float32, device=feat.device)
    _dev(out, "out", torch.float32, 3)
    _check("gat_aggregate", _lib().gat_aggregate(_ptr(row_ptr), _ptr(col_idx), n_rows, feat.shape[0],
                                                 col_idx.numel(), _ptr(weights), _ptr(feat), _feat_dtype(feat), H,
                                                 D, _ptr(out), plan.ref() if plan else None, _stream(stream)))
    return out


def gat_fused_layer(row_ptr, col_idx, v, scores=None, q=None, k=None, scale: float = 1.0, out=None,
                    plan: Plan | None = None, stream=None):
    """Fused softmax + aggregation of v with given scores, or with scores q_i . k_j computed on the fly."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col_idx, "col_idx", torch.int32, 1)
    _dev(v, "v", None, 3)
    _dev(scores, "scores", torch.float32, 2)
    _dev(q, "q", v.dtype, 3)
    _dev(k, "k", v.dtype, 3)
    n_rows = row_ptr.numel() - 1
    H, D = v.shape[1:]
    if out is None:
        out = torch.empty((n_rows, H, D), dtype=torch.float32, device=v.device)
    _dev(out, "out", torch.float32, 3)
    _check("gat_fused_layer", _lib().gat_fused_layer(_ptr(row_ptr), _ptr(col_idx), n_rows, v.shape[0],
                                                     col_idx.numel(), H, D, _feat_dtype(v), _ptr(scores), _ptr(q),
                                                     _ptr(k), float(scale), _ptr(v), _ptr(out),
                                                     plan.ref() if plan else None, _stream(stream)))
    return out


def gat_fused_layer_noalloc_bytes(n_rows, n_edges, heads, head_dim) -> int:
    return int(_lib().gat_fused_layer_noalloc_bytes(n_rows, n_edges, heads, head_dim))


def gat_fused_layer_noalloc(row_ptr, col_idx, v, out, scores=None, q=None, k=None, scale: float = 1.0, stream=None):
    """gat_fused_layer with the degree-binning plan built inside the library's own device array
    (no workspace, no allocation by the library); ``out`` (fp32 [N,H,D]) must be given."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col_idx, "col_idx", torch.int32, 1)
    _dev(v, "v", None, 3)
    _dev(scores, "scores", torch.float32, 2)
    _dev(q, "q", v.dtype, 3)
    _dev(k, "k", v.dtype, 3)
    _dev(out, "out", torch.float32, 3)
    n_rows = row_ptr.numel() - 1
    H, D = v.shape[1:]
    _check("gat_fused_layer_noalloc",
           _lib().gat_fused_layer_noalloc(_ptr(row_ptr), _ptr(col_idx), n_rows, v.shape[0], col_idx.numel(), H, D,
                                          _feat_dtype(v), _ptr(scores), _ptr(q), _ptr(k), float(scale), _ptr(v),
                                          _ptr(out), _stream(stream)))
    return out


# ----------------------------------------------------------------------------- backward
class Csc:
    """The transposed view of a graph (gat_csc) plus the device workspace that holds it."""

    def __init__(self, struct: GatCscStruct, ws: torch.Tensor):
        self.struct = struct
        self.ws = ws

    def ref(self):
        return ctypes.byref(self.struct)

    def table(self, which: str) -> torch.Tensor:
        """View of a CSC array in the workspace (int32), for inspection."""
        s = self.struct
        n = {"col_ptr": s.n_src + 1, "row_idx": s.n_edges, "perm": s.n_edges, "rows": s.n_edges}[which]
        off = {"col_ptr": s.off_col_ptr, "row_idx": s.off_row_idx, "perm": s.off_perm, "rows": s.off_rows}[which]
        return self.ws[off:off + 4 * n].view(torch.int32)


def gat_csc_workspace_bytes(n_rows, n_src, n_edges, heads, head_dim) -> int:
    return int(_lib().gat_csc_workspace_bytes(n_rows, n_src, n_edges, heads, head_dim))


def gat_csc_build(row_ptr, col_idx, n_src: int, heads: int, head_dim: int, ws: torch.Tensor | None = None,
                  stream=None) -> Csc:
    """Build the transposed view on the device (no synchronisation); allocates the workspace with
    torch unless ``ws`` (uint8, 256-byte aligned) is given."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col_idx, "col_idx", torch.int32, 1)
    n_rows, E = row_ptr.numel() - 1, col_idx.numel()
    need = gat_csc_workspace_bytes(n_rows, n_src, E, heads, head_dim)
    if need == 0:
        raise GatError("gat_csc_workspace_bytes", 2)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=row_ptr.device)
    _dev(ws, "ws", torch.uint8, 1)
    st = GatCscStruct()
    _check("gat_csc_build", _lib().gat_csc_build(_ptr(row_ptr), _ptr(col_idx), n_rows, n_src, E, heads, head_dim,
                                                 _ptr(ws), ws.numel(), ctypes.byref(st), _stream(stream)))
    return Csc(st, ws)


def gat_edge_softmax_backward(row_ptr, alpha, grad, out=None, plan: Plan | None = None, stream=None):
    """dL/dscores = alpha * (grad - sum_row alpha * grad), fp32 [E,H]; ``out`` may be ``grad``."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(alpha, "alpha", torch.float32, 2)
    _dev(grad, "grad", torch.float32, 2)
    E, H = alpha.shape
    if grad.shape != alpha.shape:
        raise ValueError("alpha and grad differ in shape")
    if out is None:
        out = torch.empty_like(alpha)
    _dev(out, "out", torch.float32, 2)
    _check("gat_edge_softmax_backward",
           _lib().gat_edge_softmax_backward(_ptr(row_ptr), row_ptr.numel() - 1, E, H, _ptr(alpha), _ptr(grad),
                                            _ptr(out), plan.ref() if plan else None, _stream(stream)))
    return out


def gat_aggregate_backward(row_ptr, col_idx, weights, feat, grad_out, csc: Csc, dweights=True, dfeat=True,
                           stream=None):
    """(dL/dweights fp32 [E,H] or None, dL/dfeat fp32 [n_src,H,D] or None).  ``dweights`` / ``dfeat``:
    True (allocate), False (skip) or an output tensor."""
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col_idx, "col_idx", torch.int32, 1)
    _dev(weights, "weights", torch.float32, 2)
    _dev(feat, "feat", None, 3)
    _dev(grad_out, "grad_out", torch.float32, 3)
    n_rows, E = row_ptr.numel() - 1, col_idx.numel()
    ns, H, D = feat.shape
    if dweights is True:
        dweights = torch.empty((E, H), dtype=torch.float32, device=feat.device)
    if dfeat is True:
        dfeat = torch.empty((ns, H, D), dtype=torch.float32, device=feat.device)
    dweights = dweights if isinstance(dweights, torch.Tensor) else None
    dfeat = dfeat if isinstance(dfeat, torch.Tensor) else None
    _dev(dweights, "dweights", torch.float32, 2)
    _dev(dfeat, "dfeat", torch.float32, 3)
    _check("gat_aggregate_backward",
           _lib().gat_aggregate_backward(_ptr(row_ptr), _ptr(col_idx), n_rows, ns, E, _ptr(weights), _ptr(feat),
                                         _feat_dtype(feat), H, D, _ptr(grad_out), _ptr(dweights), _ptr(dfeat),
                                         csc.ref(), _stream(stream)))
    return dweights, dfeat


def gat_layer_backward_workspace_bytes(n_edges, heads) -> int:
    return int(_lib().gat_layer_backward_workspace_bytes(n_edges, heads))


def gat_fused_layer_backward(row_ptr, col_idx, v, grad_out, plan: Plan, csc: Csc, scores=None, q=None, k=None,
                             scale: float = 1.0, ws: torch.Tensor | None = None, stream=None, dscores=None, dq=None,
                             dk=None, dv=None):
    """Gradients of gat_fused_layer: (dscores, None, None, dv) with scores, or (None, dq, dk, dv) with q, k.
    The output tensors may be supplied (those the mode does not use are ignored)."""
    for t, name in ((row_ptr, "row_ptr"), (col_idx, "col_idx")):
        _dev(t, name, torch.int32, 1)
    _dev(v, "v", None, 3)
    _dev(grad_out, "grad_out", torch.float32, 3)
    _dev(scores, "scores", torch.float32, 2)
    _dev(q, "q", v.dtype, 3)
    _dev(k, "k", v.dtype, 3)
    n_rows, E = row_ptr.numel() - 1, col_idx.numel()
    ns, H, D = v.shape
    dev = v.device
    need = gat_layer_backward_workspace_bytes(E, H)
    if need == 0:
        raise GatError("gat_layer_backward_workspace_bytes", 2)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(ws, "ws", torch.uint8, 1)
    layer = scores is None

    def output(t, shape, used):
        if not used:
            return None
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=dev)
        _dev(t, "gradient output", torch.float32)
        if tuple(t.shape) != shape:
            raise ValueError(f"gradient output is {tuple(t.shape)}, expected {shape}")
        return t

    dscores = output(dscores, (E, H), not layer)
    dq = output(dq, (n_rows, H, D), layer)
    dk = output(dk, (ns, H, D), layer)
    dv = output(dv, (ns, H, D), True)
    _check("gat_fused_layer_backward",
           _lib().gat_fused_layer_backward(_ptr(row_ptr), _ptr(col_idx), n_rows, ns, E, H, D, _feat_dtype(v),
                                           _ptr(scores), _ptr(q), _ptr(k), float(scale), _ptr(v),
                                           _ptr(grad_out), _ptr(dscores), _ptr(dq), _ptr(dk), _ptr(dv), plan.ref(),
                                           csc.ref(), _ptr(ws), ws.numel(), _stream(stream)))
    return dscores, dq, dk, dv


def gat_sddmm_backward_workspace_bytes(n_edges, n_src, n_dst, heads, head_dim) -> int:
    return int(_lib().gat_sddmm_backward_workspace_bytes(n_edges, n_src, n_dst, heads, head_dim))


def gat_sddmm_backward(src_idx, dst_idx, src_feat, dst_feat, grad_out, scale: float = 1.0, need_src=True,
                       need_dst=True, ws: torch.Tensor | None = None, d_src=None, d_dst=None, stream=None):
    """Gradients of gat_sddmm with respect to src_feat and dst_feat, fp32 [n,H,D] (None where not
    asked for): d_src[i] = scale * sum_{src_idx[e]=i} grad_out[e] * dst_feat[dst_idx[e]], and
    d_dst likewise."""
    _dev(src_idx, "src_idx", torch.int32, 1)
    _dev(dst_idx, "dst_idx", torch.int32, 1)
    _dev(src_feat, "src_feat", None, 3)
    _dev(dst_feat, "dst_feat", src_feat.dtype, 3)
    _dev(grad_out, "grad_out", torch.float32, 2)
    E = src_idx.numel()
    (ns, H, D), nd = src_feat.shape, dst_feat.shape[0]
    if dst_idx.numel() != E or dst_feat.shape[1:] != src_feat.shape[1:] or tuple(grad_out.shape) != (E, H):
        raise ValueError("inconsistent sddmm backward shapes")
    dev = src_feat.device
    need = gat_sddmm_backward_workspace_bytes(E, ns, nd, H, D)
    if need == 0:
        raise GatError("gat_sddmm_backward_workspace_bytes", 2)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _dev(ws, "ws", torch.uint8, 1)
    if need_src and d_src is None:
        d_src = torch.empty((ns, H, D), dtype=torch.float32, device=dev)
    if need_dst and d_dst is None:
        d_dst = torch.empty((nd, H, D), dtype=torch.float32, device=dev)
    d_src = d_src if need_src else None
    d_dst = d_dst if need_dst else None
    _dev(d_src, "d_src", torch.float32, 3)
    _dev(d_dst, "d_dst", torch.float32, 3)
    if (d_src is not None and tuple(d_src.shape) != (ns, H, D)) or (d_dst is not None and
                                                                  tuple(d_dst.shape) != (nd, H, D)):
        raise ValueError("gradient outputs must be [n_src|n_dst, H, D]")
    _check("gat_sddmm_backward",
           _lib().gat_sddmm_backward(_ptr(src_idx), _ptr(dst_idx), E, _ptr(src_feat), ns, _ptr(dst_feat), nd,
                                     _feat_dtype(src_feat), H, D, float(scale), _ptr(grad_out), _ptr(d_src),
                                     _ptr(d_dst), _ptr(ws), ws.numel(), _stream(stream)))
    return d_src, d_dst


# ----------------------------------------------------------------------------- batching
def gat_batch_csr(local_row_ptr, local_col, row_off, edge_off, src_off, stream=None, row_ptr=None, col=None):
    """Block-diagonal CSR of B graphs from their concatenated arrays and int32 offsets [B+1]
    (prefix sums of rows, edges and sources); returns (row_ptr, col_idx)."""
    for t, name in ((local_row_ptr, "local_row_ptr"), (local_col, "local_col"), (row_off, "row_off"),
                    (edge_off, "edge_off"), (src_off, "src_off")):
        _dev(t, name, torch.int32, 1)
    B = row_off.numel() - 1
    if edge_off.numel() != B + 1 or src_off.numel() != B + 1:
        raise ValueError("offset arrays differ in length")
    n_rows = local_row_ptr.numel() - B
    n_edges = local_col.numel()
    if row_ptr is None:
        row_ptr = torch.empty(n_rows + 1, dtype=torch.int32, device=row_off.device)
    if col is None:
        col = torch.empty(n_edges, dtype=torch.int32, device=row_off.device)
    _dev(row_ptr, "row_ptr", torch.int32, 1)
    _dev(col, "col", torch.int32, 1)
    if row_ptr.numel() != n_rows + 1 or col.numel() != n_edges:
        raise ValueError("output arrays of the wrong size")
    _check("gat_batch_csr", _lib().gat_batch_csr(_ptr(local_row_ptr), _ptr(local_col), _ptr(row_off),
                                                 _ptr(edge_off), _ptr(src_off), B, n_rows, n_edges, _ptr(row_ptr),
                                                 _ptr(col), _stream(stream)))
    return row_ptr, col


# ----------------------------------------------------------------------------- dense relation block
def gat_relation_block(nodes, pair_feats, edge_mask, params: dict, eps: float = 1e-5, out=None, stream=None):
    """The l2_p4 block: nodes fp32 [B,N,D], pair_feats [B,N,N,P], edge_mask [B,N,N]; params: gamma,
    beta [D], wq, wk, wv, wo [D,D], w1 [P,P], b1 [P], w2 [H,P], b2 [H] (device fp32 tensors)."""
    _dev(nodes, "nodes", torch.float32, 3)
    _dev(pair_feats, "pair_feats", torch.float32, 4)
    _dev(edge_mask, "edge_mask", torch.float32, 3)
    names = ("gamma", "beta", "wq", "wk", "wv", "wo", "w1", "b1", "w2", "b2")
    for n in names:
        _dev(params[n], n, torch.float32)
    B, N, D = nodes.shape
    P = pair_feats.shape[-1]
    H = params["w2"].shape[0]
    if pair_feats.shape[:3] != (B, N, N) or edge_mask.shape != (B, N, N):
        raise ValueError("inconsistent relation-block shapes")
    if out is None:
        out = torch.empty_like(nodes)
    _dev(out, "out", torch.float32, 3)
    _check("gat_relation_block", _lib().gat_relation_block(
        _ptr(nodes), _ptr(pair_feats), _ptr(edge_mask), *(_ptr(params[n]) for n in names[:2]), float(eps),
        *(_ptr(params[n]) for n in names[2:]), B, N, D, H, P, _ptr(out), _stream(stream)))
    return out


def gat_linear(x, w, bias=None, n_out: int = 1, y_dtype=torch.float32, out=None, stream=None):
    """y = x . w^T + bias on the matrix cores (bf16 operands, fp32 sums).  x [M, ...] fp32 or bf16 with its
    trailing dims flattened to K; w bf16 [N, K]; bias fp32 [N] or None.  Returns a list of n_out tensors
    [M, N / n_out] of y_dtype (fp32 or bf16) holding y's column blocks in order; `out` may supply them."""
    _dev(x, "x")
    _dev(w, "w", torch.bfloat16, 2)
    if bias is not None:
        _dev(bias, "bias", torch.float32, 1)
    M = x.shape[0]
    K = math.prod(x.shape[1:])
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w is {tuple(w.shape)} but x rows have {K} elements")
    if y_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y_dtype must be float32 or bfloat16")
    if n_out < 1 or N % n_out != 0:
        raise ValueError(f"{N} output columns do not split into {n_out} arrays")
    if out is None:
        out = [torch.empty((M, N // n_out), dtype=y_dtype, device=w.device) for _ in range(n_out)]
    if len(out) != n_out:
        raise ValueError(f"expected {n_out} output arrays")
    for o in out:
        _dev(o, "out", y_dtype)
        if o.numel() != M * (N // n_out):
            raise ValueError("output array of the wrong size")
    ptrs = (ctypes.c_void_p * n_out)(*(o.data_ptr() for o in out))
    _check("gat_linear", _lib().gat_linear(
        _ptr(x), _feat_dtype(x), _ptr(w), _ptr(bias), M, K, N, ptrs, n_out,
        GAT_BF16 if y_dtype == torch.bfloat16 else GAT_F32, _stream(stream)))
    return out
