"""ctypes binding of libsa (include/sa.h): argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; torch is
used here only to allocate device tensors and to name the current stream.
There is no fallback: if libsa.so is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Union

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libsa.so")

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_HIP = -3
SA_ERR_ALLOC = -4

SA_F32 = 0
SA_BF16 = 1

PATTERNS = {
    "strided_a": 0,
    "strided_b": 1,
    "fixed_a": 2,
    "fixed_b": 3,
    "dense": 4,
}

EXPORTED = [
    "sa_layout_build", "sa_layout_info", "sa_layout_export", "sa_layout_set_residue_view",
    "sa_layout_set_compact_view", "sa_layout_view_info", "sa_layout_destroy",
    "sa_fwd", "sa_bwd", "sa_bwd_workspace_size", "sa_bwd_dq_rowterms", "sa_bwd_rowterms", "sa_bwd_dkdv",
    "sa_bwd_dq", "sa_bwd_noalloc", "sa_set_fwd_form", "sa_set_split", "sa_set_one_paths",
    "sa_status_string", "sa_last_error",
]


class SAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%d): %s" % (_status_text(status), status, message))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libsa.so is not built (%s); run __graft_entry__.build() or "
                          "python block_sparse_factorized_amd/_build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, cint, flt = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    lib.sa_layout_build.argtypes = [cint, i64, i64, i64, i32, ctypes.POINTER(vp)]
    lib.sa_layout_build.restype = cint
    lib.sa_layout_info.argtypes = [vp] + [ctypes.POINTER(i64)] * 4
    lib.sa_layout_info.restype = cint
    lib.sa_layout_export.argtypes = [vp] * 8
    lib.sa_layout_export.restype = cint
    lib.sa_layout_set_residue_view.argtypes = [vp, cint]
    lib.sa_layout_set_residue_view.restype = cint
    lib.sa_layout_set_compact_view.argtypes = [vp, cint]
    lib.sa_layout_set_compact_view.restype = cint
    lib.sa_layout_view_info.argtypes = [vp, ctypes.POINTER(cint)] + [ctypes.POINTER(i64)] * 4
    lib.sa_layout_view_info.restype = cint
    lib.sa_layout_destroy.argtypes = [vp]
    lib.sa_layout_destroy.restype = None
    lib.sa_fwd.argtypes = [vp, i32, i32, i64, i32, cint, flt, vp, vp, vp, vp, vp, vp]
    lib.sa_fwd.restype = cint
    lib.sa_bwd_workspace_size.argtypes = [i32, i32, i64, i32]
    lib.sa_bwd_workspace_size.restype = sz
    lib.sa_bwd.argtypes = [vp, i32, i32, i64, i32, cint, flt] + [vp] * 10 + [sz, vp]
    lib.sa_bwd.restype = cint
    lib.sa_bwd_rowterms.argtypes = [vp, i32, i32, i64, i32, cint, flt, vp, vp, vp, vp, sz, vp]
    lib.sa_bwd_rowterms.restype = cint
    lib.sa_bwd_dkdv.argtypes = [vp, i32, i32, i64, i32, cint, flt] + [vp] * 7 + [sz, vp]
    lib.sa_bwd_dkdv.restype = cint
    lib.sa_bwd_dq_rowterms.argtypes = [vp, i32, i32, i64, i32, cint, flt] + [vp] * 8 + [sz, vp]
    lib.sa_bwd_dq_rowterms.restype = cint
    lib.sa_bwd_dq.argtypes = [vp, i32, i32, i64, i32, cint, flt] + [vp] * 6 + [sz, vp]
    lib.sa_bwd_dq.restype = cint
    lib.sa_bwd_noalloc.argtypes = [vp, i32, i32, i64, i32, cint, flt] + [vp] * 10
    lib.sa_bwd_noalloc.restype = cint
    lib.sa_set_fwd_form.argtypes = [cint]
    lib.sa_set_fwd_form.restype = cint
    lib.sa_set_split.argtypes = [cint, ctypes.POINTER(cint)]
    lib.sa_set_split.restype = cint
    lib.sa_set_one_paths.argtypes = [cint, ctypes.POINTER(cint)]
    lib.sa_set_one_paths.restype = cint
    lib.sa_status_string.argtypes = [cint]
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_last_error.argtypes = []
    lib.sa_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    """The loaded ctypes CDLL (for tests that call the C ABI directly)."""
    return _lib


def _status_text(status: int) -> str:
    return _lib.sa_status_string(status).decode()


def _check(status: int):
    if status != SA_OK:
        raise SAError(status, _lib.sa_last_error().decode())


class Layout:
    """Owning handle of an sa_layout_t."""

    def __init__(self, handle: int, pattern: str, n: int, l: int, c: int, block: int):
        self.handle = ctypes.c_void_p(handle)
        self.pattern, self.n, self.l, self.c, self.block = pattern, n, l, c, block
        self.residue_view = False
        self.compact_view = False

    def info(self) -> Dict[str, int]:
        vals = [ctypes.c_int64() for _ in range(4)]
        _check(_lib.sa_layout_info(self.handle, *[ctypes.byref(v) for v in vals]))
        return dict(zip(["nqb", "nnz", "n_masks", "allowed"], [v.value for v in vals]))

    def export(self) -> Dict[str, np.ndarray]:
        inf = self.info()
        nqb, nnz, nm = inf["nqb"], inf["nnz"], inf["n_masks"]
        nw = self.block * self.block // 64
        out = {
            "row_ptr": np.zeros(nqb + 1, np.int32), "col_idx": np.zeros(max(nnz, 1), np.int32),
            "mask_id": np.zeros(max(nnz, 1), np.int32),
            "mask_words": np.zeros((max(nm, 1), nw), np.uint64),
            "col_ptr": np.zeros(nqb + 1, np.int32), "row_idx": np.zeros(max(nnz, 1), np.int32),
            "csr_pos": np.zeros(max(nnz, 1), np.int32),
        }
        order = ["row_ptr", "col_idx", "mask_id", "mask_words", "col_ptr", "row_idx", "csr_pos"]
        _check(_lib.sa_layout_export(self.handle, *[ctypes.c_void_p(out[k].ctypes.data) for k in order]))
        for k in ("col_idx", "mask_id", "row_idx", "csr_pos"):
            out[k] = out[k][:nnz]
        out["mask_words"] = out["mask_words"][:nm]
        return out

    def set_residue_view(self, enable: bool = True) -> "Layout":
        """Run this strided-B layout's heads as dense causal attentions over
        the residue classes mod l (see sa_layout_set_residue_view)."""
        _check(_lib.sa_layout_set_residue_view(self.handle, int(bool(enable))))
        self.residue_view = bool(enable)
        return self

    def set_compact_view(self, enable: bool = True) -> "Layout":
        """Run this fixed-B layout's heads against blocks of its summary keys
        only (see sa_layout_set_compact_view)."""
        _check(_lib.sa_layout_set_compact_view(self.handle, int(bool(enable))))
        self.compact_view = bool(enable)
        return self

    def view_info(self) -> Dict[str, int]:
        """What the kernels walk for this layout (see sa_layout_view_info)."""
        kind = ctypes.c_int()
        vals = [ctypes.c_int64() for _ in range(4)]
        _check(_lib.sa_layout_view_info(self.handle, ctypes.byref(kind), *[ctypes.byref(v) for v in vals]))
        out = dict(zip(["nqb", "nkb", "nnz", "allowed"], [v.value for v in vals]))
        out["kind"] = ("layout", "residue", "compact")[kind.value]
        return out

    def close(self):
        if self.handle is not None and self.handle.value:
            _lib.sa_layout_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


FWD_FORMS = {"auto": 0, "half": 1, "paired": 2}


def sa_set_fwd_form(form: Union[str, int]) -> str:
    """Process-wide forward kernel form ("auto", "half" or "paired"; see
    sa_set_fwd_form in sa.h).  Returns the previous setting."""
    code = FWD_FORMS[form] if isinstance(form, str) else int(form)
    prev = _lib.sa_set_fwd_form(code)
    if prev < 0:
        _check(prev)
    return {v: k for k, v in FWD_FORMS.items()}[prev]


def sa_set_split(steps: int) -> int:
    """Process-wide chunking of long lists (0: chosen per call, -1: none,
    k > 0: lists longer than k in chunks of at most k; see sa_set_split in
    sa.h).  Returns the previous setting."""
    prev = ctypes.c_int()
    _check(_lib.sa_set_split(int(steps), ctypes.byref(prev)))
    return prev.value


def sa_set_one_paths(enable: bool) -> bool:
    """Process-wide switch of the one-exponential paths (see
    sa_set_one_paths in sa.h).  Returns the previous setting."""
    prev = ctypes.c_int()
    _check(_lib.sa_set_one_paths(int(bool(enable)), ctypes.byref(prev)))
    return bool(prev.value)


def sa_layout_build(pattern: Union[str, int], n: int, l: int, c: int = 1, block: int = 64) -> Layout:
    pid = PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)
    h = ctypes.c_void_p()
    _check(_lib.sa_layout_build(pid, n, l, c, block, ctypes.byref(h)))
    return Layout(h.value, pattern, n, l, c, block)


def sa_layout_info(layout: Layout) -> Dict[str, int]:
    return layout.info()


def sa_layout_export(layout: Layout) -> Dict[str, np.ndarray]:
    return layout.export()


def sa_layout_set_residue_view(layout: Layout, enable: bool = True) -> Layout:
    return layout.set_residue_view(enable)


def sa_layout_set_compact_view(layout: Layout, enable: bool = True) -> Layout:
    return layout.set_compact_view(enable)


def sa_layout_view_info(layout: Layout) -> Dict[str, int]:
    return layout.view_info()


def sa_layout_destroy(layout: Layout) -> None:
    layout.close()


def sa_bwd_workspace_size(B: int, H: int, n: int, d: int) -> int:
    return int(_lib.sa_bwd_workspace_size(B, H, n, d))


def _head_array(layouts, H: int):
    if isinstance(layouts, Layout):
        layouts = [layouts] * H
    if len(layouts) != H:
        raise ValueError("need one layout per head (%d), got %d" % (H, len(layouts)))
    arr = (ctypes.c_void_p * H)(*[lay.handle for lay in layouts])
    return arr


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError("dtype %s not supported (float32 or bfloat16)" % t.dtype)


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context in which the binding allocates the outputs and the workspace
    of a call: the stream the call's kernels run on.  torch's caching
    allocator ties a block to the stream it was allocated on, so a workspace
    freed when the call returns is reused only by later work on that same
    stream, which runs after the kernels that read it."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_tensor(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dtype, shape, device))


def sa_fwd(q, k, v, layouts: Union[Layout, Sequence[Layout]], scale: float, o=None, lse=None, stream=None):
    """O, lse = attention over the layouts' allowed pairs.  q, k, v:
    [B, H, n, d] contiguous CUDA tensors (float32 or bfloat16)."""
    import torch
    B, H, n, d = q.shape
    for name, t in (("k", k), ("v", v)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("q", q, q.shape, q.dtype, q.device)
    with _on_stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, n), torch.float32, q.device)
    heads = _head_array(layouts, H)
    _check(_lib.sa_fwd(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                       v.data_ptr(), o.data_ptr(), lse.data_ptr(), _stream_handle(stream, q.device)))
    return o, lse


def sa_bwd(q, k, v, o, lse, do, layouts: Union[Layout, Sequence[Layout]], scale: float,
           dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of L = sum(dO * O), recomputing the weights from lse."""
    import torch
    B, H, n, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, n), torch.float32, q.device)
    ws_bytes = sa_bwd_workspace_size(B, H, n, d)
    with _on_stream(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    heads = _head_array(layouts, H)
    _check(_lib.sa_bwd(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                       v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                       dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                       _stream_handle(stream, q.device)))
    return dq, dk, dv


def sa_bwd_noalloc(q, k, v, o, lse, do, layouts: Union[Layout, Sequence[Layout]], scale: float,
                   dq, dk, dv, stream=None):
    """sa_bwd with the library's own scratch for the row terms: the caller
    passes every output and nothing is allocated (see sa_bwd_noalloc in
    sa.h: one earlier sa_bwd with the same layouts, B and H is needed)."""
    import torch
    B, H, n, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check_tensor("lse", lse, (B, H, n), torch.float32, q.device)
    heads = _head_array(layouts, H)
    _check(_lib.sa_bwd_noalloc(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                               v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                               dk.data_ptr(), dv.data_ptr(), _stream_handle(stream, q.device)))
    return dq, dk, dv


def sparse_attention(q, k, v, layouts: Union[Layout, Sequence[Layout]], scale: float):
    """O = attention over the layouts' allowed pairs, differentiable in q, k
    and v.  Only O and lse are kept for the backward pass, which recomputes
    the attention weights block by block (sa_bwd); no n x n matrix is ever
    stored."""
    return _sparse_attention_fn().apply(q, k, v, layouts, float(scale))


_SPARSE_ATTENTION_FN = None


def _sparse_attention_fn():
    global _SPARSE_ATTENTION_FN
    if _SPARSE_ATTENTION_FN is None:
        import torch

        class SparseAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, layouts, scale):
                o, lse = sa_fwd(q, k, v, layouts, scale)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.layouts, ctx.scale = layouts, scale
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = sa_bwd(q, k, v, o, lse, do.contiguous(), ctx.layouts, ctx.scale)
                return dq, dk, dv, None, None

        _SPARSE_ATTENTION_FN = SparseAttention
    return _SPARSE_ATTENTION_FN


def _bwd_common(q, layouts, workspace, stream):
    import torch
    B, H, n, d = q.shape
    ws_bytes = sa_bwd_workspace_size(B, H, n, d)
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    return B, H, n, d, _head_array(layouts, H), workspace


def sa_bwd_dq_rowterms(q, k, v, o, lse, do, layouts, scale: float, workspace=None, dq=None, stream=None):
    """First kernel of sa_bwd: dQ, and the row terms of every row into
    ``workspace`` (allocated when None).  Returns (dq, workspace)."""
    import torch
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    B, H, n, d, heads, workspace = _bwd_common(q, layouts, workspace, stream)
    _check_tensor("lse", lse, (B, H, n), torch.float32, q.device)
    with _on_stream(stream):
        dq = torch.empty_like(q) if dq is None else dq
    _check_tensor("dq", dq, q.shape, q.dtype, q.device)
    _check(_lib.sa_bwd_dq_rowterms(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(), _stream_handle(stream, q.device)))
    return dq, workspace


def sa_bwd_rowterms(o, lse, do, layouts, scale: float, workspace=None, stream=None):
    """The row terms alone: -D_i = -sum_t dO_it O_it and -lse_i log2(e)
    into ``workspace`` (allocated and returned when None)."""
    import torch
    _check_tensor("do", do, o.shape, o.dtype, o.device)
    B, H, n, d, heads, workspace = _bwd_common(o, layouts, workspace, stream)
    _check_tensor("lse", lse, (B, H, n), torch.float32, o.device)
    _check(_lib.sa_bwd_rowterms(heads, B, H, n, d, _dtype_code(o), float(scale), o.data_ptr(), lse.data_ptr(),
                                do.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream_handle(stream, o.device)))
    return workspace


def sa_bwd_dkdv(q, k, v, do, layouts, scale: float, workspace, dk=None, dv=None, stream=None):
    """dK, dV (needs the row terms in ``workspace``; sa_bwd's second kernel)."""
    import torch
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    B, H, n, d, heads, workspace = _bwd_common(q, layouts, workspace, stream)
    with _on_stream(stream):
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    _check(_lib.sa_bwd_dkdv(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                            v.data_ptr(), do.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            workspace.data_ptr(), workspace.numel(), _stream_handle(stream, q.device)))
    return dk, dv


def sa_bwd_dq(q, k, v, do, layouts, scale: float, workspace, dq=None, stream=None):
    """dQ alone (needs the row terms in ``workspace``)."""
    import torch
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check_tensor(name, t, q.shape, q.dtype, q.device)
    B, H, n, d, heads, workspace = _bwd_common(q, layouts, workspace, stream)
    with _on_stream(stream):
        dq = torch.empty_like(q) if dq is None else dq
    _check_tensor("dq", dq, q.shape, q.dtype, q.device)
    _check(_lib.sa_bwd_dq(heads, B, H, n, d, _dtype_code(q), float(scale), q.data_ptr(), k.data_ptr(),
                          v.data_ptr(), do.data_ptr(), dq.data_ptr(), workspace.data_ptr(),
                          workspace.numel(), _stream_handle(stream, q.device)))
    return dq
