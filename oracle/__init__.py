"""fp64 CPU oracle for causal factorized sparse self-attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product package
``block_sparse_factorized_amd`` never does.  It shares no code with the HIP
path: the arithmetic lives in ``sa_oracle.c`` (plain C, fp64, OpenMP), built
by :func:`build` with gcc and loaded with ctypes.

Sources (page title, section): "OpenAI Sparse Transformer" (agentlenshq.com),
"Factorized Attention Patterns" and "Sparse Attention and Algorithmic
Complexity"; "Генеративное моделирование с разреженными трансформерами"
(pcnews.ru), "Разреженное внимание"; "희소 어텐션 (Sparse Attention)"
(molayo1419.me) for dot-product scores and a softmax whose weights sum to
one; "[논문 리뷰] Generating Long Sequences with Sparse Transformers"
(nubint.ai), ABSTRACT item (b), for the recomputing backward.

Pinned by the ``-m "not gpu"`` tests against: dense masked softmax brute force
(numpy, tiny N), closed-form allowed-pair counts, special cases that reduce to
O = V or to dense causal attention (torch SDPA on CPU in fp64), the
weights-sum-to-one and value-shift invariants, the two-step reachability of
the factorized patterns, and central finite differences for the backward.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

# The oracle's own numbering of the patterns (its C file defines the same).
PATTERNS = {
    "strided_a": 0,
    "strided_b": 1,
    "fixed_a": 2,
    "fixed_b": 3,
    "dense": 4,
}

_lib = None


def build() -> str:
    """Compile sa_oracle.c into oracle/_build/liboracle.so (gcc, -O2, OpenMP)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, dbl, vp, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.oracle_allowed.argtypes = [cint, i64, i64, i64, i64]
    lib.oracle_allowed.restype = cint
    lib.oracle_head_fwd.argtypes = [cint, i64, i64, i64, cint, dbl, vp, vp, vp, vp, i64, vp, vp]
    lib.oracle_head_fwd.restype = None
    lib.oracle_head_bwd.argtypes = [cint, i64, i64, i64, cint, dbl, vp, vp, vp, vp,
                                    vp, i64, vp, i64, vp, vp, vp, vp, vp]
    lib.oracle_head_bwd.restype = None
    lib.oracle_mask_dense.argtypes = [cint, i64, i64, i64, vp]
    lib.oracle_mask_dense.restype = None
    lib.oracle_row_counts.argtypes = [cint, i64, i64, i64, vp]
    lib.oracle_row_counts.restype = None
    lib.oracle_block_layout.argtypes = [cint, i64, i64, i64, i64, vp, vp, vp]
    lib.oracle_block_layout.restype = None
    lib.oracle_block_layout_sparse.argtypes = [cint, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_block_layout_sparse.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = cint
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _pid(pattern) -> int:
    return PATTERNS[pattern] if isinstance(pattern, str) else int(pattern)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def allowed(pattern, i: int, j: int, l: int, c: int = 1) -> bool:
    return bool(_load().oracle_allowed(_pid(pattern), i, j, l, c))


def mask_dense(pattern, n: int, l: int, c: int = 1) -> np.ndarray:
    """Boolean [n, n] mask of the pattern (small n only)."""
    m = np.zeros((n, n), dtype=np.uint8)
    _load().oracle_mask_dense(_pid(pattern), l, c, n, _ptr(m))
    return m.astype(bool)


def row_counts(pattern, n: int, l: int, c: int = 1) -> np.ndarray:
    """|S_i| for every row i."""
    out = np.zeros(n, dtype=np.int64)
    _load().oracle_row_counts(_pid(pattern), l, c, n, _ptr(out))
    return out


def head_fwd(pattern, l: int, c: int, q, k, v, scale: float,
             rows: Optional[Sequence[int]] = None):
    """Forward of one head.  q, k, v: [n, d].  Returns (o [n,d], lse [n]) in fp64.

    With ``rows`` only those rows are computed (the others stay 0 / nan)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    if k.shape != (n, d) or v.shape != (n, d):
        raise ValueError("q, k, v must all be [n, d]")
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.full(n, np.nan, dtype=np.float64)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    _load().oracle_head_fwd(_pid(pattern), l, c, n, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(r), 0 if r is None else len(r), _ptr(o), _ptr(lse))
    return o, lse


def head_bwd(pattern, l: int, c: int, q, k, v, dout, scale: float,
             qrows: Optional[Sequence[int]] = None, kcols: Optional[Sequence[int]] = None):
    """Backward of one head.  Returns (dq, dk, dv, o, lse) in fp64; the
    forward is recomputed inside.  With qrows/kcols only those rows of dq and
    of dk/dv are computed."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    n, d = q.shape
    if k.shape != (n, d) or v.shape != (n, d) or dout.shape != (n, d):
        raise ValueError("q, k, v, dout must all be [n, d]")
    dq = np.zeros((n, d)); dk = np.zeros((n, d)); dv = np.zeros((n, d))
    o = np.zeros((n, d)); lse = np.zeros(n)
    qr = None if qrows is None else np.ascontiguousarray(np.asarray(qrows, dtype=np.int64))
    kc = None if kcols is None else np.ascontiguousarray(np.asarray(kcols, dtype=np.int64))
    _load().oracle_head_bwd(_pid(pattern), l, c, n, d, float(scale), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(dout), _ptr(qr), 0 if qr is None else len(qr), _ptr(kc),
                            0 if kc is None else len(kc), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(o), _ptr(lse))
    return dq, dk, dv, o, lse


def block_layout(pattern, n: int, l: int, c: int, T: int):
    """Dense block view for moderate n: list of (kb list, [nblk,T,T] bool masks)
    per query block, straight from the predicate."""
    assert n % T == 0
    nb = n // T
    nblk = np.zeros(nb, dtype=np.int64)
    kbs = np.zeros(nb * nb, dtype=np.int64)
    bits = np.zeros(nb * nb * T * T, dtype=np.uint8)
    _load().oracle_block_layout(_pid(pattern), l, c, n, T, _ptr(nblk), _ptr(kbs), _ptr(bits))
    out = []
    for qb in range(nb):
        m = int(nblk[qb])
        ks = kbs[qb * nb: qb * nb + m].copy()
        tiles = bits[qb * nb * T * T: (qb * nb + m) * T * T].reshape(m, T, T).astype(bool)
        out.append((ks, tiles))
    return out


def block_layout_sparse(pattern, n: int, l: int, c: int, T: int):
    """Block view for any n: returns (row_ptr [nqb+1], kbs [nnz], pop [nnz],
    words [nnz, ceil(T*T/64)] uint64) with the row-major bit order
    bit (r*T+s) % 64 of word (r*T+s) // 64."""
    assert n % T == 0
    nb = n // T
    nw = (T * T + 63) // 64
    lib = _load()
    nblk = np.zeros(nb, dtype=np.int64)
    lib.oracle_block_layout_sparse(_pid(pattern), l, c, n, T, _ptr(nblk), None, None, None, None)
    row_ptr = np.zeros(nb + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(nblk)
    nnz = int(row_ptr[-1])
    kbs = np.zeros(max(nnz, 1), dtype=np.int64)
    pop = np.zeros(max(nnz, 1), dtype=np.int64)
    words = np.zeros((max(nnz, 1), nw), dtype=np.uint64)
    off = np.ascontiguousarray(row_ptr[:-1])
    lib.oracle_block_layout_sparse(_pid(pattern), l, c, n, T, _ptr(nblk), _ptr(off), _ptr(kbs),
                                   _ptr(pop), _ptr(words))
    return row_ptr, kbs[:nnz], pop[:nnz], words[:nnz]


def attention_fwd(q, k, v, head_patterns, scale: float, heads=None, rows=None):
    """Forward over [B, H, n, d] arrays.  head_patterns[h] = (pattern, l, c).
    heads: iterable of (b, h) to compute (default all).  Returns dict
    {(b, h): (o, lse)}."""
    B, H = q.shape[0], q.shape[1]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for (b, h) in todo:
        p, l, c = head_patterns[h]
        out[(b, h)] = head_fwd(p, l, c, q[b, h], k[b, h], v[b, h], scale, rows=rows)
    return out


def attention_bwd(q, k, v, dout, head_patterns, scale: float, heads=None, qrows=None, kcols=None):
    """Backward over [B, H, n, d] arrays; returns {(b, h): (dq, dk, dv, o, lse)}."""
    B, H = q.shape[0], q.shape[1]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for (b, h) in todo:
        p, l, c = head_patterns[h]
        out[(b, h)] = head_bwd(p, l, c, q[b, h], k[b, h], v[b, h], dout[b, h], scale,
                               qrows=qrows, kcols=kcols)
    return out
