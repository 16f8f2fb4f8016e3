"""Dense brute force used only to pin the oracle on tiny inputs.

It builds the whole N x N score matrix, fills disallowed entries with -inf and
takes a row softmax, the way dense masked attention is usually written -- the
opposite of the oracle, which never forms the matrix.  The pattern masks here
are written with numpy broadcasting, separately from the oracle's C
predicates ("OpenAI Sparse Transformer", "Factorized Attention Patterns").
"""
import numpy as np


def mask(pattern: str, n: int, l: int, c: int = 1) -> np.ndarray:
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    causal = j <= i
    if pattern == "strided_a":
        m = (i - j) < l
    elif pattern == "strided_b":
        m = np.mod(i - j, l) == 0
    elif pattern == "fixed_a":
        m = (j // l) == (i // l)
    elif pattern == "fixed_b":
        m = np.mod(j, l) >= (l - c)
    elif pattern == "dense":
        m = np.ones((n, n), dtype=bool)
    else:
        raise ValueError(pattern)
    return causal & m


def attention(q, k, v, m, scale):
    """Dense masked softmax attention in fp64.  Rows with no allowed key give
    O = 0 and lse = -inf."""
    s = scale * (q @ k.T)
    s = np.where(m, s, -np.inf)
    rowmax = s.max(axis=1, keepdims=True)
    empty = ~m.any(axis=1)
    rowmax[empty] = 0.0
    e = np.exp(s - rowmax)
    z = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty[:, None], 0.0, e / z)
        lse = np.where(empty, -np.inf, rowmax[:, 0] + np.log(z[:, 0]))
    return p @ v, lse, p
