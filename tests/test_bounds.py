"""Pins of the elementwise tolerance (tests/bounds.py) the GPU parity tests
use: it must hold for results that carry exactly the bf16 rounding the
kernels perform (simulated here in fp64 with torch's bf16 rounding), and it
must reject results with a planted mistake (the oracle run on a pattern
that drops keys, or a gradient with one block's sign flipped)."""
import numpy as np
import pytest
import torch

import oracle
from tests import bounds, brute


def bf16(a):
    """Round to bf16 (nearest even) and back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(torch.float64).numpy()


def inputs(n, d, seed, std=None):
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(d) if std is None else std
    q, k, v = (bf16(rng.standard_normal((n, d)) * s) for _ in range(3))
    do = bf16(rng.standard_normal((n, d)))
    return q, k, v, do


def simulated_kernel(pattern, l, c, q, k, v, do, scale):
    """The forward and backward with the kernels' rounding steps: P rounded
    to bf16 before P V (its sum in full precision), O rounded to bf16, D
    formed from the rounded O, P and dS rounded to bf16 before their
    products, every output rounded to bf16."""
    m = brute.mask(pattern, q.shape[0], l, c)
    s = scale * (q @ k.T)
    s = np.where(m, s, -np.inf)
    mx = s.max(1, keepdims=True)
    empty = ~m.any(1)
    mx[empty] = 0.0
    e = np.where(m, np.exp(s - mx), 0.0)
    z = e.sum(1, keepdims=True)
    z[empty] = 1.0
    o = bf16((bf16(e) @ v) / z)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, mx[:, 0] + np.log(z[:, 0]))
    p = e / z
    dd = (do * o).sum(1)
    ds = bf16(p * (do @ v.T - dd[:, None]))
    return {"o": o, "lse": lse, "dq": bf16(scale * ds @ k), "dk": bf16(scale * ds.T @ q), "dv": bf16(bf16(p).T @ do)}


def within(res, ref, bnd):
    return all(np.all(np.abs(res[t] - ref[t]) <= bnd[t]) for t in ("o", "dq", "dk", "dv"))


CASES = [("strided_a", 256, 16, 1, 16, None, 1.0), ("strided_b", 256, 16, 1, 16, None, 1.0),
         ("fixed_a", 192, 32, 1, 8, None, 0.5), ("fixed_b", 192, 32, 8, 8, None, 1.0),
         ("dense", 128, 1, 1, 16, 1.0, 1.0),            # sharp logits
         ("strided_b", 200, 7, 1, 8, 3.0, 0.5)]          # nearly one-hot rows


def oracle_all(pattern, l, c, q, k, v, do, scale):
    dq, dk, dv, o, lse = oracle.head_bwd(pattern, l, c, q, k, v, do, scale)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("pattern,n,l,c,d,std,scale", CASES)
def test_bound_holds_for_the_kernels_rounding(pattern, n, l, c, d, std, scale):
    q, k, v, do = inputs(n, d, seed=n + l + d, std=std)
    ref = oracle_all(pattern, l, c, q, k, v, do, scale)
    bnd = bounds.error_bounds(pattern, l, c, q, k, v, do, scale, ref["o"], ref["lse"])
    sim = simulated_kernel(pattern, l, c, q, k, v, do, scale)
    for t in ("o", "dq", "dk", "dv"):
        over = np.abs(sim[t] - ref[t]) - bnd[t]
        assert over.max() <= 0.0, (t, over.max())
    # and it is not vacuous: well below the size of the (non-zero) values,
    # but where the softmax is nearly one-hot (dQ, dK tiny differences)
    if std is not None and std > 1.0:
        return
    for t in ("o", "dq", "dk", "dv"):
        nz = ref[t] != 0
        assert np.median(bnd[t][nz]) < 0.2 * np.median(np.abs(ref[t][nz])), t


@pytest.mark.parametrize("pattern,n,l,c,d,std,scale", CASES[:4])
def test_bound_rejects_a_dropped_key(pattern, n, l, c, d, std, scale):
    """The oracle on a pattern that loses some allowed keys (a window one
    shorter, a stride one larger, a chunk one shorter, one summary column
    fewer) is caught by the bound of the true pattern."""
    q, k, v, do = inputs(n, d, seed=n + l + d, std=std)
    ref = oracle_all(pattern, l, c, q, k, v, do, scale)
    bnd = bounds.error_bounds(pattern, l, c, q, k, v, do, scale, ref["o"], ref["lse"])
    wrong = {"strided_a": (l - 1, c), "strided_b": (l + 1, c), "fixed_a": (l - 1, c), "fixed_b": (l, c - 1)}[pattern]
    bad = oracle_all(pattern, wrong[0], wrong[1], q, k, v, do, scale)
    assert not within(bad, ref, bnd)


def test_bound_rejects_one_flipped_block():
    """A gradient whose 32 rows of one block come out negated fails."""
    q, k, v, do = inputs(256, 16, seed=3)
    ref = oracle_all("strided_b", 16, 1, q, k, v, do, 1.0)
    bnd = bounds.error_bounds("strided_b", 16, 1, q, k, v, do, 1.0, ref["o"], ref["lse"])
    for t in ("dq", "dk", "dv"):
        bad = dict(ref)
        bad[t] = ref[t].copy()
        bad[t][96:128] *= -1.0
        assert not within(bad, ref, bnd), t
