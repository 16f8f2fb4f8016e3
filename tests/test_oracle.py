"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a dense brute force, a closed
form, a special case that reduces to a library routine, an invariant the
pages state, or finite differences.
"""
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests import brute

PATTERNS = ["strided_a", "strided_b", "fixed_a", "fixed_b", "dense"]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def row_count_closed_form(pattern, i, l, c):
    """|S_i| written out per pattern from its definition."""
    if pattern == "strided_a":
        return min(i + 1, l)
    if pattern == "strided_b":
        return i // l + 1
    if pattern == "fixed_a":
        return i % l + 1
    if pattern == "fixed_b":
        return (i // l) * c + max(0, i % l - (l - c) + 1)
    return i + 1


def total_closed_form(pattern, n, l, c):
    """Allowed-pair totals for n = m*l (the O(N sqrt N) count of "Sparse
    Attention and Algorithmic Complexity", written out per pattern)."""
    m = n // l
    assert m * l == n
    if pattern == "strided_a":
        return l * (l + 1) // 2 + (n - l) * l
    if pattern == "strided_b":
        return l * m * (m + 1) // 2
    if pattern == "fixed_a":
        return m * l * (l + 1) // 2
    if pattern == "fixed_b":
        return l * c * m * (m - 1) // 2 + m * c * (c + 1) // 2
    return n * (n + 1) // 2


CASES = [
    # (pattern, n, l, c)
    ("strided_a", 64, 8, 1), ("strided_a", 100, 7, 1), ("strided_a", 40, 64, 1),
    ("strided_b", 64, 8, 1), ("strided_b", 100, 7, 1), ("strided_b", 37, 1, 1),
    ("fixed_a", 64, 8, 1), ("fixed_a", 100, 7, 1), ("fixed_a", 50, 1, 1),
    ("fixed_b", 64, 8, 2), ("fixed_b", 100, 7, 3), ("fixed_b", 96, 16, 16), ("fixed_b", 90, 9, 1),
    ("dense", 64, 1, 1), ("dense", 33, 1, 1),
]


@pytest.mark.parametrize("pattern,n,l,c", CASES)
def test_fwd_matches_dense_bruteforce(pattern, n, l, c):
    d = 8
    # deterministic per case (Python's str hash is salted per process)
    seed = zlib.crc32(repr((pattern, n, l, c)).encode()) % 1000
    q, k, v = rnd((n, d), seed), rnd((n, d), seed + 1), rnd((n, d), seed + 2)
    scale = 0.37
    o, lse = oracle.head_fwd(pattern, l, c, q, k, v, scale)
    m = brute.mask(pattern, n, l, c)
    o_ref, lse_ref, _ = brute.attention(q, k, v, m, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=1e-12, atol=1e-12)
    assert np.all(lse[~fin] == -np.inf)


def test_fwd_tiny_workload_bruteforce():
    """The whole tiny workload (N=256, l=16, d=64) against the brute force."""
    n, d, l = 256, 64, 16
    q, k, v = (rnd((n, d), s, 1 / 8) for s in (1, 2, 3))
    for pattern in ("strided_a", "strided_b"):
        o, lse = oracle.head_fwd(pattern, l, 1, q, k, v, 1.0)
        o_ref, lse_ref, _ = brute.attention(q, k, v, brute.mask(pattern, n, l), 1.0)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("pattern,n,l,c", [
    ("strided_a", 256, 16, 1), ("strided_b", 256, 16, 1), ("fixed_a", 384, 128, 32),
    ("fixed_b", 384, 128, 32), ("fixed_b", 120, 12, 5), ("strided_a", 3072, 128, 1),
    ("strided_b", 3072, 128, 1), ("dense", 300, 1, 1), ("fixed_b", 1024, 128, 128),
])
def test_row_counts_closed_form(pattern, n, l, c):
    cnt = oracle.row_counts(pattern, n, l, c)
    exp = np.array([row_count_closed_form(pattern, i, l, c) for i in range(n)])
    assert np.array_equal(cnt, exp)
    if n % l == 0:
        assert int(cnt.sum()) == total_closed_form(pattern, n, l, c)
    if pattern == "fixed_b":
        assert int((cnt == 0).sum()) == l - c


@pytest.mark.parametrize("pattern,n,l,c", [
    ("strided_a", 96, 8, 1), ("strided_b", 96, 8, 1), ("fixed_a", 96, 8, 1), ("fixed_b", 96, 8, 3),
])
def test_zero_queries_give_uniform_weights(pattern, n, l, c):
    """Q = 0: all scores equal, so O_i is the mean of V over S_i and
    lse_i = ln |S_i| (|S_i| from the closed form)."""
    d = 5
    q = np.zeros((n, d))
    k, v = rnd((n, d), 7), rnd((n, d), 8)
    o, lse = oracle.head_fwd(pattern, l, c, q, k, v, 1.0)
    for i in range(n):
        cnt = row_count_closed_form(pattern, i, l, c)
        if cnt == 0:
            assert lse[i] == -np.inf and np.all(o[i] == 0)
            continue
        assert abs(lse[i] - math.log(cnt)) < 1e-12
    # mean over S_i, with S_i from the brute-force mask
    m = brute.mask(pattern, n, l, c)
    for i in range(n):
        if m[i].any():
            np.testing.assert_allclose(o[i], v[m[i]].mean(axis=0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("pattern,l,c", [
    ("strided_a", 1, 1), ("strided_b", 4096, 1), ("fixed_a", 1, 1),
])
def test_special_cases_self_only(pattern, l, c):
    """Patterns that reduce to attending only j = i: O = V exactly, lse = s_ii."""
    n, d = 70, 6
    q, k, v = rnd((n, d), 11), rnd((n, d), 12), rnd((n, d), 13)
    scale = 0.8
    o, lse = oracle.head_fwd(pattern, l, c, q, k, v, scale)
    np.testing.assert_allclose(o, v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, scale * np.sum(q * k, axis=1), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("pattern,l,c", [
    ("strided_a", 4096, 1), ("strided_b", 1, 1), ("fixed_a", 4096, 1), ("fixed_b", 8, 8),
    ("dense", 1, 1),
])
def test_special_cases_dense_causal_vs_sdpa(pattern, l, c):
    """Patterns that reduce to full causal attention match torch's
    scaled_dot_product_attention(is_causal=True) on the CPU in fp64."""
    n, d = 80, 16
    q, k, v = rnd((n, d), 21), rnd((n, d), 22), rnd((n, d), 23)
    scale = 0.25
    o, lse = oracle.head_fwd(pattern, l, c, q, k, v, scale)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-11, atol=1e-12)
    s = scale * (q @ k.T)
    s[np.triu_indices(n, 1)] = -np.inf
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(s), dim=1).numpy(), rtol=1e-12)


@pytest.mark.parametrize("pattern,n,l,c", [
    ("strided_a", 128, 16, 1), ("strided_b", 128, 16, 1), ("fixed_a", 128, 32, 1),
    ("fixed_b", 128, 32, 8),
])
def test_weights_sum_to_one_and_value_shift(pattern, n, l, c):
    """Softmax weights sum to one ("희소 어텐션 (Sparse Attention)"): with V a
    column of ones O = 1 on every non-empty row, and adding u to every V row
    adds u to every non-empty O row."""
    d = 4
    q, k = rnd((n, d), 31, 2.0), rnd((n, d), 32, 2.0)
    ones = np.ones((n, d))
    o1, lse = oracle.head_fwd(pattern, l, c, q, k, ones, 1.0)
    ne = np.isfinite(lse)
    np.testing.assert_allclose(o1[ne], 1.0, rtol=0, atol=1e-13)
    assert np.all(o1[~ne] == 0)
    v = rnd((n, d), 33)
    u = np.array([3.0, -1.5, 0.25, 7.0])
    o_a, _ = oracle.head_fwd(pattern, l, c, q, k, v, 1.0)
    o_b, _ = oracle.head_fwd(pattern, l, c, q, k, v + u, 1.0)
    np.testing.assert_allclose(o_b[ne] - o_a[ne], np.broadcast_to(u, o_a[ne].shape), atol=1e-12)


def _bmm(a, b):
    return (a.astype(np.int64) @ b.astype(np.int64)) > 0


@pytest.mark.parametrize("n,l", [(256, 16), (300, 17), (1024, 32), (96, 96)])
def test_two_step_reachability_strided(n, l):
    """"Factorized Attention Patterns": with the two strided heads every
    position reaches every earlier one in two steps, in either order."""
    a = oracle.mask_dense("strided_a", n, l)
    b = oracle.mask_dense("strided_b", n, l)
    tri = np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(_bmm(a, b), tri)
    assert np.array_equal(_bmm(b, a), tri)
    assert not a.all() or l >= n


@pytest.mark.parametrize("n,l,c", [(256, 16, 4), (300, 20, 1), (1024, 128, 32), (64, 8, 8)])
def test_two_step_reachability_fixed(n, l, c):
    """Fixed pattern: information flows j -> k through head A and k -> i through
    head B (with the residual path as identity), covering the causal
    triangle.  The reverse order does not, unless c = l."""
    a = oracle.mask_dense("fixed_a", n, l, c)
    b = oracle.mask_dense("fixed_b", n, l, c)
    eye = np.eye(n, dtype=bool)
    tri = np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(_bmm(eye | b, eye | a), tri)
    if c < l and n > l:
        assert not np.array_equal(_bmm(eye | a, eye | b), tri)


def test_two_step_reachability_witness_large():
    """Up to N=4096 with the closed-form middle position k instead of a
    matrix product: strided k = i - l*floor((i-j)/l); fixed k = i in the same
    chunk, else the last position of j's chunk."""
    n, l, c = 4096, 64, 16
    rng = np.random.default_rng(5)
    ii = rng.integers(0, n, 4000)
    jj = (rng.random(4000) * (ii + 1)).astype(np.int64)
    for i, j in zip(ii.tolist(), jj.tolist()):
        k = i - l * ((i - j) // l)
        assert oracle.allowed("strided_b", i, k, l) and oracle.allowed("strided_a", k, j, l)
        k2 = j + l * ((i - j) // l)
        assert oracle.allowed("strided_a", i, k2, l) and oracle.allowed("strided_b", k2, j, l)
        if i // l == j // l:
            assert oracle.allowed("fixed_a", i, j, l, c)
        else:
            k3 = (j // l) * l + l - 1
            assert oracle.allowed("fixed_b", i, k3, l, c) and oracle.allowed("fixed_a", k3, j, l, c)


@pytest.mark.parametrize("pattern,n,l,c", [
    ("strided_a", 24, 5, 1), ("strided_b", 24, 5, 1), ("fixed_a", 24, 6, 1), ("fixed_b", 24, 6, 2),
    ("dense", 20, 1, 1),
])
def test_bwd_finite_differences(pattern, n, l, c):
    """Analytic gradients of L = sum(dO * O) against central differences."""
    d = 4
    q, k, v, do = (rnd((n, d), 40 + t) for t in range(4))
    scale = 0.7
    dq, dk, dv, o, lse = oracle.head_bwd(pattern, l, c, q, k, v, do, scale)

    def loss(qq, kk, vv):
        oo, _ = oracle.head_fwd(pattern, l, c, qq, kk, vv, scale)
        return float(np.sum(oo * do))

    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-30)
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("pattern,n,l,c", [
    ("strided_a", 200, 16, 1), ("strided_b", 200, 16, 1), ("fixed_a", 200, 32, 1),
    ("fixed_b", 200, 32, 8),
])
def test_bwd_sum_identities(pattern, n, l, c):
    """sum_j dK_j = 0 (each row of dS sums to zero) and sum_j dV_j equals the
    sum of dO over non-empty rows (each row of P sums to one)."""
    d = 8
    q, k, v, do = (rnd((n, d), 50 + t, 0.5) for t in range(4))
    dq, dk, dv, o, lse = oracle.head_bwd(pattern, l, c, q, k, v, do, 1.0)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    ne = np.isfinite(lse)
    np.testing.assert_allclose(dv.sum(axis=0), do[ne].sum(axis=0), atol=1e-11)


def test_bwd_sampled_rows_match_full():
    """The sampled mode (used at full sizes) equals the full computation."""
    n, d, l, c = 300, 8, 32, 8
    q, k, v, do = (rnd((n, d), 60 + t) for t in range(4))
    full = oracle.head_bwd("fixed_b", l, c, q, k, v, do, 0.5)
    rows = [0, 5, 95, 96, 150, 299]
    part = oracle.head_bwd("fixed_b", l, c, q, k, v, do, 0.5, qrows=rows, kcols=rows)
    for a in range(3):
        np.testing.assert_array_equal(part[a][rows], full[a][rows])


def test_bwd_against_autograd_of_bruteforce():
    """dQ, dK, dV against torch autograd through the dense brute force (fp64)."""
    n, d, l = 48, 6, 8
    for pattern in ("strided_a", "strided_b", "fixed_a", "fixed_b"):
        q, k, v, do = (rnd((n, d), 70 + t) for t in range(4))
        m = torch.from_numpy(brute.mask(pattern, n, l, 3))
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        s = 0.9 * tq @ tk.T
        s = s.masked_fill(~m, float("-inf"))
        p = torch.softmax(s, dim=1)
        p = torch.nan_to_num(p, nan=0.0)
        o = p @ tv
        (o * torch.from_numpy(do)).sum().backward()
        dq, dk, dv, _, _ = oracle.head_bwd(pattern, l, 3, q, k, v, do, 0.9)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def _random_oracle_cases(count=30, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        p = str(rng.choice(["strided_a", "strided_b", "fixed_a", "fixed_b", "dense"]))
        n = int(rng.integers(1, 97))
        l = int(rng.integers(1, n + 9))
        c = int(rng.integers(1, l + 1)) if p == "fixed_b" else 1
        d = int(rng.integers(1, 9))
        scale = float(rng.choice([0.25, 1.0, 2.0]))
        out.append((p, n, l, c, d, scale))
    return out


@pytest.mark.parametrize("pattern,n,l,c,d,scale", _random_oracle_cases())
def test_random_fwd_bwd_against_autograd_of_bruteforce(pattern, n, l, c, d, scale):
    """Seeded random (pattern, n, l, c, d, scale): the oracle's O, lse and
    gradients against the dense brute force and torch autograd through it
    (fp64), including empty rows and l beyond n."""
    seed = int(1000 * scale) + n * 7 + l * 13 + c + d
    q, k, v, do = (rnd((n, d), seed + t) for t in range(4))
    m = brute.mask(pattern, n, l, c)
    o_ref, lse_ref, _ = brute.attention(q, k, v, m, scale)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    sc = (scale * tq @ tk.T).masked_fill(~torch.from_numpy(m), float("-inf"))
    pr = torch.nan_to_num(torch.softmax(sc, dim=1), nan=0.0)
    ((pr @ tv) * torch.from_numpy(do)).sum().backward()
    dq, dk, dv, o, lse = oracle.head_bwd(pattern, l, c, q, k, v, do, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin) and np.all(lse[~fin] == -np.inf)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=1e-11, atol=1e-12)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("pattern,n,l,c,T", [
    ("strided_a", 256, 16, 1, 16), ("strided_b", 256, 16, 1, 16), ("fixed_a", 512, 128, 32, 64),
    ("fixed_b", 512, 128, 32, 64), ("strided_b", 384, 40, 1, 32), ("fixed_b", 320, 20, 7, 16),
])
def test_block_layout_matches_bruteforce_mask(pattern, n, l, c, T):
    """The oracle's block view equals the brute-force mask cut into T x T tiles."""
    m = brute.mask(pattern, n, l, c)
    lay = oracle.block_layout(pattern, n, l, c, T)
    nb = n // T
    for qb in range(nb):
        tiles = m[qb * T:(qb + 1) * T].reshape(T, nb, T).transpose(1, 0, 2)
        kbs = np.nonzero(tiles.reshape(nb, -1).any(axis=1))[0]
        assert np.array_equal(lay[qb][0], kbs)
        assert np.array_equal(lay[qb][1], tiles[kbs])
    rp, kb2, pop, words = oracle.block_layout_sparse(pattern, n, l, c, T)
    for qb in range(nb):
        assert np.array_equal(kb2[rp[qb]:rp[qb + 1]], lay[qb][0])
        for a, kb in enumerate(lay[qb][0]):
            bits = np.unpackbits(words[rp[qb] + a].view(np.uint8), bitorder="little")[:T * T]
            assert np.array_equal(bits.reshape(T, T).astype(bool), lay[qb][1][a])
            assert pop[rp[qb] + a] == lay[qb][1][a].sum()


def _golden():
    with open(os.path.join(GOLDEN, "workload_blocks.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("entry", _golden()["layouts"], ids=lambda e: e["id"])
def test_block_counts_closed_form(entry):
    """Allowed-block totals of the five workloads against closed forms written
    out in tests/golden/workload_blocks.json (derivations inside)."""
    if entry["n"] > 16384:
        pytest.skip("full audio length is covered by the slow test below")
    rp, kbs, pop, _ = oracle.block_layout_sparse(entry["pattern"], entry["n"], entry["l"],
                                                 entry["c"], entry["block"])
    assert int(rp[-1]) == entry["blocks"]
    assert int(pop.sum()) == total_closed_form(entry["pattern"], entry["n"], entry["l"], entry["c"])


@pytest.mark.slow
@pytest.mark.parametrize("entry", [e for e in _golden()["layouts"] if e["n"] > 16384],
                         ids=lambda e: e["id"])
def test_block_counts_closed_form_audio(entry):
    rp, kbs, pop, _ = oracle.block_layout_sparse(entry["pattern"], entry["n"], entry["l"],
                                                 entry["c"], entry["block"])
    assert int(rp[-1]) == entry["blocks"]
    assert int(pop.sum()) == total_closed_form(entry["pattern"], entry["n"], entry["l"], entry["c"])


def test_pages_dense_memory_figure():
    """"Reducing Memory Constraints with Deep Attention": one N x N fp32 matrix
    per layer and head for 64x64x3 images, 64 layers, 4 heads is about 154 GB."""
    g = _golden()["pages"]["dense_attention_memory"]
    n = 64 * 64 * 3
    nbytes = n * n * g["layers"] * g["heads"] * 4
    assert round(nbytes / 1e9) == g["gigabytes"] or int(nbytes / 1e9) == g["gigabytes"]
