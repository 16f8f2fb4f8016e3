"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (written here, per the acceptance rules): forward O within max-abs
2e-2 (bf16 inputs) or 1e-4 (fp32 inputs) of the oracle; lse within 1e-3
(bf16) / 1e-5 (fp32) absolute on non-empty rows and exactly -inf on empty
ones; gradients within 5e-2 relative L2.  Because |O| is small for
N(0,1)/sqrt(d) inputs, O is also held to relative L2 <= 1e-2 (bf16) so a
near-zero output cannot pass, and the "sharp" inputs (N(0,1) at scale 1,
logits with standard deviation about sqrt(d)) are checked the same way.

Local bars, so that one wrong tile cannot hide in a whole-head norm:
* every group of 64 consecutive checked rows (a 64-row block of queries for
  O and dQ, of keys for dK and dV) is held to the same relative L2 bars
  (1e-2 for O, 5e-2 for gradients), against the larger of its own norm and a
  floor of a tenth of the head's RMS block norm (blocks whose reference is
  nearly zero would otherwise turn rounding into large relative errors);
* every element of a head checked whole with n <= 2048 is held to the
  first-order rounding bound of tests/bounds.py (written from the bf16
  rounding steps the kernels take), which also covers inputs whose
  gradients are tiny differences of large terms, where relative bars fail
  whatever the kernel does.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import bounds
from workloads import WORKLOADS, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_factorized_amd as sa

DEV = "cuda:0"


def layouts_for(patterns, n, block):
    cache = {}
    out = []
    for (p, l, c) in patterns:
        key = (p, l, c)
        if key not in cache:
            cache[key] = sa.sa_layout_build(p, n, l, c, block=block)
        out.append(cache[key])
    return out


def run(inputs, patterns, block, scale, backward, lays=None):
    n = inputs["q"].shape[2]
    if lays is None:
        lays = layouts_for(patterns, n, block)
    q, k, v = (inputs[t].to(DEV) for t in ("q", "k", "v"))
    o, lse = sa.sa_fwd(q, k, v, lays, scale)
    res = {"o": o, "lse": lse}
    if backward:
        do = inputs["do"].to(DEV)
        dq, dk, dv = sa.sa_bwd(q, k, v, o, lse, do, lays, scale)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    res = {k2: v2.cpu() for k2, v2 in res.items()}
    res["layouts"] = lays
    return res


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# Absolute floor of the per-block norm (an RMS of 1e-4 per element), for heads
# whose reference is exactly zero (one allowed key per row: dQ = dK = 0).
BLOCK_ABS_FLOOR_RMS = 1e-4


def block_rel_l2(g, r):
    """Largest relative L2 error over groups of 64 consecutive rows, each
    against max(its own norm, a tenth of the RMS group norm, an absolute
    floor)."""
    rows = g.shape[0]
    groups = max(1, -(-rows // 64))
    floor = max(0.1 * np.linalg.norm(r) / np.sqrt(groups), BLOCK_ABS_FLOOR_RMS * np.sqrt(min(rows, 64) * g.shape[1]))
    worst = 0.0
    for a in range(0, rows, 64):
        den = max(np.linalg.norm(r[a:a + 64]), floor)
        worst = max(worst, np.linalg.norm(g[a:a + 64] - r[a:a + 64]) / den)
    return worst


# Heads checked whole up to this length also get the elementwise bound.
ELEMENT_BOUND_MAX_N = 2048


def compare_head(inputs, res, b, h, pattern, scale, backward, fp32, rows=None, kcols=None,
                 grad_rel=("dq", "dk", "dv")):
    """Compare head (b, h).  rows: query rows checked (default all); kcols:
    key rows whose dK/dV are checked (default: the same as rows).  grad_rel:
    the gradients held to the relative bars (all of them but for inputs
    whose gradients are tiny differences of large terms, which the
    elementwise bound alone checks)."""
    pat, l, c = pattern
    q, k, v = (to_f64(inputs[t][b, h]) for t in ("q", "k", "v"))
    o_tol = 1e-4 if fp32 else 2e-2
    lse_tol = 1e-5 if fp32 else 1e-3
    kcols = rows if kcols is None else kcols
    if backward:
        do = to_f64(inputs["do"][b, h])
        rdq, rdk, rdv, ro, rlse = oracle.head_bwd(pat, l, c, q, k, v, do, scale, qrows=rows, kcols=kcols)
    else:
        ro, rlse = oracle.head_fwd(pat, l, c, q, k, v, scale, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    ksel = slice(None) if kcols is None else np.asarray(kcols)
    go = to_f64(res["o"][b, h])[sel]
    glse = res["lse"][b, h].double().numpy()[sel]
    ro, rlse = ro[sel], rlse[sel]
    err = np.abs(go - ro).max()
    assert err <= o_tol, ("O max-abs", b, h, pat, err)
    if not fp32:
        assert rel_l2(go, ro) <= 1e-2, ("O rel-L2", b, h, pat, rel_l2(go, ro))
        assert block_rel_l2(go, ro) <= 1e-2, ("O block rel-L2", b, h, pat, block_rel_l2(go, ro))
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(glse), fin), ("lse finiteness", b, h, pat)
    assert np.all(glse[~fin] == -np.inf)
    assert np.all(go[~fin] == 0.0)
    if fin.any():
        lerr = np.abs(glse[fin] - rlse[fin]).max()
        assert lerr <= lse_tol, ("lse", b, h, pat, lerr)
    if backward:
        for name, r, sl in (("dq", rdq, sel), ("dk", rdk, ksel), ("dv", rdv, ksel)):
            g = to_f64(res[name][b, h])[sl]
            assert np.all(np.isfinite(g))
            if name in grad_rel:
                e = rel_l2(g, r[sl])
                assert e <= 5e-2, (name, b, h, pat, e)
                e = block_rel_l2(g, r[sl])
                assert e <= 5e-2, (name + " block", b, h, pat, e)
    n = q.shape[0]
    if not fp32 and rows is None and kcols is None and n <= ELEMENT_BOUND_MAX_N:
        do = to_f64(inputs["do"][b, h]) if backward else np.zeros_like(q)
        bound = bounds.error_bounds(pat, l, c, q, k, v, do, scale, ro, rlse, backward=backward)
        checks = [("o", to_f64(res["o"][b, h]), ro)]
        if backward:
            checks += [("dq", to_f64(res["dq"][b, h]), rdq), ("dk", to_f64(res["dk"][b, h]), rdk),
                       ("dv", to_f64(res["dv"][b, h]), rdv)]
        for name, g, r in checks:
            over = np.abs(g - r) - bound[name]
            assert over.max() <= 0.0, (name + " elementwise bound", b, h, pat, float(over.max()),
                                       np.unravel_index(int(over.argmax()), over.shape))


def sample_heads(B, H):
    hs = {(0, 0), (0, 1 % H), (B - 1, H - 1), (B - 1, max(H - 2, 0))}
    return sorted(hs)


def test_tiny_workload_full():
    w = WORKLOADS["tiny"]
    x = workloads.make_inputs(w)
    res = run(x, w.head_patterns(), w.block, 1.0, backward=False)
    for b in range(w.batch):
        for h in range(w.heads):
            compare_head(x, res, b, h, w.head_patterns()[h], 1.0, False, fp32=True)


# ---------------------------------------------------------------------------
# Reduced sizes of every workload shape: whole tensors against the oracle.

@pytest.mark.parametrize("name,n", [("img32", 1024), ("text", 1024), ("img64", 1024), ("audio", 2048)])
def test_workload_shapes_reduced_full_compare(name, n):
    w = WORKLOADS[name]
    shape = (2, w.heads if w.heads <= 4 else 4, n, w.d)
    x = workloads.make_inputs(w, shape=shape)
    pats = w.head_patterns()[: shape[1]]
    res = run(x, pats, w.block, 1.0, backward=True)
    for b in range(shape[0]):
        for h in range(shape[1]):
            compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


# ---------------------------------------------------------------------------
# Edge cases.

EDGE = [
    # (patterns per head, n, d, note)
    ([("strided_a", 100, 1), ("strided_b", 100, 1)], 640, 64, "stride not a multiple of the block"),
    ([("strided_a", 37, 1), ("strided_b", 37, 1)], 448, 128, "odd stride, d=128"),
    ([("fixed_a", 96, 17), ("fixed_b", 96, 17)], 576, 64, "fixed, chunk not a block multiple"),
    ([("fixed_b", 256, 8)], 512, 64, "fixed B: first query blocks entirely empty"),
    ([("fixed_b", 64, 64)], 256, 64, "fixed B with c = l is dense causal"),
    ([("strided_a", 1, 1)], 192, 64, "window 1: O = V"),
    ([("strided_b", 100000, 1)], 192, 128, "stride beyond n: O = V"),
    ([("dense", 1, 1), ("strided_a", 64, 1)], 320, 64, "dense causal next to strided"),
    ([("strided_a", 64, 1)], 64, 64, "a single block"),
    ([("fixed_a", 128, 1), ("fixed_b", 128, 32), ("strided_a", 128, 1), ("strided_b", 128, 1)], 768, 64,
     "four layouts in one call"),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[3] for e in EDGE])
def test_edge_cases(case):
    pats, n, d, _ = case
    H = len(pats)
    x = workloads.custom_inputs((2, H, n, d), torch.bfloat16, seed=n + d + H)
    res = run(x, pats, 64, 1.0, backward=True)
    for b in range(2):
        for h in range(H):
            compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


def test_most_heads_and_layouts_in_one_call():
    """The largest call the head table holds: 256 heads over 8 distinct
    layouts (every pattern, views among them), forward and backward, every
    head against the oracle."""
    n, d = 256, 64
    pats = [("strided_a", 64, 1), ("strided_b", 64, 1), ("fixed_a", 64, 16), ("fixed_b", 64, 16),
            ("dense", 1, 1), ("strided_a", 3, 1), ("strided_b", 32, 1), ("fixed_b", 128, 4)]
    base = layouts_for(pats, n, 64)
    base[6].set_residue_view(True)   # strided B, l = 32: 8-row residue classes
    base[7].set_compact_view(True)   # fixed B, c = 4
    H = 256
    heads = [pats[h % 8] for h in range(H)]
    x = workloads.custom_inputs((1, H, n, d), torch.bfloat16, seed=41)
    res = run(x, heads, 64, 1.0, backward=True, lays=[base[h % 8] for h in range(H)])
    for h in range(H):
        compare_head(x, res, 0, h, heads[h], 1.0, True, fp32=False)


def test_fixed_b_empty_rows_exact():
    """Rows with no allowed key: O = 0 and lse = -inf exactly, zero gradients."""
    n, l, c = 512, 128, 32
    x = workloads.custom_inputs((1, 1, n, 64), torch.bfloat16, seed=5)
    res = run(x, [("fixed_b", l, c)], 64, 1.0, backward=True)
    empty = np.arange(l - c)
    assert torch.all(res["o"][0, 0, empty] == 0)
    assert torch.all(res["lse"][0, 0, empty] == -math.inf)
    assert torch.all(res["dq"][0, 0, empty] == 0)
    compare_head(x, res, 0, 0, ("fixed_b", l, c), 1.0, True, fp32=False)


@pytest.mark.parametrize("scale_kind", ["inv_sqrt_d", "sharp"])
def test_scales_and_sharp_logits(scale_kind):
    n, d = 768, 64
    if scale_kind == "sharp":
        x = workloads.custom_inputs((1, 2, n, d), torch.bfloat16, seed=11, std=1.0)
        scale = 1.0
    else:
        x = workloads.custom_inputs((1, 2, n, d), torch.bfloat16, seed=12, std=1.0)
        scale = 1.0 / math.sqrt(d)
    pats = [("strided_a", 128, 1), ("strided_b", 128, 1)]
    res = run(x, pats, 64, scale, backward=True)
    for h in range(2):
        compare_head(x, res, 0, h, pats[h], scale, True, fp32=False)


@pytest.fixture
def fwd_form():
    """Forces the forward kernel's form for one test, then restores the
    automatic choice."""
    forms = []

    def force(form):
        forms.append(sa.sa_set_fwd_form(form))

    yield force
    if forms:
        sa.sa_set_fwd_form(forms[0])


@pytest.fixture
def split_steps():
    """Forces the chunking of long lists (sa_set_split) for one test, then
    restores the automatic choice."""
    prev = []

    def force(steps):
        prev.append(sa.sa_set_split(steps))

    yield force
    if prev:
        sa.sa_set_split(prev[0])


def _ramp_inputs(kind, n, d, seed):
    """Q rows along one direction u and K rows placed along u by a per-key
    ramp, so scores follow the ramp: "rising" puts every row's max at its
    latest key (each block of the walk moves the running reference),
    "falling" at its first, "spikes" at a few far-out keys of either sign.
    Score differences reach about 700 (about 90 in scaled natural units)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    j = np.arange(n) / n
    if kind == "rising":
        ramp = 90.0 * j
    elif kind == "falling":
        ramp = 90.0 * (1.0 - j)
    else:
        ramp = rng.standard_normal(n) * 0.5
        hit = rng.random(n) < 0.05
        ramp[hit] = rng.choice([-1.0, 1.0], hit.sum()) * rng.uniform(20.0, 90.0, hit.sum())
    q = 8.0 * u[None, :] + 0.1 * rng.standard_normal((n, d))
    k = ramp[:, None] * u[None, :] + 0.1 * rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    do = rng.standard_normal((n, d))
    H = 4
    t = lambda a: torch.from_numpy(np.broadcast_to(a, (1, H, n, d)).copy()).to(torch.bfloat16)
    return {"q": t(q), "k": t(k), "v": t(v), "do": t(do)}


RAMP_PATTERNS = {
    # mostly full blocks: the forward's two-half form
    "full": [("dense", 1, 1), ("dense", 1, 1), ("strided_a", 512, 1), ("fixed_a", 256, 1)],
    # mostly one live half per step: the per-half form
    "sparse": [("strided_b", 128, 1), ("fixed_b", 128, 32), ("strided_b", 64, 1), ("strided_a", 64, 1)],
}


@pytest.mark.parametrize("kind", ["rising", "falling", "spikes"])
@pytest.mark.parametrize("family", ["full", "sparse"])
@pytest.mark.parametrize("form", ["half", "paired"])
@pytest.mark.parametrize("d", [64, 128])
def test_running_reference_moves(kind, family, form, d, fwd_form):
    """The forward's running reference, in each of its two forms (forced,
    whatever the automatic choice would be), at d = 64 and 128: rows whose
    max keeps rising along the walk, rows whose max comes first, and far-out
    spikes; forward and backward.  On these inputs the softmax is nearly
    one-hot, so dQ and dK are tiny differences of large terms (D_i = dO.O
    formed from the bf16-rounded O moves them by more than their own size):
    they are held to the elementwise rounding bound, which scales with the
    terms, and O and dV to every bar."""
    fwd_form(form)
    n = 1024
    x = _ramp_inputs(kind, n, d, seed=5)
    scale = 1.0 / math.sqrt(d)
    pats = RAMP_PATTERNS[family]
    res = run(x, pats, 64, scale, backward=True)
    assert torch.isfinite(res["o"]).all()
    for h in range(4):
        compare_head(x, res, 0, h, pats[h], scale, True, fp32=False, grad_rel=("dv",))


def test_forward_forms_agree():
    """Both forward forms on the same inputs, each against the oracle, and
    against each other to within rounding."""
    n, d = 1024, 64
    pats = [("strided_a", 128, 1), ("strided_b", 128, 1), ("fixed_a", 128, 32), ("fixed_b", 128, 32), ("dense", 1, 1)]
    x = workloads.custom_inputs((1, len(pats), n, d), torch.bfloat16, seed=17)
    outs = {}
    prev = sa.sa_set_fwd_form("half")
    try:
        for form in ("half", "paired"):
            sa.sa_set_fwd_form(form)
            outs[form] = run(x, pats, 64, 1.0, backward=False)
            for h in range(len(pats)):
                compare_head(x, outs[form], 0, h, pats[h], 1.0, False, fp32=False)
    finally:
        sa.sa_set_fwd_form(prev)
    assert rel_l2(outs["half"]["o"].double().numpy(), outs["paired"]["o"].double().numpy()) < 5e-3
    with pytest.raises(sa.SAError):
        sa.sa_set_fwd_form(3)


@pytest.mark.parametrize("d", [64, 128])
def test_one_element_quadrants(d):
    """Layouts whose partial quadrants leave each lane of the forward's score
    layout at most one allowed element (strided B at strides 32, 96 and 100,
    fixed B with one summary column), which take the kernels'
    one-exponential paths, beside fixed B with two summary columns (two in
    one lane: the general path)."""
    n = 1024
    pats = [("strided_b", 32, 1), ("fixed_b", 64, 1), ("strided_b", 96, 1), ("fixed_b", 128, 2),
            ("strided_b", 100, 1)]
    x = workloads.custom_inputs((2, len(pats), n, d), torch.bfloat16, seed=40 + d)
    res = run(x, pats, 64, 1.0 / math.sqrt(d), backward=True)
    for b in range(2):
        for h in range(len(pats)):
            compare_head(x, res, b, h, pats[h], 1.0 / math.sqrt(d), True, fp32=False)


@pytest.fixture
def one_paths():
    """Switches the one-exponential paths for one test, then restores them."""
    prev = []

    def force(enable):
        prev.append(sa.sa_set_one_paths(enable))

    yield force
    if prev:
        sa.sa_set_one_paths(prev[0])


@pytest.mark.parametrize("d", [64, 128])
def test_one_paths_match_general_paths(d, one_paths):
    """The same calls with the forward's and dQ's one-exponential paths on
    and off: O and dQ agree to rounding, dK and dV bit for bit (the dK/dV
    kernel has one path; the row terms the dQ kernel forms for it are the
    same either way), and both runs match the oracle.  Strided B at 128 and
    256 (diagonal blocks in every list) beside strided A and fixed B with
    one summary column."""
    n = 2048
    pats = [("strided_b", 128, 1), ("strided_a", 128, 1), ("strided_b", 256, 1), ("fixed_b", 64, 1)]
    x = workloads.custom_inputs((2, len(pats), n, d), torch.bfloat16, seed=90 + d)
    lays = layouts_for(pats, n, 64)
    one_paths(True)
    r1 = run(x, pats, 64, 1.0 / math.sqrt(d), backward=True, lays=lays)
    sa.sa_set_one_paths(False)
    r0 = run(x, pats, 64, 1.0 / math.sqrt(d), backward=True, lays=lays)
    assert torch.equal(r1["dk"], r0["dk"]) and torch.equal(r1["dv"], r0["dv"])
    for t in ("o", "dq"):
        assert torch.allclose(r1[t].float(), r0[t].float(), rtol=2e-2, atol=2e-3), t
    for res in (r1, r0):
        for b in range(2):
            for h in range(len(pats)):
                compare_head(x, res, b, h, pats[h], 1.0 / math.sqrt(d), True, fp32=False)


def test_fp32_tiny_variants():
    for pats, n in (([("fixed_a", 32, 1), ("fixed_b", 32, 8)], 256), ([("strided_a", 20, 1), ("dense", 1, 1)], 160)):
        x = workloads.custom_inputs((2, 2, n, 64), torch.float32, seed=n, with_dout=False)
        res = run(x, pats, 16, 0.5, backward=False)
        for b in range(2):
            for h in range(2):
                compare_head(x, res, b, h, pats[h], 0.5, False, fp32=True)


def test_deterministic_bitwise_repeat():
    """No atomics: two runs on the same inputs agree bit for bit."""
    w = WORKLOADS["text"]
    x = workloads.make_inputs(w, shape=(2, 4, 2048, 64))
    pats = w.head_patterns()[:4]
    r1 = run(x, pats, 64, 1.0, backward=True)
    r2 = run(x, pats, 64, 1.0, backward=True)
    for t in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(r1[t], r2[t]), t


@pytest.mark.parametrize("pats,n,d", [
    ([("fixed_a", 128, 32), ("fixed_b", 128, 32)], 512, 64),
    ([("fixed_b", 64, 16), ("strided_b", 100, 1)], 256, 64),
    ([("strided_a", 37, 1), ("fixed_b", 96, 17)], 448, 128),
    ([("fixed_b", 256, 8), ("strided_b", 128, 1)], 512, 64),
])
def test_every_output_element_written(pats, n, d):
    """Outputs pre-filled with NaN come back identical to a normal run: every
    element of O, lse, dQ, dK and dV is written (keys no query reaches get
    exact zeros), whatever the pattern leaves empty."""
    H = len(pats)
    x = workloads.custom_inputs((2, H, n, d), torch.bfloat16, seed=n + d)
    lays = layouts_for(pats, n, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full(q.shape[:3], nan, dtype=torch.float32, device=DEV)
    sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, nan) for _ in range(3))
    sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert not torch.isnan(got.float()).any(), nm
        assert torch.equal(got, want), nm


# ---------------------------------------------------------------------------
# Residue view of strided B: the same pairs, walked per residue class.

RESIDUE = [
    # (head patterns, n, d, note); strided B heads use the residue view
    ([("strided_b", 16, 1)], 1024, 64, "n/l = 64: whole blocks"),
    ([("strided_b", 8, 1)], 768, 64, "n/l = 96: ragged last block"),
    ([("strided_b", 64, 1)], 1536, 64, "n/l = 24: one ragged block"),
    ([("strided_b", 4, 1)], 1024, 64, "n/l = 256: four blocks"),
    ([("strided_b", 32, 1)], 2048, 128, "d = 128"),
    ([("strided_a", 16, 1), ("strided_b", 16, 1), ("fixed_b", 64, 16)], 1024, 64,
     "raster and residue-view heads in one call"),
]


def residue_layouts(pats, n):
    lays = layouts_for(pats, n, 64)
    for (p, _, _), lay in zip(pats, lays):
        if p == "strided_b" and not lay.residue_view:
            lay.set_residue_view(True)
    return lays


@pytest.mark.parametrize("case", RESIDUE, ids=[r[3] for r in RESIDUE])
def test_residue_view_matches_oracle(case):
    pats, n, d, _ = case
    H = len(pats)
    x = workloads.custom_inputs((2, H, n, d), torch.bfloat16, seed=7 * n + d + H)
    lays = residue_layouts(pats, n)
    dev = {t: x[t].to(DEV) for t in ("q", "k", "v", "do")}
    o, lse = sa.sa_fwd(dev["q"], dev["k"], dev["v"], lays, 1.0)
    dq, dk, dv = sa.sa_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], lays, 1.0)
    torch.cuda.synchronize()
    res = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    for b in range(2):
        for h in range(H):
            compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


def test_residue_view_every_output_written():
    pats, n, d = [("strided_b", 8, 1), ("strided_a", 8, 1)], 768, 64
    x = workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=99)
    lays = residue_layouts(pats, n)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full(q.shape[:3], nan, dtype=torch.float32, device=DEV)
    sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, nan) for _ in range(3))
    sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert not torch.isnan(got.float()).any(), nm
        assert torch.equal(got, want), nm


@pytest.mark.parametrize("name", ["img64", "audio"])
def test_residue_view_full_size_sampled(name):
    """The workload at full size with its strided-B heads in the residue view."""
    w = WORKLOADS[name]
    x = workloads.make_inputs(w)
    pats = w.head_patterns()
    lays = residue_layouts(pats, w.n)
    res = run(x, pats, w.block, 1.0, backward=True, lays=lays)
    for (b, h) in sample_heads(w.batch, w.heads):
        rows = kcols = None
        if w.n > 20000:
            rng = np.random.default_rng(h)
            rows = np.unique(np.concatenate([np.arange(0, 64), rng.integers(0, w.n, 64),
                                             np.arange(w.n - 32, w.n)]))
            kcols = np.unique(np.concatenate([np.arange(0, 16), rng.integers(0, w.n, 32),
                                              np.arange(w.n - 16, w.n)]))
        compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False, rows=rows, kcols=kcols)


# ---------------------------------------------------------------------------
# Compact view of fixed B: the same pairs, walked over the summary keys only.

COMPACT = [
    # (head patterns, n, d, note); fixed B heads use the compact view
    ([("fixed_b", 128, 32)], 1024, 64, "c = 32: two l-blocks per key block"),
    ([("fixed_b", 128, 32)], 640, 64, "160 summary keys: ragged last key block"),
    ([("fixed_b", 64, 8)], 768, 64, "c = 8: eight l-blocks per key block"),
    ([("fixed_b", 256, 128)], 1024, 64, "c = 128: two key blocks per l-block"),
    ([("fixed_b", 128, 128)], 512, 64, "c = l: no gaps (dense causal)"),
    ([("fixed_b", 128, 32)], 1024, 128, "d = 128"),
    ([("fixed_b", 32, 8)], 8192, 64, "query lists of 128 steps: the dK/dV kernel walks them in chunks"),
    ([("fixed_b", 128, 64)], 12288, 64, "lists of 192 steps: two full chunks"),
    ([("fixed_b", 64, 16)], 8192, 128, "d = 128, lists of 128 steps: a chunk of 96 and a ragged one"),
    ([("fixed_a", 128, 32), ("fixed_b", 128, 32), ("strided_b", 16, 1)], 1024, 64,
     "raster, compact and residue-view heads in one call"),
]


def view_layouts(pats, n):
    lays = layouts_for(pats, n, 64)
    for (p, _, _), lay in zip(pats, lays):
        if p == "fixed_b" and not lay.compact_view:
            lay.set_compact_view(True)
        if p == "strided_b" and not lay.residue_view:
            lay.set_residue_view(True)
    return lays


@pytest.mark.parametrize("case", COMPACT, ids=[r[3] for r in COMPACT])
def test_compact_view_matches_oracle(case):
    pats, n, d, _ = case
    H = len(pats)
    x = workloads.custom_inputs((2, H, n, d), torch.bfloat16, seed=11 * n + d + H)
    lays = view_layouts(pats, n)
    assert any(lay.view_info()["kind"] == "compact" for lay in lays)
    dev = {t: x[t].to(DEV) for t in ("q", "k", "v", "do")}
    o, lse = sa.sa_fwd(dev["q"], dev["k"], dev["v"], lays, 1.0)
    dq, dk, dv = sa.sa_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], lays, 1.0)
    torch.cuda.synchronize()
    res = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    for b in range(2):
        for h in range(H):
            compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


def test_compact_view_every_output_written():
    """NaN-filled outputs: the gaps between summary runs get exact zeros in
    dK and dV, the empty first rows O = 0 and lse = -inf."""
    pats, n, d = [("fixed_b", 128, 32), ("fixed_a", 128, 32)], 640, 64
    x = workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=98)
    lays = view_layouts(pats, n)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full(q.shape[:3], nan, dtype=torch.float32, device=DEV)
    sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, nan) for _ in range(3))
    sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert not torch.isnan(got.float()).any(), nm
        assert torch.equal(got, want), nm
    gap = (torch.arange(n, device=DEV) % 128) < 96  # non-summary positions of head 0
    assert torch.count_nonzero(dk[:, 0][:, gap]) == 0 and torch.count_nonzero(dv[:, 0][:, gap]) == 0
    assert torch.all(lse[:, 0, :96] == -math.inf) and torch.count_nonzero(o[:, 0, :96]) == 0


def test_compact_view_bitwise_repeat():
    """The compact view's dK/dV chunks are summed in a fixed order: two
    runs agree bit for bit."""
    pats, n, d = [("fixed_a", 32, 8), ("fixed_b", 32, 8)], 8192, 64
    x = workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=97)
    lays = view_layouts(pats, n)
    r1 = run(x, pats, 64, 1.0, backward=True, lays=lays)
    r2 = run(x, pats, 64, 1.0, backward=True, lays=lays)
    for t in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(r1[t], r2[t]), t


def test_compact_view_full_size_sampled():
    """The text workload at full size with its fixed-B heads in the compact view."""
    w = WORKLOADS["text"]
    x = workloads.make_inputs(w)
    pats = w.head_patterns()
    lays = view_layouts(pats, w.n)
    res = run(x, pats, w.block, 1.0, backward=True, lays=lays)
    for (b, h) in sample_heads(w.batch, w.heads):
        compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


def test_million_length_sampled():
    """n = 2^20 with l = 1024 (the length-scaling run's largest point): a
    strided-A head walked raster and a strided-B head in its residue view,
    forward and backward, sampled rows and key columns against the oracle."""
    n, d, l = 1 << 20, 64, 1024
    pats = [("strided_a", l, 1), ("strided_b", l, 1)]
    x = workloads.custom_inputs((1, 2, n, d), torch.bfloat16, seed=77)
    lays = layouts_for(pats, n, 64)
    lays[1].set_residue_view(True)
    res = run(x, pats, 64, 1.0, backward=True, lays=lays)
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([np.arange(0, 16), rng.integers(0, n, 48), np.arange(n - 16, n)]))
    kcols = np.unique(np.concatenate([np.arange(0, 8), rng.integers(0, n, 24), np.arange(n - 8, n)]))
    for h in range(2):
        compare_head(x, res, 0, h, pats[h], 1.0, True, fp32=False, rows=rows, kcols=kcols)


def test_autograd_wrapper_recomputes():
    """sparse_attention's gradients are sa_bwd's, bit for bit, and the only
    tensors it keeps besides q, k, v are O and lse (no n x n weights)."""
    pats, n, d = [("strided_a", 64, 1), ("strided_b", 64, 1)], 1024, 64
    x = workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=123)
    lays = layouts_for(pats, n, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = sa.sparse_attention(qg, kg, vg, lays, 1.0)
    saved = o.grad_fn.saved_tensors
    assert len(saved) == 5
    assert sum(t.numel() * t.element_size() for t in saved[3:]) == (
        o.numel() * o.element_size() + 2 * 2 * n * 4)  # O and lse only
    o.backward(do)
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ref_o)
    for g, r, nm in zip((qg.grad, kg.grad, vg.grad), ref, ("dq", "dk", "dv")):
        assert torch.equal(g, r), nm


def test_noncurrent_stream():
    """Kernels run on the stream they are given."""
    n = 512
    x = workloads.custom_inputs((1, 2, n, 64), torch.bfloat16, seed=21)
    lays = layouts_for([("strided_a", 64, 1), ("strided_b", 64, 1)], n, 64)
    q, k, v = (x[t].to(DEV) for t in ("q", "k", "v"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = sa.sa_fwd(q, k, v, lays, 1.0, stream=s)
    s.synchronize()
    ref_o, _ = sa.sa_fwd(q, k, v, lays, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o)


def test_bwd_on_side_stream_outside_context():
    """sa_fwd and sa_bwd given a side stream while another stream is
    current: the outputs and the workspace the binding allocates belong to
    the side stream, so allocations on the current stream made right after
    the call (and filled at once) cannot take the workspace the dK/dV
    kernel is still reading."""
    n = 2048
    pats = [("strided_a", 128, 1), ("strided_b", 128, 1), ("fixed_a", 128, 32), ("fixed_b", 128, 32)]
    x = workloads.custom_inputs((2, 4, n, 64), torch.bfloat16, seed=23)
    lays = layouts_for(pats, n, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    torch.cuda.synchronize()
    ws_elems = sa.sa_bwd_workspace_size(2, 4, n, 64) // 4
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o, lse = sa.sa_fwd(q, k, v, lays, 1.0, stream=s)
        dq, dk, dv = sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, stream=s)
        junk = [torch.full((ws_elems,), float("nan"), device=DEV) for _ in range(4)]
        s.synchronize()
        del junk
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
        for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(got, want), nm


def _sweep_cases(count=32, seed=2019):
    """Seeded random configurations: patterns mixed per head, n a multiple of
    64 (some not a multiple of l), l and c anywhere in range, d 64 or 128,
    batch and heads small, scale 1 or 1/sqrt(d), views switched on where
    they apply."""
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(count):
        n = int(rng.choice([128, 192, 384, 512, 640, 896, 1024]))
        H = int(rng.integers(1, 5))
        B = int(rng.integers(1, 3))
        d = int(rng.choice([64, 64, 128]))
        pats = []
        for _ in range(H):
            p = str(rng.choice(["strided_a", "strided_b", "fixed_a", "fixed_b", "dense"]))
            l = int(rng.choice([1, 3, 8, 16, 32, 64, 100, 128, 256, 2 * n]))
            c = int(rng.integers(1, l + 1)) if p == "fixed_b" else 1
            if p == "fixed_b" and rng.random() < 0.5:  # a power of two dividing l, for the compact view
                c = 1 << int(rng.integers(0, max(1, int(np.log2(max(l, 1))) + 1)))
                c = min(c, l)
            pats.append((p, l, c))
        scale = 1.0 if rng.random() < 0.5 else 1.0 / math.sqrt(d)
        views = bool(rng.random() < 0.5)
        out.append((idx, B, H, n, d, tuple(pats), scale, views))
    return out


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "sweep%d" % c[0])
def test_random_sweep_matches_oracle(case):
    """Every output of a seeded random configuration against the oracle."""
    idx, B, H, n, d, pats, scale, views = case
    x = workloads.custom_inputs((B, H, n, d), torch.bfloat16, seed=500 + idx)
    lays = layouts_for(list(pats), n, 64)
    if views:
        for (p, l, c), lay in zip(pats, lays):
            if p == "strided_b" and n % l == 0 and not lay.residue_view:
                lay.set_residue_view(True)
            if p == "fixed_b" and n % l == 0 and (c & (c - 1)) == 0 and not lay.compact_view:
                lay.set_compact_view(True)
    res = run(x, list(pats), 64, scale, backward=True, lays=lays)
    for b in range(B):
        for h in range(H):
            compare_head(x, res, b, h, pats[h], scale, True, fp32=False)


@pytest.mark.parametrize("case", _sweep_cases(count=16, seed=2020), ids=lambda c: "chunked%d" % c[0])
def test_random_sweep_chunked_matches_oracle(case, split_steps):
    """Seeded random configurations with every list longer than 1 to 5 steps
    walked in chunks (combining passes after each kernel) against the
    oracle, all outputs."""
    idx = case[0]
    split_steps(1 + idx % 5)
    test_random_sweep_matches_oracle(case)


def test_destroy_releases_work_lists():
    """Destroying a layout frees the cached work lists of the calls that used
    it: building, using and destroying fresh layouts over and over leaves the
    device's free memory where it was (each cycle here caches about 1 MB of
    forward work list for B = 256, H = 8, n = 4096)."""
    B, H, n, d = 256, 8, 4096, 64
    g = torch.Generator(device=DEV).manual_seed(3)
    q, k, v = (torch.randn(B, H, n, d, device=DEV, generator=g).div_(8).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=DEV)

    def cycle():
        lays = [sa.sa_layout_build("strided_a", n, 64, block=64), sa.sa_layout_build("strided_b", n, 64, block=64)]
        sa.sa_fwd(q, k, v, lays * (H // 2), 1.0, o=o, lse=lse)
        torch.cuda.synchronize()
        for lay in lays:
            lay.close()

    cycle()
    free_before = torch.cuda.mem_get_info()[0]
    for _ in range(24):
        cycle()
    free_after = torch.cuda.mem_get_info()[0]
    assert free_after >= free_before - (8 << 20), (free_before - free_after)


@pytest.mark.parametrize("steps", [0, 3])
def test_graph_capture_replays(steps, split_steps):
    """After one uncaptured call (which uploads the layouts and work lists),
    sa_fwd + sa_bwd only enqueue kernels: captured into a graph and replayed
    several times, with eager work between the replays, every replay gives
    the eager results bit for bit.  steps = 3: long lists in chunks, so the
    capture also holds the combining kernels and uses the partial-result
    buffer made by the uncaptured call (another stream's)."""
    split_steps(steps)
    n = 1024
    pats = [("strided_a", 128, 1), ("strided_b", 128, 1), ("fixed_a", 128, 32), ("fixed_b", 128, 32)]
    x = workloads.custom_inputs((2, 4, n, 64), torch.bfloat16, seed=31)
    lays = layouts_for(pats, n, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(sa.sa_bwd_workspace_size(2, 4, n, 64), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
            sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, dq, dk, dv):
            t.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), rep
        for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(got, want), (rep, nm)
        sa.sa_fwd(q, k, v, lays, 1.0)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the refused capture holds nothing
def test_capture_before_any_call_is_refused():
    """A call on a stream being captured allocates and copies nothing: with
    layouts that no call has put on the device yet, sa_fwd and sa_bwd return
    SA_ERR_UNSUPPORTED and enqueue nothing, and the capture stays usable;
    after one uncaptured call the same capture replays the eager results."""
    n = 768
    pats = [("strided_a", 64, 1), ("fixed_b", 64, 16)]
    x = workloads.custom_inputs((1, 2, n, 64), torch.bfloat16, seed=37)
    lays = layouts_for(pats, n, 64)  # fresh layouts: nothing on the device
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(sa.sa_bwd_workspace_size(1, 2, n, 64), dtype=torch.uint8, device=DEV)

    def capture():
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        errs = []
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for call in (lambda: sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse),
                             lambda: sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv, workspace=ws)):
                    try:
                        call()
                    except sa.SAError as e:
                        errs.append(e.status)
        torch.cuda.synchronize()
        return g, errs

    torch.cuda.synchronize()
    _, errs = capture()
    assert errs == [sa.SA_ERR_UNSUPPORTED, sa.SA_ERR_UNSUPPORTED]
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    torch.cuda.synchronize()
    g, errs = capture()
    assert errs == []
    for t in (o, dq, dk, dv):
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert torch.equal(got, want), nm


# ---------------------------------------------------------------------------
# Long lists walked in chunks (sa_set_split): partial results combined in
# list order by a second kernel per stage.

SPLIT = [
    # (head patterns, n, d, views, note)
    ([("strided_a", 128, 1), ("strided_b", 128, 1)], 2048, 64, False, "strided heads"),
    ([("fixed_a", 128, 32), ("fixed_b", 128, 32)], 2048, 64, False, "fixed heads: empty first rows"),
    ([("strided_b", 64, 1), ("dense", 1, 1)], 1024, 128, False, "d = 128, dense head"),
    ([("fixed_b", 128, 32), ("strided_b", 128, 1), ("strided_a", 96, 1)], 1920, 64, True,
     "compact and residue views beside a plain head, ragged last blocks"),
]


@pytest.mark.parametrize("steps", [1, 5])
@pytest.mark.parametrize("form", ["half", "paired"])
@pytest.mark.parametrize("case", SPLIT, ids=[c[4] for c in SPLIT])
def test_chunked_lists_match_oracle(case, form, steps, split_steps, fwd_form):
    """Every list longer than `steps` is walked in chunks of at most `steps`
    (one step each: a chunk often holds no allowed key of a row, whose
    partial row sum is then zero); both forward forms; against the oracle,
    every head whole with the elementwise bound."""
    pats, n, d, views, _ = case
    split_steps(steps)
    fwd_form(form)
    H = len(pats)
    x = workloads.custom_inputs((2, H, n, d), torch.bfloat16, seed=7 * n + d + steps)
    lays = view_layouts(pats, n) if views else layouts_for(pats, n, 64)
    res = run(x, pats, 64, 1.0, backward=True, lays=lays)
    for b in range(2):
        for h in range(H):
            compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False)


def test_chunked_lists_agree_with_unchunked(split_steps):
    """The same call with and without chunks: equal up to rounding order
    (bf16 outputs within a few units of the last place)."""
    pats, n, d = [("strided_a", 128, 1), ("strided_b", 128, 1), ("fixed_b", 128, 32)], 2048, 64
    x = workloads.custom_inputs((2, 3, n, d), torch.bfloat16, seed=404)
    split_steps(-1)
    r0 = run(x, pats, 64, 1.0, backward=True)
    sa.sa_set_split(3)
    r1 = run(x, pats, 64, 1.0, backward=True)
    for t in ("o", "dq", "dk", "dv"):
        a, b = r0[t].float(), r1[t].float()
        assert torch.allclose(a, b, rtol=2e-2, atol=2e-3), (t, (a - b).abs().max().item())
    fin = torch.isfinite(r0["lse"])
    assert torch.equal(fin, torch.isfinite(r1["lse"]))
    assert (r0["lse"][fin] - r1["lse"][fin]).abs().max().item() <= 1e-4


def test_chunked_bitwise_repeat_and_every_output_written(split_steps):
    """Chunks combined in a fixed order: two runs agree bit for bit, also
    with NaN-filled outputs (every element of O, lse, dQ, dK, dV written)."""
    split_steps(4)
    pats, n, d = [("strided_b", 128, 1), ("fixed_b", 64, 16)], 1472, 64
    x = workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=77)
    lays = layouts_for(pats, n, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    ref_o, ref_lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, ref_o, ref_lse, do, lays, 1.0)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full(q.shape[:3], nan, dtype=torch.float32, device=DEV)
    sa.sa_fwd(q, k, v, lays, 1.0, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, nan) for _ in range(3))
    sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
    for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        assert not torch.isnan(got.float()).any(), nm
        assert torch.equal(got, want), nm


def test_auto_chunks_underfilled_call(split_steps):
    """A batch of one with two heads leaves most compute units without a
    list of their own: the per-call rule (sa_set_split(0)) cuts the long
    lists into chunks.  Sampled rows and key columns against the oracle,
    and the results differ from the unchunked run in rounding (so chunks
    were taken)."""
    pats, n, d = [("strided_a", 128, 1), ("strided_b", 128, 1)], 8192, 64
    x = workloads.custom_inputs((1, 2, n, d), torch.bfloat16, seed=8192)
    split_steps(0)
    lays = layouts_for(pats, n, 64)
    res = run(x, pats, 64, 1.0, backward=True, lays=lays)
    rows = sorted(set(list(range(0, 64)) + list(range(4032, 4160)) + list(range(n - 96, n))))
    for h in range(2):
        compare_head(x, res, 0, h, pats[h], 1.0, True, fp32=False, rows=rows)
    sa.sa_set_split(-1)
    ref = run(x, pats, 64, 1.0, backward=True, lays=layouts_for(pats, n, 64))
    assert any(not torch.equal(res[t], ref[t]) for t in ("o", "dq", "dk", "dv"))


def test_chunked_calls_on_two_streams(split_steps):
    """Chunked calls on two streams at once use separate partial buffers:
    each stream's results equal the same call run alone."""
    split_steps(2)
    pats, n, d = [("strided_a", 128, 1), ("strided_b", 128, 1)], 2048, 64
    lays = layouts_for(pats, n, 64)
    xs = [workloads.custom_inputs((2, 2, n, d), torch.bfloat16, seed=s) for s in (5, 6)]
    dev = [{t: x[t].to(DEV) for t in ("q", "k", "v", "do")} for x in xs]
    refs = []
    for dd in dev:
        o, lse = sa.sa_fwd(dd["q"], dd["k"], dd["v"], lays, 1.0)
        refs.append((o, lse) + tuple(sa.sa_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], lays, 1.0)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for i, (st, dd) in enumerate(zip(streams, dev)):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                o, lse = sa.sa_fwd(dd["q"], dd["k"], dd["v"], lays, 1.0)
                outs[i] = (o, lse) + tuple(sa.sa_bwd(dd["q"], dd["k"], dd["v"], o, lse, dd["do"], lays, 1.0))
        torch.cuda.synchronize()
        for i in range(2):
            for got, want, nm in zip(outs[i], refs[i], ("o", "lse", "dq", "dk", "dv")):
                assert torch.equal(got, want), (rep, i, nm)


# ---------------------------------------------------------------------------
# Workloads at full size, in the launch configuration the benchmark times.

@pytest.mark.parametrize("name", ["img32", "text", "img64", "audio"])
def test_workload_full_size_sampled_heads(name):
    w = WORKLOADS[name]
    x = workloads.make_inputs(w)
    res = run(x, w.head_patterns(), w.block, 1.0, backward=True)
    for (b, h) in sample_heads(w.batch, w.heads):
        # whole heads where the oracle is quick, sampled rows otherwise
        rows = kcols = None
        if w.n > 20000:
            rng = np.random.default_rng(h)
            rows = np.unique(np.concatenate([np.arange(0, 64), rng.integers(0, w.n, 64),
                                             np.arange(w.n - 32, w.n)]))
            kcols = np.unique(np.concatenate([np.arange(0, 16), rng.integers(0, w.n, 32),
                                              np.arange(w.n - 16, w.n)]))
        compare_head(x, res, b, h, w.head_patterns()[h], 1.0, True, fp32=False, rows=rows, kcols=kcols)
    # every head is finite and empty rows (fixed B) are exactly (0, -inf)
    assert torch.isfinite(res["o"].float()).all()
    for t in ("dq", "dk", "dv"):
        assert torch.isfinite(res[t].float()).all()


def test_img64_dense_comparison_sampled_rows():
    """The dense causal comparison at the img64 shape (the launch the
    benchmark's --dense run times), forward and backward: whole 64-row
    blocks of queries (dQ) and of keys (dK, dV) at the start, the end and
    seeded places between, two heads."""
    w = WORKLOADS["img64"]
    x = workloads.make_inputs(w)
    pats = w.head_patterns(dense=True)
    res = run(x, pats, w.block, 1.0, backward=True)
    rng = np.random.default_rng(3)
    nb = w.n // 64
    blocks = sorted(set([0, 1, nb - 1] + [int(b) for b in rng.integers(2, nb - 1, 4)]))
    rows = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in blocks])
    for (b, h) in [(0, 0), (1, 15)]:
        compare_head(x, res, b, h, pats[h], 1.0, True, fp32=False, rows=rows)
    for t in ("o", "dq", "dk", "dv"):
        assert torch.isfinite(res[t].float()).all()




def test_backward_stages_match_sa_bwd():
    """sa_bwd_dq_rowterms + sa_bwd_dkdv give sa_bwd's results bit for bit;
    sa_bwd_rowterms + sa_bwd_dkdv + sa_bwd_dq give them up to the summation
    order of D_i (the same -lse log2 e, D within fp32 rounding)."""
    w = WORKLOADS["text"]
    x = workloads.make_inputs(w, shape=(1, 2, 1024, 64))
    pats = w.head_patterns()[:2]
    lays = layouts_for(pats, 1024, 64)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    o, lse = sa.sa_fwd(q, k, v, lays, 1.0)
    dq, dk, dv = sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0)
    dq1, ws1 = sa.sa_bwd_dq_rowterms(q, k, v, o, lse, do, lays, 1.0)
    dk1, dv1 = sa.sa_bwd_dkdv(q, k, v, do, lays, 1.0, ws1)
    ws2 = sa.sa_bwd_rowterms(o, lse, do, lays, 1.0)
    dk2, dv2 = sa.sa_bwd_dkdv(q, k, v, do, lays, 1.0, ws2)
    dq2 = sa.sa_bwd_dq(q, k, v, do, lays, 1.0, ws2)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq1) and torch.equal(dk, dk1) and torch.equal(dv, dv1)
    rows = 2 * 1024
    t1, t2 = ws1[:8 * rows].view(torch.float32), ws2[:8 * rows].view(torch.float32)
    assert torch.equal(t1[rows:], t2[rows:])  # -lse log2 e
    assert torch.allclose(t1[:rows], t2[:rows], rtol=1e-5, atol=1e-6)  # -D
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert rel_l2(a.float().cpu().numpy(), b.float().cpu().numpy()) < 1e-3
