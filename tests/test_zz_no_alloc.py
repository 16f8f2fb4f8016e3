"""sa_bwd_noalloc (row terms in the library's static scratch, no allocation)
against sa_bwd on the same inputs: two calls in a row, the second smaller."""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import block_sparse_factorized_amd as sa

DEV = "cuda:0"

CALLS = [
    # (B, H, n, d, head patterns, seed)
    (2, 4, 1536, 64, [("strided_a", 128, 1), ("strided_b", 128, 1), ("fixed_a", 128, 32), ("fixed_b", 128, 32)], 61),
    (1, 2, 512, 128, [("strided_a", 64, 1), ("strided_b", 64, 1)], 62),
]


@pytest.fixture
def split_steps():
    prev = []

    def force(steps):
        prev.append(sa.sa_set_split(steps))

    yield force
    if prev:
        sa.sa_set_split(prev[0])


@pytest.mark.parametrize("steps", [0, 3])
def test_noalloc_matches_sa_bwd_on_two_calls(steps, split_steps):
    """steps = 3: long lists in chunks, whose partial results go to the
    buffer the earlier sa_bwd made (no allocation either)."""
    split_steps(steps)
    free_seen = []
    for (B, H, n, d, pats, seed) in CALLS:
        lays = [sa.sa_layout_build(p, n, l, c, block=64) for (p, l, c) in pats]
        x = workloads.custom_inputs((B, H, n, d), torch.bfloat16, seed=seed)
        q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
        o, lse = sa.sa_fwd(q, k, v, lays, 1.0)
        # Nothing is on the device for these layouts' backward yet: refused, nothing launched.
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        with pytest.raises(sa.SAError) as err:
            sa.sa_bwd_noalloc(q, k, v, o, lse, do, lays, 1.0, dq, dk, dv)
        assert err.value.status == sa.SA_ERR_UNSUPPORTED
        ref = sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0)  # uploads the work lists
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        sa.sa_bwd_noalloc(q, k, v, o, lse, do, lays, 1.0, dq, dk, dv)
        torch.cuda.synchronize()
        free_seen.append(free_before - torch.cuda.mem_get_info()[0])
        for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert not torch.isnan(got.float()).any(), nm
            assert torch.equal(got, want), nm
    # the second call (the scratch array is already resident) moves no device memory
    assert free_seen[1] == 0, free_seen


def test_noalloc_rejects_beyond_scratch():
    n, d = 1 << 16, 64
    lay = sa.sa_layout_build("strided_a", n, 256, block=64)
    lib = sa.library()
    heads = (ctypes.c_void_p * 64)(*([lay.handle] * 64))
    # 1 x 64 heads x 65536 rows = 2^22 rows > 2^21: refused before any device work
    st = lib.sa_bwd_noalloc(heads, 1, 64, n, d, sa.SA_BF16, 1.0, *([ctypes.c_void_p(16)] * 9), None)
    assert st == sa.SA_ERR_INVALID_ARG
    assert b"scratch" in lib.sa_last_error()


@pytest.mark.parametrize("steps", [0, 3])
def test_noalloc_captured_replays(steps, split_steps):
    """The callers this entry point is for include graph capture: captured
    after one sa_bwd, every replay gives sa_bwd's results bit for bit, also
    with other calls on the same scratch array between the replays."""
    split_steps(steps)
    (B, H, n, d, pats, seed), (B2, H2, n2, d2, pats2, seed2) = CALLS
    lays = [sa.sa_layout_build(p, n, l, c, block=64) for (p, l, c) in pats]
    x = workloads.custom_inputs((B, H, n, d), torch.bfloat16, seed=seed)
    q, k, v, do = (x[t].to(DEV) for t in ("q", "k", "v", "do"))
    o, lse = sa.sa_fwd(q, k, v, lays, 1.0)
    ref = sa.sa_bwd(q, k, v, o, lse, do, lays, 1.0)
    # a smaller call of its own, run eagerly between the replays
    lays2 = [sa.sa_layout_build(p, n2, l, c, block=64) for (p, l, c) in pats2]
    x2 = workloads.custom_inputs((B2, H2, n2, d2), torch.bfloat16, seed=seed2)
    q2, k2, v2, do2 = (x2[t].to(DEV) for t in ("q", "k", "v", "do"))
    o2, lse2 = sa.sa_fwd(q2, k2, v2, lays2, 1.0)
    ref2 = sa.sa_bwd(q2, k2, v2, o2, lse2, do2, lays2, 1.0)
    # (an uncaptured call first: it finds the scratch array's address)
    sa.sa_bwd_noalloc(q2, k2, v2, o2, lse2, do2, lays2, 1.0, *(torch.empty_like(q2) for _ in range(3)))
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.sa_bwd_noalloc(q, k, v, o, lse, do, lays, 1.0, dq, dk, dv)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            assert torch.equal(got, want), (rep, nm)
        g2 = [torch.full_like(q2, float("nan")) for _ in range(3)]
        sa.sa_bwd_noalloc(q2, k2, v2, o2, lse2, do2, lays2, 1.0, *g2)
        torch.cuda.synchronize()
        for got, want, nm in zip(g2, ref2, ("dq", "dk", "dv")):
            assert torch.equal(got, want), (rep, "eager", nm)
