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
