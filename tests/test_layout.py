"""Host checks of the library's layout builder and C ABI (no GPU needed).

Layouts are compared bit-exactly with the oracle's direct enumeration of
the pattern predicates: the listed key blocks of every query block, and the
expanded T x T element mask of every listed block.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_factorized_amd as sa
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def expand(ex, T):
    """Expanded [nnz, T, T] masks of an exported layout (full blocks = ones)."""
    nnz = len(ex["col_idx"])
    out = np.ones((nnz, T, T), dtype=bool)
    for a in range(nnz):
        m = ex["mask_id"][a]
        if m >= 0:
            bits = np.unpackbits(ex["mask_words"][m].view(np.uint8), bitorder="little")[:T * T]
            out[a] = bits.reshape(T, T).astype(bool)
    return out


def check_against_oracle(pattern, n, l, c, T):
    lay = sa.sa_layout_build(pattern, n, l, c, block=T)
    ex = lay.export()
    info = lay.info()
    rp, kbs, pop, words = oracle.block_layout_sparse(pattern, n, l, c, T)
    assert np.array_equal(ex["row_ptr"].astype(np.int64), rp)
    assert np.array_equal(ex["col_idx"].astype(np.int64), kbs)
    got = expand(ex, T)
    nw = T * T // 64
    ref = np.unpackbits(words.view(np.uint8).reshape(-1, nw * 8), axis=1, bitorder="little")
    ref = ref[:, :T * T].reshape(-1, T, T).astype(bool)
    assert np.array_equal(got, ref)
    # full blocks are exactly those with every element allowed
    assert np.array_equal(ex["mask_id"] < 0, pop == T * T)
    assert info["allowed"] == int(pop.sum())
    assert info["nnz"] == len(kbs)
    return lay, ex


SMALL = [
    ("strided_a", 256, 16, 1, 16), ("strided_b", 256, 16, 1, 16),
    ("strided_a", 512, 40, 1, 16), ("strided_b", 512, 40, 1, 32), ("strided_b", 640, 7, 1, 64),
    ("fixed_a", 512, 128, 32, 64), ("fixed_b", 512, 128, 32, 64), ("fixed_b", 480, 24, 5, 16),
    ("fixed_b", 512, 100, 100, 64), ("fixed_a", 384, 10, 1, 32), ("dense", 384, 1, 1, 64),
    ("strided_a", 64, 1, 1, 8), ("strided_b", 128, 1000, 1, 128), ("fixed_b", 64, 128, 1, 16),
    ("strided_a", 3072, 128, 1, 64), ("strided_b", 3072, 128, 1, 64),
]


@pytest.mark.parametrize("pattern,n,l,c,T", SMALL)
def test_layout_bit_exact(pattern, n, l, c, T):
    check_against_oracle(pattern, n, l, c, T)


@pytest.mark.parametrize("pattern,n,l,c,T", [
    ("fixed_a", 12288, 128, 32, 64), ("fixed_b", 12288, 128, 32, 64),
    ("strided_a", 12288, 128, 1, 64), ("strided_b", 12288, 128, 1, 64),
])
def test_layout_bit_exact_full_size(pattern, n, l, c, T):
    check_against_oracle(pattern, n, l, c, T)


@pytest.mark.slow
@pytest.mark.parametrize("pattern", ["strided_a", "strided_b"])
def test_layout_bit_exact_audio(pattern):
    check_against_oracle(pattern, 65536, 256, 1, 64)


def _random_layout_cases(count=200, seed=1709):
    """Seeded random (pattern, n, l, c, block): every block size, n a
    multiple of the block (often not of l), l from 1 to beyond n, c anywhere
    in 1..l."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        T = int(rng.choice([8, 16, 32, 64, 128]))
        n = T * int(rng.integers(1, max(2, 1536 // T)))
        p = str(rng.choice(["strided_a", "strided_b", "fixed_a", "fixed_b", "dense"]))
        l = int(rng.integers(1, 2 * n + 2))
        c = int(rng.integers(1, l + 1)) if p == "fixed_b" else 1
        out.append((p, n, l, c, T))
    return out


@pytest.mark.parametrize("pattern,n,l,c,T", _random_layout_cases())
def test_layout_bit_exact_random(pattern, n, l, c, T):
    """Random layouts match the oracle's direct enumeration bit for bit."""
    check_against_oracle(pattern, n, l, c, T)


@pytest.mark.parametrize("pattern,n,l,c,T", SMALL[:10])
def test_transpose_and_mask_ids(pattern, n, l, c, T):
    lay = sa.sa_layout_build(pattern, n, l, c, block=T)
    ex = lay.export()
    nqb = n // T
    # transpose lists every (qb, kb) exactly once, ascending qb per kb
    pairs = set()
    for kb in range(nqb):
        seg = ex["row_idx"][ex["col_ptr"][kb]:ex["col_ptr"][kb + 1]]
        assert np.all(np.diff(seg) > 0)
        for slot in range(ex["col_ptr"][kb], ex["col_ptr"][kb + 1]):
            qb = ex["row_idx"][slot]
            pos = ex["csr_pos"][slot]
            assert ex["row_ptr"][qb] <= pos < ex["row_ptr"][qb + 1]
            assert ex["col_idx"][pos] == kb
            pairs.add((qb, kb))
    assert len(pairs) == len(ex["col_idx"])
    # mask ids appear in order of first use
    seen = [m for m in ex["mask_id"] if m >= 0]
    first = []
    for m in seen:
        if m not in first:
            first.append(m)
    assert first == list(range(len(first)))
    # the table holds no duplicates
    rows = {bytes(ex["mask_words"][m].tobytes()) for m in range(len(ex["mask_words"]))}
    assert len(rows) == len(ex["mask_words"])


@pytest.mark.parametrize("args,code", [
    (("strided_a", 100, 16, 1, 16), sa.SA_ERR_INVALID_ARG),   # n % block
    (("strided_a", 0, 16, 1, 16), sa.SA_ERR_INVALID_ARG),     # n < 1
    (("strided_a", 256, 0, 1, 16), sa.SA_ERR_INVALID_ARG),    # l < 1
    (("fixed_b", 256, 16, 0, 16), sa.SA_ERR_INVALID_ARG),     # c < 1
    (("fixed_b", 256, 16, 17, 16), sa.SA_ERR_INVALID_ARG),    # c > l
    (("strided_a", 256, 16, 1, 24), sa.SA_ERR_INVALID_ARG),   # block
    ((7, 256, 16, 1, 16), sa.SA_ERR_INVALID_ARG),             # pattern
])
def test_layout_build_errors(args, code):
    with pytest.raises(sa.SAError) as e:
        sa.sa_layout_build(args[0], args[1], args[2], args[3], block=args[4])
    assert e.value.status == code


def test_header_symbols_exported():
    """Every function include/sa.h declares is exported by libsa.so."""
    text = open(os.path.join(ROOT, "include", "sa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text))
    assert {"sa_layout_build", "sa_fwd", "sa_bwd"} <= names
    lib = ctypes.CDLL(sa.LIB_PATH)
    for name in sorted(names):
        assert hasattr(lib, name), name
    assert set(sa.EXPORTED) == names


def test_peaks_header_symbols_exported():
    """Every function include/sa_peaks.h declares is exported by libsa_peaks.so."""
    text = open(os.path.join(ROOT, "include", "sa_peaks.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(sap_[a-z0-9_]+)\s*\(", text))
    assert names == {"sap_mfma_bf16_tflops", "sap_copy_gbs"}
    lib = ctypes.CDLL(os.path.join(os.path.dirname(sa.LIB_PATH), "libsa_peaks.so"))
    for name in sorted(names):
        assert hasattr(lib, name), name


def _heads(*lays):
    return (ctypes.c_void_p * len(lays))(*[x.handle for x in lays])


def test_fwd_bwd_argument_errors_without_gpu():
    """Host-side validation returns before any device work."""
    lib = sa.library()
    lay = sa.sa_layout_build("strided_a", 256, 16, block=64)
    lay16 = sa.sa_layout_build("strided_a", 256, 16, block=16)
    h = _heads(lay, lay)
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: every case fails first
    cases = [
        (dict(B=0), sa.SA_ERR_INVALID_ARG),
        (dict(H=300), sa.SA_ERR_INVALID_ARG),
        (dict(n=512), sa.SA_ERR_INVALID_ARG),          # layout built for 256
        (dict(scale=0.0), sa.SA_ERR_INVALID_ARG),
        (dict(scale=float("nan")), sa.SA_ERR_INVALID_ARG),
        (dict(d=32), sa.SA_ERR_UNSUPPORTED),
        (dict(dtype=sa.SA_F32), sa.SA_ERR_UNSUPPORTED),  # f32 kernels need block 16
        (dict(dtype=5), sa.SA_ERR_INVALID_ARG),
        (dict(q=None), sa.SA_ERR_INVALID_ARG),
        (dict(q=ctypes.c_void_p((1 << 20) + 8)), sa.SA_ERR_INVALID_ARG),  # misaligned
    ]
    for over, code in cases:
        a = dict(heads=h, B=1, H=2, n=256, d=64, dtype=sa.SA_BF16, scale=1.0, q=p, k=p, v=p, o=p, lse=p)
        a.update(over)
        heads = _heads(*([lay] * a["H"])) if a["H"] != 2 and a["H"] <= 512 else a["heads"]
        st = lib.sa_fwd(heads, a["B"], a["H"], a["n"], a["d"], a["dtype"], a["scale"], a["q"], a["k"],
                        a["v"], a["o"], a["lse"], None)
        assert st == code, (over, st, lib.sa_last_error())
        assert lib.sa_last_error().decode() != ""
    # f32 backward is not compiled
    h16 = _heads(lay16, lay16)
    st = lib.sa_bwd(h16, 1, 2, 256, 64, sa.SA_F32, 1.0, p, p, p, p, p, p, p, p, p, p, 1 << 20, None)
    assert st == sa.SA_ERR_UNSUPPORTED
    # too small a workspace
    st = lib.sa_bwd(h, 1, 2, 256, 64, sa.SA_BF16, 1.0, p, p, p, p, p, p, p, p, p, p, 16, None)
    assert st == sa.SA_ERR_INVALID_ARG
    # nine distinct layouts in one call (at most eight)
    nine = [sa.sa_layout_build("strided_a", 256, 1 + i, block=64) for i in range(9)]
    st = lib.sa_fwd(_heads(*nine), 1, 9, 256, 64, sa.SA_BF16, 1.0, p, p, p, p, p, None)
    assert st == sa.SA_ERR_INVALID_ARG and b"distinct" in lib.sa_last_error()
    st = lib.sa_bwd(_heads(*nine), 1, 9, 256, 64, sa.SA_BF16, 1.0, p, p, p, p, p, p, p, p, p, p, 1 << 20, None)
    assert st == sa.SA_ERR_INVALID_ARG
    # NULL layout entry
    hn = (ctypes.c_void_p * 2)(lay.handle, None)
    st = lib.sa_fwd(hn, 1, 2, 256, 64, sa.SA_BF16, 1.0, p, p, p, p, p, None)
    assert st == sa.SA_ERR_INVALID_ARG
    assert sa.sa_bwd_workspace_size(2, 3, 100, 64) >= 2 * 3 * 100 * 4
    # the allocation-free backward refuses more rows than its scratch holds
    # (1 x 2 x 2^21 rows > 2^21) before any device work
    big = sa.sa_layout_build("strided_a", 1 << 21, 1024, block=64)
    st = lib.sa_bwd_noalloc(_heads(big, big), 1, 2, 1 << 21, 64, sa.SA_BF16, 1.0, p, p, p, p, p, p, p, p, p, None)
    assert st == sa.SA_ERR_INVALID_ARG and b"scratch" in lib.sa_last_error()


def test_residue_view_switch():
    """The residue view is only for strided B with block 64 and l | n; it
    leaves the layout's own listing unchanged and can be switched off."""
    lib = sa.library()
    lay = sa.sa_layout_build("strided_b", 768, 8, block=64)
    before = lay.export()
    lay.set_residue_view(True)
    lay.set_residue_view(True)  # idempotent
    after = lay.export()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    lay.set_residue_view(False)
    lay.set_residue_view(True)
    cases = [
        (("strided_a", 768, 8, 1, 64), sa.SA_ERR_UNSUPPORTED),
        (("fixed_b", 768, 128, 32, 64), sa.SA_ERR_UNSUPPORTED),
        (("strided_b", 768, 8, 1, 16), sa.SA_ERR_UNSUPPORTED),   # block 16: fp32 kernels
        (("strided_b", 768, 96 + 1, 1, 64), sa.SA_ERR_UNSUPPORTED),  # l does not divide n
    ]
    for (p, n, l, c, T), code in cases:
        x = sa.sa_layout_build(p, n, l, c, block=T)
        with pytest.raises(sa.SAError) as e:
            x.set_residue_view(True)
        assert e.value.status == code
        x.set_residue_view(False)  # switching off is always fine
    assert lib.sa_layout_set_residue_view(None, 1) == sa.SA_ERR_INVALID_ARG


def test_more_than_eight_layouts_rejected():
    lib = sa.library()
    lays = [sa.sa_layout_build("strided_a", 128, l, block=64) for l in range(1, 11)]
    p = ctypes.c_void_p(1 << 20)
    st = lib.sa_fwd(_heads(*lays), 1, len(lays), 128, 64, sa.SA_BF16, 1.0, p, p, p, p, p, None)
    assert st == sa.SA_ERR_INVALID_ARG
    assert b"distinct" in lib.sa_last_error()


def test_process_switches_validate_and_restore():
    """The process-wide test and tuning switches (no GPU needed): each
    returns the setting it replaces, refuses values outside its range with
    SA_ERR_INVALID_ARG and leaves the setting unchanged then."""
    lib = sa.library()
    prev = ctypes.c_int(-7)
    assert lib.sa_set_split(5, ctypes.byref(prev)) == sa.SA_OK and prev.value == 0
    assert lib.sa_set_split(-2, ctypes.byref(prev)) == sa.SA_ERR_INVALID_ARG
    assert b"below -1" in lib.sa_last_error()
    assert lib.sa_set_split(-1, ctypes.byref(prev)) == sa.SA_OK and prev.value == 5
    assert lib.sa_set_split(0, None) == sa.SA_OK
    assert sa.sa_set_split(0) == 0
    assert lib.sa_set_one_paths(0, ctypes.byref(prev)) == sa.SA_OK and prev.value == 1
    assert lib.sa_set_one_paths(2, ctypes.byref(prev)) == sa.SA_ERR_INVALID_ARG
    assert sa.sa_set_one_paths(True) is False
    assert sa.sa_set_one_paths(True) is True
    with pytest.raises(sa.SAError):
        sa.sa_set_split(-3)
    assert sa.sa_set_fwd_form("half") == "auto"
    with pytest.raises(sa.SAError):
        sa.sa_set_fwd_form(3)
    assert sa.sa_set_fwd_form("auto") == "half"


def test_status_strings():
    lib = sa.library()
    for code in (sa.SA_OK, sa.SA_ERR_INVALID_ARG, sa.SA_ERR_UNSUPPORTED, sa.SA_ERR_HIP, sa.SA_ERR_ALLOC):
        assert lib.sa_status_string(code)
    assert lib.sa_status_string(-99) == b"unknown status"


def test_compact_view_switch():
    """The compact view is only for fixed B with block 64, l | n and c a power
    of two; it leaves the layout's own listing unchanged, walks the same
    allowed pairs, and can be switched off."""
    lay = sa.sa_layout_build("fixed_b", 1024, 128, 32, block=64)
    before = lay.export()
    raster = lay.view_info()
    assert raster["kind"] == "layout" and raster["nkb"] == raster["nqb"] == 16
    lay.set_compact_view(True)
    lay.set_compact_view(True)  # idempotent
    after = lay.export()
    for k in before:
        assert np.array_equal(before[k], after[k]), k
    v = lay.view_info()
    assert v["kind"] == "compact" and v["allowed"] == lay.info()["allowed"]
    assert v["nqb"] == 16 and v["nkb"] == 1024 // 128 * 32 // 64
    lay.set_compact_view(False)
    assert lay.view_info()["kind"] == "layout"
    cases = [
        (("fixed_a", 768, 128, 32, 64), sa.SA_ERR_UNSUPPORTED),
        (("strided_b", 768, 8, 1, 64), sa.SA_ERR_UNSUPPORTED),
        (("fixed_b", 768, 128, 32, 16), sa.SA_ERR_UNSUPPORTED),  # block 16: fp32 kernels
        (("fixed_b", 768, 100, 32, 64), sa.SA_ERR_UNSUPPORTED),  # l does not divide n
        (("fixed_b", 768, 128, 24, 64), sa.SA_ERR_UNSUPPORTED),  # c not a power of two
    ]
    for (p, n, l, c, T), code in cases:
        bad = sa.sa_layout_build(p, n, l, c, block=T)
        with pytest.raises(sa.SAError) as e:
            bad.set_compact_view(True)
        assert e.value.status == code
        assert bad.view_info()["kind"] == "layout"


@pytest.mark.parametrize("n,l,c", [(12288, 128, 32), (1024, 128, 32), (640, 128, 32), (768, 64, 8),
                                   (1024, 256, 128), (1024, 128, 128), (4096, 256, 64), (2048, 64, 1)])
def test_compact_view_blocks(n, l, c):
    """The compact view walks exactly the fixed-B layout's allowed pairs, in
    the number of 64 x 64 blocks the summary-key prefix predicts: query block
    qb sees the first cnt(64 qb + 63) summary keys, cnt(i) = floor((i+1)/l) c
    + max(0, (i+1) mod l - (l - c)), i.e. ceil(cnt / 64) key blocks.  At the
    text workload's size that is 4656 blocks against the raster layout's 9216."""
    lay = sa.sa_layout_build("fixed_b", n, l, c, block=64)
    lay.set_compact_view(True)
    v = lay.view_info()
    assert v["allowed"] == lay.info()["allowed"]
    cnt = lambda i: (i + 1) // l * c + max(0, (i + 1) % l - (l - c))
    assert v["nnz"] == sum(-(-cnt(64 * qb + 63) // 64) for qb in range(n // 64))
    assert v["nkb"] == -(-(n // l * c) // 64)
    if (n, l, c) == (12288, 128, 32):
        assert v["nnz"] == 4656 and lay.info()["nnz"] == 9216
