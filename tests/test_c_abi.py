"""The library through its C ABI alone (tests/c_abi/abi_check.cpp): no
Python binding, no torch.  The program builds the four factorized layouts,
runs sa_fwd and sa_bwd on hipMalloc'd buffers and compares every output with
the fp64 oracle at the same tolerances as the parity tests; it also checks a
rejected call.  Built by __graft_entry__.build()."""
import os
import subprocess

import pytest

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "_build", "abi_check")


@pytest.mark.gpu
def test_c_abi_program():
    assert os.path.exists(BIN), "tests/c_abi/_build/abi_check is not built (run __graft_entry__.build())"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
