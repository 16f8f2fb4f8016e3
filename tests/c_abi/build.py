"""Compile tests/c_abi/abi_check (host code only, hipcc) against libsa.so and
the oracle's liboracle.so; both must be built first."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "_build", "abi_check")


def build() -> str:
    lib_dir = os.path.join(ROOT, "block_sparse_factorized_amd", "_lib")
    oracle_dir = os.path.join(ROOT, "oracle", "_build")
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    tmp = BIN + ".tmp%d" % os.getpid()
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "-O2", "-std=c++17",
           "-I" + os.path.join(ROOT, "include"), os.path.join(HERE, "abi_check.cpp"), "-o", tmp,
           "-L" + lib_dir, "-lsa", "-L" + oracle_dir, "-loracle",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + oracle_dir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("abi_check build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
