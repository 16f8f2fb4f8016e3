"""Build libsa.so (the C-ABI library) with hipcc for gfx950, in-tree.

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
OBJ_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libsa.so")
SOURCES = ["layout.cpp", "pack.cpp", "capi.cpp", "fwd.hip", "bwd.hip"]
# libsa_peaks.so: the micro-benchmarks of include/sa_peaks.h (not part of libsa)
PEAKS_LIB = os.path.join(OUT_DIR, "libsa_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -amdgpu-mfma-vgpr-form: keep MFMA accumulators in ordinary VGPRs, so the
# softmax's VALU work on them needs no accvgpr moves.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel whose host stub failed to instantiate must
    # fail the build, not the first dlopen.
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(6, len(SOURCES) + len(PEAKS_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAKS_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print("built", LIB)
        print("built", PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
