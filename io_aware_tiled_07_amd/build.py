"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every call recompiles; objects go to ``_build/`` next to this file and the
shared library to ``libfa.so`` in this package directory.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd128.hip", "fa_bwd_atomic.hip", "fa_fp32.hip",
           "fa_sparse.hip", "fa_fwd_fp8.hip", "fa_decode.hip"]
# MFMA results stay in arch VGPRs (the softmax reads them directly, no AGPR
# copies) everywhere except the head-dim-128 backward, whose fp32 accumulators
# need the AGPRs beside the 256 VGPRs.
AGPR_SOURCES = {"fa_bwd128.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def flags(src: str = "") -> list[str]:
    f = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-munsafe-fp-atomics",
        # inputs are finite: max/min need no NaN canonicalisation
        "-fno-honor-nans",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]
    if src not in AGPR_SOURCES:
        f += ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
    return f


def _compile(src: str, build_dir: str, extra: tuple) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags(src) + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def device_asm(src: str, extra_flags=()) -> str:
    """gfx950 assembly of one source file, compiled with the library's flags."""
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        cmd = [hipcc()] + flags(src) + list(extra_flags) + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
        return open(out).read()


def build(jobs: int = 4, extra_flags=(), lib_path: str = LIB) -> str:
    """Compile every source and link ``lib_path``. ``extra_flags`` (e.g. -D tuning
    macros) go to every hipcc compile; objects go to a build folder next to the library."""
    build_dir = BUILD if lib_path == LIB else os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(extra_flags)), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    if lib_path == LIB:
        build_ceilings()
    return lib_path


CEILINGS_SRC = "ceilings.hip"
CEILINGS = os.path.join(HERE, "fa_ceilings")


def build_ceilings() -> str:
    """Compile the unit-ceiling microbenchmarks (``csrc/ceilings.hip``) into the
    program ``fa_ceilings`` next to the library (``bench.py --ceilings`` runs it)."""
    tmp = CEILINGS + ".tmp"
    cmd = [hipcc()] + flags(CEILINGS_SRC) + [os.path.join(CSRC, CEILINGS_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEILINGS_SRC}:\n{r.stderr}")
    os.replace(tmp, CEILINGS)
    return CEILINGS


if __name__ == "__main__":
    print(build())
