"""CPU sanitizer tier: the fp64 oracle and the C ABI's host-side argument
validation built with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only), each run under its own test suite in a child process.

- oracle.c is compiled with gcc -fsanitize=address,undefined and the oracle
  pins (tests/test_oracle_pins.py) run against it (ORACLE_LIB points the
  binding at the sanitized copy).
- fa_api.cpp (every argument check of the C ABI) is compiled for the host with
  the same sanitizers (each -fsanitize= after -Xarch_host, so no GPU code is
  instrumented) and linked with the library's unmodified kernel objects; the
  C ABI tests (tests/test_abi.py) run against that library. Those tests call
  every entry point with valid and invalid arguments on a host without a GPU.

Any sanitizer report aborts the child, which fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ENV_SAN = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_child(args, preload, extra_env, timeout=600):
    env = dict(os.environ)
    env.update(ENV_SAN)
    env.update(extra_env)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, f"sanitized run failed (exit {r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return r


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None or shutil.which("gcc") is None:
        pytest.skip("gcc with libasan is not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                   check=True)
    r = _run_child(["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p", "no:cacheprovider"],
                   asan, {"ORACLE_LIB": lib, "OMP_NUM_THREADS": "4"})
    assert " passed" in r.stdout


def _clang_asan_runtime(hipcc):
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    if os.path.isabs(p) and os.path.exists(p):
        return p
    # the runtime sits in the clang resource directory next to hipcc's compiler
    r = subprocess.run([hipcc, "-print-resource-dir"], capture_output=True, text=True)
    p = os.path.join(r.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    return p if os.path.exists(p) else None


def test_c_abi_validation_under_asan_and_ubsan(tmp_path):
    from io_aware_tiled_07_amd import build as fabuild
    try:
        hipcc = fabuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")
    objs = [os.path.join(fabuild.BUILD, os.path.splitext(s)[0] + ".o") for s in fabuild.SOURCES if s != "fa_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's kernel objects are not built")
    asan = _clang_asan_runtime(hipcc)
    if asan is None:
        pytest.skip("clang's AddressSanitizer runtime is not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = str(tmp_path / "fa_api_san.o")
    lib = str(tmp_path / "libfa_san.so")
    cmd = [hipcc] + fabuild.flags("fa_api.cpp") + ["-g", "-O1"] + san + [
        "-c", os.path.join(fabuild.CSRC, "fa_api.cpp"), "-o", api_obj]
    subprocess.run(cmd, check=True, capture_output=True)
    cmd = [hipcc, f"--offload-arch={fabuild.ARCH}", "-shared", "-fPIC", "-shared-libsan"] + san + [
        "-o", lib, api_obj] + objs
    subprocess.run(cmd, check=True, capture_output=True)
    child = ("import sys, pytest\n"
             "import io_aware_tiled_07_amd as fa\n"
             f"fa._LIB_PATH = {lib!r}\n"
             "sys.exit(pytest.main(['tests/test_abi.py', '-q', '-x', '-p', 'no:cacheprovider']))\n")
    r = _run_child(["-c", child], asan, {})
    assert " passed" in r.stdout
