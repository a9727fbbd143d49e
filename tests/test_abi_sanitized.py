"""The C ABI's host-side checks (csrc/api.hip) under AddressSanitizer and
UndefinedBehaviorSanitizer.

api.hip is compiled for the host only, with both sanitizers and every report
fatal, and linked with a stub of the kernel launchers (tests/sanitize/
launch_stub.hip) and a driver (tests/sanitize/abi_checks.cpp) that calls every
entry point with bad arguments, with arguments at the limits of the size
arithmetic, with good arguments (checking which launchers run and where the
workspace parts lie) and with a failing launch.  No GPU is needed or touched.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
OUT = os.path.join(ROOT, "_build", "sanitize")

# host-only objects; -Xarch_host keeps the sanitizers off any device code
FLAGS = ["--offload-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
         "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def checker():
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("the ROCm compilers are not installed")
    os.makedirs(OUT, exist_ok=True)
    units = [
        (os.path.join(ROOT, "bitlinear_absmean_ternarise_bit_amd", "csrc", "api.hip"), "api.o", []),
        (os.path.join(ROOT, "tests", "sanitize", "launch_stub.hip"), "stub.o", []),
        (os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp"), "driver.o", ["-x", "c++"]),
    ]
    objs = []
    for src, obj, extra in units:
        out = os.path.join(OUT, obj)
        _run([HIPCC, *FLAGS, *extra, "-c", src, "-o", out])
        objs.append(out)
    exe = os.path.join(OUT, "abi_checks")
    _run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe])
    return exe


def test_abi_checks_clean_under_asan_and_ubsan(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([checker], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "Sanitizer" not in res.stderr, res.stderr
    assert ", 0 failed" in res.stdout, res.stdout
    n = int(res.stdout.split()[0])
    assert n >= 200
