"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

csrc/abi.cpp (every entry point's validation, the page allocator, the workspace layout)
is compiled with both sanitizers on its host code, linked with tests/sanitize_abi.cpp and
with the built libril.so for the kernel launchers, and run on the CPU: model descriptions
of every kind and many broken ones, the page allocator (assignment, exhaustion, double and
out-of-range release), and batch validation with fake device pointers, which the library
checks and never dereferences.  No kernel is launched.  Skipped where hipcc or the built
library is absent."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "invariant_rl_logprob_amd")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.skipif(HIPCC is None or not os.path.exists(os.path.join(PKG, "libril.so")),
                    reason="needs hipcc and the built library")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    abi, drv, exe = (str(tmp_path / n) for n in ("abi.o", "drv.o", "sanitize_abi"))
    steps = [
        [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-ffp-contract=off",
         *SAN, *inc, "-c", os.path.join(PKG, "csrc", "abi.cpp"), "-o", abi],
        [HIPCC, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-O1", "-g", "-std=c++17", *SAN, *inc, "-c",
         os.path.join(ROOT, "tests", "sanitize_abi.cpp"), "-o", drv],
        [HIPCC, *SAN, abi, drv, "-L", PKG, "-lril", f"-Wl,-rpath,{PKG}", "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    syms = subprocess.run([nm, exe], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the checks are really compiled in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-4000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
    assert "sanitized ABI checks passed" in r.stdout
