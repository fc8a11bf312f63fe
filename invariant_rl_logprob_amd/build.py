"""Build libril.so (the HIP kernels + the C ABI) in-tree for gfx950.

    python invariant_rl_logprob_amd/build.py      (or __graft_entry__.build())

Flags that are part of the numerical contract:
  -ffp-contract=off   the compiler fuses no multiply-add on its own: an FMA exists only
                      where the source writes __builtin_fmaf, identically for every
                      kernel that shares a routine;
  no -ffast-math      IEEE division/sqrt where the source asks for them;
  -Xclang -target-feature -Xclang -packed-fp32-ops   packed fp32 VALU forms are not emitted.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libril.so")
SOURCES = ["abi.cpp", "attn.hip", "prefill.hip", "mla.hip", "index.hip", "dense.hip", "lm_fp8.hip", "ssd.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    _check_undefined(tmp)
    os.replace(tmp, LIB)
    return LIB


def _check_undefined(path: str) -> None:
    """A shared library links with undefined symbols and fails only when loaded; a
    kernel template whose host launch stub was not emitted shows up here as an
    undefined ``__device_stub__`` symbol.  Refuse such a library at build time."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    r = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True)
    if r.returncode != 0:
        return  # no nm: the import check still fails loudly
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l or "_ZN3ril" in l]
    if missing:
        os.remove(path)
        raise RuntimeError("libril.so would have undefined library symbols:\n  " + "\n  ".join(missing))


if __name__ == "__main__":
    print(build(verbose=True))
