"""Builds and loads the oracle's C routines (oracle/*.c) with the host C compiler.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  ``build()`` compiles the library
in-tree (``__graft_entry__.build()`` calls it, so the built file travels with the tree);
``lib()`` loads it, compiling first if it is missing or older than a source.  The flags
keep the source's arithmetic as written: no contraction of separate multiplies and adds,
no fast-math reassociation; ``-mfma`` lets the compiler emit the hardware fused
multiply-add for ``fmaf`` (the same correctly rounded operation as the library call).
"""

import ctypes
import glob
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_c.so")
FLAGS = ["-O3", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None


def sources():
    return sorted(glob.glob(os.path.join(HERE, "*.c")))


def build(verbose: bool = False) -> str:
    fd, tmp = tempfile.mkstemp(prefix=".liboracle_c.", suffix=".so", dir=HERE)
    os.close(fd)
    cmd = ["gcc", *FLAGS, *sources(), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    try:
        subprocess.run(cmd, check=True)
        os.chmod(tmp, 0o755)
        os.replace(tmp, LIB)  # atomic: a concurrent loader sees the old file or the new one
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or any(os.path.getmtime(s) > os.path.getmtime(LIB) for s in sources()):
            build()
        c = ctypes.CDLL(LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        c.oracle_indexer_fma.argtypes = [fp, ctypes.c_int, ctypes.c_int, fp, ctypes.c_long, fp, fp]
        c.oracle_indexer_fma.restype = None
        _lib = c
    return _lib
