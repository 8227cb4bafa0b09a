"""Test-only HIP helpers (built by ``__graft_entry__.build()``, never by a
test): ``libmathprobe.so`` runs the decoder's device numerics over ranges of
inputs for the bitwise comparison with the oracle."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "math_probe.hip")
LIB_PATH = os.path.join(HERE, "libmathprobe.so")


def build() -> str:
    """Compile libmathprobe.so with the decoder library's flags."""
    import sys
    sys.path.insert(0, ROOT)
    from ctc_prefix_beam_amd.build import FLAGS
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    proc = subprocess.run([hipcc, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        p = ctypes.c_void_p
        L.math_probe.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int64, p, p, p, p]
        L.math_probe.restype = ctypes.c_int
        _lib = L
    return _lib
