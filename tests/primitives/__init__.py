"""Builds and loads the device-primitive test helper (prim_probe.hip): the
library's bf16 conversion and gate functions run on arbitrary inputs, for
the element-by-element checks in tests/test_gpu_primitives.py. Test
infrastructure only."""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parents[1]
LIB = HERE / "libprim_probe.so"
_lib = None


def build() -> Path:
    """Compiles the helper for gfx950 with the library's own flags."""
    from invariant_rmsnorm_amd import _build
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [_build.HIPCC, *_build.HIP_FLAGS, "-shared", f"-I{_build.CSRC}", f"-I{_build.INCLUDE}",
           str(HERE / "prim_probe.hip"), "-o", str(tmp)]
    out = subprocess.run(cmd, capture_output=True, text=True)
    if out.returncode:
        raise RuntimeError(out.stdout + out.stderr)
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is None:
        if not LIB.exists():
            raise ImportError(f"{LIB} is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(str(LIB))
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        lib.prim_pack_all.argtypes = [ctypes.c_uint32, i64, vp, vp]
        lib.prim_gates.argtypes = [vp, i64, vp, vp]
        _lib = lib
    return _lib
