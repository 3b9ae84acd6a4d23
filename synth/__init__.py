"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This package only draws random numbers (``synth.c``: counter-based SplitMix64
plus Box-Muller). It holds none of RMSNorm's arithmetic, and neither the CPU
oracle nor the HIP library imports it: both receive the arrays made here as
plain inputs.

bf16 tensors are returned as ``numpy.uint16`` arrays of raw bf16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_LIB_PATH = _HERE / "libsynth.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile ``synth.c`` into ``libsynth.so`` next to it (plain gcc)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             str(_HERE / "synth.c"), "-lm", "-o", str(tmp)],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build(force=False)
        lib = ctypes.CDLL(str(_LIB_PATH))
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        vp = ctypes.c_void_p
        lib.synth_u64.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_u64.restype = None
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, ctypes.c_float,
                                         ctypes.c_float, vp]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_bf16_rows.argtypes = [u64, u64, i64, i64, i64, i64,
                                               ctypes.c_float, vp, ctypes.c_int]
        lib.synth_normal_bf16_rows.restype = None
        _lib = lib
    return _lib


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def uint64s(seed: int, stream: int, n: int, first: int = 0) -> np.ndarray:
    """Raw 64-bit draws ``first .. first+n-1`` of stream (seed, stream)."""
    out = np.empty(n, dtype=np.uint64)
    if n:
        _load().synth_u64(seed, stream, first, n, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0,
               std: float = 1.0, first: int = 0) -> np.ndarray:
    """``mean + std * N(0,1)`` in fp32, ``n`` values."""
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_normal_f32(seed, stream, first, n, mean, std,
                                 out.ctypes.data)
    return out


def normal_bf16(seed: int, stream: int, rows: int, D: int, scale: float = 1.0,
                row0: int = 0, ld: int | None = None,
                out: np.ndarray | None = None) -> np.ndarray:
    """Rows ``row0 .. row0+rows-1`` of the bf16 matrix ``scale * N(0,1)``.

    Element (t, c) is drawn at counter ``t*D + c``, so any single row can be
    regenerated without the others. With ``ld > D`` the result has shape
    ``[rows, ld]`` and columns ``D..ld-1`` are zero.
    """
    ld = D if ld is None else ld
    if out is None:
        out = np.zeros((rows, ld), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    assert out.shape[0] >= rows and out.shape[1] == ld
    if rows and D:
        _load().synth_normal_bf16_rows(seed, stream, row0, rows, D, ld, scale,
                                       out.ctypes.data, _threads())
    return out


def pick_rows(seed: int, stream: int, T: int, k: int) -> np.ndarray:
    """``k`` distinct row indices of ``range(T)``, ascending, chosen as the
    rows whose 64-bit draws are smallest."""
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    h = uint64s(seed, stream, T)
    return np.sort(np.argsort(h, kind="stable")[:k]).astype(np.int64)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A seeded permutation of ``range(n)`` (rows ordered by their draws)."""
    return np.argsort(uint64s(seed, stream, n), kind="stable").astype(np.int64)


from . import workloads  # noqa: E402,F401  (recipes built on the draws above)
