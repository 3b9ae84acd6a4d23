"""Python binding of the CPU oracle (``rmsnorm_oracle.cpp``) — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library does not use it.

Arrays are numpy: bf16 values as ``uint16`` raw bits, fp32 as ``float32``,
the exact forms as ``float64``. Outputs are freshly allocated and returned.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_LIB_PATH = _HERE / "liboracle_rmsnorm.so"
_lib = None

R64, A32 = 0, 1
BF16, F16, F32 = 0, 1, 2        # storage types of activations and weights
SILU, SIGMOID = 0, 1          # gate activations
FP32_WEIGHT, CAST_INPUT = 0, 1  # gated-norm rounding conventions


def build(force: bool = True, extra_flags: tuple[str, ...] = ()) -> Path:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        subprocess.run(
            ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", *extra_flags, str(_HERE / "rmsnorm_oracle.cpp"),
             "-o", str(tmp)],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        build(force=False)
    lib = ctypes.CDLL(str(_LIB_PATH))
    i, i64, f, d, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                        ctypes.c_double, ctypes.c_void_p)
    sigs = {
        "oracle_bf16_decode": ([vp, i64, vp], None),
        "oracle_bf16_encode": ([vp, i64, vp], None),
        "oracle_weights": ([vp, i, i64, vp], i),
        "oracle_rmsnorm_fwd": ([i, vp, i64, vp, i, f, i64, i64, vp, i64, vp], i),
        "oracle_rmsnorm_residual_fwd": ([i, vp, i64, vp, i, f, i64, i64, vp, i64,
                                         vp, i64, vp], i),
        "oracle_rmsnorm_gated_fwd": ([i, vp, i64, vp, i64, vp, i, f, i64, i64, vp,
                                      i64, vp], i),
        "oracle_rmsnorm_bwd_dx": ([i, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64,
                                   vp, i64], i),
        "oracle_rmsnorm_dgamma": ([i, vp, i64, vp, i64, vp, i64, i64, vp], i),
        "oracle_rmsnorm_fwd_f64": ([vp, vp, i, d, i64, i64, vp, vp], i),
        "oracle_rmsnorm_gated_fwd_f64": ([vp, vp, vp, i, d, i64, i64, vp], i),
        "oracle_rmsnorm_bwd_f64": ([vp, vp, vp, i, d, i64, i64, vp, vp, vp], i),
        "oracle_set_mutation": ([i], None),
        "oracle_rmsnorm_gated_fwd_ex": ([i, i, i, vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64,
                                         vp], i),
        "oracle_rmsnorm_gated_fwd_f32io": ([i, i, vp, vp, vp, i, f, i64, i64, vp], i),
        "oracle_rmsnorm_gated_bwd": ([i, i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp,
                                      i64, vp, i64], i),
        "oracle_rmsnorm_gated_dgamma": ([i, i, vp, i64, vp, i64, vp, i64, vp, i64, i64, vp], i),
        "oracle_rmsnorm_gated_fwd_ex_f64": ([i, vp, vp, vp, i, d, i64, i64, vp], i),
        "oracle_rmsnorm_gated_bwd_f64": ([i, vp, vp, vp, vp, i, d, i64, i64, vp, vp, vp], i),
        "oracle_rmsnorm_add_fwd": ([i, vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64, vp, i64,
                                    vp], i),
        "oracle_rmsnorm_add_bwd": ([i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64,
                                    vp, i64, vp], i),
        "oracle_rmsnorm_add_fwd_f64": ([vp, vp, vp, i, d, i64, i64, vp, vp, vp], i),
        "oracle_rmsnorm_add_bwd_f64": ([vp, vp, vp, vp, i, d, i64, i64, vp, vp, vp], i),
        "oracle_f16_decode": ([vp, i64, vp], None),
        "oracle_f16_encode": ([vp, i64, vp], None),
        "oracle_rmsnorm_fwd_dt": ([i, i, i, vp, i64, vp, i, f, i64, i64, vp, i64, vp], i),
        "oracle_rmsnorm_bwd_dx_dt": ([i, i, i, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp,
                                      i64], i),
        "oracle_rmsnorm_dgamma_dt": ([i, i, vp, i64, vp, i64, vp, i64, i64, vp], i),
        "oracle_gemm_xwt": ([vp, i64, vp, i64, i64, i64, i64, vp, i64, vp], i),
        "oracle_rmsnorm_gated_fwd_dt": ([i, i, i, i, i, vp, i64, vp, i64, vp, i, f, i64, i64, vp,
                                         i64, vp], i),
        "oracle_rmsnorm_gated_bwd_dt": ([i, i, i, i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64,
                                         vp, i64, vp, i64], i),
        "oracle_rmsnorm_gated_dgamma_dt": ([i, i, i, vp, i64, vp, i64, vp, i64, vp, i64, i64, vp],
                                           i),
        "oracle_rmsnorm_add_fwd_dt": ([i, i, i, vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64, vp,
                                       i64, vp], i),
        "oracle_rmsnorm_add_bwd_dt": ([i, i, i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp,
                                       i64, vp, i64, vp], i),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _bf16_2d(a, D=None):
    a = np.asarray(a)
    assert a.dtype == np.uint16 and a.ndim == 2, "bf16 [T, ld] uint16"
    if a.shape[0] <= 1:
        return np.ascontiguousarray(a)
    if a.strides[1] != 2 or a.strides[0] % 2 or a.strides[0] < 2 * a.shape[1]:
        a = np.ascontiguousarray(a)
    return a


def _ld(a):
    """Row stride in elements (any value >= D for a batch of at most one row)."""
    return a.strides[0] // 2 if a.shape[0] > 1 else a.shape[1]


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: bad argument (rc={rc})")


# ---- bf16 codec ----------------------------------------------------------------

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().oracle_bf16_decode(_p(bits), bits.size, _p(out))
    return out


def bf16_encode(vals: np.ndarray) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.shape, dtype=np.uint16)
    _load().oracle_bf16_encode(_p(vals), vals.size, _p(out))
    return out


def weights(gamma: np.ndarray, zero_centered: bool) -> np.ndarray:
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty_like(gamma)
    _check(_load().oracle_weights(_p(gamma), int(zero_centered), gamma.size, _p(out)),
           "weights")
    return out


# ---- rounded forms (R64 parity reference, A32 report mode) ---------------------

def _shape(x, D):
    T = x.shape[0]
    return T, (x.shape[1] if D is None else D)


def fwd(x, gamma, zero_centered=False, eps=1e-6, mode=R64, D=None):
    """(y bf16 [T, D], rstd fp32 [T]). ``D`` < row stride lets x be strided."""
    x = _bf16_2d(x, D)
    T, D = _shape(x, D)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    y = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_fwd(mode, _p(x), _ld(x), _p(gamma),
                                      int(zero_centered), eps, T, D, _p(y), D, _p(rstd)),
           "fwd")
    return y, rstd


def residual_fwd(x, gamma, zero_centered=False, eps=1e-6, mode=R64, D=None):
    """(y, residual_out, rstd)."""
    x = _bf16_2d(x, D)
    T, D = _shape(x, D)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    y = np.empty((T, D), dtype=np.uint16)
    res = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_residual_fwd(mode, _p(x), _ld(x), _p(gamma),
                                               int(zero_centered), eps, T, D, _p(y), D,
                                               _p(res), D, _p(rstd)),
           "residual_fwd")
    return y, res, rstd


def gated_fwd(x, z, gamma, zero_centered=False, eps=1e-6, mode=R64, D=None):
    """(out bf16, rstd)."""
    x = _bf16_2d(x, D)
    z = _bf16_2d(z, D)
    T, D = _shape(x, D)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_gated_fwd(mode, _p(x), _ld(x), _p(z),
                                            _ld(z), _p(gamma),
                                            int(zero_centered), eps, T, D, _p(out), D,
                                            _p(rstd)),
           "gated_fwd")
    return out, rstd


def bwd_dx(g, x, rstd, gamma, zero_centered=False, gres=None, mode=R64, D=None):
    g = _bf16_2d(g, D)
    x = _bf16_2d(x, D)
    T, D = _shape(x, D)
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    if gres is not None:
        gres = _bf16_2d(gres, D)
    dx = np.empty((T, D), dtype=np.uint16)
    _check(_load().oracle_rmsnorm_bwd_dx(mode, _p(g), _ld(g), _p(x),
                                         _ld(x), _p(rstd), _p(gamma),
                                         int(zero_centered), T, D, _p(gres),
                                         0 if gres is None else _ld(gres),
                                         _p(dx), D),
           "bwd_dx")
    return dx


def dgamma(g, x, rstd, mode=R64, D=None):
    g = _bf16_2d(g, D)
    x = _bf16_2d(x, D)
    T, D = _shape(x, D)
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    out = np.empty(D, dtype=np.float32)
    _check(_load().oracle_rmsnorm_dgamma(mode, _p(g), _ld(g), _p(x),
                                         _ld(x), _p(rstd), T, D, _p(out)),
           "dgamma")
    return out


def bwd(g, x, rstd, gamma, zero_centered=False, gres=None, mode=R64):
    """(dx bf16 [T, D], dgamma fp32 [D])."""
    return (bwd_dx(g, x, rstd, gamma, zero_centered, gres, mode),
            dgamma(g, x, rstd, mode))


# ---- exact double forms --------------------------------------------------------

def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def fwd_f64(x, gamma, zero_centered=False, eps=1e-6):
    x, gamma = _f64(x), _f64(gamma)
    T, D = x.shape
    y = np.empty((T, D))
    rstd = np.empty(T)
    _check(_load().oracle_rmsnorm_fwd_f64(_p(x), _p(gamma), int(zero_centered), eps,
                                          T, D, _p(y), _p(rstd)), "fwd_f64")
    return y, rstd


def gated_fwd_f64(x, z, gamma, zero_centered=False, eps=1e-6):
    x, z, gamma = _f64(x), _f64(z), _f64(gamma)
    T, D = x.shape
    out = np.empty((T, D))
    _check(_load().oracle_rmsnorm_gated_fwd_f64(_p(x), _p(z), _p(gamma),
                                                int(zero_centered), eps, T, D, _p(out)),
           "gated_fwd_f64")
    return out


def bwd_f64(g, x, gamma, zero_centered=False, eps=1e-6, gres=None):
    g, x, gamma = _f64(g), _f64(x), _f64(gamma)
    gres = None if gres is None else _f64(gres)
    T, D = x.shape
    dx = np.empty((T, D))
    dg = np.empty(D)
    _check(_load().oracle_rmsnorm_bwd_f64(_p(g), _p(x), _p(gamma), int(zero_centered),
                                          eps, T, D, _p(gres), _p(dx), _p(dg)),
           "bwd_f64")
    return dx, dg


@contextlib.contextmanager
def mutation(m: int):
    """Plant one of the two defects (1: forward drops the zero-centred offset;
    2: dx's second term takes the weight twice) for the duration of a block."""
    lib = _load()
    lib.oracle_set_mutation(m)
    try:
        yield
    finally:
        lib.oracle_set_mutation(0)


# ---- gated-norm variants -------------------------------------------------------

def gated_fwd_ex(x, z, gamma, zero_centered=False, eps=1e-6, activation=SILU,
                 convention=FP32_WEIGHT, mode=R64):
    """(out bf16, rstd) for either gate activation and rounding convention."""
    x = _bf16_2d(x)
    z = _bf16_2d(z)
    T, D = x.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_gated_fwd_ex(mode, activation, convention, _p(x), _ld(x),
                                               _p(z), _ld(z), _p(gamma), int(zero_centered),
                                               eps, T, D, _p(out), D, _p(rstd)),
           "gated_fwd_ex")
    return out, rstd


def gated_fwd_f32io(x, z, gamma, zero_centered=False, eps=1e-6, activation=SILU,
                    convention=FP32_WEIGHT):
    """The gated forward on fp32 inputs and outputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    z = np.ascontiguousarray(z, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    T, D = x.shape
    out = np.empty((T, D), dtype=np.float32)
    _check(_load().oracle_rmsnorm_gated_fwd_f32io(activation, convention, _p(x), _p(z),
                                                  _p(gamma), int(zero_centered), eps, T, D,
                                                  _p(out)),
           "gated_fwd_f32io")
    return out


def gated_bwd(g, x, z, rstd, gamma, zero_centered=False, activation=SILU, mode=R64):
    """(dx bf16, dz bf16, dgamma fp32) of the gated norm (fp32 convention)."""
    g, x, z = _bf16_2d(g), _bf16_2d(x), _bf16_2d(z)
    T, D = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    dx = np.empty((T, D), dtype=np.uint16)
    dz = np.empty((T, D), dtype=np.uint16)
    dg = np.empty(D, dtype=np.float32)
    lib = _load()
    _check(lib.oracle_rmsnorm_gated_bwd(mode, activation, _p(g), _ld(g), _p(x), _ld(x), _p(z),
                                        _ld(z), _p(rstd), _p(gamma), int(zero_centered), T, D,
                                        _p(dx), D, _p(dz), D), "gated_bwd")
    _check(lib.oracle_rmsnorm_gated_dgamma(mode, activation, _p(g), _ld(g), _p(x), _ld(x), _p(z),
                                           _ld(z), _p(rstd), T, D, _p(dg)), "gated_dgamma")
    return dx, dz, dg


def gated_fwd_ex_f64(x, z, gamma, zero_centered=False, eps=1e-6, activation=SILU):
    x, z, gamma = _f64(x), _f64(z), _f64(gamma)
    T, D = x.shape
    out = np.empty((T, D))
    _check(_load().oracle_rmsnorm_gated_fwd_ex_f64(activation, _p(x), _p(z), _p(gamma),
                                                   int(zero_centered), eps, T, D, _p(out)),
           "gated_fwd_ex_f64")
    return out


def gated_bwd_f64(g, x, z, gamma, zero_centered=False, eps=1e-6, activation=SILU):
    """(dx, dz, dgamma) in double."""
    g, x, z, gamma = _f64(g), _f64(x), _f64(z), _f64(gamma)
    T, D = x.shape
    dx, dz, dg = np.empty((T, D)), np.empty((T, D)), np.empty(D)
    _check(_load().oracle_rmsnorm_gated_bwd_f64(activation, _p(g), _p(x), _p(z), _p(gamma),
                                                int(zero_centered), eps, T, D, _p(dx), _p(dz),
                                                _p(dg)),
           "gated_bwd_f64")
    return dx, dz, dg


# ---- fused add-RMSNorm ---------------------------------------------------------

def add_fwd(x, residual, gamma, zero_centered=False, eps=1e-6, mode=R64):
    """(y bf16, residual_out bf16, rstd fp32): the norm of h = x + residual
    (fp32 sum), residual_out = bf16(h)."""
    x, residual = _bf16_2d(x), _bf16_2d(residual)
    T, D = x.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    y = np.empty((T, D), dtype=np.uint16)
    rout = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_add_fwd(mode, _p(x), _ld(x), _p(residual), _ld(residual),
                                          _p(gamma), int(zero_centered), eps, T, D, _p(y), D,
                                          _p(rout), D, _p(rstd)), "add_fwd")
    return y, rout, rstd


def add_bwd(g, x, residual, rstd, gamma, zero_centered=False, g_rout=None, mode=R64,
            want_dh=True, want_dgamma=True):
    """(dh bf16, dgamma fp32) (each None unless wanted): dh is the gradient of
    x and of residual."""
    g, x, residual = _bf16_2d(g), _bf16_2d(x), _bf16_2d(residual)
    T, D = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    if g_rout is not None:
        g_rout = _bf16_2d(g_rout)
    dh = np.empty((T, D), dtype=np.uint16) if want_dh else None
    dg = np.empty(D, dtype=np.float32) if want_dgamma else None
    _check(_load().oracle_rmsnorm_add_bwd(mode, _p(g), _ld(g), _p(x), _ld(x), _p(residual),
                                          _ld(residual), _p(rstd), _p(gamma),
                                          int(zero_centered), T, D, _p(g_rout),
                                          0 if g_rout is None else _ld(g_rout), _p(dh), D,
                                          _p(dg)), "add_bwd")
    return dh, dg


def add_fwd_f64(x, residual, gamma, zero_centered=False, eps=1e-6):
    """(y, h, rstd) in double, h = x + residual."""
    x, residual, gamma = _f64(x), _f64(residual), _f64(gamma)
    T, D = x.shape
    y, h, rstd = np.empty((T, D)), np.empty((T, D)), np.empty(T)
    _check(_load().oracle_rmsnorm_add_fwd_f64(_p(x), _p(residual), _p(gamma), int(zero_centered),
                                              eps, T, D, _p(y), _p(h), _p(rstd)), "add_fwd_f64")
    return y, h, rstd


def add_bwd_f64(g, x, residual, gamma, zero_centered=False, eps=1e-6, g_rout=None):
    """(dh, dgamma) in double for L = sum g*y + sum g_rout*h."""
    g, x, residual, gamma = _f64(g), _f64(x), _f64(residual), _f64(gamma)
    g_rout = None if g_rout is None else _f64(g_rout)
    T, D = x.shape
    dh, dg = np.empty((T, D)), np.empty(D)
    _check(_load().oracle_rmsnorm_add_bwd_f64(_p(g), _p(x), _p(residual), _p(gamma),
                                              int(zero_centered), eps, T, D, _p(g_rout), _p(dh),
                                              _p(dg)), "add_bwd_f64")
    return dh, dg


# ---- activation and weight dtypes ----------------------------------------------

def f16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    _load().oracle_f16_decode(_p(bits), bits.size, _p(out))
    return out


def f16_encode(vals: np.ndarray) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.shape, dtype=np.uint16)
    _load().oracle_f16_encode(_p(vals), vals.size, _p(out))
    return out


def _weights(gamma, weight_dtype):
    """gamma as stored: fp32 values, or 16-bit patterns (uint16) for BF16/F16."""
    dt = np.float32 if weight_dtype == F32 else np.uint16
    return np.ascontiguousarray(gamma, dtype=dt)


def fwd_dt(x, gamma, zero_centered=False, eps=1e-6, act_dtype=BF16, weight_dtype=F32, mode=R64):
    """(y [T, D] in the activation type's bits, rstd fp32)."""
    x = _bf16_2d(x)
    T, D = x.shape
    gamma = _weights(gamma, weight_dtype)
    y = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_fwd_dt(mode, act_dtype, weight_dtype, _p(x), _ld(x), _p(gamma),
                                         int(zero_centered), eps, T, D, _p(y), D, _p(rstd)),
           "fwd_dt")
    return y, rstd


def bwd_dt(g, x, rstd, gamma, zero_centered=False, gres=None, act_dtype=BF16,
           weight_dtype=F32, mode=R64):
    """(dx in the activation type's bits, dgamma fp32)."""
    g, x = _bf16_2d(g), _bf16_2d(x)
    T, D = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = _weights(gamma, weight_dtype)
    if gres is not None:
        gres = _bf16_2d(gres)
    dx = np.empty((T, D), dtype=np.uint16)
    dg = np.empty(D, dtype=np.float32)
    lib = _load()
    _check(lib.oracle_rmsnorm_bwd_dx_dt(mode, act_dtype, weight_dtype, _p(g), _ld(g), _p(x),
                                        _ld(x), _p(rstd), _p(gamma), int(zero_centered), T, D,
                                        _p(gres), 0 if gres is None else _ld(gres), _p(dx), D),
           "bwd_dx_dt")
    _check(lib.oracle_rmsnorm_dgamma_dt(mode, act_dtype, _p(g), _ld(g), _p(x), _ld(x), _p(rstd),
                                        T, D, _p(dg)), "dgamma_dt")
    return dx, dg


def gated_fwd_dt(x, z, gamma, zero_centered=False, eps=1e-6, activation=SILU,
                 convention=FP32_WEIGHT, act_dtype=BF16, weight_dtype=F32, mode=R64):
    """(out in the activation type's bits, rstd fp32): the gated forward for
    bf16 / fp16 activations and fp32 / bf16 / fp16 weights."""
    x, z = _bf16_2d(x), _bf16_2d(z)
    T, D = x.shape
    gamma = _weights(gamma, weight_dtype)
    out = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_gated_fwd_dt(mode, act_dtype, weight_dtype, activation,
                                               convention, _p(x), _ld(x), _p(z), _ld(z), _p(gamma),
                                               int(zero_centered), eps, T, D, _p(out), D,
                                               _p(rstd)), "gated_fwd_dt")
    return out, rstd


def gated_bwd_dt(g, x, z, rstd, gamma, zero_centered=False, activation=SILU, act_dtype=BF16,
                 weight_dtype=F32, mode=R64):
    """(dx, dz in the activation type's bits, dgamma fp32) of the gated norm
    (fp32 convention)."""
    g, x, z = _bf16_2d(g), _bf16_2d(x), _bf16_2d(z)
    T, D = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = _weights(gamma, weight_dtype)
    dx = np.empty((T, D), dtype=np.uint16)
    dz = np.empty((T, D), dtype=np.uint16)
    dg = np.empty(D, dtype=np.float32)
    lib = _load()
    _check(lib.oracle_rmsnorm_gated_bwd_dt(mode, act_dtype, weight_dtype, activation, _p(g),
                                           _ld(g), _p(x), _ld(x), _p(z), _ld(z), _p(rstd),
                                           _p(gamma), int(zero_centered), T, D, _p(dx), D, _p(dz),
                                           D), "gated_bwd_dt")
    _check(lib.oracle_rmsnorm_gated_dgamma_dt(mode, act_dtype, activation, _p(g), _ld(g), _p(x),
                                              _ld(x), _p(z), _ld(z), _p(rstd), T, D, _p(dg)),
           "gated_dgamma_dt")
    return dx, dz, dg


def add_fwd_dt(x, residual, gamma, zero_centered=False, eps=1e-6, act_dtype=BF16,
               weight_dtype=F32, mode=R64):
    """(y, residual_out in the activation type's bits, rstd fp32) of the fused
    add-norm."""
    x, residual = _bf16_2d(x), _bf16_2d(residual)
    T, D = x.shape
    gamma = _weights(gamma, weight_dtype)
    y = np.empty((T, D), dtype=np.uint16)
    rout = np.empty((T, D), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float32)
    _check(_load().oracle_rmsnorm_add_fwd_dt(mode, act_dtype, weight_dtype, _p(x), _ld(x),
                                             _p(residual), _ld(residual), _p(gamma),
                                             int(zero_centered), eps, T, D, _p(y), D, _p(rout), D,
                                             _p(rstd)), "add_fwd_dt")
    return y, rout, rstd


def add_bwd_dt(g, x, residual, rstd, gamma, zero_centered=False, g_rout=None, act_dtype=BF16,
               weight_dtype=F32, mode=R64):
    """(dh in the activation type's bits, dgamma fp32) of the fused add-norm."""
    g, x, residual = _bf16_2d(g), _bf16_2d(x), _bf16_2d(residual)
    T, D = x.shape
    rstd = np.ascontiguousarray(rstd, dtype=np.float32)
    gamma = _weights(gamma, weight_dtype)
    if g_rout is not None:
        g_rout = _bf16_2d(g_rout)
    dh = np.empty((T, D), dtype=np.uint16)
    dg = np.empty(D, dtype=np.float32)
    _check(_load().oracle_rmsnorm_add_bwd_dt(mode, act_dtype, weight_dtype, _p(g), _ld(g), _p(x),
                                             _ld(x), _p(residual), _ld(residual), _p(rstd),
                                             _p(gamma), int(zero_centered), T, D, _p(g_rout),
                                             0 if g_rout is None else _ld(g_rout), _p(dh), D,
                                             _p(dg)), "add_bwd_dt")
    return dh, dg


# ---- batch-invariant GEMM --------------------------------------------------------

def gemm_xwt(x, w):
    """(Y bf16 [M, N], exact double sums [M, N]) of Y = X @ W.T for bf16
    X [M, K] and W [N, K]."""
    x, w = _bf16_2d(x), _bf16_2d(w)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((M, N), dtype=np.uint16)
    ye = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_gemm_xwt(_p(x), _ld(x) if M > 1 else K, _p(w), _ld(w) if N > 1 else K,
                                   M, N, K, _p(y), N, _p(ye)), "gemm_xwt")
    return y, ye
