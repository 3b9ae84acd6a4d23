"""Thin Python binding of librmsnorm_mi355x.so (the gfx950 HIP library).

The functions carry the C-ABI's names and only marshal arguments: torch
tensors supply device memory and the current stream; every step of the
computation runs in the library's kernels. There is no fallback: if the
library is missing or a call is rejected, an exception is raised.

bf16 tensors are ``torch.bfloat16`` 2-D CUDA tensors with a contiguous last
axis (any row stride); gamma, rstd and dgamma are ``torch.float32``.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "librmsnorm_mi355x.so"
_lib = None

RMSN_OK = 0
RMSN_ERR_NULL = 1
RMSN_ERR_SHAPE = 2
RMSN_ERR_UNSUPPORTED_D = 3
RMSN_ERR_MISALIGNED = 4
RMSN_ERR_EPS = 5
RMSN_ERR_ALIASING = 6
RMSN_ERR_WORKSPACE = 7
RMSN_ERR_HIP = 8
RMSN_ERR_MODE = 9

RMSN_DTYPE_BF16 = 0
RMSN_DTYPE_F16 = 1
RMSN_DTYPE_F32 = 2
_DTYPES = {torch.bfloat16: RMSN_DTYPE_BF16, torch.float16: RMSN_DTYPE_F16,
           torch.float32: RMSN_DTYPE_F32}

RMSN_GATE_SILU = 0
RMSN_GATE_SIGMOID = 1
RMSN_GATED_ROUND_FP32 = 0
RMSN_GATED_ROUND_CAST = 1

EXPORTED = (
    "rmsnorm_abi_version", "rmsnorm_status_string", "rmsnorm_fwd", "rmsnorm_residual_fwd",
    "rmsnorm_gated_fwd", "rmsnorm_gated_fwd_ex", "rmsnorm_bwd_workspace_bytes",
    "rmsnorm_bwd_partials_layout", "rmsnorm_bwd", "rmsnorm_bwd_rows", "rmsnorm_bwd_finish",
    "rmsnorm_gated_bwd", "rmsnorm_add_fwd", "rmsnorm_add_bwd", "rmsnorm_add_bwd_rows",
    "rmsnorm_fwd_dt", "rmsnorm_bwd_dt", "bigemm_bf16_xwt", "bigemm_bf16_tile",
)


class RmsnormError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}")


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(str(LIB_PATH))
    i, i64, f, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "rmsnorm_abi_version": ([], i),
        "rmsnorm_status_string": ([i], ctypes.c_char_p),
        "rmsnorm_fwd": ([vp, i64, vp, i, f, i64, i64, vp, i64, vp, vp], i),
        "rmsnorm_residual_fwd": ([vp, i64, vp, i, f, i64, i64, vp, i64, vp, i64, vp, vp], i),
        "rmsnorm_gated_fwd": ([vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64, vp, vp], i),
        "rmsnorm_gated_fwd_ex": ([vp, i64, vp, i64, vp, i, f, i64, i64, i, i, vp, i64, vp, vp], i),
        "rmsnorm_bwd_workspace_bytes": ([i64, i64], sz),
        "rmsnorm_bwd_partials_layout": ([i64, i64, vp, vp, vp], i),
        "rmsnorm_bwd": ([vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp, i64, vp, vp, sz, vp], i),
        "rmsnorm_bwd_rows": ([vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp, i64, vp, sz, vp], i),
        "rmsnorm_bwd_finish": ([vp, sz, i64, i64, vp, vp], i),
        "rmsnorm_gated_bwd": ([vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, i, vp, i64, vp, i64,
                               vp, vp, sz, vp], i),
        "rmsnorm_add_fwd": ([vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64, vp, i64, vp, vp], i),
        "rmsnorm_add_bwd": ([vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp, i64, vp,
                             vp, sz, vp], i),
        "rmsnorm_add_bwd_rows": ([vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp,
                                  i64, vp, sz, vp], i),
        "rmsnorm_fwd_dt": ([i, i, vp, i64, vp, i, f, i64, i64, vp, i64, vp, vp], i),
        "rmsnorm_bwd_dt": ([i, i, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp, i64, vp, vp,
                            sz, vp], i),
        "bigemm_bf16_xwt": ([vp, i64, vp, i64, i64, i64, i64, vp, i64, vp], i),
        "bigemm_bf16_tile": ([i64, i64, vp, vp], i),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().rmsnorm_status_string(status).decode()


def rmsnorm_abi_version() -> int:
    return load().rmsnorm_abi_version()


def rmsnorm_bwd_workspace_bytes(T: int, D: int) -> int:
    return load().rmsnorm_bwd_workspace_bytes(T, D)


def rmsnorm_bwd_partials_layout(T: int, D: int):
    """(R, S, K): rows per block, blocks per group, chunks. Chunk k holds the
    groups k, k+K, k+2K, ... of S consecutive R-row blocks."""
    out = [ctypes.c_int64(0) for _ in range(3)]
    _check("rmsnorm_bwd_partials_layout", load().rmsnorm_bwd_partials_layout(
        T, D, *(ctypes.byref(v) for v in out)))
    return tuple(v.value for v in out)


def chunk_rows(k: int, T: int, D: int):
    """Row indices of dgamma chunk k, in the order the backward adds them."""
    R, S, K = rmsnorm_bwd_partials_layout(T, D)
    nblocks = -(-T // R)
    rows = []
    for q in range(k, -(-nblocks // S), K):
        for b in range(q * S, min(nblocks, (q + 1) * S)):
            rows.extend(range(b * R, min(T, (b + 1) * R)))
    return rows[::-1]


# ---- marshalling helpers -------------------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t):
    if t is None:
        return 0
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with a contiguous last axis")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _stream(t, stream):
    if stream is not None:
        return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else stream
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn, status):
    if status != RMSN_OK:
        raise RmsnormError(fn, status)


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError(f"{name} must be {dt}, got {t.dtype}")


# ---- entry points ----------------------------------------------------------------

def rmsnorm_fwd(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None, rstd=None,
                want_rstd=True, stream=None):
    """y = bf16((x * r) * w_eff); returns (y, rstd or None)."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(gamma, torch.float32, "gamma")
    T, D = x.shape
    y = torch.empty((T, D), dtype=torch.bfloat16, device=x.device) if y is None else y
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_fwd", load().rmsnorm_fwd(
        _ptr(x), _ld(x), _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y),
        _ptr(rstd), _stream(x, stream)))
    return y, rstd


def rmsnorm_residual_fwd(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None,
                         residual_out=None, rstd=None, want_rstd=True, stream=None):
    """(y, residual_out, rstd): the forward plus a byte copy of x."""
    _dtype(x, torch.bfloat16, "x")
    T, D = x.shape
    y = torch.empty((T, D), dtype=torch.bfloat16, device=x.device) if y is None else y
    if residual_out is None:
        residual_out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_residual_fwd", load().rmsnorm_residual_fwd(
        _ptr(x), _ld(x), _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y),
        _ptr(residual_out), _ld(residual_out), _ptr(rstd), _stream(x, stream)))
    return y, residual_out, rstd


def rmsnorm_gated_fwd(x, z, gamma, zero_centered_gamma=False, eps=1e-6, *, out=None, rstd=None,
                      want_rstd=False, stream=None):
    """(out, rstd or None): out = bf16(((x * r) * w_eff) * silu(z))."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(z, torch.bfloat16, "z")
    T, D = x.shape
    out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device) if out is None else out
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_gated_fwd", load().rmsnorm_gated_fwd(
        _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(gamma), int(zero_centered_gamma), eps, T, D,
        _ptr(out), _ld(out), _ptr(rstd), _stream(x, stream)))
    return out, rstd


def rmsnorm_gated_fwd_ex(x, z, gamma, zero_centered_gamma=False, eps=1e-6, *,
                         activation=RMSN_GATE_SILU, rounding=RMSN_GATED_ROUND_FP32, out=None,
                         rstd=None, want_rstd=False, stream=None):
    """(out, rstd or None): the gated forward with a choice of activation
    (RMSN_GATE_*) and rounding convention (RMSN_GATED_ROUND_*)."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(z, torch.bfloat16, "z")
    T, D = x.shape
    out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device) if out is None else out
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_gated_fwd_ex", load().rmsnorm_gated_fwd_ex(
        _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(gamma), int(zero_centered_gamma), eps, T, D,
        int(activation), int(rounding), _ptr(out), _ld(out), _ptr(rstd), _stream(x, stream)))
    return out, rstd


def workspace_for(T, D, device):
    n = rmsnorm_bwd_workspace_bytes(T, D)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=device), n


def rmsnorm_bwd(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                dgamma=None, want_dx=True, want_dgamma=True, workspace=None, stream=None):
    """(dx or None, dgamma or None) from the saved rstd."""
    _dtype(g, torch.bfloat16, "g")
    _dtype(x, torch.bfloat16, "x")
    T, D = x.shape
    if dx is None and want_dx:
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(D, dtype=torch.float32, device=x.device)
    ws, nbytes = (None, 0)
    if dgamma is not None:
        if workspace is None:
            workspace, _ = workspace_for(T, D, x.device)
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd", load().rmsnorm_bwd(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma),
        T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx), _ptr(dgamma), _ptr(ws),
        nbytes, _stream(x, stream)))
    return dx, dgamma


def rmsnorm_bwd_rows(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                     workspace=None, stream=None):
    """Stage 1 of the backward: dx (if given) and the dgamma partials into
    ``workspace`` (if given, fp32 [chunks, D rounded up to a multiple of 8]
    viewed flat)."""
    T, D = x.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd_rows", load().rmsnorm_bwd_rows(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma),
        T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx), _ptr(workspace), nbytes,
        _stream(x, stream)))
    return dx, workspace


def rmsnorm_bwd_finish(workspace, T, D, dgamma, stream=None):
    """Stage 2 of the backward: dgamma from the partials."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd_finish", load().rmsnorm_bwd_finish(
        _ptr(workspace), nbytes, T, D, _ptr(dgamma), _stream(dgamma, stream)))
    return dgamma


def rmsnorm_gated_bwd(g, x, z, rstd, gamma, zero_centered_gamma=False, *,
                      activation=RMSN_GATE_SILU, dx=None, dz=None, dgamma=None, want_dx=True,
                      want_dz=True, want_dgamma=True, workspace=None, stream=None):
    """(dx or None, dz or None, dgamma or None): the backward of the gated
    forward (fp32 rounding convention) from the saved rstd."""
    _dtype(g, torch.bfloat16, "g")
    _dtype(x, torch.bfloat16, "x")
    _dtype(z, torch.bfloat16, "z")
    T, D = x.shape
    if dx is None and want_dx:
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if dz is None and want_dz:
        dz = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(D, dtype=torch.float32, device=x.device)
    ws, nbytes = (None, 0)
    if dgamma is not None:
        if workspace is None:
            workspace, _ = workspace_for(T, D, x.device)
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    _check("rmsnorm_gated_bwd", load().rmsnorm_gated_bwd(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, int(activation), _ptr(dx), _ld(dx), _ptr(dz), _ld(dz),
        _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dx, dz, dgamma


def rmsnorm_add_fwd(x, residual, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None,
                    residual_out=None, rstd=None, want_rstd=True, stream=None):
    """(y, residual_out, rstd or None): the norm of h = x + residual (fp32
    sum) and the updated residual bf16(h). ``y=x`` and ``residual_out=residual``
    run in place."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(residual, torch.bfloat16, "residual")
    T, D = x.shape
    y = torch.empty((T, D), dtype=torch.bfloat16, device=x.device) if y is None else y
    if residual_out is None:
        residual_out = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_add_fwd", load().rmsnorm_add_fwd(
        _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(gamma), int(zero_centered_gamma),
        eps, T, D, _ptr(y), _ld(y), _ptr(residual_out), _ld(residual_out), _ptr(rstd),
        _stream(x, stream)))
    return y, residual_out, rstd


def rmsnorm_add_bwd(g, x, residual, rstd, gamma, zero_centered_gamma=False, *,
                    g_residual_out=None, dh=None, dgamma=None, want_dh=True, want_dgamma=True,
                    workspace=None, stream=None):
    """(dh or None, dgamma or None): dh is the gradient of x and of residual."""
    _dtype(g, torch.bfloat16, "g")
    _dtype(x, torch.bfloat16, "x")
    _dtype(residual, torch.bfloat16, "residual")
    T, D = x.shape
    if dh is None and want_dh:
        dh = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(D, dtype=torch.float32, device=x.device)
    ws, nbytes = (None, 0)
    if dgamma is not None:
        if workspace is None:
            workspace, _ = workspace_for(T, D, x.device)
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    _check("rmsnorm_add_bwd", load().rmsnorm_add_bwd(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, _ptr(g_residual_out), _ld(g_residual_out), _ptr(dh),
        _ld(dh), _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dh, dgamma


def rmsnorm_add_bwd_rows(g, x, residual, rstd, gamma, zero_centered_gamma=False, *,
                         g_residual_out=None, dh=None, workspace=None, stream=None):
    """Stage 1 of the fused add backward: dh (if given) and the dgamma
    partials into ``workspace`` (if given); rmsnorm_bwd_finish completes it."""
    T, D = x.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("rmsnorm_add_bwd_rows", load().rmsnorm_add_bwd_rows(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, _ptr(g_residual_out), _ld(g_residual_out), _ptr(dh),
        _ld(dh), _ptr(workspace), nbytes, _stream(x, stream)))
    return dh, workspace


def _dt_of(t, name, allowed):
    dt = _DTYPES.get(t.dtype)
    if dt is None or dt not in allowed:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")
    return dt


def rmsnorm_fwd_dt(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None, rstd=None,
                   want_rstd=True, stream=None):
    """rmsnorm_fwd for bf16 or fp16 x (y of the same type) and fp32, bf16 or
    fp16 gamma; returns (y, rstd or None)."""
    adt = _dt_of(x, "x", (RMSN_DTYPE_BF16, RMSN_DTYPE_F16))
    wdt = _dt_of(gamma, "gamma", (RMSN_DTYPE_BF16, RMSN_DTYPE_F16, RMSN_DTYPE_F32))
    T, D = x.shape
    y = torch.empty((T, D), dtype=x.dtype, device=x.device) if y is None else y
    if rstd is None and want_rstd:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    _check("rmsnorm_fwd_dt", load().rmsnorm_fwd_dt(
        adt, wdt, _ptr(x), _ld(x), _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y),
        _ld(y), _ptr(rstd), _stream(x, stream)))
    return y, rstd


def rmsnorm_bwd_dt(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                   dgamma=None, want_dx=True, want_dgamma=True, workspace=None, stream=None):
    """rmsnorm_bwd for bf16 or fp16 activations and fp32, bf16 or fp16
    gamma; returns (dx or None, dgamma fp32 or None)."""
    adt = _dt_of(x, "x", (RMSN_DTYPE_BF16, RMSN_DTYPE_F16))
    wdt = _dt_of(gamma, "gamma", (RMSN_DTYPE_BF16, RMSN_DTYPE_F16, RMSN_DTYPE_F32))
    if g.dtype != x.dtype:
        raise TypeError("g and x must have the same dtype")
    T, D = x.shape
    if dx is None and want_dx:
        dx = torch.empty((T, D), dtype=x.dtype, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(D, dtype=torch.float32, device=x.device)
    ws, nbytes = (None, 0)
    if dgamma is not None:
        if workspace is None:
            workspace, _ = workspace_for(T, D, x.device)
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    _check("rmsnorm_bwd_dt", load().rmsnorm_bwd_dt(
        adt, wdt, _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx),
        _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dx, dgamma


def bigemm_bf16_xwt(x, w, *, y=None, stream=None):
    """Y = X @ W.T for bf16 X [M, K] and W [N, K] (K a multiple of 32), each
    row of Y independent of the batch around it."""
    _dtype(x, torch.bfloat16, "x")
    _dtype(w, torch.bfloat16, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w must have the same K")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    _check("bigemm_bf16_xwt", load().bigemm_bf16_xwt(
        _ptr(x), _ld(x), _ptr(w), _ld(w), M, N, K, _ptr(y), _ld(y), _stream(x, stream)))
    return y


def bigemm_bf16_tile(M: int, N: int):
    """(rows, columns) of the output tile bigemm_bf16_xwt uses for M x N."""
    out = [ctypes.c_int64(0) for _ in range(2)]
    _check("bigemm_bf16_tile", load().bigemm_bf16_tile(M, N, *(ctypes.byref(v) for v in out)))
    return tuple(v.value for v in out)
