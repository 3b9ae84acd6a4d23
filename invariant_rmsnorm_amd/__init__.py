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
    "rmsnorm_dgamma_chunk_rows", "rmsnorm_bwd_noalloc", "rmsnorm_gated_fwd_dt",
    "rmsnorm_gated_bwd_dt", "rmsnorm_add_fwd_dt", "rmsnorm_add_bwd_dt",
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
        "rmsnorm_dgamma_chunk_rows": ([i64], i),
        "rmsnorm_bwd_noalloc": ([vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp, i64, vp, vp], i),
        "rmsnorm_gated_fwd_dt": ([i, i, vp, i64, vp, i64, vp, i, f, i64, i64, i, i, vp, i64, vp,
                                  vp], i),
        "rmsnorm_gated_bwd_dt": ([i, i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, i, vp, i64,
                                  vp, i64, vp, vp, sz, vp], i),
        "rmsnorm_add_fwd_dt": ([i, i, vp, i64, vp, i64, vp, i, f, i64, i64, vp, i64, vp, i64, vp,
                                vp], i),
        "rmsnorm_add_bwd_dt": ([i, i, vp, i64, vp, i64, vp, i64, vp, vp, i, i64, i64, vp, i64, vp,
                                i64, vp, vp, sz, vp], i),
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


def rmsnorm_dgamma_chunk_rows(D: int) -> int:
    """Rows R of one dgamma block (a function of D alone; 0 for an invalid D)."""
    return load().rmsnorm_dgamma_chunk_rows(D)


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


def _arg(t, name, dtypes, shape, required=True):
    """Checks one tensor argument before its pointer reaches the library:
    type, dtype (one of `dtypes`), exact shape, and a memory layout the C
    side can address (1-D contiguous; 2-D with a contiguous last axis).
    Devices are checked afterwards by _same_device, so that a call with host
    tensors of the wrong dtype or shape names that mistake first."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(map(str, dtypes))}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dim() == 1 and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() == 2 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous last axis")
    return t


def _rows(x, name, dtypes):
    """The [T, D] activation that fixes a call's shape; returns (T, D)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D torch.Tensor [T, D]")
    _arg(x, name, dtypes, x.shape)
    return tuple(x.shape)


def _workspace(ws, name="workspace"):
    """A caller's dgamma workspace: fp32, contiguous; returns its bytes."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.float32 or not ws.is_contiguous():
        raise TypeError(f"{name} must be a contiguous torch.float32 tensor")
    return ws.numel() * ws.element_size()


def _same_device(*named):
    """Every given tensor must be a CUDA tensor on the first one's device."""
    ref = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor, got {t.device}")
        if ref is None:
            ref = t.device
        elif t.device != ref:
            raise ValueError(f"{name} is on {t.device}, the call's other tensors on {ref}")


# ---- entry points ----------------------------------------------------------------
# Each entry point checks every tensor argument (dtype, shape, layout,
# device) before it calls the library, so a malformed call raises here and
# never hands the kernels a pointer they would read or write out of bounds.

BF16, F32 = torch.bfloat16, torch.float32
ACT_DTYPES = (torch.bfloat16, torch.float16)
WEIGHT_DTYPES = (torch.bfloat16, torch.float16, torch.float32)


def _new(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def rmsnorm_fwd(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None, rstd=None,
                want_rstd=True, stream=None):
    """y = bf16((x * r) * w_eff); returns (y, rstd or None)."""
    T, D = _rows(x, "x", BF16)
    _arg(gamma, "gamma", F32, (D,))
    _arg(y, "y", BF16, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("gamma", gamma), ("y", y), ("rstd", rstd))
    y = _new((T, D), BF16, x) if y is None else y
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_fwd", load().rmsnorm_fwd(
        _ptr(x), _ld(x), _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y),
        _ptr(rstd), _stream(x, stream)))
    return y, rstd


def rmsnorm_residual_fwd(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None,
                         residual_out=None, rstd=None, want_rstd=True, stream=None):
    """(y, residual_out, rstd): the forward plus a byte copy of x."""
    T, D = _rows(x, "x", BF16)
    _arg(gamma, "gamma", F32, (D,))
    _arg(y, "y", BF16, (T, D), required=False)
    _arg(residual_out, "residual_out", BF16, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("gamma", gamma), ("y", y), ("residual_out", residual_out),
                 ("rstd", rstd))
    y = _new((T, D), BF16, x) if y is None else y
    if residual_out is None:
        residual_out = _new((T, D), BF16, x)
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_residual_fwd", load().rmsnorm_residual_fwd(
        _ptr(x), _ld(x), _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y),
        _ptr(residual_out), _ld(residual_out), _ptr(rstd), _stream(x, stream)))
    return y, residual_out, rstd


def _gated_args(x, z, gamma, out, rstd):
    T, D = _rows(x, "x", BF16)
    _arg(z, "z", BF16, (T, D))
    _arg(gamma, "gamma", F32, (D,))
    _arg(out, "out", BF16, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("z", z), ("gamma", gamma), ("out", out), ("rstd", rstd))
    return T, D


def rmsnorm_gated_fwd(x, z, gamma, zero_centered_gamma=False, eps=1e-6, *, out=None, rstd=None,
                      want_rstd=False, stream=None):
    """(out, rstd or None): out = bf16(((x * r) * w_eff) * silu(z))."""
    T, D = _gated_args(x, z, gamma, out, rstd)
    out = _new((T, D), BF16, x) if out is None else out
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_gated_fwd", load().rmsnorm_gated_fwd(
        _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(gamma), int(zero_centered_gamma), eps, T, D,
        _ptr(out), _ld(out), _ptr(rstd), _stream(x, stream)))
    return out, rstd


def rmsnorm_gated_fwd_ex(x, z, gamma, zero_centered_gamma=False, eps=1e-6, *,
                         activation=RMSN_GATE_SILU, rounding=RMSN_GATED_ROUND_FP32, out=None,
                         rstd=None, want_rstd=False, stream=None):
    """(out, rstd or None): the gated forward with a choice of activation
    (RMSN_GATE_*) and rounding convention (RMSN_GATED_ROUND_*)."""
    T, D = _gated_args(x, z, gamma, out, rstd)
    out = _new((T, D), BF16, x) if out is None else out
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_gated_fwd_ex", load().rmsnorm_gated_fwd_ex(
        _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(gamma), int(zero_centered_gamma), eps, T, D,
        int(activation), int(rounding), _ptr(out), _ld(out), _ptr(rstd), _stream(x, stream)))
    return out, rstd


def workspace_for(T, D, device):
    n = rmsnorm_bwd_workspace_bytes(T, D)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=device), n


def _dgamma_workspace(dgamma, workspace, T, D, like):
    """(workspace, bytes) for a call that writes dgamma (allocated when the
    caller gives none), or (None, 0) without dgamma."""
    if dgamma is None:
        return None, 0
    if workspace is None:
        workspace, _ = workspace_for(T, D, like.device)
    return workspace, _workspace(workspace)


def rmsnorm_bwd(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                dgamma=None, want_dx=True, want_dgamma=True, workspace=None, stream=None):
    """(dx or None, dgamma or None) from the saved rstd."""
    T, D = _rows(x, "x", BF16)
    _arg(g, "g", BF16, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", F32, (D,))
    _arg(g_residual, "g_residual", BF16, (T, D), required=False)
    _arg(dx, "dx", BF16, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("rstd", rstd), ("gamma", gamma), ("g_residual", g_residual),
                 ("dx", dx), ("dgamma", dgamma), ("workspace", workspace))
    if dx is None and want_dx:
        dx = _new((T, D), BF16, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
    _check("rmsnorm_bwd", load().rmsnorm_bwd(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma),
        T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx), _ptr(dgamma), _ptr(ws),
        nbytes, _stream(x, stream)))
    return dx, dgamma


def rmsnorm_bwd_noalloc(g, x, rstd, gamma, zero_centered_gamma=False, *, dx, dgamma,
                        g_residual=None, stream=None):
    """rmsnorm_bwd with the dgamma partials in the library's own device
    scratch: no workspace and no allocation, here or in the library. The
    caller passes the outputs dx and dgamma (either may be None, not both);
    calls that may overlap on one GPU race on the shared scratch."""
    T, D = _rows(x, "x", BF16)
    _arg(g, "g", BF16, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", F32, (D,))
    _arg(g_residual, "g_residual", BF16, (T, D), required=False)
    _arg(dx, "dx", BF16, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _same_device(("x", x), ("g", g), ("rstd", rstd), ("gamma", gamma), ("g_residual", g_residual),
                 ("dx", dx), ("dgamma", dgamma))
    _check("rmsnorm_bwd_noalloc", load().rmsnorm_bwd_noalloc(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma),
        T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx), _ptr(dgamma),
        _stream(x, stream)))
    return dx, dgamma


def rmsnorm_bwd_rows(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                     workspace=None, stream=None):
    """Stage 1 of the backward: dx (if given) and the dgamma partials into
    ``workspace`` (if given, fp32 [chunks, D rounded up to a multiple of 8]
    viewed flat)."""
    T, D = _rows(x, "x", BF16)
    _arg(g, "g", BF16, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", F32, (D,))
    _arg(g_residual, "g_residual", BF16, (T, D), required=False)
    _arg(dx, "dx", BF16, (T, D), required=False)
    nbytes = _workspace(workspace)
    _same_device(("x", x), ("g", g), ("rstd", rstd), ("gamma", gamma), ("g_residual", g_residual),
                 ("dx", dx), ("workspace", workspace))
    _check("rmsnorm_bwd_rows", load().rmsnorm_bwd_rows(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma),
        T, D, _ptr(g_residual), _ld(g_residual), _ptr(dx), _ld(dx), _ptr(workspace), nbytes,
        _stream(x, stream)))
    return dx, workspace


def rmsnorm_bwd_finish(workspace, T, D, dgamma, stream=None):
    """Stage 2 of the backward: dgamma from the partials."""
    _arg(dgamma, "dgamma", F32, (D,))
    nbytes = _workspace(workspace)
    _same_device(("dgamma", dgamma), ("workspace", workspace))
    _check("rmsnorm_bwd_finish", load().rmsnorm_bwd_finish(
        _ptr(workspace), nbytes, T, D, _ptr(dgamma), _stream(dgamma, stream)))
    return dgamma


def rmsnorm_gated_bwd(g, x, z, rstd, gamma, zero_centered_gamma=False, *,
                      activation=RMSN_GATE_SILU, dx=None, dz=None, dgamma=None, want_dx=True,
                      want_dz=True, want_dgamma=True, workspace=None, stream=None):
    """(dx or None, dz or None, dgamma or None): the backward of the gated
    forward (fp32 rounding convention) from the saved rstd."""
    T, D = _rows(x, "x", BF16)
    _arg(g, "g", BF16, (T, D))
    _arg(z, "z", BF16, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", F32, (D,))
    _arg(dx, "dx", BF16, (T, D), required=False)
    _arg(dz, "dz", BF16, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("z", z), ("rstd", rstd), ("gamma", gamma), ("dx", dx),
                 ("dz", dz), ("dgamma", dgamma), ("workspace", workspace))
    if dx is None and want_dx:
        dx = _new((T, D), BF16, x)
    if dz is None and want_dz:
        dz = _new((T, D), BF16, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
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
    T, D = _rows(x, "x", BF16)
    _arg(residual, "residual", BF16, (T, D))
    _arg(gamma, "gamma", F32, (D,))
    _arg(y, "y", BF16, (T, D), required=False)
    _arg(residual_out, "residual_out", BF16, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("residual", residual), ("gamma", gamma), ("y", y),
                 ("residual_out", residual_out), ("rstd", rstd))
    y = _new((T, D), BF16, x) if y is None else y
    if residual_out is None:
        residual_out = _new((T, D), BF16, x)
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_add_fwd", load().rmsnorm_add_fwd(
        _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(gamma), int(zero_centered_gamma),
        eps, T, D, _ptr(y), _ld(y), _ptr(residual_out), _ld(residual_out), _ptr(rstd),
        _stream(x, stream)))
    return y, residual_out, rstd


def _add_bwd_args(g, x, residual, rstd, gamma, g_residual_out, dh):
    T, D = _rows(x, "x", BF16)
    _arg(g, "g", BF16, (T, D))
    _arg(residual, "residual", BF16, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", F32, (D,))
    _arg(g_residual_out, "g_residual_out", BF16, (T, D), required=False)
    _arg(dh, "dh", BF16, (T, D), required=False)
    return T, D


def rmsnorm_add_bwd(g, x, residual, rstd, gamma, zero_centered_gamma=False, *,
                    g_residual_out=None, dh=None, dgamma=None, want_dh=True, want_dgamma=True,
                    workspace=None, stream=None):
    """(dh or None, dgamma or None): dh is the gradient of x and of residual."""
    T, D = _add_bwd_args(g, x, residual, rstd, gamma, g_residual_out, dh)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("residual", residual), ("rstd", rstd), ("gamma", gamma),
                 ("g_residual_out", g_residual_out), ("dh", dh), ("dgamma", dgamma),
                 ("workspace", workspace))
    if dh is None and want_dh:
        dh = _new((T, D), BF16, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
    _check("rmsnorm_add_bwd", load().rmsnorm_add_bwd(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, _ptr(g_residual_out), _ld(g_residual_out), _ptr(dh),
        _ld(dh), _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dh, dgamma


def rmsnorm_add_bwd_rows(g, x, residual, rstd, gamma, zero_centered_gamma=False, *,
                         g_residual_out=None, dh=None, workspace=None, stream=None):
    """Stage 1 of the fused add backward: dh (if given) and the dgamma
    partials into ``workspace`` (if given); rmsnorm_bwd_finish completes it."""
    T, D = _add_bwd_args(g, x, residual, rstd, gamma, g_residual_out, dh)
    nbytes = _workspace(workspace)
    _same_device(("x", x), ("g", g), ("residual", residual), ("rstd", rstd), ("gamma", gamma),
                 ("g_residual_out", g_residual_out), ("dh", dh), ("workspace", workspace))
    _check("rmsnorm_add_bwd_rows", load().rmsnorm_add_bwd_rows(
        _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(residual), _ld(residual), _ptr(rstd), _ptr(gamma),
        int(zero_centered_gamma), T, D, _ptr(g_residual_out), _ld(g_residual_out), _ptr(dh),
        _ld(dh), _ptr(workspace), nbytes, _stream(x, stream)))
    return dh, workspace


def rmsnorm_fwd_dt(x, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None, rstd=None,
                   want_rstd=True, stream=None):
    """rmsnorm_fwd for bf16 or fp16 x (y of the same type) and fp32, bf16 or
    fp16 gamma; returns (y, rstd or None)."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(y, "y", x.dtype, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("gamma", gamma), ("y", y), ("rstd", rstd))
    y = _new((T, D), x.dtype, x) if y is None else y
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_fwd_dt", load().rmsnorm_fwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(x), _ld(x), _ptr(gamma),
        int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y), _ptr(rstd), _stream(x, stream)))
    return y, rstd


def rmsnorm_bwd_dt(g, x, rstd, gamma, zero_centered_gamma=False, *, g_residual=None, dx=None,
                   dgamma=None, want_dx=True, want_dgamma=True, workspace=None, stream=None):
    """rmsnorm_bwd for bf16 or fp16 activations and fp32, bf16 or fp16
    gamma; returns (dx or None, dgamma fp32 or None)."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(g, "g", x.dtype, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(g_residual, "g_residual", x.dtype, (T, D), required=False)
    _arg(dx, "dx", x.dtype, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("rstd", rstd), ("gamma", gamma), ("g_residual", g_residual),
                 ("dx", dx), ("dgamma", dgamma), ("workspace", workspace))
    if dx is None and want_dx:
        dx = _new((T, D), x.dtype, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
    _check("rmsnorm_bwd_dt", load().rmsnorm_bwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(rstd),
        _ptr(gamma), int(zero_centered_gamma), T, D, _ptr(g_residual), _ld(g_residual),
        _ptr(dx), _ld(dx), _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dx, dgamma


def rmsnorm_gated_fwd_dt(x, z, gamma, zero_centered_gamma=False, eps=1e-6, *,
                         activation=RMSN_GATE_SILU, rounding=RMSN_GATED_ROUND_FP32, out=None,
                         rstd=None, want_rstd=False, stream=None):
    """rmsnorm_gated_fwd_ex for bf16 or fp16 x and z (out of the same type;
    the cast convention rounds to that type) and fp32, bf16 or fp16 gamma;
    returns (out, rstd or None)."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(z, "z", x.dtype, (T, D))
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(out, "out", x.dtype, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("z", z), ("gamma", gamma), ("out", out), ("rstd", rstd))
    out = _new((T, D), x.dtype, x) if out is None else out
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_gated_fwd_dt", load().rmsnorm_gated_fwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(x), _ld(x), _ptr(z), _ld(z), _ptr(gamma),
        int(zero_centered_gamma), eps, T, D, int(activation), int(rounding), _ptr(out), _ld(out),
        _ptr(rstd), _stream(x, stream)))
    return out, rstd


def rmsnorm_gated_bwd_dt(g, x, z, rstd, gamma, zero_centered_gamma=False, *,
                         activation=RMSN_GATE_SILU, dx=None, dz=None, dgamma=None, want_dx=True,
                         want_dz=True, want_dgamma=True, workspace=None, stream=None):
    """rmsnorm_gated_bwd for bf16 or fp16 activations and fp32, bf16 or fp16
    gamma; returns (dx or None, dz or None, dgamma fp32 or None)."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(g, "g", x.dtype, (T, D))
    _arg(z, "z", x.dtype, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(dx, "dx", x.dtype, (T, D), required=False)
    _arg(dz, "dz", x.dtype, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("z", z), ("rstd", rstd), ("gamma", gamma), ("dx", dx),
                 ("dz", dz), ("dgamma", dgamma), ("workspace", workspace))
    if dx is None and want_dx:
        dx = _new((T, D), x.dtype, x)
    if dz is None and want_dz:
        dz = _new((T, D), x.dtype, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
    _check("rmsnorm_gated_bwd_dt", load().rmsnorm_gated_bwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(z), _ld(z),
        _ptr(rstd), _ptr(gamma), int(zero_centered_gamma), T, D, int(activation), _ptr(dx),
        _ld(dx), _ptr(dz), _ld(dz), _ptr(dgamma), _ptr(ws), nbytes, _stream(x, stream)))
    return dx, dz, dgamma


def rmsnorm_add_fwd_dt(x, residual, gamma, zero_centered_gamma=False, eps=1e-6, *, y=None,
                       residual_out=None, rstd=None, want_rstd=True, stream=None):
    """rmsnorm_add_fwd for bf16 or fp16 x and residual (y and residual_out of
    the same type) and fp32, bf16 or fp16 gamma; returns (y, residual_out,
    rstd or None). ``y=x`` and ``residual_out=residual`` run in place."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(residual, "residual", x.dtype, (T, D))
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(y, "y", x.dtype, (T, D), required=False)
    _arg(residual_out, "residual_out", x.dtype, (T, D), required=False)
    _arg(rstd, "rstd", F32, (T,), required=False)
    _same_device(("x", x), ("residual", residual), ("gamma", gamma), ("y", y),
                 ("residual_out", residual_out), ("rstd", rstd))
    y = _new((T, D), x.dtype, x) if y is None else y
    if residual_out is None:
        residual_out = _new((T, D), x.dtype, x)
    if rstd is None and want_rstd:
        rstd = _new(T, F32, x)
    _check("rmsnorm_add_fwd_dt", load().rmsnorm_add_fwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(x), _ld(x), _ptr(residual), _ld(residual),
        _ptr(gamma), int(zero_centered_gamma), eps, T, D, _ptr(y), _ld(y), _ptr(residual_out),
        _ld(residual_out), _ptr(rstd), _stream(x, stream)))
    return y, residual_out, rstd


def rmsnorm_add_bwd_dt(g, x, residual, rstd, gamma, zero_centered_gamma=False, *,
                       g_residual_out=None, dh=None, dgamma=None, want_dh=True, want_dgamma=True,
                       workspace=None, stream=None):
    """rmsnorm_add_bwd for bf16 or fp16 activations and fp32, bf16 or fp16
    gamma; returns (dh or None, dgamma fp32 or None)."""
    T, D = _rows(x, "x", ACT_DTYPES)
    _arg(g, "g", x.dtype, (T, D))
    _arg(residual, "residual", x.dtype, (T, D))
    _arg(rstd, "rstd", F32, (T,))
    _arg(gamma, "gamma", WEIGHT_DTYPES, (D,))
    _arg(g_residual_out, "g_residual_out", x.dtype, (T, D), required=False)
    _arg(dh, "dh", x.dtype, (T, D), required=False)
    _arg(dgamma, "dgamma", F32, (D,), required=False)
    _workspace(workspace)
    _same_device(("x", x), ("g", g), ("residual", residual), ("rstd", rstd), ("gamma", gamma),
                 ("g_residual_out", g_residual_out), ("dh", dh), ("dgamma", dgamma),
                 ("workspace", workspace))
    if dh is None and want_dh:
        dh = _new((T, D), x.dtype, x)
    if dgamma is None and want_dgamma:
        dgamma = _new(D, F32, x)
    ws, nbytes = _dgamma_workspace(dgamma, workspace, T, D, x)
    _check("rmsnorm_add_bwd_dt", load().rmsnorm_add_bwd_dt(
        _DTYPES[x.dtype], _DTYPES[gamma.dtype], _ptr(g), _ld(g), _ptr(x), _ld(x), _ptr(residual),
        _ld(residual), _ptr(rstd), _ptr(gamma), int(zero_centered_gamma), T, D,
        _ptr(g_residual_out), _ld(g_residual_out), _ptr(dh), _ld(dh), _ptr(dgamma), _ptr(ws),
        nbytes, _stream(x, stream)))
    return dh, dgamma


def bigemm_bf16_xwt(x, w, *, y=None, stream=None):
    """Y = X @ W.T for bf16 X [M, K] and W [N, K] (K a multiple of 32), each
    row of Y independent of the batch around it."""
    M, K = _rows(x, "x", BF16)
    if not isinstance(w, torch.Tensor) or w.dim() != 2:
        raise ValueError("w must be a 2-D torch.Tensor [N, K]")
    N = w.shape[0]
    _arg(w, "w", BF16, (N, K))
    _arg(y, "y", BF16, (M, N), required=False)
    _same_device(("x", x), ("w", w), ("y", y))
    y = _new((M, N), BF16, x) if y is None else y
    _check("bigemm_bf16_xwt", load().bigemm_bf16_xwt(
        _ptr(x), _ld(x), _ptr(w), _ld(w), M, N, K, _ptr(y), _ld(y), _stream(x, stream)))
    return y


def bigemm_bf16_tile(M: int, N: int):
    """(rows, columns) of the output tile bigemm_bf16_xwt uses for M x N."""
    out = [ctypes.c_int64(0) for _ in range(2)]
    _check("bigemm_bf16_tile", load().bigemm_bf16_tile(M, N, *(ctypes.byref(v) for v in out)))
    return tuple(v.value for v in out)
