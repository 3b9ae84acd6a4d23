"""The C-ABI library without a GPU: it loads, exports every function that
include/rmsnorm_mi355x.h declares, and rejects every malformed call on the
host before anything is launched (fake, never-dereferenced pointers).

Rejection rules follow TransformerEngine issue "Expose Batch Invariant
Kernels", checks table (unsupported combinations are rejected, not silently
sent elsewhere) and RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual",
"Correctness / Tests" (invalid inputs)."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

import invariant_rmsnorm_amd as irn

HEADER = Path(__file__).resolve().parents[1] / "include" / "rmsnorm_mi355x.h"

A = 0x7F0000000000          # aligned fake device addresses, far apart
B = A + (1 << 36)
C = A + (2 << 36)
E = A + (3 << 36)
W = A + (4 << 36)
GAM = A + (5 << 36)
RS = A + (6 << 36)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b((?:rmsnorm|bigemm)_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = irn.load()
    names = declared_functions()
    assert set(names) == set(irn.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert irn.rmsnorm_abi_version() == 14


def test_status_strings():
    for code in range(10):
        assert irn.status_string(code).startswith("RMSN_")
    assert "unknown" in irn.status_string(99)


def fwd(**kw):
    a = dict(x=A, ld_x=4096, gamma=GAM, zc=0, eps=1e-6, T=8, D=4096, y=B, ld_y=4096, rstd=RS)
    a.update(kw)
    return irn.load().rmsnorm_fwd(a["x"], a["ld_x"], a["gamma"], a["zc"], a["eps"], a["T"], a["D"],
                                  a["y"], a["ld_y"], a["rstd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), irn.RMSN_ERR_NULL),
    (dict(y=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None), irn.RMSN_ERR_NULL),
    (dict(T=-1), irn.RMSN_ERR_SHAPE),
    (dict(D=0), irn.RMSN_ERR_SHAPE),
    (dict(D=-8), irn.RMSN_ERR_SHAPE),
    (dict(D=32776, ld_x=32776, ld_y=32776), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(D=32769, ld_x=32769, ld_y=32769), irn.RMSN_ERR_UNSUPPORTED_D),
    # D not a multiple of 8: element-wise rows, 2-byte alignment, any stride
    (dict(D=100, ld_x=99, ld_y=100), irn.RMSN_ERR_SHAPE),
    (dict(D=100, ld_x=100, ld_y=101, x=A + 1), irn.RMSN_ERR_MISALIGNED),
    (dict(D=100, ld_x=100, ld_y=101, y=B + 3), irn.RMSN_ERR_MISALIGNED),
    (dict(D=100, ld_x=101, ld_y=101, y=A + 2), irn.RMSN_ERR_ALIASING),
    (dict(D=7, ld_x=7, ld_y=7, gamma=GAM + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_x=4000), irn.RMSN_ERR_SHAPE),
    (dict(ld_y=4088), irn.RMSN_ERR_SHAPE),
    (dict(x=A + 2), irn.RMSN_ERR_MISALIGNED),
    (dict(y=B + 8), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_x=4100), irn.RMSN_ERR_MISALIGNED),
    (dict(gamma=GAM + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(rstd=RS + 2), irn.RMSN_ERR_MISALIGNED),
    (dict(eps=-1e-6), irn.RMSN_ERR_EPS),
    (dict(eps=float("nan")), irn.RMSN_ERR_EPS),
    (dict(eps=float("inf")), irn.RMSN_ERR_EPS),
    (dict(y=A), irn.RMSN_ERR_ALIASING),                       # in place
    (dict(y=A + 2 * 4096 * 4), irn.RMSN_ERR_ALIASING),         # y starts inside x
    (dict(rstd=A + 64), irn.RMSN_ERR_ALIASING),                # rstd inside x
    (dict(rstd=B + 16), irn.RMSN_ERR_ALIASING),                # rstd inside y
    (dict(gamma=B + 32), irn.RMSN_ERR_ALIASING),               # y over gamma
    (dict(T=1 << 61), irn.RMSN_ERR_SHAPE),                     # byte offsets overflow
    (dict(ld_x=(1 << 24) + 8), irn.RMSN_ERR_SHAPE),            # row stride above 2^24
])
def test_forward_rejections(kw, code):
    assert fwd(**kw) == code


def test_forward_empty_batch_is_a_noop():
    assert fwd(T=0, x=None, y=None, rstd=None, gamma=None) == irn.RMSN_OK


def test_residual_and_gated_rejections():
    lib = irn.load()
    ok = (A, 4096, GAM, 0, 1e-6, 8, 4096, B)
    assert lib.rmsnorm_residual_fwd(*ok, 4096, None, 4096, RS, None) == irn.RMSN_ERR_NULL
    assert lib.rmsnorm_residual_fwd(*ok, 4096, A, 4096, RS, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_residual_fwd(*ok, 4096, B, 4096, RS, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_residual_fwd(*ok, 4096, C + 2, 4096, RS, None) == irn.RMSN_ERR_MISALIGNED
    # gated: z required, may not alias the output
    assert lib.rmsnorm_gated_fwd(A, 4096, None, 4096, GAM, 0, 1e-6, 8, 4096, B, 4096, None,
                                 None) == irn.RMSN_ERR_NULL
    assert lib.rmsnorm_gated_fwd(A, 4096, B, 4096, GAM, 0, 1e-6, 8, 4096, B, 4096, None,
                                 None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_gated_fwd(A, 4096, C, 4000, GAM, 0, 1e-6, 8, 4096, B, 4096, None,
                                 None) == irn.RMSN_ERR_SHAPE


def bwd(**kw):
    a = dict(g=A, ld_g=4096, x=B, ld_x=4096, rstd=RS, gamma=GAM, zc=0, T=1000, D=4096, gres=None,
             ld_gres=0, dx=C, ld_dx=4096, dgamma=E, ws=W, ws_bytes=1 << 30)
    a.update(kw)
    return irn.load().rmsnorm_bwd(a["g"], a["ld_g"], a["x"], a["ld_x"], a["rstd"], a["gamma"],
                                  a["zc"], a["T"], a["D"], a["gres"], a["ld_gres"], a["dx"],
                                  a["ld_dx"], a["dgamma"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dx=None, dgamma=None), irn.RMSN_ERR_NULL),
    (dict(g=None), irn.RMSN_ERR_NULL),
    (dict(x=None), irn.RMSN_ERR_NULL),
    (dict(rstd=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None), irn.RMSN_ERR_NULL),                  # dx needs the weights
    (dict(gamma=None, dx=None), irn.RMSN_ERR_NULL),         # the kernel loads them anyway
    (dict(ws=None), irn.RMSN_ERR_WORKSPACE),
    (dict(ws_bytes=16), irn.RMSN_ERR_WORKSPACE),
    (dict(ws=W + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(dgamma=E + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(dx=A), irn.RMSN_ERR_ALIASING),
    (dict(dx=B), irn.RMSN_ERR_ALIASING),
    (dict(dgamma=RS), irn.RMSN_ERR_ALIASING),
    (dict(ws=C), irn.RMSN_ERR_ALIASING),
    (dict(gres=C, ld_gres=4096), irn.RMSN_ERR_ALIASING),
    (dict(gres=E + (1 << 30), ld_gres=100), irn.RMSN_ERR_SHAPE),
    (dict(D=32770, ld_g=32770, ld_x=32770, ld_dx=32770), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(D=4100, ld_g=4100, ld_x=4100, ld_dx=4100, x=A + 1), irn.RMSN_ERR_MISALIGNED),
    (dict(D=4100, ld_g=4100, ld_x=4101, ld_dx=4100, dx=A + 6), irn.RMSN_ERR_ALIASING),
    (dict(D=4100, ld_g=4100, ld_x=4100, ld_dx=4100, ws_bytes=16), irn.RMSN_ERR_WORKSPACE),
    (dict(T=-5), irn.RMSN_ERR_SHAPE),
])
def test_backward_rejections(kw, code):
    assert bwd(**kw) == code


def test_workspace_and_chunking_contract():
    assert irn.rmsnorm_bwd_workspace_bytes(0, 4096) == 0
    assert irn.rmsnorm_bwd_workspace_bytes(10, 0) == 0
    assert irn.rmsnorm_bwd_workspace_bytes(10, 32769) == 0
    for T, D in ((1, 128), (16, 128), (32768, 4096), (262144, 4096), (262144, 128), (1000, 2048),
                 (7, 8), (12345, 8192), (5000, 16384), (300, 32768), (777, 8200),
                 (10, 100), (3, 1), (1000, 7), (4000, 4100), (99, 32767)):
        R, S, K = irn.rmsnorm_bwd_partials_layout(T, D)
        assert R > 0 and S > 0 and 0 < K <= 512
        # partial rows of D floats rounded up to a multiple of 8
        assert irn.rmsnorm_bwd_workspace_bytes(T, D) == K * (-(-D // 8) * 8) * 4
        # R depends on D alone
        assert irn.rmsnorm_bwd_partials_layout(1, D)[0] == R
        # every row belongs to exactly one chunk
        if T <= 20000:
            rows = [r for k in range(K) for r in irn.chunk_rows(k, T, D)]
            assert sorted(rows) == list(range(T))
    # the chunk grouping is fixed per (T, D): the same plan on every call
    assert irn.rmsnorm_bwd_partials_layout(32768, 4096) == irn.rmsnorm_bwd_partials_layout(32768, 4096)
    assert irn.rmsnorm_bwd_partials_layout(0, 4096)[2] == 0


def test_dgamma_chunk_rows_depends_on_D_only():
    """rmsnorm_dgamma_chunk_rows(D) is the block height R of the partials
    layout, the same for every T; invalid D gives 0."""
    for D in (1, 7, 8, 100, 128, 1024, 2048, 4096, 4100, 8192, 8200, 16384, 32767, 32768):
        R = irn.rmsnorm_dgamma_chunk_rows(D)
        assert R > 0
        for T in (1, 17, 1000, 32768, 262144):
            assert irn.rmsnorm_bwd_partials_layout(T, D)[0] == R
    assert irn.rmsnorm_dgamma_chunk_rows(4096) == 4   # one row per wave of a 4-wave step
    for D in (0, -8, 32769, 1 << 40):
        assert irn.rmsnorm_dgamma_chunk_rows(D) == 0


def test_partials_layout_rejections():
    lib = irn.load()
    assert lib.rmsnorm_bwd_partials_layout(-1, 4096, None, None, None) == irn.RMSN_ERR_SHAPE
    assert lib.rmsnorm_bwd_partials_layout(16, 32769, None, None, None) == irn.RMSN_ERR_UNSUPPORTED_D
    assert lib.rmsnorm_bwd_partials_layout(16, 0, None, None, None) == irn.RMSN_ERR_SHAPE


def test_finish_rejections():
    lib = irn.load()
    assert lib.rmsnorm_bwd_finish(W, 1 << 30, 1000, 4096, None, None) == irn.RMSN_ERR_NULL
    assert lib.rmsnorm_bwd_finish(None, 0, 1000, 4096, E, None) == irn.RMSN_ERR_WORKSPACE
    assert lib.rmsnorm_bwd_finish(W, 64, 1000, 4096, E, None) == irn.RMSN_ERR_WORKSPACE
    assert lib.rmsnorm_bwd_finish(W, 1 << 30, 1000, 4096, W + 64, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_bwd_finish(W, 1 << 30, 1000, 32769, E, None) == irn.RMSN_ERR_UNSUPPORTED_D
    short = irn.rmsnorm_bwd_workspace_bytes(1000, 12) - 4   # one float short of the partials
    assert lib.rmsnorm_bwd_finish(W, short, 1000, 12, E, None) == irn.RMSN_ERR_WORKSPACE


Z = A + (7 << 36)
DZ = A + (8 << 36)


def gated_fwd_ex(**kw):
    a = dict(x=A, ld_x=4096, z=Z, ld_z=4096, gamma=GAM, zc=0, eps=1e-6, T=8, D=4096,
             act=irn.RMSN_GATE_SIGMOID, rounding=irn.RMSN_GATED_ROUND_CAST, out=B, ld_out=4096,
             rstd=RS)
    a.update(kw)
    return irn.load().rmsnorm_gated_fwd_ex(a["x"], a["ld_x"], a["z"], a["ld_z"], a["gamma"],
                                           a["zc"], a["eps"], a["T"], a["D"], a["act"],
                                           a["rounding"], a["out"], a["ld_out"], a["rstd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(act=2), irn.RMSN_ERR_MODE),
    (dict(act=-1), irn.RMSN_ERR_MODE),
    (dict(rounding=2), irn.RMSN_ERR_MODE),
    (dict(act=7, T=0), irn.RMSN_ERR_MODE),                  # checked even for an empty batch
    (dict(z=None), irn.RMSN_ERR_NULL),
    (dict(z=Z + 2), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_z=100), irn.RMSN_ERR_SHAPE),
    (dict(out=Z), irn.RMSN_ERR_ALIASING),
    (dict(rstd=Z + 64), irn.RMSN_ERR_ALIASING),
    (dict(D=32769, ld_x=32769, ld_z=32769, ld_out=32769), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(D=12, ld_x=13, ld_z=16, ld_out=16, z=Z + 1), irn.RMSN_ERR_MISALIGNED),   # 2-byte rule
    (dict(eps=-1.0), irn.RMSN_ERR_EPS),
])
def test_gated_forward_ex_rejections(kw, code):
    assert gated_fwd_ex(**kw) == code


def test_gated_forward_ex_empty_batch_is_a_no_op():
    assert gated_fwd_ex(T=0, x=None, z=None, out=None, gamma=None, rstd=None) == irn.RMSN_OK


def gated_bwd(**kw):
    a = dict(g=A, ld_g=4096, x=B, ld_x=4096, z=Z, ld_z=4096, rstd=RS, gamma=GAM, zc=0, T=1000,
             D=4096, act=irn.RMSN_GATE_SILU, dx=C, ld_dx=4096, dz=DZ, ld_dz=4096, dgamma=E, ws=W,
             ws_bytes=1 << 30)
    a.update(kw)
    return irn.load().rmsnorm_gated_bwd(a["g"], a["ld_g"], a["x"], a["ld_x"], a["z"], a["ld_z"],
                                        a["rstd"], a["gamma"], a["zc"], a["T"], a["D"], a["act"],
                                        a["dx"], a["ld_dx"], a["dz"], a["ld_dz"], a["dgamma"],
                                        a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(act=2), irn.RMSN_ERR_MODE),
    (dict(dx=None, dz=None, dgamma=None), irn.RMSN_ERR_NULL),
    (dict(z=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None, dx=None, dz=None), irn.RMSN_ERR_NULL),
    (dict(rstd=None), irn.RMSN_ERR_NULL),
    (dict(z=Z + 8), irn.RMSN_ERR_MISALIGNED),
    (dict(dz=DZ + 8), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_dz=4000), irn.RMSN_ERR_SHAPE),
    (dict(ld_z=4000), irn.RMSN_ERR_SHAPE),
    (dict(dz=Z), irn.RMSN_ERR_ALIASING),                    # dz over the gate input
    (dict(dz=C), irn.RMSN_ERR_ALIASING),                    # dz over dx
    (dict(dx=Z + 4096), irn.RMSN_ERR_ALIASING),             # partial overlap with z
    (dict(ws=DZ), irn.RMSN_ERR_ALIASING),
    (dict(ws=None), irn.RMSN_ERR_WORKSPACE),
    (dict(D=32772, ld_g=32772, ld_x=32772, ld_z=32772, ld_dx=32772, ld_dz=32772),
     irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(T=-1), irn.RMSN_ERR_SHAPE),
])
def test_gated_backward_rejections(kw, code):
    assert gated_bwd(**kw) == code


def test_gated_backward_accepts_dx_or_dz_alone():
    # validation only, at T = 0 (nothing launches; a non-NULL dgamma would
    # launch its zero fill, which the GPU empty-batch test covers)
    for kw in (dict(dz=None, dgamma=None), dict(dx=None, dgamma=None)):
        assert gated_bwd(T=0, **kw) == irn.RMSN_OK


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(irn, "_lib", None)
    monkeypatch.setattr(irn, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(ImportError):
        irn.load()


# ---- fused add-norm ---------------------------------------------------------------

F = A + (7 << 36)


def add_fwd(**kw):
    a = dict(x=A, ld_x=4096, res=B, ld_res=4096, gamma=GAM, zc=0, eps=1e-6, T=8, D=4096, y=C,
             ld_y=4096, rout=E, ld_rout=4096, rstd=RS)
    a.update(kw)
    return irn.load().rmsnorm_add_fwd(a["x"], a["ld_x"], a["res"], a["ld_res"], a["gamma"],
                                      a["zc"], a["eps"], a["T"], a["D"], a["y"], a["ld_y"],
                                      a["rout"], a["ld_rout"], a["rstd"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), irn.RMSN_ERR_NULL),
    (dict(res=None), irn.RMSN_ERR_NULL),
    (dict(y=None), irn.RMSN_ERR_NULL),
    (dict(rout=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None), irn.RMSN_ERR_NULL),
    (dict(T=-1), irn.RMSN_ERR_SHAPE),
    (dict(ld_res=4000), irn.RMSN_ERR_SHAPE),
    (dict(D=32769, ld_x=32769, ld_res=32769, ld_y=32769, ld_rout=32769), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(D=100, ld_x=101, ld_res=101, ld_y=101, ld_rout=101, res=B + 1), irn.RMSN_ERR_MISALIGNED),
    (dict(res=B + 2), irn.RMSN_ERR_MISALIGNED),
    (dict(rout=E + 8), irn.RMSN_ERR_MISALIGNED),
    (dict(eps=-1.0), irn.RMSN_ERR_EPS),
    (dict(y=B), irn.RMSN_ERR_ALIASING),                     # y over the residual input
    (dict(rout=A), irn.RMSN_ERR_ALIASING),                  # residual_out over x
    (dict(y=A + 2 * 4096 * 2), irn.RMSN_ERR_ALIASING),      # y over x, shifted a row
    (dict(y=A, ld_y=4104), irn.RMSN_ERR_ALIASING),          # same base, other stride
    (dict(rout=B + 16), irn.RMSN_ERR_ALIASING),             # residual_out shifted
    (dict(y=E), irn.RMSN_ERR_ALIASING),                     # the two outputs
    (dict(rstd=A + 64), irn.RMSN_ERR_ALIASING),
    (dict(x=A, res=A, y=A), irn.RMSN_ERR_ALIASING),         # in place over x, which is res too
    (dict(y=A, rout=A), irn.RMSN_ERR_ALIASING),             # both outputs on x
])
def test_add_forward_rejections(kw, code):
    # (accepted in-place calls launch kernels, so they are tested on the GPU)
    assert add_fwd(**kw) == code


def add_bwd(**kw):
    a = dict(g=A, ld_g=4096, x=B, ld_x=4096, res=F, ld_res=4096, rstd=RS, gamma=GAM, zc=0,
             T=1000, D=4096, gro=None, ld_gro=0, dh=C, ld_dh=4096, dgamma=E, ws=W,
             ws_bytes=1 << 30)
    a.update(kw)
    return irn.load().rmsnorm_add_bwd(a["g"], a["ld_g"], a["x"], a["ld_x"], a["res"], a["ld_res"],
                                      a["rstd"], a["gamma"], a["zc"], a["T"], a["D"], a["gro"],
                                      a["ld_gro"], a["dh"], a["ld_dh"], a["dgamma"], a["ws"],
                                      a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dh=None, dgamma=None), irn.RMSN_ERR_NULL),
    (dict(res=None), irn.RMSN_ERR_NULL),
    (dict(res=F + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_res=100), irn.RMSN_ERR_SHAPE),
    (dict(dh=F), irn.RMSN_ERR_ALIASING),                    # dh over the residual input
    (dict(dh=B), irn.RMSN_ERR_ALIASING),                    # dh over x (no in-place backward)
    (dict(ws=F), irn.RMSN_ERR_ALIASING),
    (dict(gro=F, ld_gro=4096, dh=F), irn.RMSN_ERR_ALIASING),
    (dict(ws=None), irn.RMSN_ERR_WORKSPACE),
    (dict(T=-2), irn.RMSN_ERR_SHAPE),
])
def test_add_backward_rejections(kw, code):
    assert add_bwd(**kw) == code


def test_add_backward_rows_rejections():
    lib = irn.load()
    args = [A, 4096, B, 4096, F, 4096, RS, GAM, 0, 1000, 4096, None, 0]
    assert lib.rmsnorm_add_bwd_rows(*args, None, 4096, None, 0, None) == irn.RMSN_ERR_NULL
    assert lib.rmsnorm_add_bwd_rows(*args, F, 4096, None, 0, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_add_bwd_rows(*args, C, 4096, W, 16, None) == irn.RMSN_ERR_WORKSPACE


# ---- storage types ------------------------------------------------------------------

def test_dtype_entry_points_reject_bad_types():
    lib = irn.load()
    ok = (A, 4096, GAM, 0, 1e-6, 8, 4096, B, 4096, RS, None)
    for adt, wdt in ((2, 2), (3, 2), (-1, 2), (0, 3), (1, 7)):
        assert lib.rmsnorm_fwd_dt(adt, wdt, *ok) == irn.RMSN_ERR_MODE
    assert lib.rmsnorm_fwd_dt(1, 0, A, 4096, GAM + 8, 0, 1e-6, 8, 4096, B, 4096, RS,
                              None) == irn.RMSN_ERR_MISALIGNED
    # rstd 8 KiB past gamma overlaps an fp32 weight vector of 4096 (16 KiB)
    assert lib.rmsnorm_fwd_dt(1, 2, A, 4096, GAM, 0, 1e-6, 8, 4096, B, 4096, GAM + 8192,
                              None) == irn.RMSN_ERR_ALIASING
    bargs = (A, 4096, B, 4096, RS, GAM, 0, 1000, 4096, None, 0, C, 4096, E, W, 1 << 30, None)
    assert lib.rmsnorm_bwd_dt(5, 2, *bargs) == irn.RMSN_ERR_MODE
    assert lib.rmsnorm_bwd_dt(1, 9, *bargs) == irn.RMSN_ERR_MODE
    assert lib.rmsnorm_bwd_dt(1, 2, A, 4096, B, 4096, RS, GAM, 0, 1000, 4096, None, 0, None, 0,
                              None, W, 1 << 30, None) == irn.RMSN_ERR_NULL


def test_gated_and_add_dtype_entry_points_reject_bad_types():
    lib = irn.load()
    gf = (A, 4096, B, 4096, GAM, 0, 1e-6, 8, 4096, 0, 0, C, 4096, RS, None)
    gb = (A, 4096, B, 4096, F, 4096, RS, GAM, 0, 1000, 4096, 0, C, 4096, E, 4096, W + 64,
          W, 1 << 30, None)
    af = (A, 4096, B, 4096, GAM, 0, 1e-6, 8, 4096, C, 4096, E, 4096, RS, None)
    ab = (A, 4096, B, 4096, F, 4096, RS, GAM, 0, 1000, 4096, None, 0, C, 4096, E, W, 1 << 30,
          None)
    for adt, wdt in ((2, 2), (3, 2), (-1, 2), (0, 3), (1, 7)):
        assert lib.rmsnorm_gated_fwd_dt(adt, wdt, *gf) == irn.RMSN_ERR_MODE
        assert lib.rmsnorm_gated_bwd_dt(adt, wdt, *gb) == irn.RMSN_ERR_MODE
        assert lib.rmsnorm_add_fwd_dt(adt, wdt, *af) == irn.RMSN_ERR_MODE
        assert lib.rmsnorm_add_bwd_dt(adt, wdt, *ab) == irn.RMSN_ERR_MODE
    # activation and rounding are checked as in the bf16 entry points
    bad_act = gf[:9] + (2,) + gf[10:]
    assert lib.rmsnorm_gated_fwd_dt(1, 0, *bad_act) == irn.RMSN_ERR_MODE
    bad_round = gf[:10] + (2,) + gf[11:]
    assert lib.rmsnorm_gated_fwd_dt(1, 0, *bad_round) == irn.RMSN_ERR_MODE
    assert lib.rmsnorm_gated_bwd_dt(1, 1, *(gb[:11] + (5,) + gb[12:])) == irn.RMSN_ERR_MODE
    # 16-bit weights keep the 16-byte alignment rule
    assert lib.rmsnorm_add_fwd_dt(1, 1, A, 4096, B, 4096, GAM + 8, 0, 1e-6, 8, 4096, C, 4096, E,
                                  4096, RS, None) == irn.RMSN_ERR_MISALIGNED
    # the weights' range follows their type: rstd 12 KiB past fp32 weights of
    # 4096 (16 KiB) overlaps them
    assert lib.rmsnorm_add_fwd_dt(1, 2, A, 4096, B, 4096, GAM, 0, 1e-6, 8, 4096, C, 4096, E,
                                  4096, GAM + 12288, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_gated_bwd_dt(1, 2, A, 4096, B, 4096, F, 4096, RS, GAM, 0, 1000, 4096, 0,
                                    C, 4096, C, 4096, None, None, 0, None) == irn.RMSN_ERR_ALIASING
    assert lib.rmsnorm_add_bwd_dt(0, 2, A, 4096, B, 4096, F, 4096, RS, GAM, 0, 1000, 4096, None,
                                  0, None, 0, None, W, 1 << 30, None) == irn.RMSN_ERR_NULL


# ---- batch-invariant GEMM -------------------------------------------------------------

def gemm(**kw):
    a = dict(x=A, ld_x=4096, w=B, ld_w=4096, M=64, N=4096, K=4096, y=C, ld_y=4096)
    a.update(kw)
    return irn.load().bigemm_bf16_xwt(a["x"], a["ld_x"], a["w"], a["ld_w"], a["M"], a["N"],
                                      a["K"], a["y"], a["ld_y"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), irn.RMSN_ERR_SHAPE),
    (dict(K=4008, ld_x=4008, ld_w=4008), irn.RMSN_ERR_UNSUPPORTED_D),   # K % 32 == 8
    (dict(K=0), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(ld_x=4088), irn.RMSN_ERR_SHAPE),
    (dict(ld_y=4000), irn.RMSN_ERR_SHAPE),
    (dict(ld_w=(1 << 21) + 8), irn.RMSN_ERR_SHAPE),
    (dict(x=None), irn.RMSN_ERR_NULL),
    (dict(y=None), irn.RMSN_ERR_NULL),
    (dict(x=A + 8), irn.RMSN_ERR_MISALIGNED),
    (dict(ld_w=4100), irn.RMSN_ERR_MISALIGNED),
    (dict(y=A + 1024), irn.RMSN_ERR_ALIASING),
    (dict(y=B), irn.RMSN_ERR_ALIASING),
    (dict(M=1 << 31), irn.RMSN_ERR_SHAPE),   # 2^32 tiles of 32 x 64: more than a grid holds
    (dict(ld_y=1 << 61), irn.RMSN_ERR_SHAPE),  # (M - 1) * ld_y would overflow int64
    (dict(ld_y=(1 << 60) // 64 + 1), irn.RMSN_ERR_SHAPE),  # just past 2^60 / M (M = 64)
])
def test_gemm_rejections(kw, code):
    assert gemm(**kw) == code


def test_gemm_empty_is_a_noop():
    assert gemm(M=0, x=None, y=None) == irn.RMSN_OK
    assert gemm(N=0, w=None, y=None) == irn.RMSN_OK


GEMM_TILES = [(256, 256), (128, 256), (128, 128), (64, 128), (32, 64)]
GEMM_ROUND_US = [113.8, 64.0, 39.6, 25.8, 19.4]  # per round of 256 tiles, K = 4096


@pytest.mark.parametrize("M,N,tile", [
    (1, 4096, (32, 64)), (128, 4096, (32, 64)), (200, 4096, (64, 128)), (300, 4096, (64, 128)),
    (500, 4096, (64, 128)), (1000, 4096, (128, 128)), (2000, 4096, (128, 256)),
    (4000, 4096, (256, 256)), (4096, 11008, (256, 256)), (8192, 4096, (256, 256)),
    (1024, 2048, (64, 128)), (100, 11008, (64, 128)), (64, 4096, (32, 64)), (0, 0, (32, 64)),
    (1000, 4100, (128, 256)),  # 264 tiles of 128 x 128 would take two rounds
])
def test_gemm_tile_choice(M, N, tile):
    """The tile with the least rounds x per-round time; ties to the larger."""
    assert irn.bigemm_bf16_tile(M, N) == tile
    def cost(t, us):
        tiles = -(-M // t[0]) * -(-N // t[1])
        return max(1, -(-tiles // 256)) * us
    costs = [cost(t, us) for t, us in zip(GEMM_TILES, GEMM_ROUND_US)]
    i = GEMM_TILES.index(tile)
    assert costs[i] == min(costs) and all(c > costs[i] for c in costs[:i])


def test_gemm_tile_rejections():
    lib = irn.load()
    v = ctypes.c_int64(0)
    assert lib.bigemm_bf16_tile(-1, 4, ctypes.byref(v), ctypes.byref(v)) == irn.RMSN_ERR_SHAPE
    assert lib.bigemm_bf16_tile(4, 4, None, ctypes.byref(v)) == irn.RMSN_ERR_NULL


def noalloc(**kw):
    a = dict(g=A, ld_g=4096, x=B, ld_x=4096, rstd=RS, gamma=GAM, zc=0, T=1000, D=4096, gres=None,
             ld_gres=0, dx=C, ld_dx=4096, dgamma=E)
    a.update(kw)
    return irn.load().rmsnorm_bwd_noalloc(a["g"], a["ld_g"], a["x"], a["ld_x"], a["rstd"],
                                          a["gamma"], a["zc"], a["T"], a["D"], a["gres"],
                                          a["ld_gres"], a["dx"], a["ld_dx"], a["dgamma"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dx=None, dgamma=None), irn.RMSN_ERR_NULL),
    (dict(g=None), irn.RMSN_ERR_NULL),
    (dict(rstd=None), irn.RMSN_ERR_NULL),
    (dict(gamma=None), irn.RMSN_ERR_NULL),
    (dict(T=-1), irn.RMSN_ERR_SHAPE),
    (dict(D=32776, ld_g=32776, ld_x=32776, ld_dx=32776), irn.RMSN_ERR_UNSUPPORTED_D),
    (dict(ld_x=4000), irn.RMSN_ERR_SHAPE),
    (dict(dgamma=E + 4), irn.RMSN_ERR_MISALIGNED),
    (dict(x=B + 2), irn.RMSN_ERR_MISALIGNED),
    (dict(dx=A), irn.RMSN_ERR_ALIASING),
    (dict(dgamma=RS), irn.RMSN_ERR_ALIASING),
])
def test_noalloc_backward_rejections(kw, code):
    """The same host checks as rmsnorm_bwd, before the scratch is looked up
    or anything is launched."""
    assert noalloc(**kw) == code


def test_noalloc_scratch_covers_every_layout():
    """Every supported (T, D) fits the library's scratch, whatever T: the
    partials layout caps the chunks, so the largest workspace is reached at
    moderate T and never grows beyond it."""
    import re as _re
    text = HEADER.read_text()
    cap = int(_re.search(r"#define RMSN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
              .expand(r"\1")) << int(_re.search(r"RMSN_NOALLOC_SCRATCH_BYTES \(\d+u << (\d+)\)",
                                                text).group(1))
    assert cap == 32 << 20
    worst = 0
    for D in list(range(1, 64)) + list(range(64, 32769, 61)) + [2048, 4096, 8192, 16384, 32768]:
        for T in (1, 1000, 1 << 20, 1 << 40):
            worst = max(worst, irn.rmsnorm_bwd_workspace_bytes(T, D))
    assert 0 < worst <= cap
