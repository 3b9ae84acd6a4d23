"""The Python binding checks every tensor argument before it calls the
library: a wrong dtype, a wrong shape, a non-contiguous vector, a host tensor
or tensors on different devices raise here, so the kernels never receive a
pointer they would read or write out of bounds. These cases run without a
GPU: they raise before any C call (the CUDA-device cases are in the GPU
suite)."""
from __future__ import annotations

import pytest
import torch

import invariant_rmsnorm_amd as irn

T, D = 8, 256
BF, F32, F16 = torch.bfloat16, torch.float32, torch.float16


def t2(dtype=BF, shape=(T, D)):
    return torch.zeros(shape, dtype=dtype)


def t1(n, dtype=F32):
    return torch.zeros(n, dtype=dtype)


def fwd_call(**kw):
    a = dict(x=t2(), gamma=t1(D))
    a.update(kw)
    x, gamma = a.pop("x"), a.pop("gamma")
    return irn.rmsnorm_fwd(x, gamma, **a)


def bwd_call(**kw):
    a = dict(g=t2(), x=t2(), rstd=t1(T), gamma=t1(D))
    a.update(kw)
    return irn.rmsnorm_bwd(a.pop("g"), a.pop("x"), a.pop("rstd"), a.pop("gamma"), **a)


@pytest.mark.parametrize("kw,exc,msg", [
    (dict(gamma=t1(D, BF)), TypeError, "gamma"),                 # bf16 weights read as fp32
    (dict(gamma=t1(D - 8)), ValueError, "gamma"),                # short weights
    (dict(x=t2(F16)), TypeError, "x"),
    (dict(x=t1(D, BF)), ValueError, "x"),                        # not 2-D
    (dict(y=t2(shape=(T - 1, D))), ValueError, "y"),             # output too small
    (dict(y=t2(F16)), TypeError, "y"),
    (dict(rstd=t1(T - 1)), ValueError, "rstd"),                  # rstd shorter than T
    (dict(rstd=t1(2 * T)[::2]), ValueError, "rstd"),             # strided vector
    (dict(x=t2(shape=(T, 2 * D))[:, ::2]), ValueError, "x"),     # last axis not contiguous
    (dict(), ValueError, "CUDA"),                                # host tensors
])
def test_forward_argument_checks(kw, exc, msg):
    with pytest.raises(exc, match=msg):
        fwd_call(**kw)


@pytest.mark.parametrize("kw,exc,msg", [
    (dict(gamma=t1(D, BF)), TypeError, "gamma"),
    (dict(rstd=t1(T, BF)), TypeError, "rstd"),
    (dict(rstd=t1(T - 1)), ValueError, "rstd"),
    (dict(g=t2(shape=(T, D + 8))), ValueError, "g"),
    (dict(g_residual=t2(F32)), TypeError, "g_residual"),
    (dict(dx=t2(shape=(T + 1, D))), ValueError, "dx"),
    (dict(dgamma=t1(D, BF)), TypeError, "dgamma"),
    (dict(dgamma=t1(D - 1)), ValueError, "dgamma"),
    (dict(workspace=t1(64, BF)), TypeError, "workspace"),
    (dict(workspace=t1(128)[::2]), TypeError, "workspace"),
    (dict(), ValueError, "CUDA"),
])
def test_backward_argument_checks(kw, exc, msg):
    with pytest.raises(exc, match=msg):
        bwd_call(**kw)


def test_every_entry_point_checks_before_the_call(monkeypatch):
    """No entry point reaches the library with malformed or host tensors: the
    library handle is replaced by one that fails the test if touched."""
    class Untouchable:
        def __getattr__(self, name):
            raise AssertionError(f"library called: {name}")
    monkeypatch.setattr(irn, "_lib", Untouchable())
    x, g, z, gamma, rstd = t2(), t2(), t2(), t1(D), t1(T)
    bad_gamma = t1(D, BF)
    calls = [
        lambda: irn.rmsnorm_fwd(x, bad_gamma),
        lambda: irn.rmsnorm_residual_fwd(x, bad_gamma),
        lambda: irn.rmsnorm_residual_fwd(x, gamma, residual_out=t2(shape=(T, 8))),
        lambda: irn.rmsnorm_gated_fwd(x, t2(shape=(T - 1, D)), gamma),
        lambda: irn.rmsnorm_gated_fwd_ex(x, z, bad_gamma),
        lambda: irn.rmsnorm_bwd(g, x, t1(T - 1), gamma),
        lambda: irn.rmsnorm_bwd_rows(g, x, rstd, bad_gamma),
        lambda: irn.rmsnorm_bwd_rows(g, x, rstd, gamma, workspace=t1(16, F16)),
        lambda: irn.rmsnorm_bwd_finish(t1(16), T, D, t1(D - 8)),
        lambda: irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma, dz=t2(F16)),
        lambda: irn.rmsnorm_add_fwd(x, t2(F16), gamma),
        lambda: irn.rmsnorm_add_bwd(g, x, z, t1(T, F16), gamma),
        lambda: irn.rmsnorm_add_bwd_rows(g, x, z, rstd, gamma, dh=t2(shape=(T, D - 8))),
        lambda: irn.rmsnorm_fwd_dt(t2(F32), gamma),
        lambda: irn.rmsnorm_fwd_dt(t2(F16), gamma, y=t2(BF)),          # y must match x's type
        lambda: irn.rmsnorm_bwd_dt(t2(F16), t2(BF), rstd, gamma),       # g and x differ
        lambda: irn.rmsnorm_bwd_dt(t2(F16), t2(F16), rstd, t1(D, torch.int32)),
        lambda: irn.rmsnorm_gated_fwd_dt(t2(F16), t2(BF), gamma),        # z must match x's type
        lambda: irn.rmsnorm_gated_fwd_dt(t2(F16), t2(F16), gamma, out=t2(BF)),
        lambda: irn.rmsnorm_gated_bwd_dt(t2(F16), t2(F16), t2(F16), rstd, t1(D - 8, F16)),
        lambda: irn.rmsnorm_gated_bwd_dt(t2(F16), t2(F16), t2(F16), rstd, gamma, dz=t2(BF)),
        lambda: irn.rmsnorm_add_fwd_dt(t2(F16), t2(F16), gamma, residual_out=t2(BF)),
        lambda: irn.rmsnorm_add_fwd_dt(t2(F32), t2(F32), gamma),         # fp32 activations
        lambda: irn.rmsnorm_add_bwd_dt(t2(F16), t2(F16), t2(BF), rstd, gamma),
        lambda: irn.rmsnorm_add_bwd_dt(t2(F16), t2(F16), t2(F16), rstd, gamma,
                                       g_residual_out=t2(BF)),
        lambda: irn.bigemm_bf16_xwt(t2(shape=(4, 64)), t2(shape=(8, 32))),
        lambda: irn.bigemm_bf16_xwt(t2(shape=(4, 64)), t2(shape=(8, 64)), y=t2(shape=(4, 4))),
        # well-formed but on the host: rejected before the call
        lambda: irn.rmsnorm_fwd(x, gamma),
        lambda: irn.rmsnorm_bwd(g, x, rstd, gamma),
        lambda: irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma),
        lambda: irn.rmsnorm_add_bwd(g, x, z, rstd, gamma),
        lambda: irn.rmsnorm_gated_fwd_dt(t2(F16), t2(F16), t1(D, F16)),
        lambda: irn.rmsnorm_gated_bwd_dt(t2(F16), t2(F16), t2(F16), rstd, gamma),
        lambda: irn.rmsnorm_add_fwd_dt(t2(F16), t2(F16), t1(D, BF)),
        lambda: irn.rmsnorm_add_bwd_dt(t2(F16), t2(F16), t2(F16), rstd, gamma),
        lambda: irn.bigemm_bf16_xwt(t2(shape=(4, 64)), t2(shape=(8, 64))),
    ]
    for i, call in enumerate(calls):
        with pytest.raises((TypeError, ValueError)):
            call()
