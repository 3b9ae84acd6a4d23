"""rmsnorm_bwd_noalloc (the backward with the dgamma partials in the
library's own device scratch) against rmsnorm_bwd with a caller workspace:
bitwise equal dx and dgamma, on two calls in a row, the second smaller than
the first (so the scratch still holds the first call's partials), plus the
dx-only and empty-batch forms. Called through the C-ABI binding."""
from __future__ import annotations

import pytest
import torch

import invariant_rmsnorm_amd as irn
import synth
from gpu_util import dev_bf16, dev_f32
from synth import workloads as wl

pytestmark = pytest.mark.gpu


def _case(T, D, zc, seed, gres):
    p = wl.tiny(zc, T=T, D=D, seed=seed, with_gres=gres)
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    gr = dev_bf16(p.gres) if gres else None
    _, rstd = irn.rmsnorm_fwd(x, gamma, zc, p.eps)
    return x, g, gr, gamma, rstd


def _compare(T, D, zc, seed, gres):
    print(f"noalloc case T={T} D={D} zc={zc} gres={gres}", flush=True)
    x, g, gr, gamma, rstd = _case(T, D, zc, seed, gres)
    dx_ref, dg_ref = irn.rmsnorm_bwd(g, x, rstd, gamma, zc, g_residual=gr)
    dx = torch.full_like(dx_ref, 7.0)
    dg = torch.full_like(dg_ref, 7.0)
    irn.rmsnorm_bwd_noalloc(g, x, rstd, gamma, zc, g_residual=gr, dx=dx, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref)
    assert torch.equal(dg.view(torch.int32), dg_ref.view(torch.int32))


def test_noalloc_matches_bwd_on_two_calls_second_smaller(gpu):
    # a 4 MiB layout (256 chunks x 4096 floats), then a smaller one that
    # leaves the first call's partials in the scratch beyond its own
    _compare(40000, 4096, False, 11001, True)
    _compare(3001, 1024, True, 11002, False)


def test_noalloc_largest_layouts_and_repeats(gpu):
    # layouts that fill the whole scratch (256 chunks x 32768 floats), the
    # second with rows not a multiple of 8
    assert irn.rmsnorm_bwd_workspace_bytes(1100, 32768) == 32 << 20
    assert irn.rmsnorm_bwd_workspace_bytes(1500, 32767) == 32 << 20
    _compare(1100, 32768, False, 11006, True)
    _compare(1500, 32767, True, 11003, False)
    _compare(77, 100, False, 11004, True)        # rows not a multiple of 8
    _compare(77, 100, False, 11004, True)        # the same call again: the same bits


def test_noalloc_dx_only_and_empty_batch(gpu):
    x, g, gr, gamma, rstd = _case(300, 2048, False, 11005, False)
    dx_ref, _ = irn.rmsnorm_bwd(g, x, rstd, gamma, want_dgamma=False)
    dx = torch.empty_like(dx_ref)
    irn.rmsnorm_bwd_noalloc(g, x, rstd, gamma, dx=dx, dgamma=None)
    _, dg_ref = irn.rmsnorm_bwd(g, x, rstd, gamma, want_dx=False)
    dg = torch.empty_like(dg_ref)
    irn.rmsnorm_bwd_noalloc(g, x, rstd, gamma, dx=None, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref) and torch.equal(dg, dg_ref)
    e = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    dg0 = torch.full((2048,), 5.0, device="cuda")
    irn.rmsnorm_bwd_noalloc(e, e, torch.empty(0, device="cuda"), gamma, dx=None, dgamma=dg0)
    torch.cuda.synchronize()
    assert torch.all(dg0 == 0)
