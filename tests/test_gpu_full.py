"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same entry points, on the same shapes).

* token norm with outlier rows, T=32768, D=4096: every element of y, rstd,
  dx (with and without the residual gradient) and dgamma against the oracle;
* gated per-head norm, 262144 x 128: every output element of the forward
  (both gates, both rounding conventions) and of the backward (dx, dz,
  dgamma; both gates);
* T=262144, D=4096, zero-centred: dgamma over all rows against the oracle,
  y/rstd/dx on sampled rows, and ten runs bitwise identical.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
from gpu_util import dev_bf16, dev_f32, host_bits
from numerics import (dgamma_rel_err, gated_dx_terms, max_ulp, rstd_rel_err, ulp_distance,
                      ulp_or_cancelled)
from synth import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _log(msg):
    print(msg, flush=True)


def test_residual_token_norm_full(gpu):
    p = wl.residual()
    _log(f"residual workload {p.T}x{p.D}: generated")
    x, g, gr, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_bf16(p.gres), dev_f32(p.gamma)
    y, res, rstd = irn.rmsnorm_residual_fwd(x, gamma, False, p.eps)
    dx, dg = irn.rmsnorm_bwd(g, x, rstd, gamma, False)
    dxr, dgr = irn.rmsnorm_bwd(g, x, rstd, gamma, False, g_residual=gr)
    torch.cuda.synchronize()
    assert torch.equal(res, x)
    assert torch.equal(dg, dgr)

    ry, rr = oracle.fwd(p.x, p.gamma, False, p.eps)
    _log("oracle forward done")
    gy, gr_ = host_bits(y), rstd.cpu().numpy()
    _log(f"y: {(gy != ry).sum()} of {gy.size} differ from the oracle; "
         f"rstd: {(gr_ != rr).sum()} of {rr.size}")
    assert max_ulp(gy, ry) <= 1
    assert rstd_rel_err(gr_, rr) <= 1e-6
    for gpu_dx, gres in ((dx, None), (dxr, p.gres)):
        rdx = oracle.bwd_dx(p.g, p.x, rr, p.gamma, False, gres)
        gdx = host_bits(gpu_dx)
        _log(f"dx (gres={gres is not None}): {(gdx != rdx).sum()} of {gdx.size} differ, "
             f"max ulp {max_ulp(gdx, rdx)}")
        assert max_ulp(gdx, rdx) <= 1
    rdg = oracle.dgamma(p.g, p.x, rr)
    err = dgamma_rel_err(dg.cpu().numpy(), rdg)
    _log(f"dgamma rel err {err:.3e}")
    assert err <= 1e-5


def test_gated_per_head_full(gpu):
    p = wl.gated()
    out, rstd = irn.rmsnorm_gated_fwd(dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma), False,
                                      p.eps, want_rstd=True)
    ro, rr = oracle.gated_fwd(p.x, p.z, p.gamma, False, p.eps)
    got = host_bits(out)
    assert max_ulp(got, ro) <= 1
    _log(f"gated: {(got != ro).sum()} of {got.size} elements 1 ulp apart")
    assert rstd_rel_err(rstd.cpu().numpy(), rr) <= 1e-6


@pytest.mark.parametrize("act,act_o", [(irn.RMSN_GATE_SILU, oracle.SILU),
                                       (irn.RMSN_GATE_SIGMOID, oracle.SIGMOID)])
def test_gated_variants_full(gpu, act, act_o):
    p = wl.gated(with_grad=True)
    x, z, gamma = dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma)
    for rounding, conv in ((irn.RMSN_GATED_ROUND_FP32, oracle.FP32_WEIGHT),
                           (irn.RMSN_GATED_ROUND_CAST, oracle.CAST_INPUT)):
        out, _ = irn.rmsnorm_gated_fwd_ex(x, z, gamma, False, p.eps, activation=act,
                                          rounding=rounding)
        ro, _ = oracle.gated_fwd_ex(p.x, p.z, p.gamma, False, p.eps, activation=act_o,
                                    convention=conv)
        got = host_bits(out)
        _log(f"gated fwd act={act} rounding={rounding}: {(got != ro).sum()} of {got.size} "
             f"elements 1 ulp apart")
        assert max_ulp(got, ro) <= 1

    g = p.g
    _, rstd = irn.rmsnorm_fwd(x, gamma, False, p.eps)
    dx, dz, dg = irn.rmsnorm_gated_bwd(dev_bf16(g), x, z, rstd, gamma, False, activation=act)
    _, rr = oracle.fwd(p.x, p.gamma, False, p.eps)
    rdx, rdz, rdg = oracle.gated_bwd(g, p.x, p.z, rr, p.gamma, False, activation=act_o)
    gdx, gdz = host_bits(dx), host_bits(dz)
    udx, udz = ulp_distance(gdx, rdx), ulp_distance(gdz, rdz)
    err = dgamma_rel_err(dg.cpu().numpy(), rdg)
    _log(f"gated bwd act={act}: dx {(udx > 0).sum()} differ (max {udx.max()} ulp), "
         f"dz {(udz > 0).sum()} differ (max {udz.max()} ulp), dgamma rel err {err:.3e}")
    terms = gated_dx_terms(g, p.x, p.z, p.gamma, False, rr, act_o == oracle.SIGMOID)
    assert ulp_or_cancelled(gdx, rdx, terms).all()
    assert udz.max() <= 1
    assert err <= 1e-5


def test_large_zero_centered_full(gpu):
    p = wl.large()
    _log(f"large workload {p.T}x{p.D}: generated")
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    y, rstd = irn.rmsnorm_fwd(x, gamma, True, p.eps)
    ws, _ = irn.workspace_for(p.T, p.D, "cuda")
    dx, dg = irn.rmsnorm_bwd(g, x, rstd, gamma, True, workspace=ws)
    torch.cuda.synchronize()

    _, rr = oracle.fwd(p.x, p.gamma, True, p.eps)
    _log("oracle forward done")
    assert rstd_rel_err(rstd.cpu().numpy(), rr) <= 1e-6
    rdg = oracle.dgamma(p.g, p.x, rr)
    err = dgamma_rel_err(dg.cpu().numpy(), rdg)
    _log(f"dgamma over {p.T} rows: rel err {err:.3e}")
    assert err <= 1e-5

    rows = np.unique(np.concatenate([[0, 1, p.T // 2, p.T - 1],
                                     np.random.default_rng(4004).integers(0, p.T, 2000)]))
    idx = torch.from_numpy(rows).cuda()
    ys, dxs = host_bits(y[idx]), host_bits(dx[idx])
    sy, sr = oracle.fwd(p.x[rows], p.gamma, True, p.eps)
    sdx = oracle.bwd_dx(p.g[rows], p.x[rows], sr, p.gamma, True)
    assert max_ulp(ys, sy) <= 1
    assert max_ulp(dxs, sdx) <= 1
    _log(f"sampled rows: y {(ys != sy).sum()}, dx {(dxs != sdx).sum()} elements differ")

    # ten runs: every output bitwise identical
    for i in range(10):
        y2, r2 = irn.rmsnorm_fwd(x, gamma, True, p.eps)
        dx2, dg2 = irn.rmsnorm_bwd(g, x, r2, gamma, True, workspace=ws)
        assert torch.equal(y, y2) and torch.equal(rstd, r2)
        assert torch.equal(dx, dx2) and torch.equal(dg.view(torch.int32), dg2.view(torch.int32))
    _log("ten repeat runs bitwise identical")
