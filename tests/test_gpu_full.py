"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the same entry points, on the same shapes).

* token norm with outlier rows, T=32768, D=4096: every element of y, rstd,
  dx (with and without the residual gradient) and dgamma against the oracle;
* gated per-head norm, 262144 x 128: every output element of the forward
  (both gates, both rounding conventions) and of the backward (dx, dz,
  dgamma; both gates);
* T=262144, D=4096, zero-centred: every element of y, rstd, dx and dgamma
  against the oracle (run over blocks of rows, and of columns for dgamma, in
  threads), and ten runs bitwise identical.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

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


def _oracle_threads():
    """Worker threads for the oracle: the host's CPU share (at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def test_large_zero_centered_full(gpu):
    p = wl.large()
    _log(f"large workload {p.T}x{p.D}: generated")
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    y, rstd = irn.rmsnorm_fwd(x, gamma, True, p.eps)
    ws, _ = irn.workspace_for(p.T, p.D, "cuda")
    dx, dg = irn.rmsnorm_bwd(g, x, rstd, gamma, True, workspace=ws)
    torch.cuda.synchronize()
    gy, gdx, grs = host_bits(y), host_bits(dx), rstd.cpu().numpy()
    _log("GPU outputs copied to the host")

    # every row: the oracle's forward and dx over blocks of rows in threads,
    # each block compared element by element with the GPU's
    rr = np.empty(p.T, np.float32)
    blocks = [(a, min(p.T, a + 2048)) for a in range(0, p.T, 2048)]

    def check(ab):
        a, b = ab
        sy, sr = oracle.fwd(p.x[a:b], p.gamma, True, p.eps)
        rr[a:b] = sr
        sdx = oracle.bwd_dx(p.g[a:b], p.x[a:b], sr, p.gamma, True)
        return (max_ulp(gy[a:b], sy), int((gy[a:b] != sy).sum()),
                max_ulp(gdx[a:b], sdx), int((gdx[a:b] != sdx).sum()),
                rstd_rel_err(grs[a:b], sr))

    with ThreadPoolExecutor(_oracle_threads()) as ex:
        res = list(ex.map(check, blocks))
    uy, ny = max(r[0] for r in res), sum(r[1] for r in res)
    udx, ndx = max(r[2] for r in res), sum(r[3] for r in res)
    ers = max(r[4] for r in res)
    _log(f"all {p.T} rows: y {ny} of {gy.size} elements differ (max {uy} ulp), "
         f"dx {ndx} differ (max {udx} ulp), rstd rel err {ers:.2e}")
    assert uy <= 1 and udx <= 1 and ers <= 1e-6

    # dgamma over all rows: the oracle over blocks of columns
    cols = np.array_split(np.arange(p.D), _oracle_threads())
    with ThreadPoolExecutor(_oracle_threads()) as ex:
        parts = list(ex.map(lambda c: oracle.dgamma(p.g[:, c[0]:c[-1] + 1],
                                                    p.x[:, c[0]:c[-1] + 1], rr), cols))
    rdg = np.concatenate(parts)
    err = dgamma_rel_err(dg.cpu().numpy(), rdg)
    _log(f"dgamma over {p.T} rows: rel err {err:.3e}")
    assert err <= 1e-5

    # ten runs: every output bitwise identical
    for i in range(10):
        y2, r2 = irn.rmsnorm_fwd(x, gamma, True, p.eps)
        dx2, dg2 = irn.rmsnorm_bwd(g, x, r2, gamma, True, workspace=ws)
        assert torch.equal(y, y2) and torch.equal(rstd, r2)
        assert torch.equal(dx, dx2) and torch.equal(dg.view(torch.int32), dg2.view(torch.int32))
    _log("ten repeat runs bitwise identical")
