"""Batch invariance on the GPU: a row's y, rstd and dx are byte-identical
whatever batch it sits in.

Methods from the pages (by title):
* TransformerEngine issue "Expose Batch Invariant Kernels", sections 1 and 3:
  one anchor row placed first / in the middle / last in batches of
  M in {1, 2, 17, 33, 128, 257, 1024}, a shuffled batch, and a non-tile-aligned
  M = 1000, compared bytewise with the M = 1 result;
* RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel":
  prefix slices n in {1, 2, 8, 16, 32, 48, 64, 256} of 512 rows, the
  non-prefix slices x[3:5] and x[:1] of 64 rows, and padding — here at hidden
  size 2048 and head size 128;
* RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual", "Correctness / Tests":
  strided inputs and batch / padding invariance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host_bits
from numerics import max_ulp, rstd_rel_err
from synth import workloads as wl

pytestmark = pytest.mark.gpu


def _fwd_bwd(x, g, gamma, zc=False, eps=1e-6):
    y, r = irn.rmsnorm_fwd(x, gamma, zc, eps)
    dx, _ = irn.rmsnorm_bwd(g, x, r, gamma, zc, want_dgamma=False)
    return y, r, dx


def _row_bytes(y, r, dx, i):
    return (host_bits(y[i:i + 1]).tobytes(), r[i:i + 1].cpu().numpy().tobytes(),
            host_bits(dx[i:i + 1]).tobytes())


@pytest.mark.parametrize("k", range(4))
def test_anchor_rows_across_batches(gpu, k):
    D = wl.SWEEP_D
    gamma_np = wl.sweep_gamma(D)
    gamma = dev_f32(gamma_np)
    ax, ag = wl.sweep_anchor(k, D)
    # the M = 1 result, itself checked against the oracle
    y1, r1, dx1 = _fwd_bwd(dev_bf16(ax[None]), dev_bf16(ag[None]), gamma)
    ref = _row_bytes(y1, r1, dx1, 0)
    oy, orr = oracle.fwd(ax[None], gamma_np)
    odx = oracle.bwd_dx(ag[None], ax[None], orr, gamma_np)
    assert max_ulp(host_bits(y1), oy) <= 1 and rstd_rel_err(r1.cpu().numpy(), orr) <= 1e-6
    assert max_ulp(host_bits(dx1), odx) <= 1
    n = 0
    for M in wl.SWEEP_M:
        for pos in wl.SWEEP_POSITIONS:
            xb, gb, i = wl.sweep_batch(k, M, pos, D)
            y, r, dx = _fwd_bwd(dev_bf16(xb), dev_bf16(gb), gamma)
            assert _row_bytes(y, r, dx, i) == ref, (k, M, pos)
            # padding rows: x = g = 0 give y = 0, dx = 0
            assert torch.all(y[M:].float() == 0) and torch.all(dx[M:].float() == 0)
            n += 1
    assert n == len(wl.SWEEP_M) * len(wl.SWEEP_POSITIONS)


@pytest.mark.parametrize("D", [128, 2048])
def test_prefix_and_offset_slices(gpu, D):
    T = 512
    x = dev_bf16(synth.normal_bf16(6000 + D, 1, T, D))
    g = dev_bf16(synth.normal_bf16(6000 + D, 2, T, D))
    gamma = dev_f32(wl.gamma_for(6000 + D, D, True))
    y, r, dx = _fwd_bwd(x, g, gamma, True)
    for n in (1, 2, 8, 16, 32, 48, 64, 256):
        ys, rs, dxs = _fwd_bwd(x[:n], g[:n], gamma, True)
        assert torch.equal(ys, y[:n]) and torch.equal(rs, r[:n]) and torch.equal(dxs, dx[:n]), n
    # non-prefix slices of the first 64 rows: x[3:5] and x[:1] (pointer offsets)
    for a, b in ((3, 5), (0, 1), (17, 64)):
        ys, rs, dxs = _fwd_bwd(x[a:b], g[a:b], gamma, True)
        assert torch.equal(ys, y[a:b]) and torch.equal(rs, r[a:b]) and torch.equal(dxs, dx[a:b])


@pytest.mark.parametrize("D", [4104, 8192, 12288, 32768])
def test_wide_rows_across_batches(gpu, D):
    """Rows spread over 2 waves (forward, D = 4104 and 8192) and 4 waves
    (forward past 8192, backward past 4096): a row's y, rstd and dx are the
    same bytes in batches of 1, 2, 3, 7 and 40 rows at every position."""
    T = 40
    x = dev_bf16(synth.normal_bf16(6300 + D, 1, T, D))
    g = dev_bf16(synth.normal_bf16(6300 + D, 2, T, D))
    gamma = dev_f32(wl.gamma_for(6300 + D, D, False))
    y, r, dx = _fwd_bwd(x, g, gamma)
    for a, b in ((0, 1), (5, 6), (39, 40), (3, 5), (10, 13), (20, 27), (0, 40)):
        ys, rs, dxs = _fwd_bwd(x[a:b], g[a:b], gamma)
        assert torch.equal(ys, y[a:b]) and torch.equal(rs, r[a:b]) and torch.equal(dxs, dx[a:b])


@pytest.mark.parametrize("D", [128, 1000, 4096])
def test_strided_rows(gpu, D):
    """Rows with a stride larger than D give the packed result bytewise."""
    T, ld = 300, D + 64
    xp = synth.normal_bf16(6100 + D, 1, T, D)
    gp = synth.normal_bf16(6100 + D, 2, T, D)
    gamma = dev_f32(wl.gamma_for(6100 + D, D, False))
    xs = torch.zeros((T, ld), dtype=torch.bfloat16, device="cuda")
    gs = torch.zeros((T, ld), dtype=torch.bfloat16, device="cuda")
    xs[:, :D] = dev_bf16(xp)
    gs[:, :D] = dev_bf16(gp)
    y, r, dx = _fwd_bwd(dev_bf16(xp), dev_bf16(gp), gamma)
    ys = torch.zeros((T, ld), dtype=torch.bfloat16, device="cuda")
    dxs = torch.zeros((T, ld), dtype=torch.bfloat16, device="cuda")
    _, r2 = irn.rmsnorm_fwd(xs[:, :D], gamma, y=ys[:, :D])
    irn.rmsnorm_bwd(gs[:, :D], xs[:, :D], r2, gamma, dx=dxs[:, :D], want_dgamma=False)
    assert torch.equal(ys[:, :D], y) and torch.equal(r2, r) and torch.equal(dxs[:, :D], dx)
    assert torch.all(ys[:, D:].float() == 0) and torch.all(dxs[:, D:].float() == 0)


@pytest.mark.parametrize("D", [20003, 32767, 32768])
def test_long_gated_and_add_rows_across_batches(gpu, D):
    """Long rows of the gated and fused-add backward (rows over 4 waves that
    load the next row during the second pass; 32767 is a row of any length
    where no lane lacks its last group): a row's dx and dz, and its dh, are
    the same bytes in batches of 1, 2, 3, 7 and 40 rows at every position."""
    T = 40
    x = dev_bf16(synth.normal_bf16(6400 + D, 1, T, D))
    g = dev_bf16(synth.normal_bf16(6400 + D, 2, T, D))
    z = dev_bf16(synth.normal_bf16(6400 + D, 5, T, D))
    gamma = dev_f32(wl.gamma_for(6400 + D, D, False))
    _, rstd = irn.rmsnorm_fwd(x, gamma)
    fdx, fdz, _ = irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma)
    _, _, hr = irn.rmsnorm_add_fwd(x, z, gamma)
    fdh, _ = irn.rmsnorm_add_bwd(g, x, z, hr, gamma, g_residual_out=x, want_dgamma=False)
    for a, b in ((0, 1), (5, 6), (39, 40), (3, 5), (10, 13), (20, 27), (0, 40)):
        pdx, pdz, _ = irn.rmsnorm_gated_bwd(g[a:b], x[a:b], z[a:b], rstd[a:b], gamma)
        assert torch.equal(pdx, fdx[a:b]) and torch.equal(pdz, fdz[a:b]), (a, b)
        pdh, _ = irn.rmsnorm_add_bwd(g[a:b], x[a:b], z[a:b], hr[a:b], gamma,
                                     g_residual_out=x[a:b], want_dgamma=False)
        assert torch.equal(pdh, fdh[a:b]), (a, b)


def test_gated_rows_across_batches(gpu):
    """Head-size rows of the gated norm are batch-invariant too."""
    D = 128
    x = dev_bf16(synth.normal_bf16(6200, 1, 1024, D))
    z = dev_bf16(synth.normal_bf16(6200, 5, 1024, D))
    gamma = dev_f32(wl.gamma_for(6200, D, False))
    full, rf = irn.rmsnorm_gated_fwd(x, z, gamma, want_rstd=True)
    for a, b in ((0, 1), (5, 6), (3, 36), (1000, 1024), (7, 1007)):
        part, rp = irn.rmsnorm_gated_fwd(x[a:b], z[a:b], gamma, want_rstd=True)
        assert torch.equal(part, full[a:b]) and torch.equal(rp, rf[a:b])
