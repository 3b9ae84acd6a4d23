"""Pins of the oracle's fused add-RMSNorm (the residual form of the norm).

Source: RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel",
the decoder-norm note: all but the first decoder norm carry a residual and
go through a fused add-and-norm that normalises the fp32 sum; the page gives
no reference arithmetic for it. The reading pinned here: h = x + residual in
fp32, the plain norm of h, the updated residual stored as bf16(h), and one
gradient dh for both x and residual.

What pins what:
  * the exact (f64) backward: central finite differences of the exact
    forward, taken separately in x and in residual, with and without a
    gradient arriving at the residual output;
  * the rounded (R64) forms: bitwise identities with the plain norm
    (residual = 0), commutativity of the fp32 sum, the zero row
    (residual = -x), torch's own rounding of the sum for residual_out, and
    rounding-aware bounds against the exact forms.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from numerics import U32, bf16_to_f64, f32_to_bf16_torch, rounding_consistent
from synth import workloads as wl


def _problem(T, D, seed, zc=False):
    x = synth.normal_bf16(seed, 1, T, D)
    res = synth.normal_bf16(seed, 4, T, D, scale=2.0)
    g = synth.normal_bf16(seed, 2, T, D)
    gro = synth.normal_bf16(seed, 5, T, D, scale=0.5)
    gamma = wl.gamma_for(seed, D, zc)
    return x, res, g, gro, gamma


def _w_eff(gamma, zc):
    return gamma.astype(np.float64) + (1.0 if zc else 0.0)


# ------------------------------------------------------ exact (f64) backward

@pytest.mark.parametrize("T,D", [(1, 8), (2, 16), (3, 128)])
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gro", [False, True])
def test_f64_add_backward_matches_finite_differences(T, D, zc, with_gro):
    x, res, g, gro, gamma = _problem(T, D, 300 + T * D, zc)
    xd, rd, gd = bf16_to_f64(x), bf16_to_f64(res), bf16_to_f64(g)
    grod = bf16_to_f64(gro) if with_gro else np.zeros_like(xd)
    eps, h = 1e-6, 1e-5
    dh, dg = oracle.add_bwd_f64(gd, xd, rd, gamma, zc, eps, g_rout=grod if with_gro else None)

    def loss(xv, rv, gam):
        y, hv, _ = oracle.add_fwd_f64(xv, rv, gam, zc, eps)
        return (gd * y).sum() + (grod * hv).sum()

    for which in ("x", "res"):
        fd = np.empty_like(xd)
        for t in range(T):
            for k in range(D):
                a, b = xd.copy(), rd.copy()
                (a if which == "x" else b)[t, k] += h
                lp = loss(a, b, gamma)
                (a if which == "x" else b)[t, k] -= 2 * h
                lm = loss(a, b, gamma)
                fd[t, k] = (lp - lm) / (2 * h)
        assert np.abs(dh - fd).max() <= 1e-7 * np.abs(fd).max(), which
    gam = gamma.astype(np.float64)
    fdg = np.empty(D)
    for j in range(D):
        gp, gm = gam.copy(), gam.copy()
        gp[j] += h
        gm[j] -= h
        fdg[j] = (loss(xd, rd, gp) - loss(xd, rd, gm)) / (2 * h)
    assert np.abs(dg - fdg).max() <= 1e-7 * np.abs(fdg).max()


def test_f64_add_with_zero_residual_is_the_plain_norm():
    x, _, g, _, gamma = _problem(4, 96, 31)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    y, hv, r = oracle.add_fwd_f64(xd, np.zeros_like(xd), gamma)
    y0, r0 = oracle.fwd_f64(xd, gamma)
    assert np.array_equal(y, y0) and np.array_equal(r, r0) and np.array_equal(hv, xd)
    dh, dg = oracle.add_bwd_f64(gd, xd, np.zeros_like(xd), gamma)
    dx0, dg0 = oracle.bwd_f64(gd, xd, gamma)
    assert np.array_equal(dh, dx0) and np.array_equal(dg, dg0)


# ------------------------------------------------------ rounded (R64) laws

@pytest.mark.parametrize("T,D,seed", [(16, 128, 1001), (5, 4096, 32), (9, 200, 33)])
@pytest.mark.parametrize("zc", [False, True])
def test_zero_residual_equals_plain_norm_bitwise(T, D, seed, zc):
    x, _, g, gro, gamma = _problem(T, D, seed, zc)
    zero = np.zeros_like(x)
    y, rout, r = oracle.add_fwd(x, zero, gamma, zc)
    y0, r0 = oracle.fwd(x, gamma, zc)
    assert np.array_equal(y, y0) and np.array_equal(r.view(np.uint32), r0.view(np.uint32))
    nz = x != 0x8000  # -0 + +0 is +0
    assert np.array_equal(rout[nz], x[nz])
    dh, dg = oracle.add_bwd(g, x, zero, r, gamma, zc, g_rout=gro)
    dx0, dg0 = oracle.bwd(g, x, r0, gamma, zc, gres=gro)
    assert np.array_equal(dh, dx0) and np.array_equal(dg.view(np.uint32), dg0.view(np.uint32))


def test_sum_commutes_bitwise():
    x, res, g, gro, gamma = _problem(12, 256, 34)
    a = oracle.add_fwd(x, res, gamma)
    b = oracle.add_fwd(res, x, gamma)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    da = oracle.add_bwd(g, x, res, a[2], gamma, g_rout=gro)
    db = oracle.add_bwd(g, res, x, a[2], gamma, g_rout=gro)
    for u, v in zip(da, db):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_residual_out_is_the_rounded_fp32_sum():
    x, res, _, _, gamma = _problem(20, 512, 35)
    _, rout, _ = oracle.add_fwd(x, res, gamma)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    rt = torch.from_numpy(res.view(np.int16)).view(torch.bfloat16).float()
    want = f32_to_bf16_torch((xt + rt).numpy())
    assert np.array_equal(rout, want)


def test_cancelled_row_is_zero():
    x, _, g, _, gamma = _problem(3, 128, 36)
    neg = x ^ np.uint16(0x8000)
    y, rout, r = oracle.add_fwd(x, neg, gamma, eps=1e-6)
    assert np.all((y & 0x7FFF) == 0) and np.all((rout & 0x7FFF) == 0)
    want = np.float32(1.0 / np.sqrt(np.float64(np.float32(1e-6))))
    assert np.all(r == want)
    # dh = g w r exactly where h = 0 (c multiplies zeros)
    dh, _ = oracle.add_bwd(g, x, neg, r, gamma)
    gw = bf16_to_f64(g).astype(np.float32) * gamma.astype(np.float32)
    assert np.array_equal(dh, f32_to_bf16_torch((gw * r[:, None]).astype(np.float32)))


def _exact(x, res, g, gro, gamma, zc, eps):
    xd, rd, gd = bf16_to_f64(x), bf16_to_f64(res), bf16_to_f64(g)
    grod = None if gro is None else bf16_to_f64(gro)
    y, hd, r = oracle.add_fwd_f64(xd, rd, gamma, zc, eps)
    dh, dg = oracle.add_bwd_f64(gd, xd, rd, gamma, zc, eps, g_rout=grod)
    return y, hd, r, dh, dg, gd


CASES = [(16, 128, 1001), (7, 4096, 37), (5, 200, 38), (3, 8, 39)]


@pytest.mark.parametrize("T,D,seed", CASES)
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gro", [False, True])
def test_r64_add_within_rounding_of_exact(T, D, seed, zc, with_gro):
    eps = 1e-6
    x, res, g, gro, gamma = _problem(T, D, seed, zc)
    gro = gro if with_gro else None
    y, rout, r = oracle.add_fwd(x, res, gamma, zc, eps)
    yd, hd, rd, dhd, dgd, gd = _exact(x, res, g, gro, gamma, zc, eps)
    # rstd: h rounded once, each square once, mean, + eps, then rsqrt (halved)
    assert np.all(np.abs(r - rd) <= 3.0 * U32 * rd)
    assert rounding_consistent(rout, hd, U32 * np.abs(hd)).all()
    # n = (h*r)*w: h (1), r (3), two products (2)
    assert rounding_consistent(y, yd, 6.1 * U32 * np.abs(yd)).all()

    dh, dg = oracle.add_bwd(g, x, res, r, gamma, zc, g_rout=gro)
    w = _w_eff(gamma, zc)
    D_ = x.shape[1]
    rr = rd[:, None]
    s = (gd * w * hd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gd * w * hd).sum(axis=1, keepdims=True)
    t1 = np.abs(gd * w) * rr
    c_abs = rr ** 3 / D_
    err = (7.6 * U32 * t1
           + np.abs(hd) * c_abs * (3.1 * U32 * s_abs + 16.0 * U32 * np.abs(s))
           + 2.1 * U32 * np.abs(dhd) + U32 * np.abs(dhd))
    assert rounding_consistent(dh, dhd, err).all()
    bound = 6.6 * U32 * (np.abs(gd * hd) * rr).sum(axis=0) + U32 * np.abs(dgd)
    assert np.all(np.abs(dg - dgd) <= bound)


def test_bounds_catch_a_dropped_residual_in_the_backward():
    """A backward that forgets the residual (normalising x alone) must fail
    the dh bound: the planted mistake is x in place of x + residual."""
    eps = 1e-6
    x, res, g, _, gamma = _problem(6, 256, 40)
    _, _, r = oracle.add_fwd(x, res, gamma, False, eps)
    dh_bad = oracle.bwd_dx(g, x, r, gamma)  # h replaced by x
    _, hd, rd, dhd, _, gd = _exact(x, res, g, None, gamma, False, eps)
    err = 8 * U32 * np.abs(dhd) + 1e-30
    assert not rounding_consistent(dh_bad, dhd, err).all()


def test_oracle_add_rows_are_batch_invariant():
    x, res, g, gro, gamma = _problem(40, 64, 41)
    y, rout, r = oracle.add_fwd(x, res, gamma)
    dh, _ = oracle.add_bwd(g, x, res, r, gamma, g_rout=gro)
    for a, b in ((0, 1), (3, 17), (39, 40)):
        ys, routs, rs = oracle.add_fwd(x[a:b], res[a:b], gamma)
        dhs, _ = oracle.add_bwd(g[a:b], x[a:b], res[a:b], rs, gamma, g_rout=gro[a:b])
        assert np.array_equal(ys, y[a:b]) and np.array_equal(routs, rout[a:b])
        assert np.array_equal(rs, r[a:b]) and np.array_equal(dhs, dh[a:b])
