"""Pins of the oracle's gated-norm variants (sigmoid gate, the cast rounding
convention, the gated backward).

Source: RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel".
There the gate activation is silu by default, with sigmoid as the other
choice. Two upstream implementations place their roundings differently. In
bf16 their outputs are more than 1e-3 apart; on fp32 inputs they match
bitwise, because the casts do nothing there. One of them does the weight
multiply in fp32. The pages do not give the backward: it is derived here by
the chain rule and pinned by finite differences.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from numerics import U32, bf16_to_f32, bf16_to_f64, f32_to_bf16_torch, rounding_consistent
from synth import workloads as wl

ACTS = [oracle.SILU, oracle.SIGMOID]


def _gate(act, z):
    s = scipy.special.expit(z)
    return z * s if act == oracle.SILU else s


def _problem(T, D, seed, zc=False):
    p = wl.tiny(zc, T=T, D=D, seed=seed, with_gate=True)
    return p


def test_fp32_silu_convention_is_the_gated_forward():
    p = _problem(9, 200, 71)
    a, ra = oracle.gated_fwd(p.x, p.z, p.gamma)
    b, rb = oracle.gated_fwd_ex(p.x, p.z, p.gamma, activation=oracle.SILU,
                                convention=oracle.FP32_WEIGHT)
    assert np.array_equal(a, b) and np.array_equal(ra, rb)


@pytest.mark.parametrize("act", ACTS)
def test_exact_gated_forward_is_norm_times_gate(act):
    p = _problem(4, 128, 72)
    xd = bf16_to_f64(p.x)
    zd = np.linspace(-20, 20, xd.size).reshape(xd.shape)
    out = oracle.gated_fwd_ex_f64(xd, zd, p.gamma, activation=act)
    y, _ = oracle.fwd_f64(xd, p.gamma)
    np.testing.assert_allclose(out, y * _gate(act, zd), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("act", ACTS)
def test_conventions_agree_bitwise_on_fp32_inputs(act):
    """With fp32 inputs the casts to the input dtype are the identity."""
    rng = np.random.default_rng(73)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    z = rng.standard_normal((64, 128)).astype(np.float32)
    gamma = wl.gamma_for(73, 128, False)
    a = oracle.gated_fwd_f32io(x, z, gamma, activation=act, convention=oracle.FP32_WEIGHT)
    b = oracle.gated_fwd_f32io(x, z, gamma, activation=act, convention=oracle.CAST_INPUT)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("act", ACTS)
def test_conventions_differ_in_bf16(act):
    """In bf16 the two conventions are more than 1e-3 apart somewhere."""
    p = _problem(512, 128, 74)
    a, _ = oracle.gated_fwd_ex(p.x, p.z, p.gamma, activation=act, convention=oracle.FP32_WEIGHT)
    b, _ = oracle.gated_fwd_ex(p.x, p.z, p.gamma, activation=act, convention=oracle.CAST_INPUT)
    diff = np.abs(bf16_to_f64(a) - bf16_to_f64(b))
    assert diff.max() > 1e-3
    assert (a != b).mean() > 0.01


def test_fp32_io_rounds_to_the_bf16_convention():
    """On bf16-valued inputs, rounding the fp32-output form once gives the
    fp32-weight convention's bf16 output."""
    p = _problem(32, 128, 75)
    out, _ = oracle.gated_fwd_ex(p.x, p.z, p.gamma)
    f = oracle.gated_fwd_f32io(bf16_to_f32(p.x), bf16_to_f32(p.z), p.gamma)
    assert np.array_equal(out, f32_to_bf16_torch(f))


def test_cast_convention_places_the_casts():
    """Sigmoid gate at z = 0 is exactly 1/2. Then the cast convention gives
    1/2 * bf16(bf16(x*r) * w), where bf16(x*r) is the plain forward with unit
    weight; the fp32 convention gives 1/2 * bf16(x*r*w), the plain forward."""
    p = _problem(16, 256, 76)
    z0 = np.zeros_like(p.x)
    cast, _ = oracle.gated_fwd_ex(p.x, z0, p.gamma, activation=oracle.SIGMOID,
                                  convention=oracle.CAST_INPUT)
    fp32, _ = oracle.gated_fwd_ex(p.x, z0, p.gamma, activation=oracle.SIGMOID,
                                  convention=oracle.FP32_WEIGHT)
    n_b, _ = oracle.fwd(p.x, np.ones(256, np.float32))
    nw = (torch.from_numpy(bf16_to_f32(n_b)) * torch.from_numpy(p.gamma)).bfloat16().double()
    assert np.array_equal(bf16_to_f64(cast), 0.5 * nw.numpy())
    y, _ = oracle.fwd(p.x, p.gamma)
    assert np.array_equal(bf16_to_f64(fp32), 0.5 * bf16_to_f64(y))


@pytest.mark.parametrize("act", ACTS)
def test_gate_derivatives_match_finite_differences(act):
    z = np.linspace(-30.0, 30.0, 601)
    h = 1e-6
    fd = (_gate(act, z + h) - _gate(act, z - h)) / (2 * h)
    # the oracle's a'(z) enters dz: with g = 1, x*r*w = 1 (constant row, w=1, eps=0)
    D = 601
    x = f32_to_bf16_torch(np.ones((1, D), np.float32))
    zb = z[None]
    _, dz, _ = oracle.gated_bwd_f64(np.ones((1, D)), bf16_to_f64(x), zb, np.ones(D), eps=0.0,
                                    activation=act)
    np.testing.assert_allclose(dz[0], fd, rtol=1e-6, atol=1e-9)
    # relative precision in the tails: with 1 - sigmoid(z) = sigmoid(-z),
    # sigmoid' = expit(z) expit(-z) and silu' = expit(z) (1 + z expit(-z))
    s, sc = scipy.special.expit(z), scipy.special.expit(-z)
    exact = s * sc if act == oracle.SIGMOID else s * (1 + z * sc)
    np.testing.assert_allclose(dz[0], exact, rtol=1e-13, atol=0)


def _gated_fd(g, x, z, gamma, zc, act, eps, h=1e-5):
    dx, dz, dg = oracle.gated_bwd_f64(g, x, z, gamma, zc, eps, act)

    def loss(xv, zv, gv):
        return (g * oracle.gated_fwd_ex_f64(xv, zv, gv, zc, eps, act)).sum()

    fx, fz = np.empty_like(x), np.empty_like(z)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fx[idx] = (loss(xp, z, gamma) - loss(xm, z, gamma)) / (2 * h)
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fz[idx] = (loss(x, zp, gamma) - loss(x, zm, gamma)) / (2 * h)
    gam = gamma.astype(np.float64)
    fg = np.empty_like(gam)
    for j in range(gam.size):
        gp, gm = gam.copy(), gam.copy()
        gp[j] += h
        gm[j] -= h
        fg[j] = (loss(x, z, gp) - loss(x, z, gm)) / (2 * h)
    rel = lambda a, b: np.abs(a - b).max() / np.abs(b).max()
    return rel(dx, fx), rel(dz, fz), rel(dg, fg)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("T,D", [(1, 8), (2, 16), (3, 40)])
def test_gated_backward_matches_finite_differences(act, zc, T, D):
    p = _problem(T, D, 77 + T * D, zc)
    e = _gated_fd(bf16_to_f64(p.g), bf16_to_f64(p.x), bf16_to_f64(p.z), p.gamma, zc, act, 1e-6)
    assert max(e) < 1e-7, e


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("T,D,seed", [(16, 128, 78), (5, 4096, 79), (7, 96, 80)])
def test_rounded_gated_backward_within_bounds_of_exact(act, T, D, seed):
    p = _problem(T, D, seed)
    _, r = oracle.fwd(p.x, p.gamma, False, p.eps)
    dx, dz, dg = oracle.gated_bwd(p.g, p.x, p.z, r, p.gamma, activation=act)
    xd, gd, zd = bf16_to_f64(p.x), bf16_to_f64(p.g), bf16_to_f64(p.z)
    ex, ez, eg = oracle.gated_bwd_f64(gd, xd, zd, p.gamma, False, p.eps, act)
    rd = oracle.fwd_f64(xd, p.gamma, False, p.eps)[1][:, None]
    w = p.gamma.astype(np.float64)
    a = _gate(act, zd)
    # dz = g * n * w * a': n (r 2.5u + mul u), nw (u), g*nw (u), a' (u), mul (u)
    assert rounding_consistent(dz, ez, 7.6 * U32 * np.abs(ez)).all()
    # dx: the plain bound with gn = g*a (one more rounding in gn and in a)
    gn = gd * a
    s = (gn * w * xd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gn * w * xd).sum(axis=1, keepdims=True)
    err = (6.6 * U32 * np.abs(gn * w) * rd
           + np.abs(xd) * rd ** 3 / D * (4.1 * U32 * s_abs + 13.0 * U32 * np.abs(s))
           + 3.1 * U32 * np.abs(ex))
    assert rounding_consistent(dx, ex, err).all()
    bound = 5.6 * U32 * (np.abs(gn * xd) * rd).sum(axis=0) + U32 * np.abs(eg)
    assert np.all(np.abs(dg - eg) <= bound)


@pytest.mark.parametrize("act", ACTS)
def test_gated_backward_special_cases(act):
    """w = 0: dx = dz = 0. Gate at z = 0: silu gives a = 0 so dx = dgamma = 0;
    sigmoid gives a = 1/2, so dx and dgamma are half the plain backward's
    with the same g (exact power-of-two scaling)."""
    p = _problem(6, 256, 81)
    _, r = oracle.fwd(p.x, p.gamma)
    dx, dz, _ = oracle.gated_bwd(p.g, p.x, p.z, r, np.zeros(256, np.float32), activation=act)
    assert np.all(bf16_to_f64(dx) == 0) and np.all(bf16_to_f64(dz) == 0)
    z0 = np.zeros_like(p.x)
    dx, _, dg = oracle.gated_bwd(p.g, p.x, z0, r, p.gamma, activation=act)
    if act == oracle.SILU:
        assert np.all(bf16_to_f64(dx) == 0) and np.all(dg == 0)
    else:
        pdx, pdg = oracle.bwd(p.g, p.x, r, p.gamma)
        assert np.array_equal(bf16_to_f64(dx), 0.5 * bf16_to_f64(pdx))
        assert np.array_equal(dg, (0.5 * pdg).astype(np.float32))
