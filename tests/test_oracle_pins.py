"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Sources (pages by title):
  [MEG] Megatron-LM PR "Fix the batch-invariant RMSNorm forward and its input
        gradient" — "What does this PR do?" items 1-2 and "How to reproduce,
        and how we checked it" (finite differences of the function's own
        forward in fp64, the weight=ones control, weight=zeros giving 0).
  [C1]  RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel" —
        the fp32 +1 offset and the SiLU-gated norm with the weight multiply in
        fp32.
  [RES] RL-Kernel PR "[DSv4][P1-5] rmsnorm_residual" — "Summary" (a byte copy
        of x) and "Implementation" (fp32 gamma, saved inverse RMS, rsqrt).

What pins what:
  * the exact (f64) forward: mean-square and scale invariants, closed forms
    for constant and one-hot rows, the zero-centred identity;
  * the exact backward: central finite differences of the exact forward
    ([MEG]'s method) and the x . dx = 0 identity at eps = 0;
  * the rounded (R64) forms: rounding-aware bounds against the exact forms,
    power-of-two scaling laws, closed forms and identities that hold bitwise;
  * the bf16 codec and the SiLU gate: torch's and scipy's library routines;
  * planted defects (the two that [MEG] fixes) must fail these checks.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from numerics import (U32, bf16_to_f32, bf16_to_f64, f32_to_bf16_torch,
                      rounding_consistent)
from synth import workloads as wl


def _problem(T, D, seed, zc, gscale=1.0):
    x = synth.normal_bf16(seed, 1, T, D)
    g = synth.normal_bf16(seed, 2, T, D, scale=gscale)
    gamma = wl.gamma_for(seed, D, zc)
    return x, g, gamma


def _w_eff(gamma, zc):
    return gamma.astype(np.float64) + (1.0 if zc else 0.0)


# ---------------------------------------------------------------- bf16 codec

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = bf16_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _edge_f32_patterns():
    pats = []
    for hi in (0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81, 0x7F7F, 0x7F80,
               0x7F7E, 0x4000, 0x0040):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            for s in (0, 0x8000_0000):
                pats.append(s | (hi << 16) | lo)
    return np.array(pats, dtype=np.uint32)


def test_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(7)
    pats = np.concatenate([rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64)
                           .astype(np.uint32), _edge_f32_patterns()])
    vals = pats.view(np.float32)
    ours = oracle.bf16_encode(vals)
    ref = f32_to_bf16_torch(vals)
    nan = np.isnan(vals)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays a quiet NaN of the same sign
    assert np.all((ours[nan] & 0x7FFF) > 0x7F80)
    assert np.all((ours[nan] & 0x0040) != 0)
    assert np.array_equal(ours[nan] >> 15, (pats[nan] >> 31).astype(np.uint16))


def test_bf16_encode_roundtrip_all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_decode(bits)
    back = oracle.bf16_encode(vals)
    finite = ~np.isnan(vals)
    assert np.array_equal(back[finite], bits[finite])


# ------------------------------------------------------- exact (f64) forward

@pytest.mark.parametrize("zc", [False, True])
def test_f64_forward_mean_square_invariant(zc):
    x, _, gamma = _problem(5, 96, 11, zc)
    xd = bf16_to_f64(x)
    for eps in (0.0, 1e-6, 0.3):
        y, r = oracle.fwd_f64(xd, gamma, zc, eps)
        m = (xd ** 2).mean(axis=1)
        u = y / _w_eff(gamma, zc)  # the normalised row x * r
        np.testing.assert_allclose((u ** 2).sum(axis=1), 96 * m / (m + eps), rtol=1e-13)
        np.testing.assert_allclose(u, xd * r[:, None], rtol=1e-13)


def test_f64_forward_closed_forms():
    D = 64
    gamma = wl.gamma_for(3, D, False)
    # constant row c: r = 1/sqrt(c^2 + eps)
    for c in (-3.0, 0.5, 7.25):
        y, r = oracle.fwd_f64(np.full((1, D), c), gamma, False, 0.01)
        assert r[0] == pytest.approx(1.0 / np.sqrt(c * c + 0.01), rel=1e-15)
        np.testing.assert_allclose(y[0], np.sign(c) * gamma * abs(c) * r[0], rtol=1e-14)
    # one-hot a*e_j, eps = 0: r = sqrt(D)/|a|, y_j = sign(a) sqrt(D) w_j
    for j, a in ((0, 2.0), (17, -0.75), (D - 1, 5.0)):
        x = np.zeros((1, D))
        x[0, j] = a
        y, r = oracle.fwd_f64(x, gamma, False, 0.0)
        assert r[0] == pytest.approx(np.sqrt(D) / abs(a), rel=1e-15)
        expect = np.zeros(D)
        expect[j] = np.sign(a) * np.sqrt(D) * gamma[j]
        np.testing.assert_allclose(y[0], expect, rtol=1e-14, atol=0)


def test_f64_forward_scale_invariance_at_eps0():
    x, _, gamma = _problem(4, 128, 12, False)
    xd = bf16_to_f64(x)
    y1, r1 = oracle.fwd_f64(xd, gamma, False, 0.0)
    y2, r2 = oracle.fwd_f64(3.7 * xd, gamma, False, 0.0)
    np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(r2 * 3.7, r1, rtol=1e-14)


def test_f64_zero_centered_is_offset_weight():
    x, g, gamma = _problem(3, 40, 13, True)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    ya, _ = oracle.fwd_f64(xd, gamma, True, 1e-6)
    yb, _ = oracle.fwd_f64(xd, gamma.astype(np.float64) + 1.0, False, 1e-6)
    assert np.array_equal(ya, yb)
    dxa, dga = oracle.bwd_f64(gd, xd, gamma, True, 1e-6)
    dxb, dgb = oracle.bwd_f64(gd, xd, gamma.astype(np.float64) + 1.0, False, 1e-6)
    assert np.array_equal(dxa, dxb) and np.array_equal(dga, dgb)


# ------------------------------------------------------ exact (f64) backward

def _fd_errors(xd, gd, gamma, zc, eps, h=1e-5):
    """Max relative errors of the analytic dx and dgamma against central
    differences of L = sum(g * y) taken through the exact forward."""
    T, D = xd.shape
    dx, dg = oracle.bwd_f64(gd, xd, gamma, zc, eps)

    def loss_rows(xv, gv_gamma):
        y, _ = oracle.fwd_f64(xv, gv_gamma, zc, eps)
        return (gd * y).sum(axis=1)

    fd_dx = np.empty_like(xd)
    for k in range(D):
        xp, xm = xd.copy(), xd.copy()
        xp[:, k] += h
        xm[:, k] -= h
        fd_dx[:, k] = (loss_rows(xp, gamma) - loss_rows(xm, gamma)) / (2 * h)
    fd_dg = np.empty(D)
    gam = gamma.astype(np.float64)
    for j in range(D):
        gp, gm = gam.copy(), gam.copy()
        gp[j] += h
        gm[j] -= h
        fd_dg[j] = (loss_rows(xd, gp).sum() - loss_rows(xd, gm).sum()) / (2 * h)
    e_dx = np.abs(dx - fd_dx).max() / np.abs(fd_dx).max()
    e_dg = np.abs(dg - fd_dg).max() / np.abs(fd_dg).max()
    return e_dx, e_dg


@pytest.mark.parametrize("T,D", [(1, 8), (2, 16), (3, 128), (1, 5), (2, 13)])
@pytest.mark.parametrize("zc", [False, True])
def test_f64_backward_matches_finite_differences(T, D, zc):
    x, g, gamma = _problem(T, D, 100 + T * D, zc)
    e_dx, e_dg = _fd_errors(bf16_to_f64(x), bf16_to_f64(g), gamma, zc, 1e-6)
    assert e_dx < 1e-7 and e_dg < 1e-7, (e_dx, e_dg)


def test_f64_backward_scale_identity_at_eps0():
    # sum_k x_k dx_k = r*s - r^3 * s * sum(x^2) / D = 0 when eps = 0
    x, g, gamma = _problem(6, 256, 21, False)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    dx, _ = oracle.bwd_f64(gd, xd, gamma, False, 0.0)
    y, r = oracle.fwd_f64(xd, gamma, False, 0.0)
    scale = (np.abs(xd * gd * gamma) * r[:, None]).sum(axis=1)
    assert np.all(np.abs((xd * dx).sum(axis=1)) <= 1e-12 * scale)


def test_f64_backward_weight_zero_gives_zero():
    x, g, _ = _problem(3, 32, 22, False)
    dx, _ = oracle.bwd_f64(bf16_to_f64(g), bf16_to_f64(x), np.zeros(32), False, 1e-6)
    assert np.all(dx == 0.0)


def test_f64_backward_residual_gradient_adds():
    x, g, gamma = _problem(2, 24, 23, False)
    gres = bf16_to_f64(synth.normal_bf16(23, 4, 2, 24))
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    dx0, dg0 = oracle.bwd_f64(gd, xd, gamma, False, 1e-6)
    dx1, dg1 = oracle.bwd_f64(gd, xd, gamma, False, 1e-6, gres=gres)
    np.testing.assert_allclose(dx1 - dx0, gres, atol=1e-15)
    assert np.array_equal(dg0, dg1)


# -------------------------------------------------- planted-defect controls

def test_weight_twice_defect_is_caught_only_with_non_unit_weights():
    """[MEG] item 2: the extra w_k factor vanishes at w = 1, so the FD check
    must use non-unit weights to see it (the weight=ones control)."""
    x, g, gamma = _problem(2, 16, 31, False)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    with oracle.mutation(2):
        e_bad, _ = _fd_errors(xd, gd, gamma, False, 1e-6)
        e_ones, _ = _fd_errors(xd, gd, np.ones(16, np.float32), False, 1e-6)
    assert e_bad > 1e-3
    assert e_ones < 1e-7


def test_dropped_offset_defect_is_caught():
    """[MEG] item 1: with the offset dropped in the forward only, FD of the
    forward disagrees with the backward, and zc(gamma=0) != plain(gamma=1)."""
    x, g, gamma = _problem(2, 16, 32, True)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    with oracle.mutation(1):
        e_dx, _ = _fd_errors(xd, gd, gamma, True, 1e-6)
        y_zc, _ = oracle.fwd(x, np.zeros(16, np.float32), True)
        y_plain, _ = oracle.fwd(x, np.ones(16, np.float32), False)
    assert e_dx > 1e-3
    assert not np.array_equal(y_zc, y_plain)


def test_rounded_bounds_catch_planted_defects():
    """A defect in the rounded form alone fails its bound against the
    (defect-free) exact form."""
    p = wl.tiny(False, T=8, D=128, seed=33)
    y, r = oracle.fwd(p.x, p.gamma)
    assert _dx_bound_ok(p, r, None).all()
    with oracle.mutation(2):
        dx_bad = oracle.bwd_dx(p.g, p.x, r, p.gamma)
    assert not _dx_bound_ok(p, r, None, dx=dx_bad).all()
    pz = wl.tiny(True, T=8, D=128, seed=34)
    assert _fwd_bound_ok(pz.x, pz.gamma, True, pz.eps).all()
    with oracle.mutation(1):
        y_bad, _ = oracle.fwd(pz.x, pz.gamma, True, pz.eps)
    assert not _fwd_bound_ok(pz.x, pz.gamma, True, pz.eps, y=y_bad).all()


# ------------------------------------------- rounded (R64) vs exact bounds

def _fwd_bound_ok(x, gamma, zc, eps, y=None):
    y0, r = oracle.fwd(x, gamma, zc, eps)
    y = y0 if y is None else y
    yd, rd = oracle.fwd_f64(bf16_to_f64(x), gamma, zc, eps)
    # rstd: three fp32 roundings before rsqrt (halved by it) plus one after
    assert np.all(np.abs(r - rd) <= 2.6 * U32 * rd)
    # n = (x*r)*w carries <= 4.5 fp32 roundoffs, then one bf16 rounding
    return rounding_consistent(y, yd, 4.6 * U32 * np.abs(yd))


def _dx_bound_ok(p, r, gres, dx=None):
    zc = p.zero_centered
    if dx is None:
        dx = oracle.bwd_dx(p.g, p.x, r, p.gamma, zc, gres)
    xd, gd = bf16_to_f64(p.x), bf16_to_f64(p.g)
    gr = None if gres is None else bf16_to_f64(gres)
    dxd, _ = oracle.bwd_f64(gd, xd, p.gamma, zc, p.eps, gres=gr)
    w = _w_eff(p.gamma, zc)
    rd = oracle.fwd_f64(xd, p.gamma, zc, p.eps)[1][:, None]
    D = xd.shape[1]
    s = (gd * w * xd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gd * w * xd).sum(axis=1, keepdims=True)
    t1 = np.abs(gd * w) * rd
    c_abs = rd ** 3 / D
    err = (4.6 * U32 * t1
           + np.abs(xd) * c_abs * (2.1 * U32 * s_abs + 13.0 * U32 * np.abs(s))
           + 2.1 * U32 * np.abs(dxd) + U32 * np.abs(dxd))
    return rounding_consistent(dx, dxd, err)


CASES = [(16, 128, 1001), (7, 4096, 17), (5, 200, 18), (3, 8, 19),
         # rows whose length is not a multiple of 8
         (9, 13, 20), (4, 1, 21), (6, 100, 22), (2, 4100, 23)]


@pytest.mark.parametrize("T,D,seed", CASES)
@pytest.mark.parametrize("zc", [False, True])
def test_r64_forward_within_rounding_of_exact(T, D, seed, zc):
    x, _, gamma = _problem(T, D, seed, zc)
    assert _fwd_bound_ok(x, gamma, zc, 1e-6).all()


@pytest.mark.parametrize("T,D,seed", CASES)
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gres", [False, True])
def test_r64_dx_within_rounding_of_exact(T, D, seed, zc, with_gres):
    p = wl.tiny(zc, T=T, D=D, seed=seed, with_gres=with_gres)
    _, r = oracle.fwd(p.x, p.gamma, zc, p.eps)
    assert _dx_bound_ok(p, r, p.gres).all()


@pytest.mark.parametrize("T,D,seed", [(16, 128, 1001), (300, 64, 5), (2, 4096, 6)])
def test_r64_dgamma_within_rounding_of_exact(T, D, seed):
    x, g, gamma = _problem(T, D, seed, False)
    _, r = oracle.fwd(x, gamma)
    dg = oracle.dgamma(g, x, r)
    xd, gd = bf16_to_f64(x), bf16_to_f64(g)
    _, dgd = oracle.bwd_f64(gd, xd, gamma, False, 1e-6)
    rd = oracle.fwd_f64(xd, gamma, False, 1e-6)[1][:, None]
    bound = 3.6 * U32 * (np.abs(gd * xd) * rd).sum(axis=0) + U32 * np.abs(dgd)
    assert np.all(np.abs(dg - dgd) <= bound)


def test_r64_gated_within_rounding_of_exact():
    p = wl.tiny(False, T=16, D=128, seed=41, with_gate=True)
    out, _ = oracle.gated_fwd(p.x, p.z, p.gamma, False, p.eps)
    outd = oracle.gated_fwd_f64(bf16_to_f64(p.x), bf16_to_f64(p.z), p.gamma, False, p.eps)
    assert rounding_consistent(out, outd, 6.6 * U32 * np.abs(outd)).all()


# ---------------------------------------------- bitwise laws of the R64 form

@pytest.mark.parametrize("T,D,seed", CASES)
def test_zero_centered_gamma0_equals_plain_gamma1(T, D, seed):
    """zc with stored gamma = 0 is w_eff = 1, exactly the plain weight 1."""
    x, g, _ = _problem(T, D, seed, False)
    gres = synth.normal_bf16(seed, 4, T, D)
    z = synth.normal_bf16(seed, 5, T, D)
    zero, one = np.zeros(D, np.float32), np.ones(D, np.float32)
    ya, ra = oracle.fwd(x, zero, True)
    yb, rb = oracle.fwd(x, one, False)
    assert np.array_equal(ya, yb) and np.array_equal(ra.view(np.uint32), rb.view(np.uint32))
    dxa = oracle.bwd_dx(g, x, ra, zero, True, gres)
    dxb = oracle.bwd_dx(g, x, rb, one, False, gres)
    assert np.array_equal(dxa, dxb)
    oa, _ = oracle.gated_fwd(x, z, zero, True)
    ob, _ = oracle.gated_fwd(x, z, one, False)
    assert np.array_equal(oa, ob)


def test_zero_weight_gives_zero_outputs():
    """[MEG]: weight = zeros gives exactly 0."""
    x, g, _ = _problem(5, 128, 51, False)
    zero = np.zeros(128, np.float32)
    y, r = oracle.fwd(x, zero)
    dx = oracle.bwd_dx(g, x, r, zero)
    assert np.all(bf16_to_f64(y) == 0.0) and np.all(bf16_to_f64(dx) == 0.0)


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_scaling_at_eps0(k):
    x, g, gamma = _problem(6, 256, 52, False)
    xs = f32_to_bf16_torch(bf16_to_f32(x) * np.float32(2.0 ** k))  # exact scaling
    y1, r1 = oracle.fwd(x, gamma, False, 0.0)
    y2, r2 = oracle.fwd(xs, gamma, False, 0.0)
    assert np.array_equal(y1, y2)
    assert np.array_equal(r2 * np.float32(2.0 ** k), r1)
    dx1 = oracle.bwd_dx(g, x, r1, gamma)
    dx2 = oracle.bwd_dx(g, xs, r2, gamma)
    assert np.array_equal(bf16_to_f64(dx2) * 2.0 ** k, bf16_to_f64(dx1))


def test_closed_forms_constant_and_one_hot_rows():
    D = 4096
    gamma = wl.gamma_for(53, D, False)
    w_b = f32_to_bf16_torch(gamma)
    for k in (-4, 0, 3):
        for sgn in (1.0, -1.0):
            x = f32_to_bf16_torch(np.full((1, D), sgn * 2.0 ** k, np.float32))
            y, r = oracle.fwd(x, gamma, False, 0.0)
            assert r[0] == np.float32(2.0 ** -k)
            expect = w_b if sgn > 0 else (w_b ^ np.uint16(0x8000))
            assert np.array_equal(y[0], expect)
    # one-hot 2^k e_j at D=4096: r = 64 * 2^-k, y_j = bf16(64 w_j), rest +-0
    for j, k in ((0, 0), (1234, 2), (D - 1, -1)):
        x = np.zeros((1, D), np.uint16)
        x[0, j] = f32_to_bf16_torch(np.array([2.0 ** k], np.float32))[0]
        y, r = oracle.fwd(x, gamma, False, 0.0)
        assert r[0] == np.float32(64.0 * 2.0 ** -k)
        yv = bf16_to_f64(y[0])
        assert yv[j] == bf16_to_f64(f32_to_bf16_torch(np.array([64.0 * gamma[j]], np.float32)))[0]
        assert np.all(np.delete(yv, j) == 0.0)


def test_mean_divides_by_D():
    """The mean is ss / D by one correctly rounded fp32 division, which for D
    not a power of two differs from multiplying by the rounded 1/D. Constant
    rows c at eps = 0 have ss = D c^2 exactly, so r = 1/|c| rounded once;
    for the rows below the multiplication by fl(1/D) would give another r."""
    decisive = 0
    for D in (7, 12, 100, 4100):
        for c in (5.0, 7.0, 11.0, 1.25, 1.75, 2.5, 15.0, 0.625):
            x = f32_to_bf16_torch(np.full((2, D), c, np.float32))
            x[1] ^= np.uint16(0x8000)  # -c
            _, r = oracle.fwd(x, np.ones(D, np.float32), False, 0.0)
            want = np.float32(1.0 / c)
            assert r[0] == want and r[1] == want, (D, c)
            ss = np.float32(D * c * c)
            by_recip = np.float32(1.0 / np.sqrt(np.float64(np.float32(ss * np.float32(1.0 / D)))))
            decisive += by_recip != want
    assert decisive >= 5


def test_single_row_dgamma_is_one_rounded_term():
    x, g, gamma = _problem(1, 512, 54, False)
    _, r = oracle.fwd(x, gamma)
    dg = oracle.dgamma(g, x, r)
    gx = bf16_to_f32(g[0]) * bf16_to_f32(x[0])  # exact in fp32
    expect = (gx * r[0]).astype(np.float32)
    assert np.array_equal(dg.view(np.uint32), expect.view(np.uint32))


def test_dgamma_empty_batch_is_zero():
    x = np.zeros((0, 64), np.uint16)
    dg = oracle.dgamma(x, x, np.zeros(0, np.float32))
    assert np.all(dg == 0.0)


def test_residual_out_is_byte_copy():
    x, _, gamma = _problem(9, 136, 55, False)
    y, res, r = oracle.residual_fwd(x, gamma)
    y2, r2 = oracle.fwd(x, gamma)
    assert np.array_equal(res, x) and np.array_equal(y, y2) and np.array_equal(r, r2)


def test_gated_silu_step_matches_scipy():
    D = 128
    x = synth.normal_bf16(56, 1, 4, D)
    zvals = np.linspace(-30.0, 30.0, 4 * D).reshape(4, D)
    gamma = wl.gamma_for(56, D, False)
    out = oracle.gated_fwd_f64(bf16_to_f64(x), zvals, gamma, False, 1e-6)
    y, _ = oracle.fwd_f64(bf16_to_f64(x), gamma, False, 1e-6)
    np.testing.assert_allclose(out, y * zvals * scipy.special.expit(zvals),
                               rtol=1e-14, atol=1e-300)


def test_gated_special_gates():
    """z = 0 gives +-0; z >= 32 has sigmoid(z) == 1 in fp32, so the gated
    output is the plain output times z (exact for z = 32)."""
    p = wl.tiny(False, T=8, D=128, seed=57)
    y, _ = oracle.fwd(p.x, p.gamma)
    z0 = np.zeros_like(p.x)
    out0, _ = oracle.gated_fwd(p.x, z0, p.gamma)
    assert np.all(bf16_to_f64(out0) == 0.0)
    z32 = np.full_like(p.x, f32_to_bf16_torch(np.array([32.0], np.float32))[0])
    out32, _ = oracle.gated_fwd(p.x, z32, p.gamma)
    assert np.array_equal(bf16_to_f64(out32), 32.0 * bf16_to_f64(y))


def test_oracle_rows_are_batch_invariant():
    """A row's outputs do not depend on the batch around it."""
    D = 2048
    gamma = wl.sweep_gamma(D)
    ax, ag = wl.sweep_anchor(0, D)
    ref_y, ref_r = oracle.fwd(ax[None], gamma)
    ref_dx = oracle.bwd_dx(ag[None], ax[None], ref_r, gamma)
    for M in (2, 17, 33):
        for pos in ("first", "middle", "last", "shuffled"):
            x, g, i = wl.sweep_batch(0, M, pos, D)
            y, r = oracle.fwd(x, gamma)
            dx = oracle.bwd_dx(g, x, r, gamma)
            assert np.array_equal(y[i], ref_y[0]) and r[i] == ref_r[0]
            assert np.array_equal(dx[i], ref_dx[0])


def test_strided_rows_match_packed():
    x, g, gamma = _problem(5, 96, 58, False)
    big = np.zeros((5, 128), np.uint16)
    big[:, :96] = x
    y1, r1 = oracle.fwd(x, gamma)
    y2, r2 = oracle.fwd(big[:, :96], gamma)
    assert np.array_equal(y1, y2) and np.array_equal(r1, r2)


def test_a32_stays_within_its_own_bound_of_r64():
    """Report mode: ascending-fp32 sums differ from R64 by at most the
    classical recursive-summation bound (D-1)*u*sum|terms|."""
    x, _, gamma = _problem(8, 4096, 59, False)
    _, r64 = oracle.fwd(x, gamma, mode=oracle.R64)
    _, r32 = oracle.fwd(x, gamma, mode=oracle.A32)
    rel = np.abs(r32.astype(np.float64) / r64 - 1.0)
    assert np.all(rel <= 0.5 * 4095 * U32 + 3 * U32)
    assert rel.max() > 0  # the two conventions are distinguishable
