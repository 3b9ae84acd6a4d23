"""GPU parity of the gated norm's variants against the CPU oracle: both gate
activations (silu, sigmoid), both rounding conventions of the forward, and
the gated backward (dx, dz, dgamma), through the C-ABI binding.

Tolerances: out and dz <= 1 bf16 ulp; rstd <= 1e-6 relative; dgamma <= 1e-5
relative in the infinity norm (with the fp32-partial overflow rule of
numerics.dgamma_check). dx <= 1 bf16 ulp, or, where dx is a
cancelling difference, within ulp + 2^-20 of the magnitude of its terms:
the kernel's gate is within a few fp32 ulp of the oracle's (correctly
rounded) one, and cancellation magnifies that relative to dx.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host_bits
from numerics import (bf16_to_f32, bf16_to_f64, dgamma_check, dgamma_term_stats,
                      dgamma_terms_f32, gated_dx_terms, max_ulp, rstd_rel_err, ulp_distance,
                      ulp_or_cancelled)
from synth import workloads as wl

pytestmark = pytest.mark.gpu

ACTS = [(irn.RMSN_GATE_SILU, oracle.SILU), (irn.RMSN_GATE_SIGMOID, oracle.SIGMOID)]
ROUNDINGS = [(irn.RMSN_GATED_ROUND_FP32, oracle.FP32_WEIGHT),
             (irn.RMSN_GATED_ROUND_CAST, oracle.CAST_INPUT)]
WIDTHS = [8, 64, 96, 128, 136, 1024, 2560, 4096, 4104, 5632, 6144, 8192, 8200, 16384, 18440,
          32768]
# not multiples of 8: rows of any alignment
# (32767: 4096 groups, so no lane lacks its last one, at 16 vectors per lane)
ODD_WIDTHS = [5, 13, 100, 1001, 4100, 12290, 20003, 32767]


def _rows_for(D):
    return 1037 if D <= 2048 else 261 if D <= 8192 else 97


def _gpu_bwd(p, act, rstd=None, **kw):
    x, g, z, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_bf16(p.z), dev_f32(p.gamma)
    if rstd is None:
        _, rstd = irn.rmsnorm_fwd(x, gamma, p.zero_centered, p.eps)
    return irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma, p.zero_centered, activation=act, **kw)


def _dgamma_ok(gpu, ref, p, act_o):
    """The shared dgamma rule (numerics.dgamma_check): infinity-norm relative
    error <= 1e-5 over ordinary columns, non-finite terms propagated alike,
    and columns whose terms' magnitudes add up to 2^127 or more (where the
    GPU's fp32 chunk partials may overflow and the oracle's double sum does
    not) held to the error bound of an fp32 sum. The terms are
    fp32(fp32(gn*x)*r) with gn = fp32(g*a(z))."""
    z = bf16_to_f64(p.z)
    _, rr = oracle.fwd(p.x, p.gamma, p.zero_centered, p.eps)
    with np.errstate(invalid="ignore", over="ignore"):
        s = scipy.special.expit(z)
        a = (s if act_o == oracle.SIGMOID else z * s).astype(np.float32)
        gn = bf16_to_f32(p.g) * a            # fp32(g * a(z)), as both sides round it
    mag, nonfinite = dgamma_term_stats(dgamma_terms_f32(gn, bf16_to_f32(p.x), rr))
    ok, report = dgamma_check(gpu, ref, mag, nonfinite, p.T + 512)
    print(f"gated dgamma: {report}", flush=True)
    return ok


def _check_bwd(p, act, act_o, label):
    dx, dz, dg = _gpu_bwd(p, act)
    _, rr = oracle.fwd(p.x, p.gamma, p.zero_centered, p.eps)
    rdx, rdz, rdg = oracle.gated_bwd(p.g, p.x, p.z, rr, p.gamma, p.zero_centered, activation=act_o)
    gdx, gdz = host_bits(dx), host_bits(dz)
    terms = gated_dx_terms(p.g, p.x, p.z, p.gamma, p.zero_centered, rr, act_o == oracle.SIGMOID)
    ok = ulp_or_cancelled(gdx, rdx, terms)
    assert ok.all(), (label, int((~ok).sum()), int(ulp_distance(gdx, rdx).max()))
    assert max_ulp(gdz, rdz) <= 1, label
    assert _dgamma_ok(dg.cpu().numpy(), rdg, p, act_o), label
    return gdx, rdx


@pytest.mark.parametrize("rounding,rounding_o", ROUNDINGS)
@pytest.mark.parametrize("act,act_o", ACTS)
@pytest.mark.parametrize("D", WIDTHS + ODD_WIDTHS)
def test_gated_forward_variants(gpu, D, act, act_o, rounding, rounding_o):
    """Every geometry class at a T spanning several steps plus a ragged tail."""
    zc = D % 16 == 8
    p = wl.tiny(zc, T=_rows_for(D), D=D, seed=9400 + D, with_gate=True)
    out, rstd = irn.rmsnorm_gated_fwd_ex(dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma), zc, p.eps,
                                         activation=act, rounding=rounding, want_rstd=True)
    ro, rr = oracle.gated_fwd_ex(p.x, p.z, p.gamma, zc, p.eps, activation=act_o,
                                 convention=rounding_o)
    assert max_ulp(host_bits(out), ro) <= 1
    assert rstd_rel_err(rstd.cpu().numpy(), rr) <= 1e-6


def test_silu_fp32_is_the_gated_forward(gpu):
    p = wl.tiny(False, T=300, D=128, seed=9500, with_gate=True)
    x, z, gamma = dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma)
    a, ra = irn.rmsnorm_gated_fwd(x, z, gamma, want_rstd=True)
    b, rb = irn.rmsnorm_gated_fwd_ex(x, z, gamma, want_rstd=True)
    assert torch.equal(a, b) and torch.equal(ra, rb)


@pytest.mark.parametrize("act,act_o", ACTS)
def test_rounding_conventions_differ_in_bf16(gpu, act, act_o):
    """The two conventions are more than 1e-3 apart somewhere in bf16."""
    p = wl.tiny(False, T=512, D=128, seed=9510, with_gate=True)
    x, z, gamma = dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma)
    f, _ = irn.rmsnorm_gated_fwd_ex(x, z, gamma, activation=act,
                                    rounding=irn.RMSN_GATED_ROUND_FP32)
    c, _ = irn.rmsnorm_gated_fwd_ex(x, z, gamma, activation=act,
                                    rounding=irn.RMSN_GATED_ROUND_CAST)
    assert (f.float() - c.float()).abs().max().item() > 1e-3


@pytest.mark.parametrize("act,act_o", ACTS)
@pytest.mark.parametrize("D", WIDTHS)
def test_gated_backward_widths(gpu, D, act, act_o):
    zc = D % 16 == 8
    p = wl.tiny(zc, T=_rows_for(D), D=D, seed=9600 + D, with_gate=True)
    _check_bwd(p, act, act_o, (D, act))


@pytest.mark.parametrize("act,act_o", ACTS)
@pytest.mark.parametrize("D", [128, 4096])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 513, 2049])
def test_gated_backward_ragged(gpu, T, D, act, act_o):
    p = wl.tiny(False, T=T, D=D, seed=9700 + T, with_gate=True)
    _check_bwd(p, act, act_o, (T, D, act))


@pytest.mark.parametrize("act,act_o", ACTS)
def test_gated_backward_tiny_fixture(gpu, act, act_o):
    for zc in (False, True):
        p = wl.tiny(zc, with_gate=True)
        _check_bwd(p, act, act_o, (zc, act))


@pytest.mark.parametrize("D", [128, 4096])
def test_gated_backward_output_subsets(gpu, D):
    """Each output alone (or any pair) has the bits of the full call's."""
    p = wl.tiny(False, T=333, D=D, seed=9800, with_gate=True)
    x, g, z, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_bf16(p.z), dev_f32(p.gamma)
    _, rstd = irn.rmsnorm_fwd(x, gamma)
    full = irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma)
    for want in ((1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 1, 0), (0, 1, 1), (1, 0, 1)):
        got = irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma, want_dx=bool(want[0]),
                                    want_dz=bool(want[1]), want_dgamma=bool(want[2]))
        for w, a, b in zip(want, got, full):
            if w:
                assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else
                                   a.view(torch.int32),
                                   b.view(torch.int16) if b.dtype == torch.bfloat16 else
                                   b.view(torch.int32)), want
            else:
                assert a is None


def test_gate_at_zero_closed_forms(gpu):
    """z = 0: sigmoid gives a = 1/2 exactly, so dx and dgamma are exactly half
    the plain backward's and out half the plain forward's; silu gives a = 0,
    so dx = 0 and dgamma = 0, and dz = g*((x*r)*w)/2 (silu'(0) = 1/2)."""
    p = wl.tiny(False, T=200, D=4096, seed=9900, with_gate=True)
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    z0 = torch.zeros_like(x)
    y, rstd = irn.rmsnorm_fwd(x, gamma)
    pdx, pdg = irn.rmsnorm_bwd(g, x, rstd, gamma)
    out, _ = irn.rmsnorm_gated_fwd_ex(x, z0, gamma, activation=irn.RMSN_GATE_SIGMOID)
    assert torch.equal(out.float(), 0.5 * y.float())
    dx, dz, dg = irn.rmsnorm_gated_bwd(g, x, z0, rstd, gamma, activation=irn.RMSN_GATE_SIGMOID)
    assert torch.equal(dx.float(), 0.5 * pdx.float())
    assert torch.equal(dg, 0.5 * pdg)
    dx, dz, dg = irn.rmsnorm_gated_bwd(g, x, z0, rstd, gamma, activation=irn.RMSN_GATE_SILU)
    assert torch.all(dx.float() == 0) and torch.all(dg == 0)
    nw = (x.float() * rstd[:, None]) * gamma[None, :]
    assert torch.equal(dz.float(), ((g.float() * nw) * 0.5).bfloat16().float())


def _edge_problem(D, seed):
    """Normal x and g; z rows holding the gate's special values (infinities,
    NaN, bf16's largest and subnormal values, zeros of both signs, large
    arguments of either sign) and one all-zero x row."""
    rng = np.random.default_rng(seed)
    p = wl.tiny(False, T=8, D=D, seed=seed, with_gate=True)
    z = p.z.copy()
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0000, 0x8000,
                         0x42C8, 0xC2C8, 0x4120, 0xC120, 0x42B0, 0xC2B0], np.uint16)
    for t in range(4):
        z[t] = specials[rng.integers(0, specials.size, D)]
    p.z = z
    p.x = p.x.copy()
    p.x[5] = 0
    return p


@pytest.mark.parametrize("act,act_o", ACTS)
@pytest.mark.parametrize("D", [128, 4096])
def test_gated_edge_values(gpu, D, act, act_o):
    p = _edge_problem(D, 9950 + D)
    x, z, gamma = dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma)
    for rounding, rounding_o in ROUNDINGS:
        out, _ = irn.rmsnorm_gated_fwd_ex(x, z, gamma, activation=act, rounding=rounding)
        ro, _ = oracle.gated_fwd_ex(p.x, p.z, p.gamma, activation=act_o, convention=rounding_o)
        assert max_ulp(host_bits(out), ro) <= 1, rounding
    _check_bwd(p, act, act_o, ("edge", D, act))


@pytest.mark.parametrize("act,act_o", ACTS)
def test_gated_backward_rows_across_batches(gpu, act, act_o):
    """dx and dz of a row do not depend on the batch around it."""
    D = 128
    x = dev_bf16(synth.normal_bf16(6300, 1, 1024, D))
    g = dev_bf16(synth.normal_bf16(6300, 2, 1024, D))
    z = dev_bf16(synth.normal_bf16(6300, 5, 1024, D))
    gamma = dev_f32(wl.gamma_for(6300, D, False))
    _, rstd = irn.rmsnorm_fwd(x, gamma)
    fdx, fdz, _ = irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma, activation=act)
    for a, b in ((0, 1), (5, 6), (3, 36), (1000, 1024), (7, 1007)):
        pdx, pdz, _ = irn.rmsnorm_gated_bwd(g[a:b], x[a:b], z[a:b], rstd[a:b], gamma,
                                            activation=act)
        assert torch.equal(pdx, fdx[a:b]) and torch.equal(pdz, fdz[a:b]), (a, b)


def test_gated_backward_empty_batch(gpu):
    D = 256
    e = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    gamma = torch.ones(D, device="cuda")
    dg = torch.full((D,), 7.0, device="cuda")
    dx, dz, dg = irn.rmsnorm_gated_bwd(e, e, e, torch.empty(0, device="cuda"), gamma, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)


def test_gated_repeat_runs_bitwise(gpu):
    p = wl.tiny(True, T=3000, D=4096, seed=9990, with_gate=True)
    first = _gpu_bwd(p, irn.RMSN_GATE_SILU)
    for _ in range(3):
        again = _gpu_bwd(p, irn.RMSN_GATE_SILU)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("act,act_o", ACTS)
@pytest.mark.parametrize("D", ODD_WIDTHS)
def test_gated_backward_odd_widths(gpu, D, act, act_o):
    """Rows not a multiple of 8 (any alignment): dx, dz and dgamma against
    the oracle, over a few steps and a ragged tail."""
    zc = D % 2 == 1
    p = wl.tiny(zc, T=_rows_for(D), D=D, seed=9650 + D, with_gate=True)
    _check_bwd(p, act, act_o, (D, act))


@pytest.mark.parametrize("D", [100, 4100])
def test_gated_backward_odd_rows_strided(gpu, D):
    """Rows of D not a multiple of 8 in wider buffers at an odd element
    offset: the same bits as the contiguous call, nothing written outside."""
    p = wl.tiny(False, T=333, D=D, seed=9660 + D, with_gate=True)
    dx, dz, dg = _gpu_bwd(p, irn.RMSN_GATE_SILU)
    ld = D + 3

    def wide(bits):
        buf = torch.zeros((p.T, ld), dtype=torch.bfloat16, device="cuda")
        buf[:, 1:1 + D] = dev_bf16(bits)
        return buf[:, 1:1 + D]

    x, g, z = wide(p.x), wide(p.g), wide(p.z)
    gamma = dev_f32(p.gamma)
    _, rstd = irn.rmsnorm_fwd(x, gamma, False, p.eps)
    dxw = torch.full((p.T, ld), 5.0, dtype=torch.bfloat16, device="cuda")
    dzw = torch.full((p.T, ld), 5.0, dtype=torch.bfloat16, device="cuda")
    _, _, dg2 = irn.rmsnorm_gated_bwd(g, x, z, rstd, gamma, activation=irn.RMSN_GATE_SILU,
                                      dx=dxw[:, 1:1 + D], dz=dzw[:, 1:1 + D])
    torch.cuda.synchronize()
    assert torch.equal(dxw[:, 1:1 + D], dx) and torch.equal(dzw[:, 1:1 + D], dz)
    assert torch.equal(dg2, dg)
    assert torch.all(dxw[:, 0].float() == 5.0) and torch.all(dxw[:, 1 + D:].float() == 5.0)
    assert torch.all(dzw[:, 0].float() == 5.0) and torch.all(dzw[:, 1 + D:].float() == 5.0)
