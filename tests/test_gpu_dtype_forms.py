"""GPU parity of the gated norm and the fused add-norm in other storage types
(rmsnorm_gated_fwd_dt, rmsnorm_gated_bwd_dt, rmsnorm_add_fwd_dt,
rmsnorm_add_bwd_dt) against the CPU oracle's _dt forms: fp16 activations
and bf16 / fp16 / fp32 weights, rows of every geometry class and of lengths
that are not multiples of 8.

Sources: RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel"
(fp16 checked beside bf16; the gated conventions, one casting to the input
dtype; the fused add of the decoder norms); Megatron-LM PR "Fix the
batch-invariant RMSNorm forward and its input gradient", item 1 (weights
cast to fp32, then offset).

Tolerances: out, y, residual_out, dz and dh <= 1 ulp of their storage type
(ordered integers of the bits); rstd <= 1e-6 relative; dgamma <= 1e-5
relative in the infinity norm, under the fp32-partial overflow rule of
numerics.dgamma_check. The gated dx <= 1 ulp, or where it is a cancelling
difference within ulp + 2^-20 of the magnitude of its terms (the kernel's
gate is within a few fp32 ulps of the oracle's correctly rounded one).
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from numerics import (dgamma_check, dgamma_rel_err, dgamma_term_stats, dgamma_terms_f32,
                      max_ulp, rstd_rel_err, ulp_distance)
from synth import workloads as wl

pytestmark = pytest.mark.gpu

ACT = {"bf16": (torch.bfloat16, oracle.BF16), "f16": (torch.float16, oracle.F16)}
WEIGHT = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16),
          "f16": (torch.float16, oracle.F16)}
GATES = [(irn.RMSN_GATE_SILU, oracle.SILU), (irn.RMSN_GATE_SIGMOID, oracle.SIGMOID)]
ROUNDINGS = [(irn.RMSN_GATED_ROUND_FP32, oracle.FP32_WEIGHT),
             (irn.RMSN_GATED_ROUND_CAST, oracle.CAST_INPUT)]
# every geometry class (one to four waves per row, several rows per wave),
# rows of 16-byte groups and rows that are not
WIDTHS = [8, 96, 128, 136, 1024, 4096, 4104, 8192, 12288, 32768]
ODD_WIDTHS = [5, 100, 1001, 4100, 20003]


def _rows_for(D):
    return 1037 if D <= 2048 else 261 if D <= 8192 else 97


def _bits(seed, stream, T, D, act, scale=1.0):
    v = synth.normal_f32(seed, stream, T * D, 0.0, scale).reshape(T, D)
    return torch.from_numpy(v).to(ACT[act][0]).view(torch.int16).numpy().view(np.uint16)


def _dev(bits, act):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(ACT[act][0]).cuda()


def _host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _to_f32(bits, act):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(ACT[act][0]) \
        .float().numpy()


def _weights(seed, D, zc, wt):
    t = torch.from_numpy(wl.gamma_for(seed, D, zc)).to(WEIGHT[wt][0])
    stored = t.numpy() if wt == "f32" else t.view(torch.int16).numpy().view(np.uint16)
    return t.cuda(), stored, t.float().numpy()


def _gate(act_o, z):
    s = scipy.special.expit(z)
    return s if act_o == oracle.SIGMOID else z * s


def _ulp(v, act):
    """Spacing of the storage type's values at |v| (subnormal spacing below
    its smallest normal)."""
    bits, emin = (8, -125) if act == "bf16" else (11, -13)
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, np.maximum(e, emin) - bits)


def _ulp_or_cancelled(got, ref, terms, act, k=2.0 ** -20):
    d = ulp_distance(got, ref)
    g, r = _to_f32(got, act).astype(np.float64), _to_f32(ref, act).astype(np.float64)
    with np.errstate(invalid="ignore"):
        near = np.abs(g - r) <= _ulp(r, act) + k * np.abs(terms)
    return (d <= 1) | near


# ---- gated norm --------------------------------------------------------------------

def _gated_problem(seed, T, D, act):
    return (_bits(seed, 1, T, D, act), _bits(seed, 5, T, D, act, 2.0),
            _bits(seed, 2, T, D, act))


def _check_gated(act, wt, T, D, zc, gate, gate_o, rounding, rounding_o, seed, backward=True):
    x, z, g = _gated_problem(seed, T, D, act)
    gamma, gstored, w32 = _weights(seed, D, zc, wt)
    a_o, w_o = ACT[act][1], WEIGHT[wt][1]
    out, r = irn.rmsnorm_gated_fwd_dt(_dev(x, act), _dev(z, act), gamma, zc, 1e-6,
                                      activation=gate, rounding=rounding, want_rstd=True)
    ro, rr = oracle.gated_fwd_dt(x, z, gstored, zc, 1e-6, gate_o, rounding_o, a_o, w_o)
    label = (act, wt, T, D, zc, gate, rounding)
    assert max_ulp(_host(out), ro) <= 1, label
    assert rstd_rel_err(r.cpu().numpy(), rr) <= 1e-6, label
    if not backward:
        return
    dx, dz, dg = irn.rmsnorm_gated_bwd_dt(_dev(g, act), _dev(x, act), _dev(z, act), r, gamma, zc,
                                          activation=gate)
    torch.cuda.synchronize()
    rdx, rdz, rdg = oracle.gated_bwd_dt(g, x, z, rr, gstored, zc, gate_o, a_o, w_o)
    assert max_ulp(_host(dz), rdz) <= 1, label
    xf, gf, zf = (_to_f32(b, act).astype(np.float64) for b in (x, g, z))
    w = w32.astype(np.float64) + (1.0 if zc else 0.0)
    rd = rr.astype(np.float64)[:, None]
    gw = gf * _gate(gate_o, zf) * w
    terms = np.abs(gw * rd) + np.abs(xf) * rd ** 3 * np.abs(gw * xf).sum(1, keepdims=True) / D
    ok = _ulp_or_cancelled(_host(dx), rdx, terms, act)
    assert ok.all(), (label, int((~ok).sum()))
    with np.errstate(invalid="ignore", over="ignore"):
        a32 = _gate(gate_o, zf).astype(np.float32)
    gn = _to_f32(g, act) * a32
    mag, nonfinite = dgamma_term_stats(dgamma_terms_f32(gn, _to_f32(x, act), rr))
    good, report = dgamma_check(dg.cpu().numpy(), rdg, mag, nonfinite, T + 512)
    assert good, (label, report)


@pytest.mark.parametrize("wt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("rounding,rounding_o", ROUNDINGS)
@pytest.mark.parametrize("gate,gate_o", GATES)
def test_gated_types(gpu, act, wt, gate, gate_o, rounding, rounding_o):
    _check_gated(act, wt, 37, 4096, wt == "f16", gate, gate_o, rounding, rounding_o, 1800)


@pytest.mark.parametrize("gate,gate_o", GATES)
@pytest.mark.parametrize("D", WIDTHS + ODD_WIDTHS)
def test_gated_f16_widths(gpu, D, gate, gate_o):
    zc = D % 16 == 8
    _check_gated("f16", "bf16" if D % 2 else "f32", _rows_for(D), D, zc, gate, gate_o,
                 irn.RMSN_GATED_ROUND_FP32, oracle.FP32_WEIGHT, 1810 + D)


@pytest.mark.parametrize("gate,gate_o", GATES)
@pytest.mark.parametrize("D", [128, 4096, 4104, 4100, 20003])
def test_gated_f16_cast_widths(gpu, D, gate, gate_o):
    """The cast convention rounds its two intermediates to fp16."""
    _check_gated("f16", "f16", _rows_for(D), D, False, gate, gate_o, irn.RMSN_GATED_ROUND_CAST,
                 oracle.CAST_INPUT, 1820 + D, backward=False)


def test_gated_f16_cast_differs_from_fp32_convention(gpu):
    x, z, _ = _gated_problem(1830, 512, 128, "f16")
    gamma, _, _ = _weights(1830, 128, False, "f32")
    f, _ = irn.rmsnorm_gated_fwd_dt(_dev(x, "f16"), _dev(z, "f16"), gamma,
                                    rounding=irn.RMSN_GATED_ROUND_FP32)
    c, _ = irn.rmsnorm_gated_fwd_dt(_dev(x, "f16"), _dev(z, "f16"), gamma,
                                    rounding=irn.RMSN_GATED_ROUND_CAST)
    assert (f != c).any()


# ---- fused add-norm ------------------------------------------------------------------

def _check_add(act, wt, T, D, zc, with_gro, seed):
    x, res = _bits(seed, 1, T, D, act), _bits(seed, 6, T, D, act, 2.0)
    g = _bits(seed, 2, T, D, act)
    gro = _bits(seed, 4, T, D, act, 0.5) if with_gro else None
    gamma, gstored, _ = _weights(seed, D, zc, wt)
    a_o, w_o = ACT[act][1], WEIGHT[wt][1]
    y, rout, r = irn.rmsnorm_add_fwd_dt(_dev(x, act), _dev(res, act), gamma, zc, 1e-6)
    ry, rrout, rr = oracle.add_fwd_dt(x, res, gstored, zc, 1e-6, a_o, w_o)
    label = (act, wt, T, D, zc, with_gro)
    assert max_ulp(_host(y), ry) <= 1, label
    assert np.array_equal(_host(rout), rrout), label  # one fp32 add, one rounding: exact
    assert rstd_rel_err(r.cpu().numpy(), rr) <= 1e-6, label
    dh, dg = irn.rmsnorm_add_bwd_dt(_dev(g, act), _dev(x, act), _dev(res, act), r, gamma, zc,
                                    g_residual_out=None if gro is None else _dev(gro, act))
    torch.cuda.synchronize()
    rdh, rdg = oracle.add_bwd_dt(g, x, res, rr, gstored, zc, g_rout=gro, act_dtype=a_o,
                                 weight_dtype=w_o)
    assert max_ulp(_host(dh), rdh) <= 1, label
    assert dgamma_rel_err(dg.cpu().numpy(), rdg) <= 1e-5, label


@pytest.mark.parametrize("wt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("zc", [False, True])
def test_add_types(gpu, act, wt, zc):
    _check_add(act, wt, 37, 4096, zc, True, 1840)


@pytest.mark.parametrize("with_gro", [False, True])
@pytest.mark.parametrize("D", WIDTHS + ODD_WIDTHS)
def test_add_f16_widths(gpu, D, with_gro):
    _check_add("f16", "f16" if D % 2 else "f32", _rows_for(D), D, D % 16 == 8, with_gro, 1850 + D)


@pytest.mark.parametrize("T", [1, 2, 63, 65, 513])
def test_add_f16_ragged_batches(gpu, T):
    _check_add("f16", "bf16", T, 2048, True, True, 1860 + T)


def test_add_f16_in_place(gpu):
    """y over x and residual_out over the residual input give the bytes of
    the out-of-place call."""
    T, D = 300, 4100
    x, res = _bits(1870, 1, T, D, "f16"), _bits(1870, 6, T, D, "f16", 2.0)
    gamma, _, _ = _weights(1870, D, False, "f16")
    y0, ro0, r0 = irn.rmsnorm_add_fwd_dt(_dev(x, "f16"), _dev(res, "f16"), gamma)
    xd, rd = _dev(x, "f16"), _dev(res, "f16")
    y1, ro1, r1 = irn.rmsnorm_add_fwd_dt(xd, rd, gamma, y=xd, residual_out=rd)
    assert y1.data_ptr() == xd.data_ptr() and ro1.data_ptr() == rd.data_ptr()
    assert torch.equal(y0, xd) and torch.equal(ro0, rd) and torch.equal(r0, r1)


# ---- shared properties ---------------------------------------------------------------

def test_16bit_weights_equal_fp32_weights_bitwise(gpu):
    """A bf16 / fp16 weight gives the bytes of its exact fp32 value, gated
    and fused add alike."""
    T, D = 100, 4096
    x, z, g = (_dev(b, "f16") for b in _gated_problem(1880, T, D, "f16"))
    for wt in ("bf16", "f16"):
        w16, _, _ = _weights(1880, D, True, wt)
        w32 = w16.float()
        for gate, _ in GATES:
            o16, r16 = irn.rmsnorm_gated_fwd_dt(x, z, w16, True, activation=gate, want_rstd=True)
            o32, r32 = irn.rmsnorm_gated_fwd_dt(x, z, w32, True, activation=gate, want_rstd=True)
            assert torch.equal(o16, o32) and torch.equal(r16, r32)
            b16 = irn.rmsnorm_gated_bwd_dt(g, x, z, r16, w16, True, activation=gate)
            b32 = irn.rmsnorm_gated_bwd_dt(g, x, z, r32, w32, True, activation=gate)
            assert all(torch.equal(u, v) for u, v in zip(b16, b32))
        a16 = irn.rmsnorm_add_fwd_dt(x, z, w16, True)
        a32 = irn.rmsnorm_add_fwd_dt(x, z, w32, True)
        assert all(torch.equal(u, v) for u, v in zip(a16, a32))
        d16 = irn.rmsnorm_add_bwd_dt(g, x, z, a16[2], w16, True, g_residual_out=g)
        d32 = irn.rmsnorm_add_bwd_dt(g, x, z, a32[2], w32, True, g_residual_out=g)
        assert all(torch.equal(u, v) for u, v in zip(d16, d32))


def test_bf16_dt_forms_equal_the_bf16_entry_points(gpu):
    """With bf16 activations and fp32 weights the _dt entry points are the
    bf16 ones, byte for byte."""
    T, D = 300, 4100
    x, z, g = (_dev(b, "bf16") for b in _gated_problem(1890, T, D, "bf16"))
    gamma, _, _ = _weights(1890, D, False, "f32")
    for gate, _ in GATES:
        for rnd, _ in ROUNDINGS:
            a = irn.rmsnorm_gated_fwd_dt(x, z, gamma, activation=gate, rounding=rnd,
                                         want_rstd=True)
            b = irn.rmsnorm_gated_fwd_ex(x, z, gamma, activation=gate, rounding=rnd,
                                         want_rstd=True)
            assert all(torch.equal(u, v) for u, v in zip(a, b))
        a = irn.rmsnorm_gated_bwd_dt(g, x, z, b[1], gamma, activation=gate)
        c = irn.rmsnorm_gated_bwd(g, x, z, b[1], gamma, activation=gate)
        assert all(torch.equal(u, v) for u, v in zip(a, c))
    a = irn.rmsnorm_add_fwd_dt(x, z, gamma)
    b = irn.rmsnorm_add_fwd(x, z, gamma)
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    a = irn.rmsnorm_add_bwd_dt(g, x, z, b[2], gamma, g_residual_out=g)
    c = irn.rmsnorm_add_bwd(g, x, z, b[2], gamma, g_residual_out=g)
    assert all(torch.equal(u, v) for u, v in zip(a, c))


@pytest.mark.parametrize("D", [4096, 4100])
def test_f16_rows_across_batches(gpu, D):
    """Every per-row output of the fp16 gated and fused-add forms is the same
    in any slice of the batch."""
    T = 300
    x, z, g = (_dev(b, "f16") for b in _gated_problem(1900 + D, T, D, "f16"))
    gamma, _, _ = _weights(1900, D, False, "f16")
    o, r = irn.rmsnorm_gated_fwd_dt(x, z, gamma, want_rstd=True)
    dx, dz, _ = irn.rmsnorm_gated_bwd_dt(g, x, z, r, gamma, want_dgamma=False)
    y, ro, ra = irn.rmsnorm_add_fwd_dt(x, z, gamma)
    dh, _ = irn.rmsnorm_add_bwd_dt(g, x, z, ra, gamma, want_dgamma=False)
    for a, b in ((0, 1), (7, 8), (3, 70), (299, 300), (100, 300)):
        os_, rs = irn.rmsnorm_gated_fwd_dt(x[a:b], z[a:b], gamma, want_rstd=True)
        dxs, dzs, _ = irn.rmsnorm_gated_bwd_dt(g[a:b], x[a:b], z[a:b], rs, gamma,
                                              want_dgamma=False)
        assert torch.equal(os_, o[a:b]) and torch.equal(rs, r[a:b])
        assert torch.equal(dxs, dx[a:b]) and torch.equal(dzs, dz[a:b])
        ys, ros, ras = irn.rmsnorm_add_fwd_dt(x[a:b], z[a:b], gamma)
        dhs, _ = irn.rmsnorm_add_bwd_dt(g[a:b], x[a:b], z[a:b], ras, gamma, want_dgamma=False)
        assert torch.equal(ys, y[a:b]) and torch.equal(ros, ro[a:b]) and torch.equal(ras, ra[a:b])
        assert torch.equal(dhs, dh[a:b])
