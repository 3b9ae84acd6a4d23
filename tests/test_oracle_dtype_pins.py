"""Pins of the oracle's storage types: the binary16 codec, fp16 activations
and bf16 / fp16 weights.

Sources: RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel"
(the contract's fp16 rows beside bf16); Megatron-LM PR "Fix the
batch-invariant RMSNorm forward and its input gradient", item 1 (the weight
is cast to fp32, then offset by one).

What pins what:
  * the binary16 codec: numpy's float16 conversions (all 2^16 patterns for
    decoding, 4M fp32 patterns plus ties, overflow and subnormals for
    encoding);
  * the _dt forms with (bf16, fp32): bitwise equal to the bf16 / fp32
    functions, pinned elsewhere (a second code path);
  * bf16 and fp16 weights: bitwise equal to passing their exact fp32 values;
  * fp16 activations: rounding-aware bounds against the exact (f64) forms,
    whose own pins are finite differences and closed forms; exact-arithmetic
    inputs; overflow to infinity;
  * the gated norm and the fused add-norm in these types: with (bf16, fp32)
    bitwise equal to their bf16 functions; 16-bit weights equal to their fp32
    values; fp16 within rounding of the exact forms; the cast convention's
    two intermediate roundings go to the activations' type (a sigmoid gate at
    z = 0 is exactly 1/2, which exposes them); binary16 overflow of the
    stored residual sum.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from numerics import U32
from synth import workloads as wl


def _f16_bits(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def _f16_val(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(ours[nan]))
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


def test_f16_encode_matches_numpy_rne():
    rng = np.random.default_rng(16)
    pats = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    # concentrate on binary16's range, ties and its subnormal / overflow edges
    near = (rng.integers(0x33000000, 0x47800000, size=1 << 20, dtype=np.uint64)
            .astype(np.uint32))
    ties = (np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
            .astype(np.float32).view(np.uint32) + np.uint32(0x1000))  # halfway up
    edges = np.array([0x477FE000, 0x477FEFFF, 0x477FF000, 0x477FF001, 0x7F800000, 0xFF800000,
                      0x7FC00000, 0x7F800001, 0x00000001, 0x33000000, 0x33000001, 0x387FC000,
                      0x38800000, 0x80000000, 0x3F800000, 0xC7800000], np.uint32)
    vals = np.concatenate([pats, near, ties, edges]).view(np.float32)
    ours = oracle.f16_encode(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    nan = np.isnan(vals)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all((ours[nan] & 0x0200) != 0)


@pytest.mark.parametrize("zc", [False, True])
def test_dt_forms_equal_the_bf16_fp32_functions(zc):
    p = wl.tiny(zc, T=33, D=384, seed=1601, with_gres=True)
    y, r = oracle.fwd_dt(p.x, p.gamma, zc, p.eps)
    y0, r0 = oracle.fwd(p.x, p.gamma, zc, p.eps)
    assert np.array_equal(y, y0) and np.array_equal(r.view(np.uint32), r0.view(np.uint32))
    dx, dg = oracle.bwd_dt(p.g, p.x, r, p.gamma, zc, gres=p.gres)
    dx0, dg0 = oracle.bwd(p.g, p.x, r0, p.gamma, zc, p.gres)
    assert np.array_equal(dx, dx0) and np.array_equal(dg.view(np.uint32), dg0.view(np.uint32))


@pytest.mark.parametrize("weight_dtype", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("act_dtype", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("zc", [False, True])
def test_16bit_weights_equal_their_fp32_values(weight_dtype, act_dtype, zc):
    """The cast to fp32 is exact, so a bf16 / fp16 weight behaves exactly as
    its fp32 value; the +1 offset follows the cast."""
    D = 256
    x = synth.normal_bf16(1602, 1, 20, D)
    g = synth.normal_bf16(1602, 2, 20, D)
    if act_dtype == oracle.F16:  # reuse the draws as fp16 patterns of similar size
        x = _f16_bits(synth.normal_f32(1602, 1, 20 * D).reshape(20, D))
        g = _f16_bits(synth.normal_f32(1602, 2, 20 * D).reshape(20, D))
    w32 = wl.gamma_for(1602, D, zc)
    if weight_dtype == oracle.BF16:
        wbits = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        wval = torch.from_numpy(wbits.view(np.int16)).view(torch.bfloat16).float().numpy()
    else:
        wbits = _f16_bits(w32)
        wval = wbits.view(np.float16).astype(np.float32)
    y, r = oracle.fwd_dt(x, wbits, zc, 1e-6, act_dtype, weight_dtype)
    y0, r0 = oracle.fwd_dt(x, wval, zc, 1e-6, act_dtype, oracle.F32)
    assert np.array_equal(y, y0) and np.array_equal(r, r0)
    dx, dg = oracle.bwd_dt(g, x, r, wbits, zc, act_dtype=act_dtype, weight_dtype=weight_dtype)
    dx0, dg0 = oracle.bwd_dt(g, x, r, wval, zc, act_dtype=act_dtype, weight_dtype=oracle.F32)
    assert np.array_equal(dx, dx0) and np.array_equal(dg, dg0)
    if zc:  # the offset is applied to the widened weight: gamma -> gamma + 1
        y1, _ = oracle.fwd_dt(x, (wval.astype(np.float64) + 1.0).astype(np.float32), False,
                              1e-6, act_dtype, oracle.F32)
        assert np.array_equal(y, y1)


def _f16_rounding_consistent(res_bits, exact, err):
    """A binary16 result is the nearest value to `exact` unless `exact` lies
    within `err` of a rounding midpoint (numpy's RNE gives the nearest)."""
    res = _f16_val(res_bits)
    with np.errstate(over="ignore"):
        nearest = exact.astype(np.float16).astype(np.float64)
    return np.abs(res - exact) <= np.abs(nearest - exact) + 2.0 * err + 1e-300


@pytest.mark.parametrize("T,D,seed", [(16, 128, 1603), (5, 4096, 1604), (9, 200, 1605)])
@pytest.mark.parametrize("zc", [False, True])
def test_f16_activations_within_rounding_of_exact(T, D, seed, zc):
    eps = 1e-6
    xv = synth.normal_f32(seed, 1, T * D).reshape(T, D)
    gv = synth.normal_f32(seed, 2, T * D).reshape(T, D)
    x, g = _f16_bits(xv), _f16_bits(gv)
    gamma = wl.gamma_for(seed, D, zc)
    y, r = oracle.fwd_dt(x, gamma, zc, eps, oracle.F16)
    xd, gd = _f16_val(x), _f16_val(g)
    yd, rd = oracle.fwd_f64(xd, gamma, zc, eps)
    assert np.all(np.abs(r - rd) <= 2.6 * U32 * rd)
    assert _f16_rounding_consistent(y, yd, 4.6 * U32 * np.abs(yd)).all()
    dx, dg = oracle.bwd_dt(g, x, r, gamma, zc, act_dtype=oracle.F16)
    dxd, dgd = oracle.bwd_f64(gd, xd, gamma, zc, eps)
    w = gamma.astype(np.float64) + (1.0 if zc else 0.0)
    rr = rd[:, None]
    s = (gd * w * xd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gd * w * xd).sum(axis=1, keepdims=True)
    err = (4.6 * U32 * np.abs(gd * w) * rr
           + np.abs(xd) * rr ** 3 / D * (2.1 * U32 * s_abs + 13.0 * U32 * np.abs(s))
           + 3.1 * U32 * np.abs(dxd))
    assert _f16_rounding_consistent(dx, dxd, err).all()
    bound = 3.6 * U32 * (np.abs(gd * xd) * rr).sum(axis=0) + U32 * np.abs(dgd)
    assert np.all(np.abs(dg - dgd) <= bound)


def test_f16_exact_arithmetic_and_overflow():
    """Dyadic inputs whose row mean square is a power of four give exact
    results at eps = 0; outputs past 65504 round to infinity."""
    D = 64
    x = np.full((2, D), 2.0, np.float32)        # r = 1/2
    x[1, ::2] = -2.0
    gamma = np.full(D, 3.0, np.float32)
    y, r = oracle.fwd_dt(_f16_bits(x), gamma, False, 0.0, oracle.F16)
    assert np.all(r == 0.5)
    assert np.array_equal(_f16_val(y), np.sign(x) * 3.0)
    big = np.full(D, 70000.0, np.float32)
    y, _ = oracle.fwd_dt(_f16_bits(x), big, False, 0.0, oracle.F16)
    assert np.all(np.isinf(_f16_val(y))) and np.array_equal(np.sign(_f16_val(y)), np.sign(x))


# ---- gated norm and fused add-norm in other storage types -----------------------

ACTS = [oracle.SILU, oracle.SIGMOID]


def _f16_problem(seed, T, D, scales=(1.0, 1.0, 1.0)):
    """fp16 patterns of N(0, s^2) draws for three operands."""
    return tuple(_f16_bits(synth.normal_f32(seed, 1 + i, T * D).reshape(T, D) * s)
                 for i, s in enumerate(scales))


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("act", ACTS)
def test_gated_dt_forms_equal_the_bf16_functions(zc, act):
    p = wl.tiny(zc, T=21, D=320, seed=1610, with_gate=True)
    for conv in (oracle.FP32_WEIGHT, oracle.CAST_INPUT):
        o, r = oracle.gated_fwd_dt(p.x, p.z, p.gamma, zc, p.eps, act, conv)
        o0, r0 = oracle.gated_fwd_ex(p.x, p.z, p.gamma, zc, p.eps, act, conv)
        assert np.array_equal(o, o0) and np.array_equal(r.view(np.uint32), r0.view(np.uint32))
    dx, dz, dg = oracle.gated_bwd_dt(p.g, p.x, p.z, r, p.gamma, zc, act)
    dx0, dz0, dg0 = oracle.gated_bwd(p.g, p.x, p.z, r, p.gamma, zc, act)
    assert np.array_equal(dx, dx0) and np.array_equal(dz, dz0)
    assert np.array_equal(dg.view(np.uint32), dg0.view(np.uint32))


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gro", [False, True])
def test_add_dt_forms_equal_the_bf16_functions(zc, with_gro):
    T, D, seed = 19, 264, 1611
    x = synth.normal_bf16(seed, 1, T, D)
    res = synth.normal_bf16(seed, 4, T, D, scale=2.0)
    g = synth.normal_bf16(seed, 2, T, D)
    gro = synth.normal_bf16(seed, 5, T, D, scale=0.5) if with_gro else None
    gamma = wl.gamma_for(seed, D, zc)
    y, ro, r = oracle.add_fwd_dt(x, res, gamma, zc)
    y0, ro0, r0 = oracle.add_fwd(x, res, gamma, zc)
    assert np.array_equal(y, y0) and np.array_equal(ro, ro0)
    assert np.array_equal(r.view(np.uint32), r0.view(np.uint32))
    dh, dg = oracle.add_bwd_dt(g, x, res, r, gamma, zc, g_rout=gro)
    dh0, dg0 = oracle.add_bwd(g, x, res, r, gamma, zc, g_rout=gro)
    assert np.array_equal(dh, dh0) and np.array_equal(dg.view(np.uint32), dg0.view(np.uint32))


def _weights16(w32, weight_dtype):
    if weight_dtype == oracle.BF16:
        bits = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        val = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    else:
        bits = _f16_bits(w32)
        val = bits.view(np.float16).astype(np.float32)
    return bits, val


@pytest.mark.parametrize("weight_dtype", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("act_dtype", [oracle.BF16, oracle.F16])
@pytest.mark.parametrize("zc", [False, True])
def test_gated_add_16bit_weights_equal_their_fp32_values(weight_dtype, act_dtype, zc):
    T, D, seed = 12, 256, 1612
    if act_dtype == oracle.F16:
        x, z, g = _f16_problem(seed, T, D, (1.0, 3.0, 1.0))
    else:
        x, z, g = (synth.normal_bf16(seed, 1 + i, T, D, scale=s)
                   for i, s in enumerate((1.0, 3.0, 1.0)))
    wbits, wval = _weights16(wl.gamma_for(seed, D, zc), weight_dtype)
    F32 = oracle.F32
    for act in ACTS:
        for conv in (oracle.FP32_WEIGHT, oracle.CAST_INPUT):
            o, r = oracle.gated_fwd_dt(x, z, wbits, zc, 1e-6, act, conv, act_dtype, weight_dtype)
            o0, r0 = oracle.gated_fwd_dt(x, z, wval, zc, 1e-6, act, conv, act_dtype, F32)
            assert np.array_equal(o, o0) and np.array_equal(r, r0)
        b = oracle.gated_bwd_dt(g, x, z, r, wbits, zc, act, act_dtype, weight_dtype)
        b0 = oracle.gated_bwd_dt(g, x, z, r, wval, zc, act, act_dtype, F32)
        assert all(np.array_equal(u, v) for u, v in zip(b, b0))
    y, ro, r = oracle.add_fwd_dt(x, z, wbits, zc, 1e-6, act_dtype, weight_dtype)
    y0, ro0, r0 = oracle.add_fwd_dt(x, z, wval, zc, 1e-6, act_dtype, F32)
    assert np.array_equal(y, y0) and np.array_equal(ro, ro0) and np.array_equal(r, r0)
    dh, dg = oracle.add_bwd_dt(g, x, z, r, wbits, zc, g_rout=g, act_dtype=act_dtype,
                               weight_dtype=weight_dtype)
    dh0, dg0 = oracle.add_bwd_dt(g, x, z, r, wval, zc, g_rout=g, act_dtype=act_dtype,
                                 weight_dtype=F32)
    assert np.array_equal(dh, dh0) and np.array_equal(dg, dg0)


def _gate(act, z):
    import scipy.special
    s = scipy.special.expit(z)
    return z * s if act == oracle.SILU else s


@pytest.mark.parametrize("T,D,seed", [(16, 128, 1613), (5, 4096, 1614), (7, 200, 1615)])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("zc", [False, True])
def test_f16_gated_within_rounding_of_exact(T, D, seed, act, zc):
    eps = 1e-6
    x, z, g = _f16_problem(seed, T, D, (1.0, 3.0, 1.0))
    gamma = wl.gamma_for(seed, D, zc)
    out, r = oracle.gated_fwd_dt(x, z, gamma, zc, eps, act, act_dtype=oracle.F16)
    xd, zd, gd = _f16_val(x), _f16_val(z), _f16_val(g)
    ex = oracle.gated_fwd_ex_f64(xd, zd, gamma, zc, eps, act)
    rd = oracle.fwd_f64(xd, gamma, zc, eps)[1]
    assert np.all(np.abs(r - rd) <= 2.6 * U32 * rd)
    # x*r (r 2.6u + u), *w (u), the gate in fp32 (u), *a (u)
    assert _f16_rounding_consistent(out, ex, 6.6 * U32 * np.abs(ex)).all()
    dx, dz, dg = oracle.gated_bwd_dt(g, x, z, r, gamma, zc, act, act_dtype=oracle.F16)
    edx, edz, edg = oracle.gated_bwd_f64(gd, xd, zd, gamma, zc, eps, act)
    w = gamma.astype(np.float64) + (1.0 if zc else 0.0)
    rr = rd[:, None]
    assert _f16_rounding_consistent(dz, edz, 7.6 * U32 * np.abs(edz)).all()
    gn = gd * _gate(act, zd)
    s = (gn * w * xd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gn * w * xd).sum(axis=1, keepdims=True)
    err = (6.6 * U32 * np.abs(gn * w) * rr
           + np.abs(xd) * rr ** 3 / D * (4.1 * U32 * s_abs + 13.0 * U32 * np.abs(s))
           + 3.1 * U32 * np.abs(edx))
    assert _f16_rounding_consistent(dx, edx, err).all()
    bound = 5.6 * U32 * (np.abs(gn * xd) * rr).sum(axis=0) + U32 * np.abs(edg)
    assert np.all(np.abs(dg - edg) <= bound)


@pytest.mark.parametrize("act_dtype", [oracle.BF16, oracle.F16])
def test_cast_convention_rounds_to_the_activation_type(act_dtype):
    """A sigmoid gate at z = 0 is exactly 1/2. The cast convention then gives
    1/2 * q(q(q(x*r) * w)) with q the rounding to the activations' type and
    q(x*r) the plain forward with unit weight; the fp32 convention gives
    1/2 * q(x*r*w), the plain forward. Inputs keep every output normal, so
    halving is exact."""
    T, D, seed = 12, 256, 1616
    rng = np.random.default_rng(seed)
    mag = rng.uniform(0.5, 2.0, (T, D)) * rng.choice([-1.0, 1.0], (T, D))
    gamma = rng.uniform(0.5, 1.5, D).astype(np.float32)
    if act_dtype == oracle.F16:
        x = _f16_bits(mag)
        val, enc = (lambda b: _f16_val(b)), (lambda v: _f16_bits(v))
    else:
        x = torch.from_numpy(mag.astype(np.float32)).bfloat16().view(torch.int16).numpy() \
            .view(np.uint16)
        val = lambda b: torch.from_numpy(np.asarray(b).view(np.int16)).view(torch.bfloat16) \
            .double().numpy()
        enc = lambda v: torch.from_numpy(np.asarray(v, np.float32)).bfloat16() \
            .view(torch.int16).numpy().view(np.uint16)
    z0 = np.zeros_like(x)
    cast, _ = oracle.gated_fwd_dt(x, z0, gamma, False, 1e-6, oracle.SIGMOID, oracle.CAST_INPUT,
                                  act_dtype)
    fp32, _ = oracle.gated_fwd_dt(x, z0, gamma, False, 1e-6, oracle.SIGMOID, oracle.FP32_WEIGHT,
                                  act_dtype)
    n, _ = oracle.fwd_dt(x, np.ones(D, np.float32), False, 1e-6, act_dtype)
    nw = enc((val(n).astype(np.float32) * gamma).astype(np.float32))
    assert np.array_equal(val(cast), 0.5 * val(nw))
    y, _ = oracle.fwd_dt(x, gamma, False, 1e-6, act_dtype)
    assert np.array_equal(val(fp32), 0.5 * val(y))
    assert (cast != fp32).any()


@pytest.mark.parametrize("T,D,seed", [(16, 128, 1617), (7, 4096, 1618), (5, 200, 1619)])
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gro", [False, True])
def test_f16_add_within_rounding_of_exact(T, D, seed, zc, with_gro):
    eps = 1e-6
    x, res, g = _f16_problem(seed, T, D, (1.0, 2.0, 1.0))
    gro = _f16_bits(synth.normal_f32(seed, 5, T * D).reshape(T, D) * 0.5) if with_gro else None
    gamma = wl.gamma_for(seed, D, zc)
    y, rout, r = oracle.add_fwd_dt(x, res, gamma, zc, eps, oracle.F16)
    xd, resd, gd = _f16_val(x), _f16_val(res), _f16_val(g)
    grod = None if gro is None else _f16_val(gro)
    yd, hd, rd = oracle.add_fwd_f64(xd, resd, gamma, zc, eps)
    assert np.all(np.abs(r - rd) <= 3.0 * U32 * rd)
    assert _f16_rounding_consistent(rout, hd, U32 * np.abs(hd)).all()
    assert _f16_rounding_consistent(y, yd, 6.1 * U32 * np.abs(yd)).all()
    dh, dg = oracle.add_bwd_dt(g, x, res, r, gamma, zc, g_rout=gro, act_dtype=oracle.F16)
    dhd, dgd = oracle.add_bwd_f64(gd, xd, resd, gamma, zc, eps, g_rout=grod)
    w = gamma.astype(np.float64) + (1.0 if zc else 0.0)
    rr = rd[:, None]
    s = (gd * w * hd).sum(axis=1, keepdims=True)
    s_abs = np.abs(gd * w * hd).sum(axis=1, keepdims=True)
    err = (7.6 * U32 * np.abs(gd * w) * rr
           + np.abs(hd) * rr ** 3 / D * (3.1 * U32 * s_abs + 16.0 * U32 * np.abs(s))
           + 3.1 * U32 * np.abs(dhd))
    assert _f16_rounding_consistent(dh, dhd, err).all()
    bound = 6.6 * U32 * (np.abs(gd * hd) * rr).sum(axis=0) + U32 * np.abs(dgd)
    assert np.all(np.abs(dg - dgd) <= bound)


def test_f16_add_residual_out_overflows_to_infinity():
    """h = x + residual is formed in fp32; past binary16's range the stored
    residual_out is infinite while y, normalised, stays finite."""
    D = 64
    x = _f16_bits(np.full((1, D), 60000.0))
    res = _f16_bits(np.full((1, D), 30000.0))
    y, ro, r = oracle.add_fwd_dt(x, res, np.ones(D, np.float32), False, 0.0, oracle.F16)
    assert np.all(np.isinf(_f16_val(ro)))
    assert np.array_equal(_f16_val(y), np.ones((1, D)))
    assert abs(float(r[0]) * 90000.0 - 1.0) <= 3.0 * U32
