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
    inputs; overflow to infinity.
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
