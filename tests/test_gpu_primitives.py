"""The library's device primitives, element by element (the helper in
tests/primitives runs the library's own functions on arbitrary inputs):

* the fp32 -> bf16 conversion every kernel stores with (rmsn::pack2,
  gfx950's v_cvt_pk_bf16_f32) on all 2^32 fp32 bit patterns, against the
  oracle's codec (round to nearest even, subnormals kept, overflow to
  infinity): bitwise for every non-NaN input, a NaN of the same sign for
  every NaN input (the payload may differ);
* the gate functions of the gated norm on every 256th fp32 bit pattern plus
  the special values, against double-precision references from
  scipy.special.expit: the forward's sigmoid_fast and gate_fast (stated to
  about 2^-16 relative) and the backward's gate and gate_and_grad (stated to
  a few fp32 ulp). Relative errors are taken against max(|ref|, 2^-126), so
  results in the subnormal range are held to the same absolute error as
  the smallest normal ones, with an allowance for a subnormal sigmoid
  scaled by z; silu' near its root against the magnitude of its terms;
  non-finite references must be matched exactly (NaN for NaN).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import primitives

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, os.cpu_count() or 1))


def _log(msg):
    print(msg, flush=True)


def test_bf16_conversion_on_every_fp32_pattern(gpu):
    lib = primitives.load()
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int16, device=gpu)
    stream = torch.cuda.current_stream(gpu).cuda_stream
    step = chunk // THREADS
    total_nan = 0
    with ThreadPoolExecutor(THREADS) as pool:
        for c in range(1 << 32 >> 28):
            first = c * chunk
            assert lib.prim_pack_all(first, chunk, out.data_ptr(), stream) == 0
            got = out.cpu().numpy().view(np.uint16)
            bits = np.arange(first, first + chunk, dtype=np.uint32)
            vals = bits.view(np.float32)
            ref = np.empty(chunk, np.uint16)

            def enc(i):
                ref[i * step:(i + 1) * step] = oracle.bf16_encode(vals[i * step:(i + 1) * step])

            list(pool.map(enc, range(THREADS)))
            nan_in = (bits & 0x7FFFFFFF) > 0x7F800000
            diff = got != ref
            # non-NaN inputs: bitwise
            bad = diff & ~nan_in
            assert not bad.any(), (c, hex(int(bits[bad][0])), hex(int(got[bad][0])),
                                   hex(int(ref[bad][0])))
            # NaN inputs: a NaN of the same sign
            g = got[nan_in]
            assert (((g & 0x7FFF) > 0x7F80) & ((g & 0x8000) == ((bits[nan_in] >> 16) & 0x8000))).all(), c
            total_nan += int(nan_in.sum())
    _log(f"bf16 conversion: all 2^32 fp32 patterns match the oracle codec "
         f"({total_nan} NaN inputs gave NaN of the same sign)")


def _gate_inputs():
    bits = np.arange(0, 1 << 32, 256, dtype=np.uint64).astype(np.uint32)
    z = bits.view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 88.0, -88.0, 103.0,
                        -103.0, 128.0, -128.0, 30.0, -30.0, 16.635532, -16.635532],
                       dtype=np.float32)
    return np.concatenate([z, special])


def _err(got, ref, z, scale=None):
    """Relative error against max(scale, 2^-126) (scale = |ref| unless the
    function is a cancelling difference: then the magnitude of its terms),
    less the allowance for a
    subnormal intermediate: where sigmoid(z) is below 2^-126 (z < -87.3) it
    carries an absolute rounding of up to 2^-149, which silu = z * sigmoid
    and the derivatives scale by up to 1 + |z|; that allowance is
    (1 + |z|) * 2^-148 in absolute terms. Also whether every non-finite
    reference is matched exactly (NaN for NaN)."""
    got = got.astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        fin = np.isfinite(ref)
        slack = (1.0 + np.abs(z)) * 2.0 ** -148
        excess = np.maximum(np.abs(got - ref) - slack, 0.0)
        scale = np.abs(ref) if scale is None else scale
        err = np.where(fin, excess / np.maximum(scale, 2.0 ** -126), 0.0)
        nonfin_ok = np.where(fin, True, (np.isnan(ref) & np.isnan(got)) | (got == ref))
    return err, nonfin_ok


def test_gate_functions_over_the_fp32_range(gpu):
    lib = primitives.load()
    z = _gate_inputs()
    n = z.size
    zd = torch.from_numpy(z).to(gpu)
    out = torch.empty(6 * n, dtype=torch.float32, device=gpu)
    assert lib.prim_gates(zd.data_ptr(), n, out.data_ptr(),
                          torch.cuda.current_stream(gpu).cuda_stream) == 0
    o = out.view(n, 6).cpu().numpy()
    with np.errstate(invalid="ignore", over="ignore"):
        z64 = z.astype(np.float64)
        s = scipy.special.expit(z64)
        sc = scipy.special.expit(-z64)          # 1 - sigmoid, without cancellation
        refs = {
            # the forward's lean gate: about 2^-16 relative
            "sigmoid_fast": (o[:, 0], s, 2.0 ** -16),
            "gate_fast silu": (o[:, 1], z64 * s, 2.0 ** -16),
            # the backward's gate and its derivative: a few fp32 ulp
            "gate sigmoid": (o[:, 2], s, 2.0 ** -21),
            "gate silu": (o[:, 3], z64 * s, 2.0 ** -21),
            "sigmoid'": (o[:, 4], s * sc, 2.0 ** -21),
            # silu' = s (1 + z (1 - s)) cancels near its root z = -1.2785:
            # there the error is measured against its terms, s (1 + |z (1 - s)|)
            "silu'": (o[:, 5], s * (1.0 + z64 * sc), 2.0 ** -21, s * (1.0 + np.abs(z64 * sc))),
        }
    failed = []
    for name, (got, ref, bound, *scale) in refs.items():
        err, nonfin_ok = _err(got, ref, z64, scale[0] if scale else None)
        worst = int(np.argmax(err))
        _log(f"{name}: max relative error {err.max():.3e} (2^{np.log2(max(err.max(), 1e-300)):.2f}) "
             f"at z = {z[worst]!r}; bound 2^{np.log2(bound):.0f}; non-finite matched: "
             f"{bool(nonfin_ok.all())}")
        if not (nonfin_ok.all() and err.max() <= bound):
            failed.append(name)
    assert not failed, failed
