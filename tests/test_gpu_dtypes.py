"""GPU parity of the storage-type entry points (rmsnorm_fwd_dt,
rmsnorm_bwd_dt) against the CPU oracle's _dt forms: fp16 activations and
bf16 / fp16 / fp32 weights.

Sources: RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA kernel"
(fp16 is checked beside bf16); Megatron-LM PR "Fix the batch-invariant
RMSNorm forward and its input gradient", item 1 (the weight is cast to fp32,
then offset). Tolerances: y and dx <= 1 ulp of their storage type (ordered
integers of the bits), rstd <= 1e-6 relative, dgamma <= 1e-5 relative in the
infinity norm.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from numerics import dgamma_rel_err, max_ulp, rstd_rel_err
from synth import workloads as wl

pytestmark = pytest.mark.gpu

ACT = {"bf16": (torch.bfloat16, oracle.BF16), "f16": (torch.float16, oracle.F16)}
WEIGHT = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16),
          "f16": (torch.float16, oracle.F16)}


def _act_bits(seed, stream, T, D, act, scale=1.0):
    """Seeded N(0, scale^2) activations stored as `act`, as 16-bit patterns."""
    v = synth.normal_f32(seed, stream, T * D, 0.0, scale).reshape(T, D)
    t = torch.from_numpy(v).to(ACT[act][0])
    return t.view(torch.int16).numpy().view(np.uint16)


def _dev(bits, act):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(ACT[act][0]).cuda()


def _host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _weights(seed, D, zc, wt):
    w32 = wl.gamma_for(seed, D, zc)
    t = torch.from_numpy(w32).to(WEIGHT[wt][0])
    stored = t.numpy() if wt == "f32" else t.view(torch.int16).numpy().view(np.uint16)
    return t.cuda(), stored


def _check(act, wt, T, D, zc, with_gres, seed):
    x = _act_bits(seed, 1, T, D, act)
    g = _act_bits(seed, 2, T, D, act)
    gr = _act_bits(seed, 4, T, D, act) if with_gres else None
    gamma, gstored = _weights(seed, D, zc, wt)
    y, r = irn.rmsnorm_fwd_dt(_dev(x, act), gamma, zc, 1e-6)
    dx, dg = irn.rmsnorm_bwd_dt(_dev(g, act), _dev(x, act), r, gamma, zc,
                                g_residual=None if gr is None else _dev(gr, act))
    torch.cuda.synchronize()
    a_o, w_o = ACT[act][1], WEIGHT[wt][1]
    ry, rr = oracle.fwd_dt(x, gstored, zc, 1e-6, a_o, w_o)
    rdx, rdg = oracle.bwd_dt(g, x, rr, gstored, zc, gres=gr, act_dtype=a_o, weight_dtype=w_o)
    label = (act, wt, T, D, zc, with_gres)
    assert max_ulp(_host(y), ry) <= 1, label
    assert rstd_rel_err(r.cpu().numpy(), rr) <= 1e-6, label
    assert max_ulp(_host(dx), rdx) <= 1, label
    assert dgamma_rel_err(dg.cpu().numpy(), rdg) <= 1e-5, label
    return y, r, dx, dg


@pytest.mark.parametrize("wt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("zc", [False, True])
def test_dtypes_small(gpu, act, wt, zc):
    _check(act, wt, 37, 4096, zc, True, 1700)


@pytest.mark.parametrize("D", [8, 24, 128, 136, 1024, 2048, 4104, 8192, 12288, 32768])
def test_f16_widths(gpu, D):
    T = 1037 if D <= 2048 else 97
    _check("f16", "bf16" if D % 16 else "f32", T, D, D % 16 == 8, True, 1710 + D)


@pytest.mark.parametrize("T", [1, 2, 63, 65, 513])
def test_f16_ragged_batches(gpu, T):
    _check("f16", "f16", T, 2048, False, False, 1720 + T)


def test_16bit_weights_equal_fp32_weights_bitwise(gpu):
    """A bf16 / fp16 weight gives the same bytes as its exact fp32 value."""
    D, T = 4096, 100
    x = _dev(_act_bits(1730, 1, T, D, "bf16"), "bf16")
    g = _dev(_act_bits(1730, 2, T, D, "bf16"), "bf16")
    for wt in ("bf16", "f16"):
        w16, _ = _weights(1730, D, True, wt)
        w32 = w16.float()
        y16, r16 = irn.rmsnorm_fwd_dt(x, w16, True)
        y32, r32 = irn.rmsnorm_fwd(x, w32, True)
        assert torch.equal(y16, y32) and torch.equal(r16, r32)
        dx16, dg16 = irn.rmsnorm_bwd_dt(g, x, r16, w16, True)
        dx32, dg32 = irn.rmsnorm_bwd(g, x, r32, w32, True)
        assert torch.equal(dx16, dx32) and torch.equal(dg16, dg32)


def test_f16_overflow_and_subnormal_outputs(gpu):
    """|y| past 65504 becomes infinity; tiny results stay fp16 subnormals."""
    D = 256
    x = torch.full((2, D), 2.0, dtype=torch.float16, device="cuda")
    x[1, ::2] = -2.0
    big = torch.full((D,), 70000.0, device="cuda")
    y, r = irn.rmsnorm_fwd_dt(x, big, eps=0.0)
    assert torch.all(torch.isinf(y)) and torch.equal(torch.sign(y), torch.sign(x))
    tiny = torch.full((D,), 2.0 ** -20, device="cuda")
    y, _ = irn.rmsnorm_fwd_dt(x, tiny, eps=0.0)
    assert torch.equal(y.float(), torch.sign(x).float() * 2.0 ** -20)  # 2^-20 is subnormal in fp16


def test_f16_rows_across_batches(gpu):
    D, T = 2048, 300
    x = _dev(_act_bits(1740, 1, T, D, "f16"), "f16")
    g = _dev(_act_bits(1740, 2, T, D, "f16"), "f16")
    gamma, _ = _weights(1740, D, False, "f16")
    y, r = irn.rmsnorm_fwd_dt(x, gamma)
    dx, _ = irn.rmsnorm_bwd_dt(g, x, r, gamma, want_dgamma=False)
    for a, b in ((0, 1), (7, 8), (3, 70), (299, 300), (100, 300)):
        ys, rs = irn.rmsnorm_fwd_dt(x[a:b], gamma)
        dxs, _ = irn.rmsnorm_bwd_dt(g[a:b], x[a:b], rs, gamma, want_dgamma=False)
        assert torch.equal(ys, y[a:b]) and torch.equal(rs, r[a:b]) and torch.equal(dxs, dx[a:b])


@pytest.mark.slow
def test_f16_full_size(gpu):
    """T = 32768, D = 4096 in fp16 with fp16 weights: every element."""
    _check("f16", "f16", 32768, 4096, False, True, 1750)
