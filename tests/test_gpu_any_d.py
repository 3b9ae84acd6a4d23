"""GPU parity for rows whose length D is not a multiple of 8.

Such rows move element by element (2-byte accesses) through the same
kernels and geometry as 16-byte rows; a lane's group of 8 is strided by the
row's lane count, so their reduction tree is D's own (still fixed by D
alone). Checked here against the CPU oracle, element by element:
- the plain, residual-copy and residual-gradient forms;
- bf16 and fp16 activations, with fp32 and 16-bit weights;
- odd row strides and bases 2 bytes off 16-byte alignment, with nothing
  written outside the row;
- anchor rows bitwise equal across batch sizes and positions;
- the two dgamma stages with partial rows padded to a multiple of 8;
- the mean as a true division: constant rows give the closed-form rstd.
The gated and fused-add forms take the same odd widths in their own test
files. Tolerances are those of the other parity tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host_bits, run_fwd_bwd
from numerics import dgamma_rel_err, f32_to_bf16_torch, max_ulp, rstd_rel_err
from synth import workloads as wl

pytestmark = pytest.mark.gpu

# One width per geometry class: 1 or 2 lanes per row, 4..32 lanes (masked),
# one wave (1..8 groups per lane), rows over 2 and 4 waves in the forward
# and over 4 waves in the backward, up to the largest row.
ODD_WIDTHS = [1, 2, 3, 5, 7, 9, 13, 15, 17, 31, 33, 63, 65, 100, 127, 129, 255, 257, 500, 513,
              1000, 1023, 1025, 2047, 2049, 3000, 4095, 4097, 4100, 5001, 8191, 8193, 8199,
              12290, 16383, 16385, 18435, 24577, 32767]


def _oracle_all(p, gres):
    y, r = oracle.fwd(p.x, p.gamma, p.zero_centered, p.eps)
    dx, dg = oracle.bwd(p.g, p.x, r, p.gamma, p.zero_centered, p.gres if gres else None)
    return {"y": y, "rstd": r, "dx": dx, "dgamma": dg}


def _assert_parity(got, ref, label):
    assert max_ulp(got["y"], ref["y"]) <= 1, label
    assert rstd_rel_err(got["rstd"], ref["rstd"]) <= 1e-6, label
    assert max_ulp(got["dx"], ref["dx"]) <= 1, label
    assert dgamma_rel_err(got["dgamma"], ref["dgamma"]) <= 1e-5, label


@pytest.mark.parametrize("D", ODD_WIDTHS)
def test_odd_widths(gpu, D):
    """Every geometry class at a T spanning several steps and a ragged
    tail, with the residual gradient; both gamma modes across the set."""
    T = 1037 if D <= 2048 else 261 if D <= 8192 else 97
    p = wl.tiny(D % 2 == 1, T=T, D=D, seed=11000 + D, with_gres=True)
    _assert_parity(run_fwd_bwd(p, True), _oracle_all(p, True), D)
    if D in (7, 100, 4100):
        _assert_parity(run_fwd_bwd(p, False), _oracle_all(p, False), (D, "no gres"))


def _strided(bits, pad_left, pad_right, fill):
    """Device bf16 [T, D] view at column pad_left of a [T, D + pads] buffer
    (row stride D + pads, base pad_left elements in), the rest `fill`."""
    T, D = bits.shape
    buf = np.full((T, D + pad_left + pad_right), fill, np.uint16)
    buf[:, pad_left:pad_left + D] = bits
    t = dev_bf16(buf)
    return t, t[:, pad_left:pad_left + D]


@pytest.mark.parametrize("D", [5, 100, 1001, 4100, 9999])
def test_odd_strides_and_offsets(gpu, D):
    """Row strides of D + 3 .. D + 7 elements and bases 2 to 6 bytes past
    a 16-byte boundary give the same bytes as packed rows, and nothing
    outside the rows is written."""
    T = 67
    p = wl.tiny(False, T=T, D=D, seed=11500 + D, with_gres=True)
    gamma = dev_f32(p.gamma)
    ref_y, ref_r = irn.rmsnorm_fwd(dev_bf16(p.x), gamma)
    ref_dx, ref_dg = irn.rmsnorm_bwd(dev_bf16(p.g), dev_bf16(p.x), ref_r, gamma,
                                     g_residual=dev_bf16(p.gres))
    sentinel = 0x7FC1  # a NaN pattern no result has
    _, x = _strided(p.x, 1, 2, 0)
    _, g = _strided(p.g, 3, 4, 0)
    _, gr = _strided(p.gres, 2, 3, 0)
    ybuf, y = _strided(np.zeros((T, D), np.uint16), 1, 4, sentinel)
    rbuf, res = _strided(np.zeros((T, D), np.uint16), 3, 2, sentinel)
    dxbuf, dx = _strided(np.zeros((T, D), np.uint16), 2, 5, sentinel)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    irn.rmsnorm_residual_fwd(x, gamma, y=y, residual_out=res, rstd=rstd)
    dg = torch.empty(D, dtype=torch.float32, device="cuda")
    irn.rmsnorm_bwd(g, x, rstd, gamma, g_residual=gr, dx=dx, dgamma=dg)
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(rstd, ref_r)
    assert np.array_equal(host_bits(res), p.x)
    assert torch.equal(dx, ref_dx) and torch.equal(dg, ref_dg)
    for buf, left in ((ybuf, 1), (rbuf, 3), (dxbuf, 2)):
        b = host_bits(buf)
        assert np.all(b[:, :left] == sentinel) and np.all(b[:, left + D:] == sentinel)


@pytest.mark.parametrize("D", [3, 100, 4100, 12290])
def test_odd_rows_across_batches(gpu, D):
    """An anchor row's y, rstd and dx are bitwise the same in batches of
    1, 2, 17 and 300 rows, first, in the middle and last."""
    fill = wl.tiny(False, T=300, D=D, seed=11600 + D)
    anchor = wl.tiny(False, T=1, D=D, seed=11700 + D)
    gamma = dev_f32(fill.gamma)

    def run(xb, gb):
        x, g = dev_bf16(xb), dev_bf16(gb)
        y, r = irn.rmsnorm_fwd(x, gamma)
        dx, _ = irn.rmsnorm_bwd(g, x, r, gamma, want_dgamma=False)
        return host_bits(y), r.cpu().numpy(), host_bits(dx)

    y1, r1, dx1 = run(anchor.x, anchor.g)
    for M in (1, 2, 17, 300):
        for pos in sorted({0, M // 2, M - 1}):
            xb, gb = fill.x[:M].copy(), fill.g[:M].copy()
            xb[pos], gb[pos] = anchor.x[0], anchor.g[0]
            y, r, dx = run(xb, gb)
            assert np.array_equal(y[pos], y1[0]), (M, pos)
            assert r[pos].view(np.uint32) == r1[0].view(np.uint32), (M, pos)
            assert np.array_equal(dx[pos], dx1[0]), (M, pos)


def test_constant_rows_divide_by_D(gpu):
    """At eps = 0 a constant row c has ss = D c^2 exactly and rstd = 1/|c|
    rounded once; at D = 7, 12, 100 and 4100 a multiplication by the rounded
    1/D would give a different rstd for several of these c."""
    cs = np.array([5.0, 7.0, 11.0, 1.25, 1.75, 2.5, 15.0, 0.625], np.float32)
    for D in (7, 12, 100, 4100):
        x = f32_to_bf16_torch(np.repeat(np.concatenate([cs, -cs])[:, None], D, axis=1))
        _, r = irn.rmsnorm_fwd(dev_bf16(x), torch.ones(D, device="cuda"), eps=0.0)
        want = np.float32(1.0) / np.concatenate([cs, cs]).astype(np.float64)
        assert np.array_equal(r.cpu().numpy(), want.astype(np.float32)), D


ACT = {"bf16": (torch.bfloat16, oracle.BF16), "f16": (torch.float16, oracle.F16)}
WEIGHT = {"f32": (torch.float32, oracle.F32), "bf16": (torch.bfloat16, oracle.BF16),
          "f16": (torch.float16, oracle.F16)}


def _bits(seed, stream, T, D, act):
    v = synth.normal_f32(seed, stream, T * D, 0.0, 1.0).reshape(T, D)
    return torch.from_numpy(v).to(ACT[act][0]).view(torch.int16).numpy().view(np.uint16)


def _dev(bits, act):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(ACT[act][0]).cuda()


@pytest.mark.parametrize("act,wt", [("f16", "f32"), ("f16", "bf16"), ("bf16", "f16"),
                                    ("f16", "f16")])
@pytest.mark.parametrize("D", [5, 100, 4100, 12290])
def test_odd_widths_storage_types(gpu, act, wt, D):
    T = 301 if D <= 4100 else 61
    zc = D % 2 == 0
    x, g, gr = (_bits(11800 + D, s, T, D, act) for s in (1, 2, 4))
    w = torch.from_numpy(wl.gamma_for(11800 + D, D, zc)).to(WEIGHT[wt][0])
    stored = w.numpy() if wt == "f32" else w.view(torch.int16).numpy().view(np.uint16)
    y, r = irn.rmsnorm_fwd_dt(_dev(x, act), w.cuda(), zc, 1e-6)
    dx, dg = irn.rmsnorm_bwd_dt(_dev(g, act), _dev(x, act), r, w.cuda(), zc, g_residual=_dev(gr, act))
    torch.cuda.synchronize()
    a_o, w_o = ACT[act][1], WEIGHT[wt][1]
    ry, rr = oracle.fwd_dt(x, stored, zc, 1e-6, a_o, w_o)
    rdx, rdg = oracle.bwd_dt(g, x, rr, stored, zc, gres=gr, act_dtype=a_o, weight_dtype=w_o)
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert max_ulp(host(y), ry) <= 1
    assert rstd_rel_err(r.cpu().numpy(), rr) <= 1e-6
    assert max_ulp(host(dx), rdx) <= 1
    assert dgamma_rel_err(dg.cpu().numpy(), rdg) <= 1e-5


@pytest.mark.parametrize("D", [13, 100, 4100])
def test_odd_backward_stages_and_padded_partials(gpu, D):
    """bwd == bwd_rows + bwd_finish bitwise; chunk partial rows are D
    rounded up to a multiple of 8 floats, the padding columns zero, and
    the partials add up to dgamma."""
    p = wl.tiny(False, T=3000, D=D, seed=11900 + D)
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    _, r = irn.rmsnorm_fwd(x, gamma)
    dx, dg = irn.rmsnorm_bwd(g, x, r, gamma)
    ws, nbytes = irn.workspace_for(p.T, D, "cuda")
    Dp = -(-D // 8) * 8
    _, _, K = irn.rmsnorm_bwd_partials_layout(p.T, D)
    assert nbytes == K * Dp * 4
    dx2 = torch.empty_like(dx)
    irn.rmsnorm_bwd_rows(g, x, r, gamma, dx=dx2, workspace=ws)
    dg2 = torch.empty_like(dg)
    irn.rmsnorm_bwd_finish(ws, p.T, D, dg2)
    assert torch.equal(dx, dx2) and torch.equal(dg, dg2)
    part = ws[: K * Dp].view(K, Dp).double().cpu().numpy()
    assert np.all(part[:, D:] == 0)
    ref_dg = oracle.dgamma(p.g, p.x, oracle.fwd(p.x, p.gamma)[1])
    assert dgamma_rel_err(part[:, :D].sum(axis=0), ref_dg) <= 1e-5
    assert dgamma_rel_err(dg.cpu().numpy(), ref_dg) <= 1e-5
