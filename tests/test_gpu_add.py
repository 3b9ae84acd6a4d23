"""GPU parity of the fused add-norm (rmsnorm_add_fwd / rmsnorm_add_bwd)
against the CPU oracle, through the C-ABI.

The form is RL-Kernel PR "C1: zero-centred RMSNorm references and CUDA
kernel", decoder-norm note: the fused add normalises the fp32 sum
h = x + residual and carries the updated residual forward. Tolerances as for
the plain norm: y and dh <= 1 bf16 ulp, rstd <= 1e-6 relative, dgamma
<= 1e-5 relative in the infinity norm; the updated residual bf16(h) is
computed identically on both sides and must match bitwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
from gpu_util import dev_bf16, dev_f32, host_bits
from numerics import dgamma_rel_err, max_ulp, rstd_rel_err, ulp_distance
from synth import workloads as wl

pytestmark = pytest.mark.gpu

WIDTHS = [8, 16, 24, 64, 96, 128, 136, 256, 520, 1024, 2048, 2560, 4096, 4104, 5120, 8192,
          8200, 12288, 16384, 20480, 32768]
# not multiples of 8: element-wise rows
WIDTHS += [3, 13, 100, 1001, 4100, 12290, 20003]
# no lane lacking its last group: 14 and 16 vectors per lane
WIDTHS += [28671, 32767]


def _run(p, with_gro, zc=None):
    zc = p.zero_centered if zc is None else zc
    x, res, g, gamma = dev_bf16(p.x), dev_bf16(p.residual), dev_bf16(p.g), dev_f32(p.gamma)
    gro = dev_bf16(p.gres) if with_gro else None
    y, rout, rstd = irn.rmsnorm_add_fwd(x, res, gamma, zc, p.eps)
    dh, dg = irn.rmsnorm_add_bwd(g, x, res, rstd, gamma, zc, g_residual_out=gro)
    torch.cuda.synchronize()
    return {"y": host_bits(y), "rout": host_bits(rout), "rstd": rstd.cpu().numpy(),
            "dh": host_bits(dh), "dgamma": dg.cpu().numpy()}


def _oracle(p, with_gro, zc=None):
    zc = p.zero_centered if zc is None else zc
    y, rout, r = oracle.add_fwd(p.x, p.residual, p.gamma, zc, p.eps)
    dh, dg = oracle.add_bwd(p.g, p.x, p.residual, r, p.gamma, zc,
                            g_rout=p.gres if with_gro else None)
    return {"y": y, "rout": rout, "rstd": r, "dh": dh, "dgamma": dg}


def _assert_parity(got, ref, label):
    assert np.array_equal(got["rout"], ref["rout"]), label
    assert max_ulp(got["y"], ref["y"]) <= 1, label
    assert rstd_rel_err(got["rstd"], ref["rstd"]) <= 1e-6, label
    assert max_ulp(got["dh"], ref["dh"]) <= 1, label
    assert dgamma_rel_err(got["dgamma"], ref["dgamma"]) <= 1e-5, label


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("with_gro", [False, True])
def test_add_tiny_fixture(gpu, zc, with_gro):
    p = wl.tiny(zc, with_gres=True, with_residual=True)
    _assert_parity(_run(p, with_gro), _oracle(p, with_gro), (zc, with_gro))


@pytest.mark.parametrize("D", WIDTHS)
def test_add_widths(gpu, D):
    """Every geometry class at a T spanning several steps plus a ragged tail."""
    T = 1037 if D <= 2048 else 261 if D <= 8192 else 97
    p = wl.tiny(D % 16 == 8, T=T, D=D, seed=8500 + D, with_gres=True, with_residual=True)
    _assert_parity(_run(p, True), _oracle(p, True), D)


@pytest.mark.parametrize("D", [128, 4096])
@pytest.mark.parametrize("T", [1, 2, 5, 63, 65, 513, 2049])
def test_add_ragged_batches(gpu, D, T):
    p = wl.tiny(False, T=T, D=D, seed=8600 + T, with_gres=True, with_residual=True)
    _assert_parity(_run(p, False), _oracle(p, False), (T, D))


def test_add_edge_rows(gpu):
    """A cancelled row (residual = -x), an all-zero row, rows whose sum
    overflows to infinity, a NaN input and large-magnitude rows: the same
    IEEE outcomes as the oracle (NaN where the oracle has NaN)."""
    D = 256
    p = wl.tiny(False, T=12, D=D, seed=8700, with_gres=True, with_residual=True)
    x, res = p.x.copy(), p.residual.copy()
    res[0] = x[0] ^ np.uint16(0x8000)        # h = 0
    x[1] = 0
    res[1] = 0                               # zero row
    x[2, :] = 0x7F00                         # 1.7e38 + 1.7e38 overflows
    res[2, :] = 0x7F00
    x[3, 5] = 0x7FC0                         # NaN
    x[4] = (x[4] & np.uint16(0x807F)) | np.uint16(0x5F00)   # |x| ~ 2^63
    p.x, p.residual = x, res
    got, ref = _run(p, True), _oracle(p, True)
    assert np.array_equal(got["rout"], ref["rout"])
    for k in ("y", "dh"):
        assert ulp_distance(got[k], ref[k]).max() <= 1, k
    rr, gr = ref["rstd"], got["rstd"]
    assert np.array_equal(np.isnan(rr), np.isnan(gr))
    fin = np.isfinite(rr)
    assert rstd_rel_err(gr[fin], rr[fin]) <= 1e-6
    assert np.array_equal(gr[~fin], rr[~fin]) or np.all(np.isnan(rr[~fin]))


@pytest.mark.parametrize("D", [4096, 4100, 13])
def test_add_in_place(gpu, D):
    """y = x and residual_out = residual in place give the out-of-place bytes."""
    p = wl.tiny(True, T=777, D=D, seed=8800 + D, with_residual=True)
    x, res, gamma = dev_bf16(p.x), dev_bf16(p.residual), dev_f32(p.gamma)
    y0, rout0, r0 = irn.rmsnorm_add_fwd(x, res, gamma, True, p.eps)
    x2, res2 = x.clone(), res.clone()
    y, rout, r = irn.rmsnorm_add_fwd(x2, res2, gamma, True, p.eps, y=x2, residual_out=res2)
    torch.cuda.synchronize()
    assert y.data_ptr() == x2.data_ptr() and rout.data_ptr() == res2.data_ptr()
    assert torch.equal(x2, y0) and torch.equal(res2, rout0) and torch.equal(r, r0)
    # only one of the two in place
    x3, res3 = x.clone(), res.clone()
    irn.rmsnorm_add_fwd(x3, res3, gamma, True, p.eps, residual_out=res3)
    torch.cuda.synchronize()
    assert torch.equal(res3, rout0) and torch.equal(x3, x)


def test_add_backward_stages(gpu):
    """add_bwd == add_bwd_rows + bwd_finish bitwise; the chunk partials add
    up to dgamma."""
    p = wl.tiny(False, T=3000, D=1024, seed=8900, with_gres=True, with_residual=True)
    x, res, g, gamma = dev_bf16(p.x), dev_bf16(p.residual), dev_bf16(p.g), dev_f32(p.gamma)
    gro = dev_bf16(p.gres)
    _, _, r = irn.rmsnorm_add_fwd(x, res, gamma)
    dh, dg = irn.rmsnorm_add_bwd(g, x, res, r, gamma, g_residual_out=gro)
    ws, _ = irn.workspace_for(p.T, p.D, "cuda")
    dh2 = torch.empty_like(dh)
    irn.rmsnorm_add_bwd_rows(g, x, res, r, gamma, g_residual_out=gro, dh=dh2, workspace=ws)
    dg2 = torch.empty_like(dg)
    irn.rmsnorm_bwd_finish(ws, p.T, p.D, dg2)
    assert torch.equal(dh, dh2) and torch.equal(dg, dg2)
    dh_only, none = irn.rmsnorm_add_bwd(g, x, res, r, gamma, g_residual_out=gro,
                                        want_dgamma=False)
    none2, dg_only = irn.rmsnorm_add_bwd(g, x, res, r, gamma, want_dh=False)
    assert none is None and none2 is None
    assert torch.equal(dh_only, dh) and torch.equal(dg_only, dg)


def test_add_rows_across_batches(gpu):
    """A row's y, residual_out, rstd and dh do not depend on the batch."""
    p = wl.tiny(False, T=1024, D=2048, seed=9900, with_gres=True, with_residual=True)
    x, res, g, gamma = dev_bf16(p.x), dev_bf16(p.residual), dev_bf16(p.g), dev_f32(p.gamma)
    gro = dev_bf16(p.gres)

    def run(a, b):
        y, ro, r = irn.rmsnorm_add_fwd(x[a:b], res[a:b], gamma)
        dh, _ = irn.rmsnorm_add_bwd(g[a:b], x[a:b], res[a:b], r, gamma,
                                    g_residual_out=gro[a:b], want_dgamma=False)
        return [host_bits(y), host_bits(ro), r.cpu().numpy(), host_bits(dh)]

    full = run(0, 1024)
    for a, b in ((0, 1), (5, 6), (3, 36), (1000, 1024), (7, 1007), (511, 1024)):
        part = run(a, b)
        for u, v in zip(part, full):
            assert u.tobytes() == v[a:b].tobytes(), (a, b)
    # a row inside a padded batch (zero rows appended)
    xp = torch.cat([x[:17], torch.zeros_like(x[:5])])
    rp = torch.cat([res[:17], torch.zeros_like(res[:5])])
    y, ro, r = irn.rmsnorm_add_fwd(xp, rp, gamma)
    assert host_bits(y[:17]).tobytes() == full[0][:17].tobytes()
    assert r[:17].cpu().numpy().tobytes() == full[2][:17].tobytes()


def test_add_strided_inputs(gpu):
    """Row strides wider than D give the packed result."""
    p = wl.tiny(False, T=100, D=1024, seed=9901, with_residual=True)
    x, res, gamma = dev_bf16(p.x), dev_bf16(p.residual), dev_f32(p.gamma)
    wide = torch.zeros((100, 1536), dtype=torch.bfloat16, device="cuda")
    wide[:, 256:1280] = res
    y0, ro0, r0 = irn.rmsnorm_add_fwd(x, res, gamma)
    y1, ro1, r1 = irn.rmsnorm_add_fwd(x, wide[:, 256:1280], gamma)
    assert torch.equal(y0, y1) and torch.equal(ro0, ro1) and torch.equal(r0, r1)


@pytest.mark.slow
def test_add_full_size(gpu):
    """The fused add workload at T=32768, D=4096: every element."""
    p = wl.fused_add()
    got = _run(p, True)
    ref = _oracle(p, True)
    print(f"fused add: y {(got['y'] != ref['y']).sum()}, dh {(got['dh'] != ref['dh']).sum()} "
          f"of {got['y'].size} elements differ", flush=True)
    _assert_parity(got, ref, "full")
