"""GPU parity: the HIP library (through its C-ABI) against the CPU oracle,
element by element, on seeded inputs small enough for the oracle.

Tolerances: y / gated out <= 1 bf16 ulp, rstd <= 1e-6 relative,
dx <= 1 bf16 ulp (with the cancellation rule in numerics.py), dgamma <= 1e-5
relative in the infinity norm. Exact-arithmetic inputs must match bitwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host_bits, run_fwd_bwd
from numerics import (bf16_to_f32, bf16_to_f64, dgamma_check, dgamma_rel_err,
                      dgamma_term_stats, dgamma_terms_f32, f32_to_bf16_torch, max_ulp,
                      rstd_rel_err)
from synth import workloads as wl

pytestmark = pytest.mark.gpu


def oracle_all(p, gres=False):
    y, r = oracle.fwd(p.x, p.gamma, p.zero_centered, p.eps)
    out = {"y": y, "rstd": r}
    if p.g is not None:
        dx, dg = oracle.bwd(p.g, p.x, r, p.gamma, p.zero_centered, p.gres if gres else None)
        out["dx"], out["dgamma"] = dx, dg
    return out


def assert_parity(p, got, ref, gres=False, label=""):
    assert max_ulp(got["y"], ref["y"]) <= 1, label
    assert rstd_rel_err(got["rstd"], ref["rstd"]) <= 1e-6, label
    if "dx" in ref:
        assert max_ulp(got["dx"], ref["dx"]) <= 1, label
        assert dgamma_rel_err(got["dgamma"], ref["dgamma"]) <= 1e-5, label


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("gres", [False, True])
def test_tiny_fixture(gpu, zc, gres):
    p = wl.tiny(zc, with_gres=True)
    assert_parity(p, run_fwd_bwd(p, gres), oracle_all(p, gres), gres, p.name)


@pytest.mark.parametrize("T", [1, 7, 16])
@pytest.mark.parametrize("D", [128, 4096])
@pytest.mark.parametrize("zc", [False, True])
def test_token_and_width_grid(gpu, T, D, zc):
    p = wl.tiny(zc, T=T, D=D, seed=7000 + T + D, with_gres=True)
    for gres in (False, True):
        assert_parity(p, run_fwd_bwd(p, gres), oracle_all(p, gres), gres, (T, D, zc, gres))


WIDTHS = [8, 16, 24, 40, 64, 96, 128, 136, 256, 264, 384, 512, 520, 1024, 1536, 2048, 2560,
          3072, 4096, 4104, 5120, 6144, 7168, 8192,
          # rows over 2 waves (8192 < D <= 16384) and 4 waves (D <= 32768)
          8200, 9216, 12288, 16384, 16392, 18432, 20480, 24576, 28680, 32768]


@pytest.mark.parametrize("D", WIDTHS)
def test_widths(gpu, D):
    """Every geometry class (lanes per row 1..64 in one wave, 128 and 256
    over 2 and 4 waves; 1..16 vectors per lane, masked and unmasked) at a T
    spanning several steps plus a ragged tail."""
    T = 1037 if D <= 2048 else 261 if D <= 8192 else 97
    p = wl.tiny(D % 16 == 8, T=T, D=D, seed=8000 + D, with_gres=True)
    assert_parity(p, run_fwd_bwd(p, True), oracle_all(p, True), True, D)


@pytest.mark.parametrize("D", [16392, 18432, 20480, 24576, 28680, 32768])
def test_long_rows_without_residual_gradient(gpu, D):
    """Rows over 4 waves past the two-set pipeline (9 to 16 vectors per
    lane: the next row loaded into the registers the second pass frees),
    plain backward, 66 chunks of up to 4 row steps each."""
    p = wl.tiny(D % 16 == 8, T=261, D=D, seed=8500 + D)
    assert_parity(p, run_fwd_bwd(p, False), oracle_all(p, False), False, D)


@pytest.mark.parametrize("D", [128, 4096])
@pytest.mark.parametrize("T", [2, 3, 4, 5, 31, 63, 64, 65, 127, 129, 511, 513, 2049])
def test_ragged_batches(gpu, D, T):
    p = wl.tiny(False, T=T, D=D, seed=9000 + T)
    assert_parity(p, run_fwd_bwd(p), oracle_all(p), False, (T, D))


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("D", [128, 2048, 4096])
def test_residual_forward(gpu, zc, D):
    p = wl.tiny(zc, T=77, D=D, seed=9100 + D)
    x, gamma = dev_bf16(p.x), dev_f32(p.gamma)
    y, res, rstd = irn.rmsnorm_residual_fwd(x, gamma, zc, p.eps)
    ry, rres, rr = oracle.residual_fwd(p.x, p.gamma, zc, p.eps)
    assert np.array_equal(host_bits(res), p.x)  # byte copy
    assert max_ulp(host_bits(y), ry) <= 1
    assert rstd_rel_err(rstd.cpu().numpy(), rr) <= 1e-6
    y2, r2 = irn.rmsnorm_fwd(x, gamma, zc, p.eps)
    assert torch.equal(y, y2) and torch.equal(rstd, r2)


@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("D", [64, 128, 256, 4096])
def test_gated_forward(gpu, zc, D):
    p = wl.tiny(zc, T=300, D=D, seed=9200 + D, with_gate=True)
    out, rstd = irn.rmsnorm_gated_fwd(dev_bf16(p.x), dev_bf16(p.z), dev_f32(p.gamma), zc, p.eps,
                                      want_rstd=True)
    ro, rr = oracle.gated_fwd(p.x, p.z, p.gamma, zc, p.eps)
    assert max_ulp(host_bits(out), ro) <= 1
    assert rstd_rel_err(rstd.cpu().numpy(), rr) <= 1e-6


def test_gated_special_gates(gpu):
    """z = 0 gives +-0 and z = 32 gives exactly 32 * the plain output."""
    p = wl.tiny(False, T=64, D=128, seed=9300)
    x, gamma = dev_bf16(p.x), dev_f32(p.gamma)
    y, _ = irn.rmsnorm_fwd(x, gamma)
    z0 = torch.zeros_like(x)
    out0, _ = irn.rmsnorm_gated_fwd(x, z0, gamma)
    assert torch.all(out0.float() == 0)
    out32, _ = irn.rmsnorm_gated_fwd(x, torch.full_like(x, 32.0), gamma)
    assert torch.equal(out32.float(), 32.0 * y.float())


def _edge_rows(D, rng):
    bmax = f32_to_bf16_torch(np.array([3.3895314e38], np.float32))[0]
    sub = np.uint16(0x0001)
    rows = [
        np.zeros(D, np.uint16),                                      # zero row
        np.full(D, 0x8000, np.uint16),                               # -0 row
        f32_to_bf16_torch(50.0 * rng.standard_normal(D).astype(np.float32)),  # outliers
        np.where(rng.random(D) < 0.5, bmax, bmax | 0x8000).astype(np.uint16),  # +-bf16 max
        np.where(rng.random(D) < 0.5, sub, sub | 0x8000).astype(np.uint16),    # subnormals
        f32_to_bf16_torch((1e-20 * rng.standard_normal(D)).astype(np.float32)),  # tiny normals
        f32_to_bf16_torch(np.where(np.arange(D) == 3, 1.0, 0.0).astype(np.float32)),  # one-hot
    ]
    inf_row = f32_to_bf16_torch(rng.standard_normal(D).astype(np.float32))
    inf_row[5] = 0x7F80
    nan_row = f32_to_bf16_torch(rng.standard_normal(D).astype(np.float32))
    nan_row[7] = 0x7FC0
    rows += [inf_row, nan_row]
    return np.stack(rows)


def _edge_dgamma_ok(gpu_dg, p, rstd_ref, label):
    """dgamma of an edge batch under the shared rule (numerics.dgamma_check);
    the terms are fp32((g*x)*r) per row, rounded as both sides round them."""
    ref = oracle.dgamma(p.g, p.x, rstd_ref)
    mag, nonfinite = dgamma_term_stats(
        dgamma_terms_f32(bf16_to_f32(p.g), bf16_to_f32(p.x), rstd_ref))
    ok, report = dgamma_check(gpu_dg, ref, mag, nonfinite, p.T + 512)
    print(f"edge dgamma {label}: {report}", flush=True)
    assert ok, (label, report)


@pytest.mark.parametrize("D", [128, 4096])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_edge_values(gpu, D, eps):
    rng = np.random.default_rng(D)
    x = _edge_rows(D, rng)
    T = x.shape[0]
    g = synth.normal_bf16(9400, 2, T, D)
    gamma = wl.gamma_for(9400, D, False)
    p = wl.Problem("edge", T, D, eps, False, gamma, x, g)
    got, ref = run_fwd_bwd(p), oracle_all(p)
    assert max_ulp(got["y"], ref["y"]) <= 1
    assert rstd_rel_err(got["rstd"], ref["rstd"]) <= 1e-6
    # dx within 1 ulp; NaN/inf positions must agree exactly
    assert max_ulp(got["dx"], ref["dx"]) <= 1
    nan_g = np.isnan(bf16_to_f64(got["dx"]))
    nan_r = np.isnan(bf16_to_f64(ref["dx"]))
    assert np.array_equal(nan_g, nan_r)
    # dgamma over all edge rows (the NaN row makes every column NaN; with
    # eps = 0 the zero rows do too), then over the rows without a NaN input
    _edge_dgamma_ok(got["dgamma"], p, ref["rstd"], (D, eps, "all rows"))
    finite = np.array([not np.isnan(bf16_to_f64(r)).any() for r in x])
    q = wl.Problem("edge-finite", int(finite.sum()), D, eps, False, gamma, x[finite], g[finite])
    _edge_dgamma_ok(run_fwd_bwd(q)["dgamma"], q, oracle_all(q)["rstd"], (D, eps, "finite rows"))


@pytest.mark.parametrize("D", [128, 4096])
def test_dgamma_partial_overflow(gpu, D):
    """dgamma terms of +-2^126 that cancel: 64 rows of x = 1 carry g = +2^126
    and 64 more g = -2^126 in their first 2 columns (N(0,1) elsewhere), among
    N(0,1) rows. The oracle's double sum of those columns is small and finite;
    an fp32 running sum passes FLT_MAX after four such terms, so the GPU's
    chunk partials may overflow there. Checked under the shared overflow
    rule; y, rstd and dx (no sums across rows) against the oracle as usual."""
    rng = np.random.default_rng(9450 + D)
    T = 600
    xf = rng.standard_normal((T, D)).astype(np.float32)
    gf = rng.standard_normal((T, D)).astype(np.float32)
    rows = rng.permutation(T)[:128]
    xf[rows] = 1.0
    gf[rows[:64], :2] = 2.0 ** 126
    gf[rows[64:], :2] = -(2.0 ** 126)
    x, g = f32_to_bf16_torch(xf), f32_to_bf16_torch(gf)
    gamma = wl.gamma_for(9450, D, False)
    p = wl.Problem("huge-g", T, D, 1e-6, False, gamma, x, g)
    got, ref = run_fwd_bwd(p), oracle_all(p)
    assert max_ulp(got["y"], ref["y"]) <= 1
    assert rstd_rel_err(got["rstd"], ref["rstd"]) <= 1e-6
    assert max_ulp(got["dx"], ref["dx"]) <= 1
    assert np.isfinite(ref["dgamma"][:2]).all()   # the double sums stay finite
    _edge_dgamma_ok(got["dgamma"], p, ref["rstd"], (D, "huge g"))


def _exact_problem(T, D, seed, zc):
    """Dyadic inputs for which every sum is exact in any order (eps = 0):
    row t has |x| = 2^k_t, g in {j/8}, w_eff in {m/16}."""
    rng = np.random.default_rng(seed)
    k = rng.integers(-3, 4, size=T)
    sign = np.where(rng.random((T, D)) < 0.5, -1.0, 1.0)
    x = f32_to_bf16_torch((sign * 2.0 ** k[:, None]).astype(np.float32))
    g = f32_to_bf16_torch((rng.integers(-16, 17, size=(T, D)) / 8.0).astype(np.float32))
    w = rng.integers(8, 25, size=D) / 16.0
    gamma = (w - 1.0 if zc else w).astype(np.float32)
    return wl.Problem("exact", T, D, 0.0, zc, gamma, x, g,
                      gres=f32_to_bf16_torch((rng.integers(-8, 9, size=(T, D)) / 8.0)
                                             .astype(np.float32)))


@pytest.mark.parametrize("D", [8, 128, 2048, 4096, 8192, 16384, 32768])
@pytest.mark.parametrize("zc", [False, True])
def test_exact_arithmetic_bitwise(gpu, D, zc):
    p = _exact_problem(301, D, D + zc, zc)
    for gres in (False, True):
        got, ref = run_fwd_bwd(p, gres), oracle_all(p, gres)
        assert np.array_equal(got["y"], ref["y"])
        assert np.array_equal(got["rstd"].view(np.uint32), ref["rstd"].view(np.uint32))
        assert np.array_equal(got["dx"], ref["dx"])
        assert np.array_equal(got["dgamma"].view(np.uint32), ref["dgamma"].view(np.uint32))


def test_zero_centered_gamma0_equals_plain_gamma1(gpu):
    p = wl.tiny(False, T=99, D=4096, seed=9500, with_gres=True)
    x, g, gr = dev_bf16(p.x), dev_bf16(p.g), dev_bf16(p.gres)
    zero = torch.zeros(4096, device="cuda")
    one = torch.ones(4096, device="cuda")
    ya, ra = irn.rmsnorm_fwd(x, zero, True)
    yb, rb = irn.rmsnorm_fwd(x, one, False)
    assert torch.equal(ya, yb) and torch.equal(ra, rb)
    dxa, dga = irn.rmsnorm_bwd(g, x, ra, zero, True, g_residual=gr)
    dxb, dgb = irn.rmsnorm_bwd(g, x, rb, one, False, g_residual=gr)
    assert torch.equal(dxa, dxb) and torch.equal(dga, dgb)


def test_zero_weight_gives_zero(gpu):
    p = wl.tiny(False, T=50, D=2048, seed=9600)
    x, g = dev_bf16(p.x), dev_bf16(p.g)
    zero = torch.zeros(2048, device="cuda")
    y, r = irn.rmsnorm_fwd(x, zero)
    dx, _ = irn.rmsnorm_bwd(g, x, r, zero)
    assert torch.all(y.float() == 0) and torch.all(dx.float() == 0)


@pytest.mark.parametrize("D", [128, 4096])
def test_backward_stages_and_partials(gpu, D):
    """bwd == bwd_rows + bwd_finish bitwise; the per-chunk partials add up to
    dgamma; a single row's dgamma is the one rounded term."""
    p = wl.tiny(False, T=3000, D=D, seed=9700 + D)
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    _, r = irn.rmsnorm_fwd(x, gamma)
    dx, dg = irn.rmsnorm_bwd(g, x, r, gamma)
    ws, _ = irn.workspace_for(p.T, D, "cuda")
    dx2 = torch.empty_like(dx)
    irn.rmsnorm_bwd_rows(g, x, r, gamma, dx=dx2, workspace=ws)
    dg2 = torch.empty_like(dg)
    irn.rmsnorm_bwd_finish(ws, p.T, D, dg2)
    assert torch.equal(dx, dx2) and torch.equal(dg, dg2)
    _, _, K = irn.rmsnorm_bwd_partials_layout(p.T, D)
    part = ws[: K * D].view(K, D).double().cpu().numpy()
    ref_dg = oracle.dgamma(p.g, p.x, oracle.fwd(p.x, p.gamma)[1])
    assert dgamma_rel_err(part.sum(axis=0), ref_dg) <= 1e-5
    # chunk k's partial is the oracle's dgamma over chunk k's rows
    _, r_ref = oracle.fwd(p.x, p.gamma)
    for k in (0, K // 2, K - 1):
        rows = np.array(irn.chunk_rows(k, p.T, D))
        want = oracle.dgamma(p.g[rows], p.x[rows], r_ref[rows])
        assert dgamma_rel_err(part[k], want) <= 1e-5
    # T = 1
    _, r1 = irn.rmsnorm_fwd(x[:1], gamma)
    _, dg1 = irn.rmsnorm_bwd(g[:1], x[:1], r1, gamma, want_dx=False)
    gx = (g[:1].float() * x[:1].float())[0]
    assert torch.equal(dg1, gx * r1[0])


def test_dx_only_and_dgamma_only(gpu):
    p = wl.tiny(True, T=513, D=1024, seed=9800)
    x, g, gamma = dev_bf16(p.x), dev_bf16(p.g), dev_f32(p.gamma)
    _, r = irn.rmsnorm_fwd(x, gamma, True)
    dx, dg = irn.rmsnorm_bwd(g, x, r, gamma, True)
    dx_only, none = irn.rmsnorm_bwd(g, x, r, gamma, True, want_dgamma=False)
    none2, dg_only = irn.rmsnorm_bwd(g, x, r, gamma, True, want_dx=False)
    assert none is None and none2 is None
    assert torch.equal(dx, dx_only) and torch.equal(dg, dg_only)


def test_empty_batch(gpu):
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    gamma = torch.ones(4096, device="cuda")
    y, r = irn.rmsnorm_fwd(x, gamma)
    assert y.shape == (0, 4096)
    dg = torch.full((4096,), 7.0, device="cuda")
    irn.rmsnorm_bwd(x, x, r, gamma, dgamma=dg, want_dx=False)
    torch.cuda.synchronize()
    assert torch.all(dg == 0)


def test_rejections_write_nothing(gpu):
    D = 256
    x = dev_bf16(synth.normal_bf16(1, 1, 10, D))
    gamma = torch.ones(D, device="cuda")
    y = torch.full((10, D), 3.0, dtype=torch.bfloat16, device="cuda")
    # a 2-byte offset base is misaligned for rows of a multiple of 8 elements
    with pytest.raises(irn.RmsnormError) as e:
        xx = x.view(-1)[1:].as_strided((9, D), (D, 1))
        irn.rmsnorm_fwd(xx, gamma, y=y[:9])
    assert e.value.status == irn.RMSN_ERR_MISALIGNED
    with pytest.raises(irn.RmsnormError) as e:
        irn.rmsnorm_fwd(x, gamma, y=x)  # in place
    assert e.value.status == irn.RMSN_ERR_ALIASING
    with pytest.raises(irn.RmsnormError) as e:
        irn.rmsnorm_fwd(x, gamma, eps=float("nan"), y=y)
    assert e.value.status == irn.RMSN_ERR_EPS
    torch.cuda.synchronize()
    assert torch.all(y.float() == 3.0)


def test_binding_rejects_before_launch(gpu):
    """Malformed tensors on the GPU (bf16 weights where fp32 is required, an
    rstd shorter than T, a host gamma beside CUDA activations) raise in the
    binding; nothing is launched and the outputs keep their contents."""
    D, T = 256, 10
    x = dev_bf16(synth.normal_bf16(2, 1, T, D))
    g = dev_bf16(synth.normal_bf16(2, 2, T, D))
    gamma = torch.ones(D, device="cuda")
    y = torch.full((T, D), 3.0, dtype=torch.bfloat16, device="cuda")
    dx = torch.full((T, D), 3.0, dtype=torch.bfloat16, device="cuda")
    rstd = torch.ones(T, device="cuda")
    with pytest.raises(TypeError, match="gamma"):
        irn.rmsnorm_fwd(x, gamma.to(torch.bfloat16), y=y)
    with pytest.raises(ValueError, match="rstd"):
        irn.rmsnorm_bwd(g, x, rstd[: T - 1], gamma, dx=dx)
    with pytest.raises(ValueError, match="CUDA"):
        irn.rmsnorm_bwd(g, x, rstd, gamma.cpu(), dx=dx)
    with pytest.raises(ValueError, match="dx"):
        irn.rmsnorm_bwd(g, x, rstd, gamma, dx=dx[:, : D - 8])
    torch.cuda.synchronize()
    assert torch.all(y.float() == 3.0) and torch.all(dx.float() == 3.0)
