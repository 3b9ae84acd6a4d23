"""GPU checks of the batch-invariant BF16 GEMM (bigemm_bf16_xwt) against
the CPU oracle, following TransformerEngine issue "Expose Batch Invariant
Kernels", point 3: one anchor row placed first / in the middle / last in
batches of M in {1, 2, 17, 33, 128, 257, 1024}, a shuffled batch and a
non-tile-aligned M = 1000, compared bytewise with the M = 1 result; accuracy
against an exact (double) product.

Tolerance against the oracle's exact sums: the fp32 accumulation over K
terms is within gamma_K = K u / (1 - K u) of sum |x w| (u = 2^-24), so the
bf16 result must be a correct rounding of a value within that bound of the
exact sum (numerics.rounding_consistent). Integer inputs whose sums are
exact in fp32 must match the oracle bitwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import invariant_rmsnorm_amd as irn
import oracle
import synth
from gpu_util import dev_bf16, host_bits
from numerics import U32, bf16_to_f64, f32_to_bf16_torch, rounding_consistent

pytestmark = pytest.mark.gpu


def _check_parity(x, w, y_bits):
    _, ye = oracle.gemm_xwt(x, w)
    K = x.shape[1]
    scale = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(w)).T
    gamma = K * U32 / (1 - K * U32)
    ok = rounding_consistent(y_bits, ye, gamma * scale)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} outside the accumulation bound"


@pytest.mark.parametrize("M,N,K", [(1, 128, 32), (5, 64, 64), (64, 96, 128), (33, 200, 160),
                                   (70, 130, 192), (17, 300, 256), (256, 128, 96),
                                   (300, 257, 512), (257, 1000, 1024), (1000, 1024, 2048)])
def test_gemm_parity(gpu, M, N, K):
    x = synth.normal_bf16(2100 + M, 1, M, K)
    w = synth.normal_bf16(2100 + M, 2, N, K)
    y = irn.bigemm_bf16_xwt(dev_bf16(x), dev_bf16(w))
    torch.cuda.synchronize()
    _check_parity(x, w, host_bits(y))


@pytest.mark.parametrize("M,N,K", [(3, 40, 32), (300, 200, 640), (129, 1030, 1024)])
def test_gemm_exact_integers_bitwise(gpu, M, N, K):
    rng = np.random.default_rng(M + N + K)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    wi = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    x, w = f32_to_bf16_torch(xi), f32_to_bf16_torch(wi)
    y = irn.bigemm_bf16_xwt(dev_bf16(x), dev_bf16(w))
    ref, _ = oracle.gemm_xwt(x, w)
    assert np.array_equal(host_bits(y), ref)


def test_gemm_strided_operands(gpu):
    M, N, K = 200, 300, 256
    x = synth.normal_bf16(2120, 1, M, K)
    w = synth.normal_bf16(2120, 2, N, K)
    xd, wd = dev_bf16(x), dev_bf16(w)
    xs = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros((N, K + 32), dtype=torch.bfloat16, device="cuda")
    xs[:, :K] = xd
    ws[:, 32:] = wd
    ys = torch.zeros((M, N + 3), dtype=torch.bfloat16, device="cuda")
    irn.bigemm_bf16_xwt(xs[:, :K], ws[:, 32:], y=ys[:, :N])
    y = irn.bigemm_bf16_xwt(xd, wd)
    assert torch.equal(ys[:, :N], y)
    assert torch.all(ys[:, N:] == 0)  # nothing written past N


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 352), (4096, 4096, 320), (600, 4096, 288)])
def test_gemm_strided_operands_large_tiles(gpu, M, N, K):
    """Row strides above K and offset bases on the tiles whose operands go
    straight into LDS (128 x 128, 256 x 256 and 64 x 128 here; K ends in a
    half stage in two of them): the same bytes as contiguous operands,
    nothing written past N."""
    assert irn.bigemm_bf16_tile(M, N)[0] >= 64
    x = synth.normal_bf16(2125 + M, 1, M, K)
    w = synth.normal_bf16(2125 + M, 2, N, K)
    xd, wd = dev_bf16(x), dev_bf16(w)
    xs = torch.zeros((M, K + 40), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros((N, K + 24), dtype=torch.bfloat16, device="cuda")
    xs[:, 8:K + 8] = xd
    ws[:, 24:] = wd
    ys = torch.zeros((M, N + 5), dtype=torch.bfloat16, device="cuda")
    irn.bigemm_bf16_xwt(xs[:, 8:K + 8], ws[:, 24:], y=ys[:, :N])
    y = irn.bigemm_bf16_xwt(xd, wd)
    assert torch.equal(ys[:, :N], y)
    assert torch.all(ys[:, N:] == 0)
    rows = [0, M // 2, M - 1]
    _check_parity(x[rows], w, host_bits(y)[rows])


M_SET = (1, 2, 17, 33, 128, 257, 1024)


def test_gemm_anchor_rows_across_batches(gpu):
    """The page's check: anchor rows, bitwise equal to their M = 1 result in
    every batch size and position; padding and shuffles; M = 1000."""
    N = K = 2048
    w = dev_bf16(synth.normal_bf16(2130, 2, N, K))
    filler = synth.normal_bf16(2131, 1, 1024, K)
    for a in range(3):
        anchor = synth.normal_bf16(2132 + a, 1, 1, K)
        ref = irn.bigemm_bf16_xwt(dev_bf16(anchor), w)
        _check_parity(anchor, host_bits(w), host_bits(ref))
        for M in M_SET + (1000,):
            for pos in sorted({0, M // 2, M - 1}):
                xb = filler[:M].copy()
                xb[pos] = anchor[0]
                y = irn.bigemm_bf16_xwt(dev_bf16(xb), w)
                assert torch.equal(y[pos:pos + 1], ref), (a, M, pos)
        # shuffled batch with zero padding rows appended
        perm = np.random.default_rng(2140 + a).permutation(300)
        xb = np.concatenate([filler[:299], anchor, np.zeros((7, K), np.uint16)])[perm.tolist() + list(range(300, 307))]
        pos = int(np.where(perm == 299)[0][0])
        y = irn.bigemm_bf16_xwt(dev_bf16(xb), w)
        assert torch.equal(y[pos:pos + 1], ref)
        assert torch.all(y[300:].float() == 0)


def test_gemm_row_slices_equal_full_batch(gpu):
    """Every slice of a batch gives the same bytes as the full batch."""
    M, N, K = 1024, 1024, 1024
    x = dev_bf16(synth.normal_bf16(2150, 1, M, K))
    w = dev_bf16(synth.normal_bf16(2150, 2, N, K))
    full = irn.bigemm_bf16_xwt(x, w)
    for a, b in ((0, 1), (3, 5), (255, 257), (100, 1000), (1000, 1024), (0, 1024)):
        assert torch.equal(irn.bigemm_bf16_xwt(x[a:b], w), full[a:b]), (a, b)


def test_gemm_every_tile_gives_the_same_rows(gpu):
    """Batch sizes chosen so that each of the five output tiles is used
    (N = 4000 and M not multiples of any tile; K = 544 ends in a half
    stage): the first and the last M rows of the 4000-row batch computed
    alone equal the same rows of the full batch bitwise, and sampled rows
    agree with the oracle."""
    Mfull, N, K = 4000, 4000, 544
    Ms = (1, 200, 300, 500, 1000, 2000, 3900)
    assert {irn.bigemm_bf16_tile(M, N) for M in Ms} == {
        (256, 256), (128, 256), (128, 128), (64, 128), (32, 64)}
    xh = synth.normal_bf16(2170, 1, Mfull, K)
    wh = synth.normal_bf16(2170, 2, N, K)
    x, w = dev_bf16(xh), dev_bf16(wh)
    full = irn.bigemm_bf16_xwt(x, w)
    for M in Ms:
        assert torch.equal(irn.bigemm_bf16_xwt(x[:M], w), full[:M]), M
        assert torch.equal(irn.bigemm_bf16_xwt(x[Mfull - M:], w), full[Mfull - M:]), M
    rows = [0, 31, 255, 1999, 3998, 3999]
    _check_parity(xh[rows], wh, host_bits(full)[rows])


@pytest.mark.slow
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (4096, 11008, 4096), (4096, 4096, 11008)])
def test_gemm_full_size_sampled(gpu, M, N, K):
    """Shapes of the batch-invariant GEMM cost table: 64 sampled rows
    against the oracle."""
    x = synth.normal_bf16(2160 + N + K, 1, M, K)
    w = synth.normal_bf16(2160 + N + K, 2, N, K)
    y = irn.bigemm_bf16_xwt(dev_bf16(x), dev_bf16(w))
    rows = np.random.default_rng(2160).choice(M, 64, replace=False)
    _check_parity(x[rows], w, host_bits(y)[rows])
