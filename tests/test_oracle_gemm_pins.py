"""Pins of the oracle's batch-invariant GEMM, Y = X @ W.T in bf16
(TransformerEngine issue "Expose Batch Invariant Kernels", point 3).

What pins what (none re-types the oracle's sum):
  * W = identity gives X back, and a one-hot row of X picks a column of W;
  * the roles of X and W swap exactly: gemm(X, W) == gemm(W, X).T bitwise;
  * small-integer inputs: numpy's int64 matmul, exact, then torch's bf16
    rounding;
  * power-of-two scaling of X scales Y exactly;
  * the exact sums against numpy's float64 matmul (a library routine).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from numerics import bf16_to_f64, f32_to_bf16_torch


def _bits(v):
    return f32_to_bf16_torch(np.asarray(v, dtype=np.float32))


def test_identity_weight_returns_x():
    K = 96
    x = synth.normal_bf16(2001, 1, 13, K)
    w = _bits(np.eye(K))
    y, ye = oracle.gemm_xwt(x, w)
    assert np.array_equal(y, x)
    assert np.array_equal(ye, bf16_to_f64(x))


def test_one_hot_rows_pick_columns_of_w():
    K, N = 64, 40
    w = synth.normal_bf16(2002, 2, N, K)
    x = np.zeros((3, K), np.float32)
    x[0, 5] = 1.0
    x[1, 63] = -2.0
    x[2, 0] = 0.5
    y, _ = oracle.gemm_xwt(_bits(x), w)
    wv = bf16_to_f64(w)
    assert np.array_equal(y[0], _bits(wv[:, 5]))
    assert np.array_equal(y[1], _bits(-2.0 * wv[:, 63]))
    assert np.array_equal(y[2], _bits(0.5 * wv[:, 0]))


def test_roles_of_x_and_w_swap_exactly():
    x = synth.normal_bf16(2003, 1, 17, 200)
    w = synth.normal_bf16(2003, 2, 29, 200)
    y, ye = oracle.gemm_xwt(x, w)
    yt, yte = oracle.gemm_xwt(w, x)
    assert np.array_equal(y, yt.T) and np.array_equal(ye, yte.T)


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (7, 5, 64), (33, 17, 512)])
def test_small_integers_match_integer_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + K)
    xi = rng.integers(-16, 17, size=(M, K))
    wi = rng.integers(-16, 17, size=(N, K))
    y, ye = oracle.gemm_xwt(_bits(xi), _bits(wi))
    exact = xi.astype(np.int64) @ wi.astype(np.int64).T
    assert np.array_equal(ye, exact.astype(np.float64))
    assert np.array_equal(y, _bits(exact.astype(np.float32)))


def test_power_of_two_scaling_is_exact():
    x = synth.normal_bf16(2004, 1, 9, 128)
    w = synth.normal_bf16(2004, 2, 11, 128)
    y, _ = oracle.gemm_xwt(x, w)
    y8, _ = oracle.gemm_xwt(_bits(8.0 * bf16_to_f64(x)), w)
    assert np.array_equal(bf16_to_f64(y8), 8.0 * bf16_to_f64(y))


def test_exact_sums_match_float64_matmul():
    x = synth.normal_bf16(2005, 1, 20, 1024)
    w = synth.normal_bf16(2005, 2, 30, 1024)
    _, ye = oracle.gemm_xwt(x, w)
    ref = bf16_to_f64(x) @ bf16_to_f64(w).T
    scale = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(w)).T
    assert np.all(np.abs(ye - ref) <= 1e-13 * scale)
