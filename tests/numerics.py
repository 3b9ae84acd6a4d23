"""Comparison helpers for the tests (numpy / torch library routines only).

Nothing here computes RMSNorm: these functions compare bf16 results with
exact or reference values, using torch's own bf16 conversions so that the
comparisons do not rely on the oracle's codec.
"""
from __future__ import annotations

import numpy as np
import torch

U32 = 2.0 ** -24  # fp32 unit roundoff


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bits (torch's conversion)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    t = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()


def f32_to_bf16_torch(v: np.ndarray) -> np.ndarray:
    """torch's fp32 -> bf16 conversion (round to nearest even), as bits."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers ordered like the values; +0 and -0 both map to 0."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits & 0x7FFF) > 0x7F80


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordered(a) - ordered(b)|; NaN vs NaN counts 0, NaN vs number a huge value."""
    d = np.abs(ordered(a) - ordered(b))
    na, nb = is_nan_bf16(a), is_nan_bf16(b)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, 1 << 20, d)


def rounding_consistent(res_bits: np.ndarray, exact: np.ndarray,
                        err_bound: np.ndarray | float) -> np.ndarray:
    """Mask of elements where a bf16 result is a correct rounding of a value
    within ``err_bound`` of ``exact``.

    A result equal to bf16_rne(exact) always passes; the other bf16 neighbour
    passes only when ``exact`` lies within ``err_bound`` of the midpoint
    between them. Formally: |res - exact| <= |nearest - exact| + 2*err_bound.
    """
    res = bf16_to_f64(res_bits)
    exact = np.asarray(exact, dtype=np.float64)
    nearest = bf16_to_f64(f32_to_bf16_torch(exact.astype(np.float32)))
    with np.errstate(invalid="ignore"):
        ok = np.abs(res - exact) <= np.abs(nearest - exact) + 2.0 * err_bound + 1e-300
        same_nonfinite = (~np.isfinite(res)) & (~np.isfinite(exact)) & (
            (np.isnan(res) & np.isnan(exact)) | (res == exact))
    return ok | same_nonfinite


# ---- GPU-vs-oracle tolerances ------------------------------------------------
# y, gated out and dx: <= 1 bf16 ulp (ordered-integer distance, +0 == -0, NaN
# matches NaN). rstd: <= 1e-6 relative. dgamma: infinity-norm relative
# <= 1e-5, i.e. max|gpu - ref| <= 1e-5 * max|ref|.

def max_ulp(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    if a_bits.size == 0:
        return 0
    return int(ulp_distance(a_bits, b_bits).max())


def rstd_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = gpu.astype(np.float64)
    ref = ref.astype(np.float64)
    both_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    both_nan = np.isnan(gpu) & np.isnan(ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.abs(gpu - ref) / np.abs(ref)
    rel = np.where(both_inf | both_nan | ((gpu == 0) & (ref == 0)), 0.0, rel)
    rel = np.where(np.isnan(rel), np.inf, rel)
    return float(rel.max()) if rel.size else 0.0


def dgamma_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    scale = np.abs(ref.astype(np.float64)).max()
    if scale == 0:
        return float(np.abs(gpu).max())
    return float(np.abs(gpu.astype(np.float64) - ref).max() / scale)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits; subnormal spacing
    2^-133 below 2^-126)."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def ulp_or_cancelled(got_bits: np.ndarray, ref_bits: np.ndarray, terms: np.ndarray,
                     k: float = 2.0 ** -20) -> np.ndarray:
    """Mask: within 1 bf16 ulp of the reference or, for a result that is a
    difference of terms whose magnitudes add to ``terms``, within
    ulp(ref) + k * terms. The second branch covers inputs that carry a few
    fp32 ulps of approximation error (the gate a(z)): relative to the terms
    such an error is tiny, but a cancelling difference magnifies it relative
    to the result."""
    d = ulp_distance(got_bits, ref_bits)
    got, ref = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    with np.errstate(invalid="ignore"):
        near = np.abs(got - ref) <= bf16_ulp(ref) + k * np.abs(terms)
    return (d <= 1) | near


def gated_dx_terms(g_bits, x_bits, z_bits, gamma, zero_centered, rstd, sigmoid):
    """Magnitude of the two terms of the gated dx, per element, in double:
    |gn w r| + |x| r^3 sum_i |gn_i w_i x_i| / D, with gn = g a(z) and a the
    sigmoid (``sigmoid``) or silu gate (scipy's expit)."""
    import scipy.special
    g, x, z = bf16_to_f64(g_bits), bf16_to_f64(x_bits), bf16_to_f64(z_bits)
    w = np.asarray(gamma, np.float64) + (1.0 if zero_centered else 0.0)
    s = scipy.special.expit(z)
    with np.errstate(invalid="ignore", over="ignore"):
        a = s if sigmoid else z * s
        gw = g * a * w
        r = np.asarray(rstd, np.float64)[:, None]
        D = x.shape[1]
        return np.abs(gw * r) + np.abs(x) * r ** 3 * np.abs(gw * x).sum(1, keepdims=True) / D


# ---- dgamma under fp32 partial overflow ---------------------------------------
# The GPU sums a column's dgamma terms in fp32 per chunk, then the chunk
# partials in fp32; the oracle sums the same fp32 terms in double and rounds
# once. Where the terms' magnitudes add up to about FLT_MAX, an fp32 partial
# may overflow to +-inf (or meet an infinity of the other sign: NaN) although
# the double sum is finite, and a finite fp32 result there carries a rounding
# error relative to that magnitude rather than to the result. Columns whose
# sum of |term| reaches DGAMMA_OVERFLOW_MAG are therefore held only to the
# error bound of an fp32 sum of their terms, and may be non-finite; every
# other column must meet the infinity-norm tolerance, and a column with a
# non-finite term must match the oracle's infinity or NaN exactly.
DGAMMA_OVERFLOW_MAG = 2.0 ** 127


def dgamma_terms_f32(g32: np.ndarray, x32: np.ndarray, rstd: np.ndarray) -> np.ndarray:
    """The dgamma terms as both sides round them, fp32((g * x) * r) per
    element (numpy float32 products: IEEE, round to nearest even, no fused
    multiply-add), returned as float64. A product past FLT_MAX is inf and
    inf * 0 is NaN, as on both sides; a double product would hide that."""
    with np.errstate(invalid="ignore", over="ignore"):
        t = (np.asarray(g32, np.float32) * np.asarray(x32, np.float32)) * \
            np.asarray(rstd, np.float32)[:, None]
    return t.astype(np.float64)


def dgamma_term_stats(terms: np.ndarray):
    """Per column of a [T, D] array of dgamma terms (double): the sum of the
    finite terms' magnitudes, and whether any term is not finite."""
    with np.errstate(invalid="ignore", over="ignore"):
        a = np.abs(terms)
    fin = np.isfinite(a)
    return np.where(fin, a, 0.0).sum(0), (~fin).any(0)


def dgamma_check(gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray, nonfinite: np.ndarray,
                 n_terms: int, tol: float = 1e-5):
    """(ok, report) for a GPU dgamma against the oracle's under the rule
    above. `mag` and `nonfinite` come from dgamma_term_stats; `n_terms`
    bounds the length of any fp32 summation chain (rows plus chunks)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    big = mag >= DGAMMA_OVERFLOW_MAG
    special = nonfinite & ~big
    plain = ~big & ~nonfinite
    report = {"columns": int(gpu.size), "overflow_prone": int(big.sum()),
              "nonfinite_terms": int(special.sum())}
    ok = True
    # ordinary columns: finite, infinity-norm relative error
    if plain.any():
        g, r = gpu[plain], ref[plain]
        ok &= bool(np.isfinite(g).all())
        err = dgamma_rel_err(g, r) if np.isfinite(g).all() else float("inf")
        report["rel_err"] = err
        ok &= err <= tol
    # a non-finite term: both sides propagate it the same way
    if special.any():
        g, r = gpu[special], ref[special]
        same = (np.isnan(g) & np.isnan(r)) | (g == r)
        ok &= bool(same.all())
    # overflow-prone columns: any non-finite value, or a finite one within
    # the error bound of an fp32 sum of n_terms terms of total magnitude mag
    if big.any():
        g, r, m = gpu[big], ref[big], mag[big]
        fin = np.isfinite(g)
        with np.errstate(invalid="ignore", over="ignore"):
            within = (np.abs(g - r) <= n_terms * U32 * m) | ~np.isfinite(r)
        ok &= bool((~fin | within).all())
    return bool(ok), report
