"""Named synthetic workloads (shapes, distributions and seeds).

Every tensor is drawn from ``synth`` with a fixed (seed, stream) pair, so the
same bytes are produced on any machine and for any thread count. Streams:
1 = x, 2 = upstream gradient g, 3 = gamma, 4 = residual gradient,
5 = gate z, 6 = residual input of the fused add, 9 = outlier-row choice,
10 = outlier-row values.

The workloads follow the pages' synthetic recipes: rows of ``randn``
activations and gradients, fp32 weights drawn as ``1 + N(0, 0.1)`` (or
``N(0, 0.1)`` for the zero-centred convention, where the stored weight is the
offset from one), head dimension 128 for the gated norm and hidden size 2048
or 4096 for the token norms.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import normal_bf16, normal_f32, permutation, pick_rows

S_X, S_G, S_GAMMA, S_GRES, S_Z, S_RES_IN, S_OUTLIER_PICK, S_OUTLIER_VAL = 1, 2, 3, 4, 5, 6, 9, 10


@dataclass
class Problem:
    name: str
    T: int
    D: int
    eps: float
    zero_centered: bool
    gamma: np.ndarray                    # fp32 [D]
    x: np.ndarray                        # bf16 bits [T, D]
    g: np.ndarray | None = None          # bf16 bits [T, D]
    gres: np.ndarray | None = None       # bf16 bits [T, D]
    z: np.ndarray | None = None          # bf16 bits [T, D]
    residual: np.ndarray | None = None   # bf16 bits [T, D] (fused add input)
    meta: dict = field(default_factory=dict)


def gamma_for(seed: int, D: int, zero_centered: bool) -> np.ndarray:
    """fp32 weights: ``1 + N(0,0.1)`` plain, ``N(0,0.1)`` zero-centred."""
    return normal_f32(seed, S_GAMMA, D, 0.0 if zero_centered else 1.0, 0.1)


def tiny(zero_centered: bool, T: int = 16, D: int = 128, seed: int = 1001,
         with_gres: bool = False, with_gate: bool = False,
         with_residual: bool = False) -> Problem:
    """Small fixture: x, g ~ N(0,1); non-unit weights; eps = 1e-6."""
    p = Problem(
        name=f"tiny_T{T}_D{D}_zc{int(zero_centered)}", T=T, D=D, eps=1e-6,
        zero_centered=zero_centered, gamma=gamma_for(seed, D, zero_centered),
        x=normal_bf16(seed, S_X, T, D), g=normal_bf16(seed, S_G, T, D))
    if with_gres:
        p.gres = normal_bf16(seed, S_GRES, T, D)
    if with_gate:
        p.z = normal_bf16(seed, S_Z, T, D)
    if with_residual:
        p.residual = normal_bf16(seed, S_RES_IN, T, D)
    return p


def outlier_rows(seed: int, T: int, frac: float = 0.01) -> np.ndarray:
    return pick_rows(seed, S_OUTLIER_PICK, T, int(round(frac * T)))


def residual(T: int = 32768, D: int = 4096, seed: int = 2002,
             with_gres: bool = True, rows: np.ndarray | None = None) -> Problem:
    """Token norm with outliers: x ~ N(0,1) except round(1% of T) seeded rows
    drawn as 50 * N(0,1); g (and the residual-branch gradient) ~ N(0,1);
    gamma = 1 + N(0,0.1); eps = 1e-6.

    With ``rows`` given, only those rows of the full [T, D] workload are
    produced (in that order), for checks that sample a large problem.
    """
    out_rows = outlier_rows(seed, T)
    idx = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    x = _rows_of(seed, S_X, idx, D, 1.0)
    is_out = np.isin(idx, out_rows)
    if is_out.any():
        x[is_out] = _rows_of(seed, S_OUTLIER_VAL, idx[is_out], D, 50.0)
    p = Problem(name=f"residual_T{T}_D{D}", T=T, D=D, eps=1e-6, zero_centered=False,
                gamma=gamma_for(seed, D, False), x=x,
                g=_rows_of(seed, S_G, idx, D, 1.0),
                meta={"outlier_rows": out_rows})
    if with_gres:
        p.gres = _rows_of(seed, S_GRES, idx, D, 1.0)
    return p


def gated(T: int = 262144, D: int = 128, seed: int = 3003,
          rows: np.ndarray | None = None, with_grad: bool = False) -> Problem:
    """Gated per-head norm: x, z ~ N(0,1); gamma = 1 + N(0,0.1); with
    ``with_grad`` also an upstream gradient g ~ N(0,1) for the backward."""
    idx = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    return Problem(name=f"gated_T{T}_D{D}", T=T, D=D, eps=1e-6, zero_centered=False,
                   gamma=gamma_for(seed, D, False),
                   x=_rows_of(seed, S_X, idx, D, 1.0),
                   g=_rows_of(seed, S_G, idx, D, 1.0) if with_grad else None,
                   z=_rows_of(seed, S_Z, idx, D, 1.0))


def fused_add(T: int = 32768, D: int = 4096, seed: int = 6006,
              rows: np.ndarray | None = None, with_gres: bool = True) -> Problem:
    """Fused add-norm of a decoder layer: x (the sublayer output) and the
    residual stream ~ N(0,1); g ~ N(0,1); the gradient arriving at the
    updated residual (``gres``) ~ N(0,1); gamma = 1 + N(0,0.1); eps = 1e-6."""
    idx = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    p = Problem(name=f"fused_add_T{T}_D{D}", T=T, D=D, eps=1e-6, zero_centered=False,
                gamma=gamma_for(seed, D, False), x=_rows_of(seed, S_X, idx, D, 1.0),
                g=_rows_of(seed, S_G, idx, D, 1.0),
                residual=_rows_of(seed, S_RES_IN, idx, D, 1.0))
    if with_gres:
        p.gres = _rows_of(seed, S_GRES, idx, D, 1.0)
    return p


def large(T: int = 262144, D: int = 4096, seed: int = 4004,
          rows: np.ndarray | None = None) -> Problem:
    """Large fwd+bwd: x ~ N(0,1); g = 0.01 * N(0,1); stored gamma drawn as
    1 + N(0,0.1) with the zero-centred flag on (so w_eff = gamma + 1)."""
    idx = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    return Problem(name=f"large_T{T}_D{D}", T=T, D=D, eps=1e-6, zero_centered=True,
                   gamma=normal_f32(seed, S_GAMMA, D, 1.0, 0.1),
                   x=_rows_of(seed, S_X, idx, D, 1.0),
                   g=_rows_of(seed, S_G, idx, D, 0.01))


# --- batch-composition sweep ------------------------------------------------

SWEEP_D = 2048
SWEEP_M = (1, 2, 17, 33, 128, 257, 1000, 1024)
SWEEP_POSITIONS = ("first", "middle", "last", "shuffled")
SWEEP_ANCHOR_SEEDS = (5001, 5002, 5003, 5004)
SWEEP_FILLER_SEED = 5100
SWEEP_SHUFFLE_SEED = 5200
SWEEP_GAMMA_SEED = 5000
SWEEP_PAD_ROWS = 5


def sweep_anchor(k: int, D: int = SWEEP_D) -> tuple[np.ndarray, np.ndarray]:
    """Anchor ``k``'s (x row, g row), each bf16 bits [D]."""
    s = SWEEP_ANCHOR_SEEDS[k]
    return normal_bf16(s, S_X, 1, D)[0], normal_bf16(s, S_G, 1, D)[0]


def sweep_gamma(D: int = SWEEP_D) -> np.ndarray:
    return gamma_for(SWEEP_GAMMA_SEED, D, False)


def sweep_batch(k: int, M: int, position: str, D: int = SWEEP_D,
                pad: int = SWEEP_PAD_ROWS) -> tuple[np.ndarray, np.ndarray, int]:
    """A batch of ``M`` real rows holding anchor ``k`` plus ``pad`` zero rows.

    The other M-1 real rows are filler rows ~ N(0,1). Returns (x, g, row
    index of the anchor). ``position`` is first / middle (M//2) / last, or
    shuffled: the real rows are permuted by a seeded permutation.
    """
    ax, ag = sweep_anchor(k, D)
    x = np.zeros((M + pad, D), dtype=np.uint16)
    g = np.zeros((M + pad, D), dtype=np.uint16)
    if M > 1:
        x[: M - 1] = normal_bf16(SWEEP_FILLER_SEED, S_X, M - 1, D)
        g[: M - 1] = normal_bf16(SWEEP_FILLER_SEED, S_G, M - 1, D)
    if position == "first":
        pos = 0
    elif position == "middle":
        pos = M // 2
    elif position in ("last", "shuffled"):
        pos = M - 1
    else:
        raise ValueError(position)
    # make room for the anchor at `pos`, keeping filler order
    x[pos + 1: M] = x[pos: M - 1].copy()
    g[pos + 1: M] = g[pos: M - 1].copy()
    x[pos], g[pos] = ax, ag
    if position == "shuffled":
        perm = permutation(SWEEP_SHUFFLE_SEED, 1000 + M, M)
        x[:M], g[:M] = x[perm], g[perm]
        pos = int(np.nonzero(perm == M - 1)[0][0])
    return x, g, pos


def _rows_of(seed: int, stream: int, idx: np.ndarray, D: int, scale: float) -> np.ndarray:
    """Rows ``idx`` of the [*, D] matrix ``scale * N(0,1)`` of (seed, stream)."""
    n = len(idx)
    out = np.empty((n, D), dtype=np.uint16)
    if n == 0:
        return out
    # contiguous runs are produced in one call each
    starts = np.flatnonzero(np.diff(idx, prepend=idx[0] - 2) != 1)
    ends = np.append(starts[1:], n)
    for a, b in zip(starts, ends):
        normal_bf16(seed, stream, int(b - a), D, scale, row0=int(idx[a]),
                    out=out[a:b])
    return out
