"""The input generator is deterministic, row-addressable and independent of
its thread count (so any row of a large workload can be regenerated)."""
import numpy as np

import synth
from synth import workloads as wl


def test_rows_regenerate_independently():
    full = synth.normal_bf16(9, 1, 300, 72)
    part = synth.normal_bf16(9, 1, 5, 72, row0=123)
    assert np.array_equal(full[123:128], part)


def test_strided_output_leaves_padding():
    a = synth.normal_bf16(9, 1, 300, 72, ld=80)
    assert np.array_equal(a[:, :72], synth.normal_bf16(9, 1, 300, 72))
    assert np.all(a[:, 72:] == 0)


def test_streams_and_seeds_differ():
    a = synth.normal_bf16(9, 1, 4, 64)
    assert not np.array_equal(a, synth.normal_bf16(9, 2, 4, 64))
    assert not np.array_equal(a, synth.normal_bf16(10, 1, 4, 64))


def test_normal_moments():
    v = synth.normal_f32(3, 1, 1 << 18)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_sampled_rows_of_named_workloads():
    p = wl.residual(T=512, D=64)
    rows = np.array([0, 1, 2, int(p.meta["outlier_rows"][0]), 511])
    q = wl.residual(T=512, D=64, rows=rows)
    assert np.array_equal(q.x, p.x[rows]) and np.array_equal(q.g, p.g[rows])
    assert len(p.meta["outlier_rows"]) == round(0.01 * 512)


def test_sweep_batch_places_anchor():
    for pos in wl.SWEEP_POSITIONS:
        x, g, i = wl.sweep_batch(1, 33, pos, D=64)
        ax, ag = wl.sweep_anchor(1, D=64)
        assert np.array_equal(x[i], ax) and np.array_equal(g[i], ag)
        assert np.all(x[33:] == 0) and x.shape[0] == 33 + wl.SWEEP_PAD_ROWS
