"""The seeded input recipe (gla_inputs.py) against the distributions it states (CPU).

q, v ~ N(0, 1); k ~ N(0, 1) / sqrt(d_k); log_gate = logsigmoid(z) / 16, or logsigmoid(2 z) / 8 for
the heavy gate, with z ~ N(0, 1); values rounded to the I/O dtype.  The expected means of the gates
come from Gauss-Hermite quadrature of the log-sigmoid, not from the generator.
"""
import numpy as np
import pytest
import torch

import gla_inputs

EXPECTED = {  # workload -> (B, H, grid_h, grid_w, dtype, gate, directions)
    1: (1, 2, 40, 40, "f32", "light", (0,)),
    2: (1, 6, 40, 40, "f16", "light", (0, 1, 2, 3)),
    3: (8, 6, 40, 40, "f16", "heavy", (0, 1, 2, 3)),
    4: (1, 16, 64, 64, "bf16", "light", (2, 3)),
    5: (1, 16, 128, 128, "f16", "light", (0, 1, 2, 3)),
}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def mean_log_sigmoid(scale):
    """E[log sigmoid(scale * z)], z ~ N(0, 1), by Gauss-Hermite quadrature."""
    x, w = np.polynomial.hermite_e.hermegauss(80)
    return float(np.sum(w * -np.logaddexp(0.0, -scale * x)) / np.sqrt(2 * np.pi))


@pytest.mark.parametrize("idx", sorted(EXPECTED))
def test_workload_shapes_and_dtypes(idx):
    B, H, gh, gw, dtype, gate, dirs = EXPECTED[idx]
    w = gla_inputs.workload(idx)
    assert (w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.dtype, w.gate, tuple(w.directions)) == \
        (B, H, gh, gw, 64, 64, dtype, gate, dirs)


@pytest.mark.parametrize("idx", [2, 3])
def test_workload_inputs_follow_the_recipe(idx):
    w = gla_inputs.workload(idx)
    q, k, v, g = gla_inputs.workload_inputs(w, 0)
    for t, last in ((q, 64), (k, 64), (v, 64), (g, 64)):
        assert t.dtype == TORCH_DTYPE[w.dtype] and tuple(t.shape) == (w.B, w.H, w.grid_h, w.grid_w, last)
    qf, kf, vf, gf = (t.double() for t in (q, k, v, g))
    assert abs(float(qf.std()) - 1) < 0.02 and abs(float(vf.std()) - 1) < 0.02
    assert abs(float(kf.std()) - 1 / 8) < 0.0025 and abs(float(kf.mean())) < 0.002
    assert bool((gf <= 0).all())
    scale, div = (2.0, 8.0) if w.gate == "heavy" else (1.0, 16.0)
    want = mean_log_sigmoid(scale) / div
    assert abs(float(gf.mean()) - want) < 0.01 * abs(want), (float(gf.mean()), want)
    # a 64-token chunk's total log-decay along the scan averages 64 times that
    assert abs(float(gf.reshape(-1, 64, 64).sum(1).mean()) - 64 * want) < 0.02 * 64 * abs(want)


def test_seeds_are_fixed_per_workload_and_layer():
    w = gla_inputs.workload(2)
    a = gla_inputs.workload_inputs(w, 1)
    b = gla_inputs.workload_inputs(w, 1)
    c = gla_inputs.workload_inputs(w, 2)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[0], c[0])


@pytest.mark.parametrize("scale", [1.0, 2.0])
def test_quadrature_matches_adaptive_integration(scale):
    """The Gauss-Hermite expectation against scipy's adaptive quadrature of the same integral."""
    from scipy import integrate

    f = lambda x: -np.logaddexp(0.0, -scale * x) * np.exp(-x * x / 2) / np.sqrt(2 * np.pi)  # noqa: E731
    val, _ = integrate.quad(f, -np.inf, np.inf, epsabs=1e-12)
    assert abs(mean_log_sigmoid(scale) - val) < 1e-8
