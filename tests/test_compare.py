"""The parity metric itself (CPU only)."""
import numpy as np
import torch

from oracle.compare import parity_errors, ulp, TOLERANCE


def test_ulp_values():
    assert ulp(1.0, "f16") == 2.0 ** -10
    assert ulp(1.5, "bf16") == 2.0 ** -7
    assert ulp(3.0, "f32") == 2.0 ** -22
    assert ulp(0.0, "f16") == 2.0 ** -24          # fp16 subnormal spacing
    assert ulp(2.0 ** -100, "bf16") == 2.0 ** -107
    assert ulp(1e-45, "bf16") == 2.0 ** -133        # below the smallest normal


def test_exact_rounding_has_zero_excess():
    rng = np.random.default_rng(0)
    # float32-representable values, so each cast below is one rounding
    o = (rng.standard_normal(50000) * 3.0).astype(np.float32).astype(np.float64)
    for dt, td in (("f16", torch.float16), ("bf16", torch.bfloat16), ("f32", torch.float32)):
        y = torch.from_numpy(o).to(td).double().numpy()
        e = parity_errors(y, o, dt)
        assert e["err_excess"] == 0.0
        assert e["err_raw"] <= e["rounding_floor"] * 1.0000001
    # bfloat16 rounding alone exceeds 1e-2 of rms on heavy-tailed data: why bf16 gates on excess
    o2 = o.copy()
    o2[0] = 25.0
    y2 = torch.from_numpy(o2).to(torch.bfloat16).double().numpy()
    e = parity_errors(y2, o2, "bf16")
    assert e["err_raw"] > TOLERANCE["bf16"] * 0.5 and e["err_excess"] == 0.0 and e["ok"]


def test_injected_error_is_measured():
    rng = np.random.default_rng(1)
    o = rng.standard_normal(1000)
    rms = np.sqrt(np.mean(o * o))
    y = o.copy()
    y[5] += 0.05 * rms
    e = parity_errors(y, o, "f32")
    assert abs(e["err_raw"] - 0.05) < 1e-9 and not e["ok"]
    y = torch.from_numpy(o).to(torch.float16).double().numpy()
    y[7] += 0.02 * rms
    e = parity_errors(y, o, "f16")
    assert e["err_excess"] > 0.019 and not e["ok"]


def test_non_finite_fails():
    o = np.ones(10)
    y = o.copy()
    y[3] = np.nan
    e = parity_errors(y, o, "f16")
    assert not e["ok"] and e["err_raw"] == float("inf")
