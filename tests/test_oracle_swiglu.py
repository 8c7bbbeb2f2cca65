"""Pins for the Spatial SwiGLU oracle (CPU only).

The pages give the block's structure in one sentence (a 3 x 3 per-channel
convolution in the value branch of SwiGLU), so the pins come from what that
structure fixes: the convolution against scipy's 2-D cross-correlation, the
reduction to plain SwiGLU (torch's SiLU and matmul) when the kernel is a
centred delta, a brute-force loop evaluation on a tiny grid, locality of the
3 x 3 neighbourhood, zero padding at the grid border, and closed-form SiLU
values.  A flipped or transposed kernel, swapped gate/value columns, another
activation, a dropped bias or another padding rule each fail one of them.
"""
import math

import numpy as np
import pytest
import scipy.signal
import torch

import gla_inputs
from oracle import swiglu


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


def rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


@pytest.mark.parametrize("gh,gw", [(1, 1), (1, 6), (5, 1), (4, 7), (9, 3)])
def test_conv_matches_scipy_cross_correlation(gh, gw):
    rng = np.random.default_rng(gh * 10 + gw)
    F = 5
    val = rand(rng, 2, gh, gw, F)
    w = rand(rng, 3, 3, F)  # asymmetric: a flip or a transpose changes the result
    got = swiglu.depthwise3x3(val, w)
    for b in range(2):
        for f in range(F):
            ref = scipy.signal.correlate2d(val[b, :, :, f], w[:, :, f], mode="same", boundary="fill")
            assert np.allclose(got[b, :, :, f], ref, rtol=0, atol=1e-12)


def test_centred_delta_kernel_is_plain_swiglu():
    rng = np.random.default_rng(1)
    B, gh, gw, C, F = 2, 4, 5, 6, 7
    x, w_in, w_out = rand(rng, B, gh, gw, C), rand(rng, C, 2 * F), rand(rng, F, C)
    delta = np.zeros((3, 3, F))
    delta[1, 1, :] = 1.0
    got = swiglu.spatial_swiglu(x, w_in, delta, None, w_out)
    xt, wt, ot = (torch.from_numpy(a) for a in (x, w_in, w_out))
    u = xt @ wt
    ref = (torch.nn.functional.silu(u[..., :F]) * u[..., F:]) @ ot
    assert rel(got, ref.numpy()) < 1e-13


def test_brute_force_tiny_grid():
    rng = np.random.default_rng(2)
    B, gh, gw, C, F = 1, 2, 3, 2, 3
    x, w_in, cw, cb, w_out = (rand(rng, B, gh, gw, C), rand(rng, C, 2 * F), rand(rng, 3, 3, F),
                              rand(rng, F), rand(rng, F, C))
    got = swiglu.spatial_swiglu(x, w_in, cw, cb, w_out)
    for y in range(gh):
        for c0 in range(gw):
            for c in range(C):
                total = 0.0
                for f in range(F):
                    g = sum(x[0, y, c0, k] * w_in[k, f] for k in range(C))
                    conv = cb[f]
                    for dy in range(3):
                        for dx in range(3):
                            yy, xx = y + dy - 1, c0 + dx - 1
                            if 0 <= yy < gh and 0 <= xx < gw:
                                conv += cw[dy, dx, f] * sum(x[0, yy, xx, k] * w_in[k, F + f]
                                                            for k in range(C))
                    total += g / (1.0 + math.exp(-g)) * conv * w_out[f, c]
                assert abs(got[0, y, c0, c] - total) < 1e-12


def test_changes_stay_in_the_3x3_neighbourhood():
    rng = np.random.default_rng(3)
    B, gh, gw, C, F = 1, 7, 8, 4, 6
    x, w_in, cw, cb, w_out = (rand(rng, B, gh, gw, C), rand(rng, C, 2 * F), rand(rng, 3, 3, F),
                              rand(rng, F), rand(rng, F, C))
    base = swiglu.spatial_swiglu(x, w_in, cw, cb, w_out)
    x2 = x.copy()
    x2[0, 3, 4, :] += 1.0
    diff = np.abs(swiglu.spatial_swiglu(x2, w_in, cw, cb, w_out) - base).max(axis=-1)[0]
    for y in range(gh):
        for c in range(gw):
            near = abs(y - 3) <= 1 and abs(c - 4) <= 1
            assert (diff[y, c] > 1e-9) == near, (y, c)


def test_zero_padding_at_the_border():
    """A grid embedded in a larger one with zero margins gives the same interior outputs: the
    value branch of a zero token is zero, as the padding assumes."""
    rng = np.random.default_rng(4)
    B, gh, gw, C, F = 1, 4, 5, 3, 4
    x, w_in, cw, cb, w_out = (rand(rng, B, gh, gw, C), rand(rng, C, 2 * F), rand(rng, 3, 3, F),
                              rand(rng, F), rand(rng, F, C))
    big = np.zeros((B, gh + 4, gw + 4, C))
    big[:, 2:gh + 2, 2:gw + 2, :] = x
    small_out = swiglu.spatial_swiglu(x, w_in, cw, cb, w_out)
    big_out = swiglu.spatial_swiglu(big, w_in, cw, cb, w_out)
    assert rel(big_out[:, 2:gh + 2, 2:gw + 2, :], small_out) < 1e-14
    assert np.all(big_out[:, 0, :, :] == 0.0)  # SiLU(0) = 0 on zero tokens


def test_silu_closed_forms():
    assert swiglu.silu(0.0) == 0.0
    assert abs(swiglu.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    z = np.linspace(-30, 30, 121)
    assert np.allclose(swiglu.silu(z) - swiglu.silu(-z), z, rtol=0, atol=1e-12)
    assert swiglu.silu(800.0) == 800.0 and swiglu.silu(-800.0) == 0.0


def test_gate_of_zero_blocks_everything():
    rng = np.random.default_rng(5)
    x, w_in, cw, cb, w_out = (rand(rng, 1, 3, 3, 4), rand(rng, 4, 10), rand(rng, 3, 3, 5),
                              rand(rng, 5), rand(rng, 5, 4))
    w_in[:, :5] = 0.0
    assert np.all(swiglu.spatial_swiglu(x, w_in, cw, cb, w_out) == 0.0)


def test_generator_shapes_and_dtypes():
    x, w_in, cw, cb, w_out = gla_inputs.make_swiglu_inputs(2, 3, 4, 16, 24, "bf16", seed=1)
    assert x.shape == (2, 3, 4, 16) and w_in.shape == (16, 48) and cw.shape == (3, 3, 24)
    assert cb.shape == (24,) and w_out.shape == (24, 16) and x.dtype == torch.bfloat16
    assert gla_inputs.make_swiglu_inputs(1, 2, 2, 8, 8, "f32", bias=False)[3] is None


# ---- pin strength: each plausible slip, planted in the oracle, fails some pin ----------------

def _mutant_conv(kind):
    real = swiglu.depthwise3x3

    def conv(val, conv_w, conv_b=None):
        w = np.asarray(conv_w, dtype=np.float64)
        if kind == "flipped":      # convolution instead of cross-correlation
            w = w[::-1, ::-1]
        elif kind == "transposed":  # dy and dx exchanged
            w = np.transpose(w, (1, 0, 2))
        elif kind == "no_bias":
            conv_b = None
        elif kind == "wrap":        # periodic instead of zero padding
            val = np.asarray(val, dtype=np.float64)
            acc = np.zeros_like(val)
            for dy in range(3):
                for dx in range(3):
                    acc += w[dy, dx] * np.roll(val, (1 - dy, 1 - dx), axis=(1, 2))
            return acc + (np.asarray(conv_b, dtype=np.float64) if conv_b is not None else 0.0)
        return real(val, w, conv_b)
    return conv


PINS = [test_conv_matches_scipy_cross_correlation, test_centred_delta_kernel_is_plain_swiglu,
        test_brute_force_tiny_grid, test_changes_stay_in_the_3x3_neighbourhood,
        test_zero_padding_at_the_border, test_silu_closed_forms, test_gate_of_zero_blocks_everything]


def _some_pin_fails():
    for pin in PINS:
        try:
            if pin is test_conv_matches_scipy_cross_correlation:
                pin(4, 7)
            else:
                pin()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("kind", ["flipped", "transposed", "no_bias", "wrap"])
def test_pins_catch_convolution_slips(kind, monkeypatch):
    monkeypatch.setattr(swiglu, "depthwise3x3", _mutant_conv(kind))
    assert _some_pin_fails()


@pytest.mark.parametrize("kind", ["sigmoid", "swapped_branches", "relu"])
def test_pins_catch_gate_slips(kind, monkeypatch):
    real = swiglu.spatial_swiglu
    if kind == "sigmoid":
        monkeypatch.setattr(swiglu, "silu", lambda z: 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64))))
    elif kind == "relu":
        monkeypatch.setattr(swiglu, "silu", lambda z: np.maximum(np.asarray(z, dtype=np.float64), 0.0))
    else:
        def swapped(x, w_in, conv_w, conv_b, w_out, return_hidden=False):
            w = np.asarray(w_in, dtype=np.float64)
            F = w.shape[1] // 2
            return real(x, np.concatenate([w[:, F:], w[:, :F]], axis=1), conv_w, conv_b, w_out,
                        return_hidden)
        monkeypatch.setattr(swiglu, "spatial_swiglu", swapped)
    assert _some_pin_fails()
