"""fp64 CPU oracle for GTR's Spatial SwiGLU block (test infrastructure only).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the HIP library.

What the pages fix.  Every GTR layer pairs the GLA token mixer with a
Spatial SwiGLU block that handles neighbouring positions (the x-techcon
article on GTR, section 架构 / Architecture); the abstract page calls these
"spatially enhanced SwiGLU blocks".  The same section says the block adds a
3 x 3 per-channel (depthwise) convolution to its value branch, so that
adjacent patches exchange information directly.

Reading (the pages give nothing more; stated as assumptions):
  * SwiGLU as usual: a gate branch SiLU(x W_g) times a value branch x W_v,
    then an output projection W_o.  The convolution acts on the value branch
    after its projection:  out = (SiLU(x W_g) * (DWConv3x3(x W_v) + b)) W_o.
  * The convolution runs over the patch grid with zero padding (same size),
    as a cross-correlation: tap (dy, dx) multiplies the value at grid
    position (row + dy - 1, col + dx - 1).
  * No normalisation, residual or bias other than the convolution's own;
    those belong to the layer around the block.

Layouts: x and out [B][grid_h][grid_w][C]; w_in [C][2F] with the gate
projection in columns [0, F) and the value projection in [F, 2F);
conv_w [3][3][F]; conv_b [F] (optional); w_out [F][C].
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def silu(z):
    """z * sigmoid(z), written so that large |z| neither overflows nor loses z."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z >= 0, z / (1.0 + np.exp(-np.abs(z))), z * np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))


def depthwise3x3(val, conv_w, conv_b=None):
    """Per-channel 3 x 3 cross-correlation over the grid, zero padding.

    val [B][gh][gw][F], conv_w [3][3][F], conv_b [F] or None."""
    val = _f64(val)
    w = _f64(conv_w)
    B, gh, gw, F = val.shape
    pad = np.zeros((B, gh + 2, gw + 2, F))
    pad[:, 1:gh + 1, 1:gw + 1, :] = val
    acc = np.zeros_like(val)
    for dy in range(3):
        for dx in range(3):
            acc += w[dy, dx] * pad[:, dy:dy + gh, dx:dx + gw, :]
    if conv_b is not None:
        acc += _f64(conv_b)
    return acc


def spatial_swiglu(x, w_in, conv_w, conv_b, w_out, return_hidden=False):
    """out = (SiLU(x W_g) * (DWConv3x3(x W_v) + b)) W_o in fp64 (see the module docstring)."""
    x = _f64(x)
    w_in = _f64(w_in)
    w_out = _f64(w_out)
    C = x.shape[-1]
    F = w_out.shape[0]
    if w_in.shape != (C, 2 * F) or w_out.shape != (F, C):
        raise ValueError(f"weights {w_in.shape}, {w_out.shape} do not match C={C}, F={F}")
    u = x @ w_in
    gate, val = u[..., :F], u[..., F:]
    hidden = silu(gate) * depthwise3x3(val, conv_w, conv_b)
    out = hidden @ w_out
    return (out, hidden) if return_hidden else out
