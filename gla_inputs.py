"""Seeded synthetic inputs for the GTR gated-linear-attention forward pass.

This module is the only code shared by the HIP path's tests/benchmark and the
fp64 oracle: it draws random tensors and holds none of the attention
arithmetic.

Workloads.  The patch grids follow the GTR pages: images are cut into patches
at stride 16 (x-techcon article on GTR, section 架构), so a 640x640 detection
input gives a 40x40 grid (same article, section 迁移: detection runs at
640x640) and a 1024x1024 input gives 64x64 (section 部署: rotated detection and
semantic segmentation at 1024x1024).  The 128x128 grid is the 16,384-token
point of the isolated operator test (section 算子).  The pages give no batch,
head count or head width for the operator test; the values below are the
benchmark's own choice.

Recipe (per call): ``torch.Generator('cpu').manual_seed(1000*cfg + layer)``;
draw q, k, v, z ~ N(0, 1) as float32 of shape [B, H, grid_h, grid_w, d] in that
order; k /= sqrt(d_k); log_gate = logsigmoid(z)/16 ("light" gate) or
logsigmoid(2 z)/8 ("heavy" gate); then round-to-nearest-even to the I/O dtype.
The oracle reads the rounded values, widened exactly to float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

DIR_NAMES = ("L->R", "R->L", "T->B", "B->T")


@dataclass(frozen=True)
class Workload:
    index: int            # 1-based workload number, used in the seed
    name: str
    B: int
    H: int
    grid_h: int
    grid_w: int
    d_k: int
    d_v: int
    dtype: str            # "f32" | "f16" | "bf16"
    gate: str             # "light" | "heavy"
    directions: tuple     # scan directions run, in order, as one step

    @property
    def n_tok(self) -> int:
        return self.grid_h * self.grid_w


WORKLOADS = (
    Workload(1, "grid40x40_f32_b1h2_lr", 1, 2, 40, 40, 64, 64, "f32", "light", (0,)),
    Workload(2, "grid40x40_f16_b1h6_4dir", 1, 6, 40, 40, 64, 64, "f16", "light", (0, 1, 2, 3)),
    Workload(3, "grid40x40_f16_b8h6_heavygate_4dir", 8, 6, 40, 40, 64, 64, "f16", "heavy", (0, 1, 2, 3)),
    Workload(4, "grid64x64_bf16_b1h16_tb_bt", 1, 16, 64, 64, 64, 64, "bf16", "light", (2, 3)),
    Workload(5, "grid128x128_f16_b1h16_4dir", 1, 16, 128, 128, 64, 64, "f16", "light", (0, 1, 2, 3)),
)


def workload(idx_or_name) -> Workload:
    for w in WORKLOADS:
        if w.index == idx_or_name or w.name == idx_or_name:
            return w
    raise KeyError(idx_or_name)


TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def make_inputs(B, H, grid_h, grid_w, d_k=64, d_v=64, dtype="f16", gate="light", seed=0):
    """Return (q, k, v, log_gate) as CPU tensors of the I/O dtype, [B,H,gh,gw,d]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shp_k = (B, H, grid_h, grid_w, d_k)
    shp_v = (B, H, grid_h, grid_w, d_v)
    q = torch.randn(shp_k, generator=g, dtype=torch.float32)
    k = torch.randn(shp_k, generator=g, dtype=torch.float32)
    v = torch.randn(shp_v, generator=g, dtype=torch.float32)
    z = torch.randn(shp_k, generator=g, dtype=torch.float32)
    k = k / math.sqrt(d_k)
    if gate == "light":
        log_gate = torch.nn.functional.logsigmoid(z) / 16.0
    elif gate == "heavy":
        log_gate = torch.nn.functional.logsigmoid(2.0 * z) / 8.0
    elif gate == "ones":          # alpha = 1: no decay at all
        log_gate = torch.zeros_like(z)
    elif gate.startswith("const:"):  # the same log-gate everywhere
        log_gate = torch.full_like(z, float(gate.split(":", 1)[1]))
    elif gate.startswith("scale:"):  # logsigmoid(z) times a factor (stress)
        log_gate = torch.nn.functional.logsigmoid(z) * float(gate.split(":", 1)[1])
    elif gate == "mixed_extreme":  # most tokens light, some tokens nearly reset the state
        log_gate = torch.nn.functional.logsigmoid(z) / 16.0
        sel = torch.rand(shp_k[:4] + (1,), generator=g) < 0.05
        log_gate = torch.where(sel, torch.full_like(log_gate, -30.0), log_gate)
    else:
        raise ValueError(f"unknown gate recipe {gate!r}")
    td = TORCH_DTYPES[dtype]
    return q.to(td), k.to(td), v.to(td), log_gate.to(td)


def workload_inputs(w: Workload, layer: int):
    """Inputs of call ``layer`` (0-based position in the step) of workload ``w``."""
    return make_inputs(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.dtype, w.gate,
                       seed=1000 * w.index + layer)


# ---- Spatial SwiGLU block (the layer's other half) ------------------------------------------
#
# Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw, in this order and as float32,
# x ~ N(0, 1) [B, grid_h, grid_w, C], w_in ~ N(0, 1/C) [C, 2F], conv_w ~ N(0, 1/9) [3, 3, F],
# conv_b ~ N(0, 0.1^2) [F] and w_out ~ N(0, 1/F) [F, C]; then round to the I/O dtype.  The
# pages give neither the channel width nor the hidden width of the block; the workloads take
# C = heads x 64 of the matching attention workload and F = 8C/3 rounded up to a multiple
# of 64 (the usual SwiGLU width).

@dataclass(frozen=True)
class SwigluWorkload:
    name: str
    B: int
    grid_h: int
    grid_w: int
    C: int
    F: int
    dtype: str
    seed: int

    @property
    def n_tok(self) -> int:
        return self.grid_h * self.grid_w


SWIGLU_WORKLOADS = (
    SwigluWorkload("swiglu_grid40x40_c384_f1024_f16", 1, 40, 40, 384, 1024, "f16", 7001),
    SwigluWorkload("swiglu_grid128x128_c1024_f2752_f16", 1, 128, 128, 1024, 2752, "f16", 7002),
)


def swiglu_workload(idx_or_name) -> SwigluWorkload:
    for i, w in enumerate(SWIGLU_WORKLOADS, start=1):
        if i == idx_or_name or w.name == idx_or_name:
            return w
    raise KeyError(idx_or_name)


def make_swiglu_inputs(B, grid_h, grid_w, C, F, dtype="f16", seed=0, bias=True):
    """Return (x, w_in, conv_w, conv_b or None, w_out) as CPU tensors of the I/O dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn((B, grid_h, grid_w, C), generator=g, dtype=torch.float32)
    w_in = torch.randn((C, 2 * F), generator=g, dtype=torch.float32) / math.sqrt(C)
    conv_w = torch.randn((3, 3, F), generator=g, dtype=torch.float32) / 3.0
    conv_b = torch.randn((F,), generator=g, dtype=torch.float32) * 0.1
    w_out = torch.randn((F, C), generator=g, dtype=torch.float32) / math.sqrt(F)
    t = TORCH_DTYPES[dtype]
    return (x.to(t), w_in.to(t), conv_w.to(t), conv_b.to(t) if bias else None, w_out.to(t))


def make_output_grad(shape, dtype="f16", seed=0):
    """dL/dout for the backward pass: N(0, 1) of the given shape, rounded to the I/O dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(TORCH_DTYPES[dtype])
