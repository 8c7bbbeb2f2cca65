"""fp64 CPU oracle for the GTR gated-linear-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and this package imports nothing from the
HIP side.

The arithmetic lives in ``gla_oracle.c`` (a plain token-by-token fp64
recurrence, see its header for the passages it follows).  This module only
compiles that file with gcc, loads it with ctypes and marshals arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "_gla_oracle.so")
# The pin-strength test points this at deliberately broken copies of the oracle.
_LIB = os.environ.get("GLA_ORACLE_LIB_OVERRIDE", _DEFAULT_LIB)
_lib = None

DIRECTIONS = {0: "L->R", 1: "R->L", 2: "T->B", 3: "B->T"}


def build(verbose: bool = False) -> str:
    """Compile gla_oracle.c into oracle/_gla_oracle.so with gcc (always rebuilds)."""
    return build_from(_SRC, _DEFAULT_LIB, verbose)


def build_from(src: str, lib: str, verbose: bool = False) -> str:
    tmp = lib + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gla_oracle_f64.restype = ctypes.c_int
    lib.gla_oracle_f64.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_int] * 7 + [dp, dp, ctypes.c_int]
    lib.gla_oracle_bwd_f64.restype = ctypes.c_int
    lib.gla_oracle_bwd_f64.argtypes = [dp] * 12 + [ctypes.c_int] * 8
    lib.gla_oracle_scan_index.restype = ctypes.c_long
    lib.gla_oracle_scan_index.argtypes = [ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_int]
    _lib = lib
    return lib


def to_f64(x) -> np.ndarray:
    """Exact widening of a float16/bfloat16/float32/float64 array (numpy or torch CPU)."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype, widen in torch first
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def scan_index(t: int, grid_h: int, grid_w: int, direction: int) -> int:
    """Grid index visited at scan position t (the C oracle's own map)."""
    return int(_load().gla_oracle_scan_index(t, grid_h, grid_w, direction))


def scan_order(grid_h: int, grid_w: int, direction: int) -> list[int]:
    return [scan_index(t, grid_h, grid_w, direction) for t in range(grid_h * grid_w)]


def gla_forward(q, k, v, log_gate, direction: int, s0=None, want_state: bool = False,
                n_threads: int = 0, return_threads: bool = False):
    """Token-by-token fp64 GLA forward.

    q, k, log_gate: [B, H, grid_h, grid_w, d_k]; v: [B, H, grid_h, grid_w, d_v].
    s0 (optional): [B, H, d_k, d_v] initial state.  Returns out [B, H, grid_h,
    grid_w, d_v] as float64 (plus the final state when ``want_state``, plus the
    OpenMP thread count when ``return_threads``).
    """
    q, k, v, g = to_f64(q), to_f64(k), to_f64(v), to_f64(log_gate)
    if q.ndim != 5 or k.shape != q.shape or g.shape != q.shape or v.ndim != 5 \
            or v.shape[:4] != q.shape[:4]:
        raise ValueError(f"bad shapes q{q.shape} k{k.shape} v{v.shape} g{g.shape}")
    B, H, gh, gw, dk = q.shape
    dv = v.shape[4]
    out = np.empty((B, H, gh, gw, dv), dtype=np.float64)
    s0a = None
    if s0 is not None:
        s0a = to_f64(s0)
        if s0a.shape != (B, H, dk, dv):
            raise ValueError(f"bad s0 shape {s0a.shape}")
    sf = np.empty((B, H, dk, dv), dtype=np.float64) if want_state else None
    rc = _load().gla_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out),
                                B, H, gh, gw, dk, dv, int(direction), _ptr(s0a), _ptr(sf),
                                int(n_threads))
    if rc < 0:
        raise ValueError(f"gla_oracle_f64 failed with code {rc}")
    res = [out]
    if want_state:
        res.append(sf)
    if return_threads:
        res.append(rc)
    return res[0] if len(res) == 1 else tuple(res)


def gla_backward(q, k, v, log_gate, dout, direction: int, s0=None, ds_final=None,
                 want_ds0: bool = False, n_threads: int = 0):
    """Token-by-token fp64 gradients of the forward pass (see gla_oracle_bwd_f64).

    Returns (dq, dk, dv, dlog_gate) as float64 in the layouts of q, k, v and
    log_gate, plus ds0 when ``want_ds0``.  ds_final is dL/dS_final (optional)."""
    q, k, v, g, do = to_f64(q), to_f64(k), to_f64(v), to_f64(log_gate), to_f64(dout)
    B, H, gh, gw, dk_ = q.shape
    dv_ = v.shape[4]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:4] != q.shape[:4] or do.shape != v.shape:
        raise ValueError("bad shapes")
    st = (B, H, dk_, dv_)
    s0a = to_f64(s0) if s0 is not None else None
    dsf = to_f64(ds_final) if ds_final is not None else None
    for a in (s0a, dsf):
        if a is not None and a.shape != st:
            raise ValueError(f"bad state shape {a.shape}")
    dq, dk = np.empty_like(q), np.empty_like(k)
    dv, dg = np.empty_like(v), np.empty_like(g)
    ds0 = np.empty(st, dtype=np.float64) if want_ds0 else None
    rc = _load().gla_oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(do), _ptr(s0a),
                                    _ptr(dsf), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(ds0),
                                    B, H, gh, gw, dk_, dv_, int(direction), int(n_threads))
    if rc < 0:
        raise ValueError(f"gla_oracle_bwd_f64 failed with code {rc}")
    return (dq, dk, dv, dg, ds0) if want_ds0 else (dq, dk, dv, dg)
