"""MI355X (gfx950) chunkwise forward pass of key-only-gated linear attention.

Thin ctypes binding over ``libgtr_gla.so`` (built from ``csrc/`` by
``build.py``).  The functions below carry the C names of ``include/gtr_gla.h``
and only marshal arguments: every step of the computation runs in the HIP
kernels of the library.  PyTorch is used for device memory and streams.

There is no fallback: if the library is not built, or no GPU is present, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that the library binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgtr_gla.so")

GTR_DIR_L2R, GTR_DIR_R2L, GTR_DIR_T2B, GTR_DIR_B2T = 0, 1, 2, 3
GTR_DTYPE_F32, GTR_DTYPE_F16, GTR_DTYPE_BF16 = 0, 1, 2
GTR_PATH_AUTO, GTR_PATH_FUSED, GTR_PATH_SPLIT = 0, 1, 2
ERRORS = {
    0: "GTR_OK", -1: "GTR_ERR_INVALID_ARG", -2: "GTR_ERR_UNSUPPORTED", -3: "GTR_ERR_ALIGNMENT",
    -4: "GTR_ERR_ALIAS", -5: "GTR_ERR_NO_DEVICE", -6: "GTR_ERR_POINTER", -7: "GTR_ERR_ALLOC",
    -8: "GTR_ERR_CAPTURE", -9: "GTR_ERR_LAUNCH", -10: "GTR_ERR_TIMEOUT", -11: "GTR_ERR_SCRATCH",
}
DTYPE_CODES = {torch.float32: GTR_DTYPE_F32, torch.float16: GTR_DTYPE_F16,
               torch.bfloat16: GTR_DTYPE_BF16}

# Every symbol include/gtr_gla.h and include/gtr_swiglu.h declare.
EXPORTS = ("gtr_gla_fwd", "gtr_gla_fwd_static", "gtr_gla_fwd_f32", "gtr_gla_fwd_f16", "gtr_gla_fwd_bf16",
           "gtr_gla_fwd_ex", "gtr_gla_check", "gtr_gla_workspace_bytes",
           "gtr_gla_workspace_bytes_ex", "gtr_gla_plan",
           "gtr_gla_last_error", "gtr_gla_version", "gtr_gla_release_workspaces",
           "gtr_gla_profile_begin", "gtr_gla_profile_end", "gtr_gla_kernel_name",
           "gtr_gla_stream_status", "gtr_gla_bwd", "gtr_swiglu_fwd", "gtr_swiglu_workspace_bytes")


class GlaError(RuntimeError):
    def __init__(self, code: int, message: str):
        self.code = code
        super().__init__(f"{ERRORS.get(code, code)}: {message}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m recurrent_vision_backbone_chunkwise_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
    fp = ctypes.c_void_p
    sig = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i]
    L.gtr_gla_fwd.argtypes = sig + [i, st]
    L.gtr_gla_fwd_static.argtypes = sig + [i, st]
    for name in ("gtr_gla_fwd_f32", "gtr_gla_fwd_f16", "gtr_gla_fwd_bf16"):
        getattr(L, name).argtypes = sig + [st]
    L.gtr_gla_fwd_ex.argtypes = sig + [i, fp, fp, i, i, st]
    L.gtr_gla_check.argtypes = sig + [i, fp, fp, i, i]
    ip = ctypes.POINTER(ctypes.c_int)
    L.gtr_gla_plan.argtypes = [i] * 8 + [ip, ip, ip]
    for name in ("gtr_gla_fwd", "gtr_gla_fwd_static", "gtr_gla_fwd_f32", "gtr_gla_fwd_f16", "gtr_gla_fwd_bf16",
                 "gtr_gla_fwd_ex", "gtr_gla_check", "gtr_gla_version", "gtr_gla_plan"):
        getattr(L, name).restype = ctypes.c_int
    L.gtr_gla_workspace_bytes.argtypes = [i] * 7
    L.gtr_gla_workspace_bytes.restype = ctypes.c_size_t
    L.gtr_gla_workspace_bytes_ex.argtypes = [i] * 9
    L.gtr_gla_workspace_bytes_ex.restype = ctypes.c_size_t
    L.gtr_gla_last_error.argtypes = []
    L.gtr_gla_last_error.restype = ctypes.c_char_p
    L.gtr_gla_release_workspaces.argtypes = []
    L.gtr_gla_release_workspaces.restype = None
    L.gtr_gla_profile_begin.argtypes = []
    L.gtr_gla_profile_begin.restype = None
    L.gtr_gla_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), i]
    L.gtr_gla_profile_end.restype = ctypes.c_int
    L.gtr_gla_kernel_name.argtypes = [i]
    L.gtr_gla_kernel_name.restype = ctypes.c_char_p
    L.gtr_gla_stream_status.argtypes = [st]
    L.gtr_gla_stream_status.restype = i
    L.gtr_gla_bwd.argtypes = [vp] * 5 + [fp, fp] + [vp] * 4 + [fp] + [i] * 8 + [st]
    L.gtr_gla_bwd.restype = i
    L.gtr_swiglu_fwd.argtypes = [vp] * 6 + [i] * 6 + [st]
    L.gtr_swiglu_fwd.restype = i
    L.gtr_swiglu_workspace_bytes.argtypes = [i] * 6
    L.gtr_swiglu_workspace_bytes.restype = ctypes.c_size_t
    _lib = L
    return L


def hip_runtimes_mapped() -> list[str]:
    """Paths of every HIP runtime mapped into this process (must be exactly one)."""
    with open("/proc/self/maps") as f:
        return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})


def gtr_gla_last_error() -> str:
    return lib().gtr_gla_last_error().decode()


def gtr_gla_version() -> int:
    return lib().gtr_gla_version()


def gtr_gla_workspace_bytes(B, H, grid_h, grid_w, d_k=64, d_v=64, dtype=GTR_DTYPE_F16) -> int:
    return lib().gtr_gla_workspace_bytes(B, H, grid_h, grid_w, d_k, d_v, dtype)


def gtr_gla_workspace_bytes_ex(B, H, grid_h, grid_w, d_k=64, d_v=64, dtype=GTR_DTYPE_F16,
                               chunks_per_segment=0, path=GTR_PATH_AUTO) -> int:
    return lib().gtr_gla_workspace_bytes_ex(B, H, grid_h, grid_w, d_k, d_v, dtype,
                                            chunks_per_segment, path)


def gtr_gla_plan(B, H, grid_h, grid_w, chunks_per_segment=0, path=GTR_PATH_AUTO, d_k=64,
                 d_v=64) -> dict:
    """{"seg_len", "n_seg", "fused"} the library uses for this shape."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().gtr_gla_plan(B, H, grid_h, grid_w, d_k, d_v, chunks_per_segment, path,
                              ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"seg_len": a.value, "n_seg": b.value, "fused": bool(c.value)}


def gtr_gla_release_workspaces() -> None:
    lib().gtr_gla_release_workspaces()


def gtr_gla_profile_begin() -> None:
    lib().gtr_gla_profile_begin()


def gtr_gla_profile_end() -> dict:
    """{kernel name: (total ms, launches)} for the kernels launched since profile_begin."""
    n = 16
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    rc = lib().gtr_gla_profile_end(ms, cnt, n)
    if rc < 0:
        raise GlaError(rc, "profiling events could not be read")
    return {lib().gtr_gla_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(rc)}


def gtr_gla_kernel_name(kernel: int) -> str:
    return lib().gtr_gla_kernel_name(kernel).decode()


def gtr_gla_stream_status(stream=None) -> None:
    """Synchronises `stream`; raises GlaError (GTR_ERR_TIMEOUT) if a one-launch wait on it gave up."""
    _check(lib().gtr_gla_stream_status(_stream_handle(stream)))


def _check(rc: int) -> None:
    if rc != 0:
        raise GlaError(rc, gtr_gla_last_error())


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _shapes(q, k, v, log_gate, out):
    for name, t in (("q", q), ("k", k), ("v", v), ("log_gate", log_gate), ("out", out)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 5:
            raise ValueError(f"{name} must be [B, H, grid_h, grid_w, d], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, gh, gw, dk = q.shape
    dv = v.shape[4]
    if k.shape != q.shape or log_gate.shape != q.shape or v.shape[:4] != q.shape[:4] \
            or out.shape != v.shape:
        raise ValueError("shape mismatch between q, k, v, log_gate and out")
    return B, H, gh, gw, dk, dv


def gtr_gla_fwd(q, k, v, log_gate, out, direction: int, stream=None) -> None:
    """out <- GLA forward of (q, k, v, log_gate) along `direction` (asynchronous)."""
    B, H, gh, gw, dk, dv = _shapes(q, k, v, log_gate, out)
    _check(lib().gtr_gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gate.data_ptr(),
                             out.data_ptr(), B, H, gh, gw, dk, dv, int(direction),
                             DTYPE_CODES[q.dtype], _stream_handle(stream)))


def gtr_gla_fwd_static(q, k, v, log_gate, out, direction: int, stream=None) -> None:
    """gtr_gla_fwd with its working memory in the library's fixed device array (no allocation)."""
    B, H, gh, gw, dk, dv = _shapes(q, k, v, log_gate, out)
    _check(lib().gtr_gla_fwd_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gate.data_ptr(),
                                    out.data_ptr(), B, H, gh, gw, dk, dv, int(direction),
                                    DTYPE_CODES[q.dtype], _stream_handle(stream)))


def gtr_gla_fwd_ex(q, k, v, log_gate, out, direction: int, s0=None, s_final=None,
                   chunks_per_segment: int = 0, path: int = GTR_PATH_AUTO, stream=None) -> None:
    """Extended call: optional initial state s0 / final state s_final (float32 [B,H,d_k,d_v])."""
    B, H, gh, gw, dk, dv = _shapes(q, k, v, log_gate, out)
    for name, t in (("s0", s0), ("s_final", s_final)):
        if t is None:
            continue
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() \
                or tuple(t.shape) != (B, H, dk, dv):
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [B, H, d_k, d_v]")
    _check(lib().gtr_gla_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gate.data_ptr(),
                                out.data_ptr(), B, H, gh, gw, dk, dv, int(direction),
                                DTYPE_CODES[q.dtype],
                                s0.data_ptr() if s0 is not None else None,
                                s_final.data_ptr() if s_final is not None else None,
                                int(chunks_per_segment), int(path), _stream_handle(stream)))


def gla_forward(q, k, v, log_gate, direction: int, s0=None, want_state: bool = False,
                chunks_per_segment: int = 0, path: int = GTR_PATH_AUTO, stream=None):
    """Allocating convenience wrapper: returns out (and the final state when asked)."""
    out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    s_final = None
    if want_state:
        s_final = torch.empty(q.shape[0], q.shape[1], q.shape[4], v.shape[4],
                              dtype=torch.float32, device=q.device)
    gtr_gla_fwd_ex(q, k, v, log_gate, out, direction, s0=s0, s_final=s_final,
                   chunks_per_segment=chunks_per_segment, path=path, stream=stream)
    return (out, s_final) if want_state else out


def gtr_gla_bwd(q, k, v, log_gate, dout, dq, dk, dv, dlog_gate, direction: int, s0=None,
                ds_final=None, ds0=None, stream=None) -> None:
    """Gradients of gtr_gla_fwd_ex (asynchronous): dq, dk, dlog_gate like q, dv like v; ds0
    (optional, float32 [B, H, d_k, d_v]) receives dL/ds0.  ds_final is dL/ds_final."""
    B, H, gh, gw, d_k, d_v = _shapes(q, k, v, log_gate, dout)
    for name, t, like in (("dq", dq, q), ("dk", dk, q), ("dv", dv, v), ("dlog_gate", dlog_gate, q)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() \
                or t.shape != like.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor shaped and typed like its input")
    for name, t in (("s0", s0), ("ds_final", ds_final), ("ds0", ds0)):
        if t is not None and (not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous()
                              or tuple(t.shape) != (B, H, d_k, d_v)):
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor [B, H, d_k, d_v]")
    ptr = lambda t: t.data_ptr() if t is not None else None
    _check(lib().gtr_gla_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_gate.data_ptr(),
                             dout.data_ptr(), ptr(s0), ptr(ds_final), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), dlog_gate.data_ptr(), ptr(ds0), B, H, gh, gw, d_k, d_v,
                             int(direction), DTYPE_CODES[q.dtype], _stream_handle(stream)))


def gla_backward(q, k, v, log_gate, dout, direction: int, s0=None, ds_final=None,
                 want_ds0: bool = False, stream=None):
    """Allocating wrapper: returns (dq, dk, dv, dlog_gate) and ds0 when asked."""
    dq, dk, dlg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(log_gate)
    dv = torch.empty_like(v)
    ds0 = None
    if want_ds0:
        ds0 = torch.empty(q.shape[0], q.shape[1], q.shape[4], v.shape[4], dtype=torch.float32,
                          device=q.device)
    gtr_gla_bwd(q, k, v, log_gate, dout, dq, dk, dv, dlg, direction, s0=s0, ds_final=ds_final,
                ds0=ds0, stream=stream)
    return (dq, dk, dv, dlg, ds0) if want_ds0 else (dq, dk, dv, dlg)


# ---- Spatial SwiGLU block (include/gtr_swiglu.h) ------------------------------------------------

def gtr_swiglu_workspace_bytes(B, grid_h, grid_w, C, F, dtype=GTR_DTYPE_F16) -> int:
    return lib().gtr_swiglu_workspace_bytes(B, grid_h, grid_w, C, F, dtype)


def gtr_swiglu_fwd(x, w_in, conv_w, conv_b, w_out, out, stream=None) -> None:
    """out <- Spatial SwiGLU of x (asynchronous).  x, out [B, grid_h, grid_w, C]; w_in [C, 2F];
    conv_w [3, 3, F]; conv_b [F] or None; w_out [F, C]; one dtype throughout."""
    named = (("x", x), ("w_in", w_in), ("conv_w", conv_w), ("conv_b", conv_b), ("w_out", w_out),
             ("out", out))
    for name, t in named:
        if t is None and name == "conv_b":
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.dtype != x.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, x has {x.dtype}")
    if x.dtype not in DTYPE_CODES or x.dim() != 4:
        raise ValueError("x must be [B, grid_h, grid_w, C] of float32, float16 or bfloat16")
    B, gh, gw, C = x.shape
    F = w_out.shape[0]
    if tuple(w_in.shape) != (C, 2 * F) or tuple(conv_w.shape) != (3, 3, F) \
            or tuple(w_out.shape) != (F, C) or out.shape != x.shape \
            or (conv_b is not None and tuple(conv_b.shape) != (F,)):
        raise ValueError("shape mismatch between x, w_in, conv_w, conv_b, w_out and out")
    _check(lib().gtr_swiglu_fwd(x.data_ptr(), w_in.data_ptr(), conv_w.data_ptr(),
                                conv_b.data_ptr() if conv_b is not None else None,
                                w_out.data_ptr(), out.data_ptr(), B, gh, gw, C, F,
                                DTYPE_CODES[x.dtype], _stream_handle(stream)))


def swiglu_forward(x, w_in, conv_w, conv_b, w_out, stream=None):
    """Allocating convenience wrapper around gtr_swiglu_fwd."""
    out = torch.empty_like(x)
    gtr_swiglu_fwd(x, w_in, conv_w, conv_b, w_out, out, stream=stream)
    return out
