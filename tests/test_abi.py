"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented codes before touching the HIP
runtime.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import recurrent_vision_backbone_chunkwise_amd as gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gtr_gla.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gtr_gla.h", "gtr_swiglu.h")]


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gtr_[a-z]\w*)\s*\(", text)))


def declared_constants():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(GTR_\w+)\s+\(?(-?\d+)\)?", text)}


def test_library_exports_every_declared_symbol():
    L = gla.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(gla.EXPORTS) == names


def test_binding_constants_match_header():
    c = declared_constants()
    assert c["GTR_DIR_L2R"] == gla.GTR_DIR_L2R and c["GTR_DIR_B2T"] == gla.GTR_DIR_B2T
    assert c["GTR_DTYPE_BF16"] == gla.GTR_DTYPE_BF16
    for code, name in gla.ERRORS.items():
        assert c[name] == code


def test_version_and_sizes():
    assert gla.gtr_gla_version() == 10000
    split = gla.GTR_PATH_SPLIT
    fused = gla.GTR_PATH_FUSED
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 64, 64, 1, 1, split) == 6 * 25 * (2 * 4096 + 64) * 4
    # one-launch path: a payload slot per segment (state and decays; no entering states), then a
    # 32-word header, a 128-byte work line for each of 16 XCD ids and a 64-bit flag per segment;
    # a single segment needs no payload
    sync = lambda flags: (32 + 16 * 32 + 2 * flags) * 4
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 64, 64, 1, 1, fused) == \
        6 * 25 * (4096 + 64) * 4 + sync(6 * 25)
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 8, 8, 64, 64, 1, 1, fused) == sync(6)
    # two key blocks: a slot per segment and key block; fp32 I/O keeps at most 2 chunks per segment
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 128, 64, 1, 0, fused) == \
        6 * 9 * 2 * (4096 + 64) * 4 + sync(6 * 9)
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 128, 64, 0, 0, fused) == \
        6 * 13 * 2 * (4096 + 64) * 4 + sync(6 * 13)
    # head dims: value columns in 64-wide blocks are sequences of their own, key blocks share one
    per = (2 * 4096 + 64) * 4
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 32, 64, 1, 1, split) == 6 * 25 * per
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 64, 128, 1, 1, split) == 12 * 25 * per
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 128, 64, 1, 1, split) == 6 * 25 * 2 * per
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 132, 64, 1, 0, 0) == 0
    assert gla.gtr_gla_workspace_bytes_ex(0, 6, 40, 40, 64, 64, 1, 0, 0) == 0
    assert gla.gtr_gla_workspace_bytes_ex(1, 6, 40, 40, 64, 64, 1, 0, 3) == 0
    # the seven-argument form is the library's own choice of path and segment length
    for shape in [(1, 6, 40, 40, 64, 64, 1), (8, 6, 40, 40, 64, 64, 1), (1, 16, 128, 128, 64, 64, 1),
                  (1, 2, 40, 40, 64, 64, 0), (1, 16, 64, 64, 64, 64, 2), (1, 4, 33, 17, 128, 96, 1)]:
        assert gla.gtr_gla_workspace_bytes(*shape) == gla.gtr_gla_workspace_bytes_ex(*shape, 0, 0) > 0
    assert gla.gtr_gla_workspace_bytes(1, 6, 40, 40, 132, 64, 1) == 0
    assert gla.gtr_gla_workspace_bytes(1, 6, 40, 40, 64, 64, 3) == 0


def test_workspace_bytes_signatures_through_ctypes():
    """The boundary's sizing call takes (B, H, grid_h, grid_w, d_k, d_v, dtype); the _ex form adds
    the segment length and path of gtr_gla_fwd_ex."""
    import ctypes
    L = ctypes.CDLL(gla.LIB_PATH)
    f7, f9 = L.gtr_gla_workspace_bytes, L.gtr_gla_workspace_bytes_ex
    f7.argtypes, f7.restype = [ctypes.c_int] * 7, ctypes.c_size_t
    f9.argtypes, f9.restype = [ctypes.c_int] * 9, ctypes.c_size_t
    assert f7(1, 6, 40, 40, 64, 64, 1) == f9(1, 6, 40, 40, 64, 64, 1, 0, 0) > 0
    assert f7(1, 16, 128, 128, 64, 64, 1) == f9(1, 16, 128, 128, 64, 64, 1, 0, 0) > 0
    assert f9(1, 6, 40, 40, 64, 64, 1, 1, 2) == 6 * 25 * (2 * 4096 + 64) * 4
    assert f7(-1, 6, 40, 40, 64, 64, 1) == 0



def test_plans():
    # one launch caps segments at 3 chunks
    pl = gla.gtr_gla_plan(1, 16, 128, 128, path=gla.GTR_PATH_FUSED)
    assert pl["fused"] and pl["seg_len"] == 3 and pl["n_seg"] == 86
    pl = gla.gtr_gla_plan(1, 16, 128, 128, chunks_per_segment=9, path=gla.GTR_PATH_FUSED)
    assert pl["fused"] and pl["seg_len"] == 3
    pl = gla.gtr_gla_plan(1, 16, 128, 128)
    assert not pl["fused"] and pl["seg_len"] * pl["n_seg"] >= 256
    pl = gla.gtr_gla_plan(1, 16, 128, 128, path=gla.GTR_PATH_SPLIT)
    assert not pl["fused"] and pl["seg_len"] * pl["n_seg"] >= 256
    pl = gla.gtr_gla_plan(1, 6, 40, 40, path=gla.GTR_PATH_FUSED)
    assert pl["fused"] and pl["seg_len"] == 3 and pl["n_seg"] == 9
    pl = gla.gtr_gla_plan(1, 6, 40, 40)  # few short sequences: three launches
    assert not pl["fused"] and pl["seg_len"] == 1
    pl = gla.gtr_gla_plan(8, 6, 40, 40)  # many short sequences: one launch
    assert pl["fused"] and pl["seg_len"] == 3 and pl["n_seg"] == 9
    pl = gla.gtr_gla_plan(1, 16, 64, 64)  # 64 chunks per sequence: three launches
    assert not pl["fused"] and pl["seg_len"] == 2
    pl = gla.gtr_gla_plan(1, 6, 40, 40, chunks_per_segment=4)
    assert pl["seg_len"] == 4 and pl["n_seg"] == 7 and not pl["fused"]
    pl = gla.gtr_gla_plan(1, 6, 40, 40, chunks_per_segment=3, path=gla.GTR_PATH_FUSED)
    assert pl["seg_len"] == 3 and pl["n_seg"] == 9 and pl["fused"]
    pl = gla.gtr_gla_plan(1, 1, 1, 1, chunks_per_segment=9)
    assert pl["seg_len"] == 1 and pl["n_seg"] == 1
    assert gla.gtr_gla_plan(1, 1, 0, 1) == {"seg_len": 0, "n_seg": 0, "fused": False}  # no tokens
    # the one-launch path takes any length; only its per-sequence payload slots (16,640 bytes per
    # segment, 32-bit byte offsets) bound the segment count
    assert gla.gtr_gla_plan(1, 1, 769, 64, path=gla.GTR_PATH_FUSED)["n_seg"] == 257
    assert gla.gtr_gla_plan(1, 1, 2048, 4096, path=gla.GTR_PATH_FUSED)["n_seg"] == 43691
    with pytest.raises(gla.GlaError):
        gla.gtr_gla_plan(1, 1, 2048, 4096, chunks_per_segment=1, path=gla.GTR_PATH_FUSED)
    assert gla.gtr_gla_plan(1, 1, 769, 64, chunks_per_segment=3)["fused"] is False
    with pytest.raises(gla.GlaError):
        gla.gtr_gla_plan(1, 1, -1, 1)
    # head dims: the kernels walk one sequence per 64-wide value block; d_k > 64 takes three
    # launches unless the one-launch path is asked for (it then keeps both key blocks' states)
    assert gla.gtr_gla_plan(8, 6, 40, 40, d_k=32, d_v=32)["fused"]
    assert not gla.gtr_gla_plan(8, 6, 40, 40, d_k=128, d_v=64)["fused"]
    pl = gla.gtr_gla_plan(8, 6, 40, 40, path=gla.GTR_PATH_FUSED, d_k=128)
    assert pl["fused"] and pl["seg_len"] == 3 and pl["n_seg"] == 9
    assert gla.gtr_gla_plan(1, 6, 40, 40, d_k=64, d_v=128) == gla.gtr_gla_plan(1, 12, 40, 40)


def test_automatic_choice():
    """The one launch for sequences of 2 to 48 chunks, at least one sequence per XCD, with the
    shortest segments (two or more per sequence) whose count fits about one round of resident
    workgroups (512 at 16-bit I/O; 3-chunk segments up to 768); three launches otherwise."""
    def auto(B, H, gh, gw):
        pl = gla.gtr_gla_plan(B, H, gh, gw)
        return pl["seg_len"] if pl["fused"] else 0

    assert auto(4, 6, 24, 24) == 1      # 24 sequences x 9 chunks: 216 one-chunk segments
    assert auto(1, 8, 40, 40) == 1      # 8 x 25 = 200
    assert auto(2, 16, 32, 32) == 1     # 32 x 16 = 512, the most that fit
    assert auto(1, 16, 48, 48) == 2     # 16 x 36 = 576 one-chunk segments, 288 of two chunks
    assert auto(32, 6, 16, 16) == 2     # 192 x 4 = 768, then 384
    assert auto(8, 6, 40, 40) == 3      # 48 x 25: 1200, 624, then 432 of three chunks
    assert auto(16, 6, 32, 32) == 3     # 96 x 16: 1536, 768, then 576 <= 768
    assert auto(16, 6, 40, 40) == 0     # 96 x 25: 864 three-chunk segments, more than a round
    assert auto(1, 6, 40, 40) == 0      # fewer sequences than XCDs
    assert auto(1, 12, 64, 64) == 0     # 64 chunks per sequence
    assert auto(1, 16, 56, 56) == 0     # 49 chunks
    assert auto(16, 8, 8, 8) == 0       # one chunk: a single segment per sequence
    assert auto(16, 8, 8, 16) == 1      # two chunks: two one-chunk segments
    assert gla.gtr_gla_plan(8, 6, 40, 40, d_k=128)["fused"] is False  # two key blocks
    # fp32 I/O runs the one launch at one workgroup per CU (256 resident): 24 x 16 = 384 one-chunk
    # segments do not fit, 192 of two chunks do; the workspace follows the plan of the call's type
    ws = gla.lib().gtr_gla_workspace_bytes_ex
    ws.argtypes, ws.restype = [ctypes.c_int] * 9, ctypes.c_size_t
    fused = gla.GTR_PATH_FUSED
    assert ws(4, 6, 32, 32, 64, 64, gla.GTR_DTYPE_F32, 0, 0) == ws(4, 6, 32, 32, 64, 64, gla.GTR_DTYPE_F32, 2, fused)
    assert ws(4, 6, 32, 32, 64, 64, gla.GTR_DTYPE_F16, 0, 0) == ws(4, 6, 32, 32, 64, 64, gla.GTR_DTYPE_F16, 1, fused)
    assert auto(4, 6, 32, 32) == 1


A = 0x10000  # fake, 16-byte aligned, never dereferenced


def call(q=A, k=A + 0x100000, v=A + 0x200000, g=A + 0x300000, out=A + 0x400000, B=1, H=1, gh=4,
         gw=4, dk=64, dv=64, d=0, dt=1, s0=None, sf=None, seg=0, path=0):
    return gla.lib().gtr_gla_fwd_ex(q, k, v, g, out, B, H, gh, gw, dk, dv, d, dt, s0, sf, seg, path,
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(B=-1), -1), (dict(H=-1), -1), (dict(gh=-1), -1),
    (dict(dk=0), -1),
    (dict(d=4), -1), (dict(d=-1), -1), (dict(dt=3), -1), (dict(gh=1 << 12, gw=1 << 11 | 1), -1),
    (dict(path=3), -1), (dict(path=-1), -1),
    (dict(B=1 << 11, H=1 << 10), -1),
    (dict(dk=132), -2), (dict(dv=30), -2), (dict(dk=256), -2), (dict(dk=132, path=1), -2),
    (dict(gh=1 << 11, gw=1 << 12, dk=128, dt=0), -1),  # 2^23 rows of 512 bytes: past 2^31 bytes
    (dict(k=A + 0x100008), -3), (dict(out=A + 0x400004), -3), (dict(s0=A + 0x500002), -3),
    (dict(out=A + 0x200000), -4), (dict(out=A + 0x300000 + 0x400), -4),
    (dict(sf=A + 0x400000), -4), (dict(s0=A + 0x500000, sf=A + 0x500000), -4),
])
def test_argument_errors_before_any_hip_call(kw, code):
    assert call(**kw) == code
    assert gla.gtr_gla_last_error() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(gh=0), dict(gw=0), dict(B=0, gh=0),
                                dict(B=0, q=None, k=None, v=None, g=None, out=None),
                                dict(gh=0, q=None, k=None, v=None, g=None, out=None),
                                dict(B=0, sf=A + 0x500000)])
def test_empty_calls_succeed_without_device_work(kw):
    """No sequence or no token: nothing to compute; null tensor pointers are allowed."""
    assert call(**kw) == 0
    assert gla.gtr_gla_workspace_bytes(kw.get("B", 1), kw.get("H", 1), kw.get("gh", 4), kw.get("gw", 4),
                                       64, 64, 1) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK),
                    reason="a GPU is visible")
def test_valid_call_without_gpu_reports_no_device():
    assert call() == -5
    assert "device" in gla.gtr_gla_last_error()
    assert call(gh=0, sf=A + 0x500000) == -5  # no tokens but a final state to write
    assert call(q=None) == -1  # argument errors still come first


def test_typed_entry_points_validate_too():
    L = gla.lib()
    for fn in (L.gtr_gla_fwd_f32, L.gtr_gla_fwd_f16, L.gtr_gla_fwd_bf16):
        assert fn(A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, 1, 1, 4, 4, 64, 64, 7,
                  None) == -1
    assert L.gtr_gla_fwd(A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, 1, 1, 4, 4, 64,
                         64, 0, 5, None) == -1


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 2, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        gla.gtr_gla_fwd(x, x, x, x, x.clone(), 0)


def test_single_hip_runtime_mapped():
    gla.lib()
    assert len(gla.hip_runtimes_mapped()) == 1


# ---- Spatial SwiGLU entry point ------------------------------------------------------------

def swiglu_call(x=A, w_in=A + 0x1000000, conv_w=A + 0x2000000, conv_b=A + 0x3000000,
                w_out=A + 0x4000000, out=A + 0x5000000, B=1, gh=4, gw=4, C=16, F=32, dt=1):
    return gla.lib().gtr_swiglu_fwd(x, w_in, conv_w, conv_b, w_out, out, B, gh, gw, C, F, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), -1), (dict(B=-1), -1), (dict(gh=-2), -1), (dict(x=None), -1), (dict(w_out=None), -1),
    (dict(B=1 << 10, gh=1 << 8, gw=1 << 7), -1),
    (dict(C=12), -2), (dict(F=4), -2), (dict(C=0), -2), (dict(F=1 << 17), -2),
    (dict(x=A + 8), -3), (dict(conv_b=A + 0x3000004), -3),
    (dict(out=A), -4), (dict(out=A + 0x1000000 + 64), -4),
])
def test_swiglu_argument_errors_before_any_hip_call(kw, code):
    assert swiglu_call(**kw) == code
    assert gla.gtr_gla_last_error() != ""


def test_swiglu_empty_calls_and_sizes():
    assert swiglu_call(B=0, x=None, out=None) == 0
    assert swiglu_call(gh=0) == 0
    assert gla.gtr_swiglu_workspace_bytes(1, 40, 40, 384, 1024, 1) == 1600 * 2048 * 2 + 1600 * 1024 * 2
    assert gla.gtr_swiglu_workspace_bytes(1, 40, 40, 384, 1024, 2) == 1600 * 2048 * 4 + 1600 * 1024 * 2
    assert gla.gtr_swiglu_workspace_bytes(1, 40, 40, 384, 1024, 0) == 1600 * 2048 * 4 + 1600 * 1024 * 4
    assert gla.gtr_swiglu_workspace_bytes(0, 40, 40, 384, 1024, 1) == 0
    assert gla.gtr_swiglu_workspace_bytes(1, 40, 40, 12, 1024, 1) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK),
                    reason="a GPU is visible")
def test_swiglu_valid_call_without_gpu_reports_no_device():
    assert swiglu_call() == -5
    assert swiglu_call(conv_b=None) == -5


# ---- backward entry point --------------------------------------------------------------------

def bwd_call(q=A, k=A + 0x100000, v=A + 0x200000, g=A + 0x300000, do=A + 0x400000, s0=None, dsf=None,
             dq=A + 0x500000, dk=A + 0x600000, dv=A + 0x700000, dg=A + 0x800000, ds0=None, B=1, H=1,
             gh=4, gw=4, dkk=64, dvv=64, d=0, dt=1):
    return gla.lib().gtr_gla_bwd(q, k, v, g, do, s0, dsf, dq, dk, dv, dg, ds0, B, H, gh, gw, dkk, dvv, d, dt,
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=4), -1), (dict(dt=3), -1), (dict(B=-1), -1), (dict(q=None), -1), (dict(dg=None), -1),
    (dict(do=None), -1), (dict(gh=1 << 12, gw=1 << 11 | 1), -1), (dict(B=1 << 10, H=1 << 10, gh=2048, gw=4096), -1),
    (dict(dkk=132), -2), (dict(dvv=132), -2), (dict(dvv=30), -2),
    (dict(dq=A + 0x500008), -3), (dict(ds0=A + 0x900004), -3),
    (dict(dq=A), -4), (dict(dv=A + 0x400000), -4), (dict(dk=A + 0x500000), -4),
])
def test_backward_argument_errors_before_any_hip_call(kw, code):
    assert bwd_call(**kw) == code
    assert gla.gtr_gla_last_error() != ""


def test_backward_empty_calls():
    assert bwd_call(B=0) == 0
    assert bwd_call(gh=0, q=None, k=None, v=None, g=None, do=None, dq=None, dk=None, dv=None, dg=None) == 0


@pytest.mark.skipif(os.path.exists("/dev/kfd") and os.access("/dev/kfd", os.R_OK),
                    reason="a GPU is visible")
def test_backward_valid_call_without_gpu_reports_no_device():
    assert bwd_call() == -5
    assert bwd_call(gh=0, ds0=A + 0x900000, dsf=A + 0xa00000) == -5  # no tokens, ds0 = ds_final


def test_kernel_names_match_the_header():
    """gtr_gla_kernel_name() gives the ids gtr_gla.h documents for gtr_gla_profile_end()."""
    names = ["gla_seg_state", "gla_seg_scan", "gla_seg_out", "gla_fused", "swiglu_gemm_in",
             "swiglu_mix", "swiglu_gemm_out", "gla_bwd_dqk", "gla_bwd_dgate",
             "gla_bwd_ds0"]
    L = gla.lib()
    assert [L.gtr_gla_kernel_name(i).decode() for i in range(len(names))] == names
    assert L.gtr_gla_kernel_name(len(names)) == b"" and L.gtr_gla_kernel_name(-1) == b""
    header = open(os.path.join(ROOT, "include", "gtr_gla.h")).read()
    assert f"number of kernel ids ({len(names)})" in header
    for i, n in enumerate(names):
        assert f"{i} {n}" in header, n
