"""gtr_gla_fwd_static: the forward pass with its working memory in the library's
fixed device array (no allocation), checked against gtr_gla_fwd (needs an MI355X).

Two calls in a row, the second on a smaller input, each against gtr_gla_fwd on
the same inputs at the parity bar of oracle/compare.py, and bitwise against
the three-launch path with the same segment length; a shape whose boundary
states need longer segments to fit; a shape that cannot fit is refused with
GTR_ERR_SCRATCH; free device memory does not change across calls.
"""
import ctypes
import sys

import pytest
import torch

import gla_inputs
import recurrent_vision_backbone_chunkwise_amd as gla
from oracle.compare import parity_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 32 << 20  # GTR_GLA_STATIC_SCRATCH_BYTES


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def raw_static(q, k, v, g, out, direction):
    """The C entry point through ctypes, returning its code."""
    B, H, gh, gw, dk = q.shape
    dv = v.shape[-1]
    return gla.lib().gtr_gla_fwd_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                        out.data_ptr(), B, H, gh, gw, dk, dv, direction,
                                        gla.DTYPE_CODES[q.dtype], None)


def inputs(B, H, gh, gw, dtype, seed):
    return [x.to(DEV) for x in gla_inputs.make_inputs(B, H, gh, gw, 64, 64, dtype, "light", seed=seed)]


def states_bytes(seqs, n_seg):
    return seqs * n_seg * (2 * 4096 + 64) * 4 if n_seg > 1 else 0


def test_two_calls_match_the_allocating_entry_point():
    cases = [(2, 8, 128, 128, "f16", 0), (1, 3, 40, 40, "bf16", 3)]  # the second is smaller
    for i, (B, H, gh, gw, dtype, d) in enumerate(cases):
        note(f"static call {i}: B={B} H={H} grid={gh}x{gw} {dtype} dir={d}")
        q, k, v, g = inputs(B, H, gh, gw, dtype, seed=40 + i)
        ref = torch.empty_like(v)
        gla.gtr_gla_fwd(q, k, v, g, ref, d)
        plan = gla.gtr_gla_plan(B, H, gh, gw, path=gla.GTR_PATH_SPLIT)
        assert states_bytes(B * H, plan["n_seg"]) <= SCRATCH
        split = torch.empty_like(v)
        gla.gtr_gla_fwd_ex(q, k, v, g, split, d, chunks_per_segment=plan["seg_len"], path=gla.GTR_PATH_SPLIT)
        out = torch.full_like(v, float("nan"))
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        assert raw_static(q, k, v, g, out, d) == 0, gla.gtr_gla_last_error()
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free_before, "the static entry point allocated device memory"
        e = parity_errors(out.double().cpu().numpy(), ref.double().cpu().numpy(), dtype)
        assert e["ok"], e
        assert torch.equal(out, split), "same kernels and segment length: bitwise equal"


def test_segments_lengthen_to_fit():
    """64 sequences of 100 chunks: the planner's 5-chunk segments need 40 MiB of states, more
    than the array holds, so the call lengthens them; results still match gtr_gla_fwd."""
    B, H, gh, gw = 1, 64, 80, 80
    plan = gla.gtr_gla_plan(B, H, gh, gw, path=gla.GTR_PATH_SPLIT)
    assert states_bytes(B * H, plan["n_seg"]) > SCRATCH
    note(f"lengthened segments: {plan}")
    q, k, v, g = inputs(B, H, gh, gw, "f16", seed=7)
    ref = torch.empty_like(v)
    gla.gtr_gla_fwd(q, k, v, g, ref, 2)
    out = torch.full_like(v, float("nan"))
    for _ in range(2):  # twice in a row on the shared array
        assert raw_static(q, k, v, g, out, 2) == 0, gla.gtr_gla_last_error()
    torch.cuda.synchronize()
    e = parity_errors(out.double().cpu().numpy(), ref.double().cpu().numpy(), "f16")
    assert e["ok"], e


def test_too_large_is_refused_without_launching():
    """200 sequences of 256 chunks need 53 MB of states even with 32-chunk segments."""
    B, H, gh, gw = 1, 200, 128, 128
    note("refused shape")
    q, k, v, g = (torch.zeros(B, H, gh, gw, 64, dtype=torch.float16, device=DEV) for _ in range(4))
    out = torch.full_like(v, float("nan"))
    assert raw_static(q, k, v, g, out, 0) == -11  # GTR_ERR_SCRATCH
    msg = gla.gtr_gla_last_error()
    assert "gtr_gla_fwd_static" in msg and str(SCRATCH) in msg, msg
    torch.cuda.synchronize()
    assert torch.isnan(out).all(), "a refused call ran"
    with pytest.raises(gla.GlaError):
        gla.gtr_gla_fwd_static(q, k, v, g, out, 0)
