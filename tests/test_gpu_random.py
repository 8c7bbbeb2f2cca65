"""Seeded random configurations through the C ABI vs the fp64 oracles (needs an MI355X).

Each case draws, from its own seed, every knob the entry points take at once: batch and
heads, a grid of 1..48 x 1..48 cells (ragged chunk tails, single tokens, long thin grids),
head dims (any multiple of 4 up to 128, so one or two 64-wide key and value blocks), I/O
type, scan direction, gate recipe, launch structure and segment length, and whether an
initial state is passed or a final state asked for.  The fixed test suites cover each knob
on its own; these cases cover them together.  Gates as in the fixed suites.
"""
import sys

import numpy as np
import pytest
import torch

import gla_inputs
import oracle
import recurrent_vision_backbone_chunkwise_amd as gla
from oracle.compare import parity_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = ("f32", "f16", "bf16")
GATES = ("light", "heavy", "mixed_extreme", "ones")
PATHS = (gla.GTR_PATH_AUTO, gla.GTR_PATH_FUSED, gla.GTR_PATH_SPLIT)


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def draw(seed):
    r = np.random.RandomState(seed)
    return dict(B=int(r.randint(1, 3)), H=int(r.randint(1, 4)), gh=int(r.randint(1, 49)),
                gw=int(r.randint(1, 49)), dk=4 * int(r.randint(1, 33)), dv=4 * int(r.randint(1, 33)),
                dtype=DTYPES[r.randint(3)], direction=int(r.randint(4)), gate=GATES[r.randint(len(GATES))],
                path=int(PATHS[r.randint(3)]), seg=int(r.randint(0, 4)), s0=bool(r.randint(2)),
                want_state=bool(r.randint(2)))


def state_tolerance_dtype(dtype):
    # the final state is fp32, formed from 16-bit operands for 16-bit I/O
    return "f32" if dtype == "f32" else "f16"


@pytest.mark.parametrize("seed", range(40))
def test_forward_random_configuration(seed):
    c = draw(7000 + seed)
    note(f"forward seed={seed} {c}")
    q, k, v, g = gla_inputs.make_inputs(c["B"], c["H"], c["gh"], c["gw"], c["dk"], c["dv"], c["dtype"],
                                        c["gate"], seed=7100 + seed)
    s0 = None
    if c["s0"]:
        s0 = torch.randn(c["B"], c["H"], c["dk"], c["dv"], generator=torch.Generator().manual_seed(7200 + seed)) * 0.5
    res = gla.gla_forward(*(t.to(DEV) for t in (q, k, v, g)), c["direction"],
                          s0=s0.to(DEV) if s0 is not None else None, want_state=c["want_state"],
                          chunks_per_segment=c["seg"], path=c["path"])
    torch.cuda.synchronize()
    y, sf = res if c["want_state"] else (res, None)
    ref = oracle.gla_forward(q, k, v, g, c["direction"], s0=s0.double().numpy() if s0 is not None else None,
                             want_state=c["want_state"])
    ref, sref = ref if c["want_state"] else (ref, None)
    e = parity_errors(y.double().cpu().numpy(), ref, c["dtype"])
    assert e["ok"], f"{c}: out {e}"
    if c["want_state"]:
        es = parity_errors(sf.double().cpu().numpy(), sref, state_tolerance_dtype(c["dtype"]))
        assert es["ok"], f"{c}: s_final {es}"


def draw_many(seed):
    """Like draw, with 2 to 60 sequences (B*H, twice with d_v > 64) on grids of up to 40x40, so that the
    automatic choice takes the one launch with 1-, 2- or 3-chunk segments for many of them."""
    r = np.random.RandomState(seed)
    c = draw(seed)
    c.update(B=int(r.randint(1, 7)), H=int(r.randint(2, 11)), gh=int(r.randint(4, 41)), gw=int(r.randint(4, 41)),
             dk=64 if r.randint(3) else 4 * int(r.randint(1, 17)), dv=64 if r.randint(3) else 4 * int(r.randint(1, 33)),
             path=int(gla.GTR_PATH_AUTO), seg=0)
    if seed % 6 == 4:  # 24 sequences of 23 to 25 chunks: 2-chunk segments
        c.update(B=4, H=6, gh=40, gw=int(r.randint(36, 41)), dk=64, dv=64)
    if seed % 6 == 5:  # 48 sequences of 21 to 25 chunks: 3-chunk segments
        c.update(B=8, H=6, gh=int(r.randint(36, 41)), gw=int(r.randint(36, 41)), dk=64, dv=64)
    return c


@pytest.mark.parametrize("seed", range(24))
def test_forward_random_many_sequences(seed):
    c = draw_many(9000 + seed)
    plan = gla.gtr_gla_plan(c["B"], c["H"], c["gh"], c["gw"], 0, gla.GTR_PATH_AUTO, c["dk"], c["dv"])
    note(f"forward many seed={seed} {c} plan={plan}")
    q, k, v, g = gla_inputs.make_inputs(c["B"], c["H"], c["gh"], c["gw"], c["dk"], c["dv"], c["dtype"],
                                        c["gate"], seed=9100 + seed)
    s0 = None
    if c["s0"]:
        s0 = torch.randn(c["B"], c["H"], c["dk"], c["dv"], generator=torch.Generator().manual_seed(9200 + seed)) * 0.5
    res = gla.gla_forward(*(t.to(DEV) for t in (q, k, v, g)), c["direction"],
                          s0=s0.to(DEV) if s0 is not None else None, want_state=c["want_state"])
    gla.gtr_gla_stream_status()
    y, sf = res if c["want_state"] else (res, None)
    ref = oracle.gla_forward(q, k, v, g, c["direction"], s0=s0.double().numpy() if s0 is not None else None,
                             want_state=c["want_state"])
    ref, sref = ref if c["want_state"] else (ref, None)
    e = parity_errors(y.double().cpu().numpy(), ref, c["dtype"])
    assert e["ok"], f"{c}: out {e}"
    if c["want_state"]:
        es = parity_errors(sf.double().cpu().numpy(), sref, state_tolerance_dtype(c["dtype"]))
        assert es["ok"], f"{c}: s_final {es}"


def test_many_sequence_draws_reach_every_automatic_plan():
    """The draws above cover three launches and the one launch with 1-, 2- and 3-chunk segments
    (host-side check of the plans the seeds give)."""
    lens = set()
    for seed in range(24):
        c = draw_many(9000 + seed)
        pl = gla.gtr_gla_plan(c["B"], c["H"], c["gh"], c["gw"], 0, gla.GTR_PATH_AUTO, c["dk"], c["dv"])
        lens.add(pl["seg_len"] if pl["fused"] else 0)
    assert {0, 1, 2, 3} <= lens, lens


@pytest.mark.parametrize("seed", range(24))
def test_backward_random_configuration(seed):
    c = draw(8000 + seed)
    note(f"backward seed={seed} {c}")
    q, k, v, g = gla_inputs.make_inputs(c["B"], c["H"], c["gh"], c["gw"], c["dk"], c["dv"], c["dtype"],
                                        c["gate"], seed=8100 + seed)
    dout = gla_inputs.make_output_grad(v.shape, c["dtype"], seed=8200 + seed)
    gen = torch.Generator().manual_seed(8300 + seed)
    s0 = torch.randn(c["B"], c["H"], c["dk"], c["dv"], generator=gen) * 0.5 if c["s0"] else None
    dsf = torch.randn(c["B"], c["H"], c["dk"], c["dv"], generator=gen) * 0.1 if c["want_state"] else None
    got = gla.gla_backward(*(t.to(DEV) for t in (q, k, v, g, dout)), c["direction"],
                           s0=s0.to(DEV) if s0 is not None else None,
                           ds_final=dsf.to(DEV) if dsf is not None else None, want_ds0=True)
    torch.cuda.synchronize()
    ref = oracle.gla_backward(q, k, v, g, dout, c["direction"],
                              s0=s0.double().numpy() if s0 is not None else None,
                              ds_final=dsf.double().numpy() if dsf is not None else None, want_ds0=True)
    for name, y, o in zip(("dq", "dk", "dv", "dlog_gate", "ds0"), got, ref):
        e = parity_errors(y.double().cpu().numpy(), o, state_tolerance_dtype(c["dtype"]) if name == "ds0" else c["dtype"])
        if e["rounding_floor"] > e["tol"]:
            # the output type cannot hold these gradients at all (e.g. after a reset gate): judge
            # what it can hold
            assert e["err_excess"] <= e["tol"], f"{c}: {name} {e}"
        else:
            assert e["ok"], f"{c}: {name} {e}"
