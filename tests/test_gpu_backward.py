"""Backward pass through the C ABI (gtr_gla_bwd) vs the fp64 backward oracle (needs an MI355X).

Every gradient uses the forward pass's gate: max|y - o| / rms(o) <= 1e-4 (fp32 I/O),
<= 1e-2 (fp16 I/O), and for bf16 the excess over the output's half-ulp <= 1e-2.
"""
import sys

import pytest
import torch

import gla_inputs
import oracle
import recurrent_vision_backbone_chunkwise_amd as gla
from oracle.compare import parity_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = ("f32", "f16", "bf16")
NAMES = ("dq", "dk", "dv", "dlog_gate", "ds0")


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def check(q, k, v, g, direction, dtype, label, s0=None, dsf=None, seed=0):
    dout = gla_inputs.make_output_grad(v.shape, dtype, seed=seed)
    note(f"bwd {label} dir={direction} dtype={dtype} shape={tuple(q.shape)} dv={v.shape[-1]} "
         f"s0={s0 is not None} dsf={dsf is not None}")
    dev = [t.to(DEV) for t in (q, k, v, g, dout)]
    got = gla.gla_backward(*dev, direction, s0=s0.to(DEV) if s0 is not None else None,
                           ds_final=dsf.to(DEV) if dsf is not None else None, want_ds0=True)
    torch.cuda.synchronize()
    ref = oracle.gla_backward(q, k, v, g, dout, direction, s0=s0.double().numpy() if s0 is not None else None,
                              ds_final=dsf.double().numpy() if dsf is not None else None, want_ds0=True)
    errs = {}
    for name, y, o in zip(NAMES, got, ref):
        # ds0 is fp32, formed from 16-bit operands for 16-bit I/O (as the forward's final state)
        e = parity_errors(y.double().cpu().numpy(), o, ("f32" if dtype == "f32" else "f16") if name == "ds0" else dtype)
        errs[name] = round(e["err_raw"], 6)
        if e["rounding_floor"] > e["tol"]:
            # the output type cannot hold these gradients (e.g. ~1e-13 in fp16): judge what it can
            assert e["err_excess"] <= e["tol"], f"{label} {name}: {e}"
        else:
            assert e["ok"], f"{label} {name}: {e}"
    return errs


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("direction", [0, 1, 2, 3])
@pytest.mark.parametrize("grid", [(1, 1), (1, 63), (7, 9), (9, 17), (13, 11), (8, 8), (8, 24), (16, 16)],
                         ids=lambda g: f"{g[0]}x{g[1]}")
def test_small_grids(grid, direction, dtype):
    gh, gw = grid
    q, k, v, g = gla_inputs.make_inputs(2, 3, gh, gw, 64, 64, dtype, "light", seed=gh * 100 + gw + direction)
    check(q, k, v, g, direction, dtype, f"{gh}x{gw}", seed=direction)


@pytest.mark.parametrize("dtype", DTYPES)
def test_initial_and_final_state(dtype):
    q, k, v, g = gla_inputs.make_inputs(1, 2, 11, 13, 64, 64, dtype, "light", seed=31)
    gen = torch.Generator().manual_seed(32)
    s0 = torch.randn(1, 2, 64, 64, generator=gen) * 0.5
    dsf = torch.randn(1, 2, 64, 64, generator=gen) * 0.1
    for d in range(4):
        check(q, k, v, g, d, dtype, "state", s0=s0, dsf=dsf, seed=33 + d)


@pytest.mark.parametrize("gate", ["const:-30", "mixed_extreme", "ones", "scale:4"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_extremes(gate, dtype):
    q, k, v, g = gla_inputs.make_inputs(1, 2, 19, 23, 64, 64, dtype, gate, seed=34)
    for d in (0, 3):
        check(q, k, v, g, d, dtype, f"gate={gate}", seed=35 + d)


@pytest.mark.parametrize("dims", [(32, 32), (64, 32), (32, 64), (4, 8), (48, 60)], ids=lambda d: f"dk{d[0]}_dv{d[1]}")
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_head_dims(dims, dtype):
    dk, dv = dims
    q, k, v, g = gla_inputs.make_inputs(2, 2, 9, 17, dk, dv, dtype, "light", seed=dk + dv)
    gen = torch.Generator().manual_seed(dk * dv)
    s0 = torch.randn(2, 2, dk, dv, generator=gen) * 0.5
    dsf = torch.randn(2, 2, dk, dv, generator=gen) * 0.1
    for d in (1, 2):
        check(q, k, v, g, d, dtype, f"dk={dk} dv={dv}", s0=s0, dsf=dsf, seed=36 + d)


@pytest.mark.parametrize("dims", [(128, 64), (96, 32), (68, 64), (128, 4), (64, 128), (32, 100), (128, 128),
                                  (100, 68)], ids=lambda d: f"dk{d[0]}_dv{d[1]}")
@pytest.mark.parametrize("dtype", DTYPES)
def test_wide_heads(dims, dtype):
    """Heads wider than 64: both key blocks' states in one pass, dv summed over them in fp32, and
    dq, dk, dlog_gate, ds0 per key block as slices of the key-side rows; each value block's states
    as a sequence of its own, and dq and dk summed over the value blocks in fp32."""
    dk, dv = dims
    q, k, v, g = gla_inputs.make_inputs(2, 2, 9, 17, dk, dv, dtype, "light", seed=dk * 3 + dv)
    gen = torch.Generator().manual_seed(dk + 5 * dv)
    s0 = torch.randn(2, 2, dk, dv, generator=gen) * 0.5
    dsf = torch.randn(2, 2, dk, dv, generator=gen) * 0.1
    check(q, k, v, g, 0, dtype, f"dk={dk} dv={dv}", seed=50)
    check(q, k, v, g, 3, dtype, f"dk={dk} dv={dv} with states", s0=s0, dsf=dsf, seed=51)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wide_heads_long(dtype):
    """128 x 128 heads over 4,096 tokens (64 chunks per scan) with extreme gates on some dims."""
    q, k, v, g = gla_inputs.make_inputs(1, 2, 64, 64, 128, 128, dtype, "mixed_extreme", seed=52)
    gen = torch.Generator().manual_seed(53)
    s0 = torch.randn(1, 2, 128, 128, generator=gen) * 0.5
    dsf = torch.randn(1, 2, 128, 128, generator=gen) * 0.1
    for d in (1, 2):
        note(f"errors {check(q, k, v, g, d, dtype, '64x64 dk=dv=128', s0=s0, dsf=dsf, seed=54 + d)}")


@pytest.mark.parametrize("widx", [2, 4])
def test_workload_shapes(widx):
    w = gla_inputs.workload(widx)
    q, k, v, g = gla_inputs.workload_inputs(w, 0)
    note(f"errors {check(q, k, v, g, w.directions[0], w.dtype, w.name, seed=37)}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16k_tokens(dtype):
    """128x128, two heads, 16-bit I/O: 256 chunks along the forward and the reversed scan."""
    q, k, v, g = gla_inputs.make_inputs(1, 2, 128, 128, 64, 64, dtype, "light", seed=45)
    for d in (1, 2):
        note(f"errors {check(q, k, v, g, d, dtype, '128x128', seed=46 + d)}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_long_sequence(dtype):
    """144 chunks: both state scans run 143 or 144 steps; with s0 and dL/dS_final."""
    q, k, v, g = gla_inputs.make_inputs(1, 1, 96, 96, 64, 64, dtype, "light", seed=39)
    s0 = torch.randn(1, 1, 64, 64, generator=torch.Generator().manual_seed(40)) * 0.5
    dsf = torch.randn(1, 1, 64, 64, generator=torch.Generator().manual_seed(41))
    for d in (0, 2):
        note(f"errors {check(q, k, v, g, d, dtype, '96x96', s0=s0, dsf=dsf, seed=42 + d)}")


def test_unsupported_width_and_empty_calls():
    q, k, v, g = (t.to(DEV) for t in gla_inputs.make_inputs(1, 1, 4, 4, 64, 64, "f16", "light", seed=38))
    v = torch.zeros(1, 1, 4, 4, 132, dtype=torch.float16, device=DEV)
    with pytest.raises(gla.GlaError) as ex:  # d_v above 128
        gla.gla_backward(q, k, v, g, torch.zeros_like(v), 0)
    assert ex.value.code == -2
    x = torch.empty(2, 3, 0, 5, 64, dtype=torch.float16, device=DEV)
    dsf = torch.randn(2, 3, 64, 64, device=DEV)
    res = gla.gla_backward(x, x, x, x, x, 1, ds_final=dsf, want_ds0=True)
    torch.cuda.synchronize()
    assert torch.equal(res[4], dsf)  # no tokens: the final state is the initial one


def test_repeat_calls_are_bitwise_equal():
    q, k, v, g = (t.to(DEV) for t in gla_inputs.make_inputs(1, 4, 23, 29, 64, 64, "bf16", "light", seed=39))
    dout = gla_inputs.make_output_grad(v.shape, "bf16", seed=40).to(DEV)
    first = gla.gla_backward(q, k, v, g, dout, 2)
    for _ in range(3):
        again = gla.gla_backward(q, k, v, g, dout, 2)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_workspace_allocation_failure(monkeypatch):
    """A failed backward-workspace allocation returns GTR_ERR_ALLOC and runs nothing; the next
    call allocates and matches the oracle."""
    q, k, v, g = gla_inputs.make_inputs(1, 2, 9, 17, 64, 64, "f16", "light", seed=43)
    dout = gla_inputs.make_output_grad(v.shape, "f16", seed=44)
    dev = [t.to(DEV) for t in (q, k, v, g, dout)]
    s = torch.cuda.Stream()  # no workspace yet
    outs = [torch.full_like(t, float("nan")) for t in (dev[0], dev[1], dev[2], dev[3])]
    note("bwd allocation failure")
    monkeypatch.setenv("GTR_GLA_TEST_FAIL_ALLOC", "1")
    with pytest.raises(gla.GlaError) as ex:
        gla.gtr_gla_bwd(*dev, *outs, 1, stream=s)
    torch.cuda.synchronize()
    assert ex.value.code == -7 and all(torch.isnan(o).all() for o in outs)
    monkeypatch.delenv("GTR_GLA_TEST_FAIL_ALLOC")
    gla.gtr_gla_bwd(*dev, *outs, 1, stream=s)
    torch.cuda.synchronize()
    ref = oracle.gla_backward(q, k, v, g, dout, 1)
    for name, y, o in zip(NAMES, outs, ref):
        e = parity_errors(y.double().cpu().numpy(), o, "f16")
        assert e["ok"] or (e["rounding_floor"] > e["tol"] and e["err_excess"] <= e["tol"]), (name, e)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)], ids=lambda d: f"dk{d[0]}_dv{d[1]}")
def test_graph_replays_match_eager(dims):
    """The reversed scan and dv run on a second stream forked from the caller's and joined back:
    captured in a HIP graph (after one eager call), every replay gives bitwise the eager result,
    with eager work between the replays."""
    dk_, dv_ = dims
    q, k, v, g = (t.to(DEV) for t in gla_inputs.make_inputs(1, 3, 23, 29, dk_, dv_, "f16", "light", seed=61))
    dout = gla_inputs.make_output_grad(v.shape, "f16", seed=62).to(DEV)
    gen = torch.Generator().manual_seed(63)
    s0 = (torch.randn(1, 3, dk_, dv_, generator=gen) * 0.5).to(DEV)
    dsf = (torch.randn(1, 3, dk_, dv_, generator=gen) * 0.1).to(DEV)
    outs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
            torch.empty(1, 3, dk_, dv_, device=DEV)]
    stream = torch.cuda.Stream()

    def call():
        gla.gtr_gla_bwd(q, k, v, g, dout, outs[0], outs[1], outs[2], outs[3], 2, s0=s0, ds_final=dsf,
                        ds0=outs[4], stream=stream)

    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))  # eager work between the replays, on the default stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(NAMES, outs, eager):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager call"



def test_two_streams_side_by_side():
    """Calls on two caller streams, each with its own workspace and second stream, run side by
    side and give bitwise the results of the same calls made one at a time."""
    def inputs(seed, shape):
        q, k, v, g = (t.to(DEV) for t in gla_inputs.make_inputs(*shape, 64, 64, "f16", "light", seed=seed))
        return q, k, v, g, gla_inputs.make_output_grad(v.shape, "f16", seed=seed + 1).to(DEV)
    a = inputs(81, (1, 4, 40, 40))
    b = inputs(83, (2, 3, 33, 29))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):
        ref_a = gla.gla_backward(*a, 2, want_ds0=True, stream=sa)
    torch.cuda.synchronize()
    with torch.cuda.stream(sb):
        ref_b = gla.gla_backward(*b, 1, want_ds0=True, stream=sb)
    torch.cuda.synchronize()
    for rep in range(3):
        note(f"two streams, repeat {rep}")
        with torch.cuda.stream(sa):
            got_a = gla.gla_backward(*a, 2, want_ds0=True, stream=sa)
        with torch.cuda.stream(sb):
            got_b = gla.gla_backward(*b, 1, want_ds0=True, stream=sb)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, got_a, ref_a):
            assert torch.equal(x, y), f"stream a, repeat {rep}: {name}"
        for name, x, y in zip(NAMES, got_b, ref_b):
            assert torch.equal(x, y), f"stream b, repeat {rep}: {name}"
