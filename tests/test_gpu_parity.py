"""HIP path vs the fp64 oracle, element by element (needs an MI355X).

Every call goes through the C ABI (libgtr_gla.so) via the thin binding; the
oracle runs on the host on the same seeded inputs.  Gate: max|y - o| / rms(o)
<= 1e-4 for fp32 I/O and <= 1e-2 for fp16 I/O; bf16 I/O is gated on the same
bound after removing the half-ulp that rounding the exact result to bf16
costs by itself (see oracle/compare.py).
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


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def gpu_run(q, k, v, g, direction, **kw):
    args = [x.to(DEV) for x in (q, k, v, g)]
    res = gla.gla_forward(*args, direction, **kw)
    torch.cuda.synchronize()
    return res


def check(q, k, v, g, direction, dtype, label, **kw):
    note(f"{label} dir={direction} dtype={dtype} shape={tuple(q.shape)} {kw}")
    y = gpu_run(q, k, v, g, direction, **kw)
    ref = oracle.gla_forward(q, k, v, g, direction)
    e = parity_errors(y.double().cpu().numpy(), ref, dtype)
    assert e["ok"], f"{label}: {e}"
    return e


# ---- small grids: several tiles, ragged tails, degenerate shapes ---------------------

SMALL_GRIDS = [(1, 1), (1, 63), (1, 65), (8, 8), (7, 9), (5, 13), (9, 17), (13, 11), (3, 100),
               (100, 3), (16, 16)]


PATHS = {"fused": 1, "split": 2}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("direction", [0, 1, 2, 3])
@pytest.mark.parametrize("grid", SMALL_GRIDS, ids=lambda g: f"{g[0]}x{g[1]}")
def test_small_grids(grid, direction, dtype, path):
    gh, gw = grid
    q, k, v, g = gla_inputs.make_inputs(2, 3, gh, gw, 64, 64, dtype, "light",
                                        seed=gh * 1000 + gw * 10 + direction)
    check(q, k, v, g, direction, dtype, f"small {gh}x{gw}", path=PATHS[path], chunks_per_segment=1)


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("seg", [1, 2, 3, 4, 6, 7, 0])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_segment_lengths(seg, dtype, path):
    q, k, v, g = gla_inputs.make_inputs(1, 4, 17, 19, 64, 64, dtype, "heavy", seed=77 + seg)
    check(q, k, v, g, 3, dtype, f"seg_len={seg}", chunks_per_segment=seg, path=PATHS[path])


# ---- the five benchmark workloads at full size, every listed direction ----------------

@pytest.mark.parametrize("path", ["auto", "fused", "split"])
@pytest.mark.parametrize("widx", [1, 2, 3, 4, 5])
def test_workloads_full_size(widx, path):
    w = gla_inputs.workload(widx)
    for layer, d in enumerate(w.directions):
        q, k, v, g = gla_inputs.workload_inputs(w, layer)
        e = check(q, k, v, g, d, w.dtype, w.name, path=PATHS.get(path, 0))
        note(f"  {w.name} dir={d}: err_raw={e['err_raw']:.3g} err_excess={e['err_excess']:.3g}")


# ---- gates that stress the exponent range ------------------------------------------------

@pytest.mark.parametrize("gate", ["ones", "scale:4", "const:-30", "const:-1000", "mixed_extreme",
                                  "const:-0.7"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_extremes(gate, dtype):
    q, k, v, g = gla_inputs.make_inputs(1, 2, 19, 23, 64, 64, dtype, gate, seed=5)
    for d, path in ((0, 1), (2, 2)):
        check(q, k, v, g, d, dtype, f"gate={gate}", path=path, chunks_per_segment=2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_values_near_the_fp16_operand_limits(dtype):
    """16-bit I/O runs on fp16 operands (include/gtr_gla.h, value range).  Close to each limit the
    result still meets the tolerance: |q|, |k| up to ~100 with within-chunk scores up to ~2.5e4 and a
    steep gate whose 16-token products (~2^-14) push the diagonal midpoint factors to ~2^7; then a
    unit gate over 40,960 tokens of positive keys and values, whose state grows to ~2.6e4."""
    cast = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    gen = torch.Generator().manual_seed(31)
    shape = (1, 2, 16, 20, 64)
    q = torch.randn(shape, generator=gen) * 25
    k = torch.randn(shape, generator=gen) * 25
    v = torch.randn(shape, generator=gen)
    g = -0.6 + 0.05 * torch.randn(shape, generator=gen)
    q, k, v, g = (t.to(cast).float().to(cast) for t in (q, k, v, g))
    chunks = [t.float().reshape(2, 320, 64)[:, :256].reshape(2, 4, 64, 64) for t in (q, k)]
    scores = torch.einsum("hctd,hcsd->hcts", *chunks).abs().max()
    assert 5e3 < float(scores) < 6.5e4 and float(q.abs().max()) < 256 and float(k.abs().max()) < 256
    for d in (0, 2):
        check(q, k, v, g, d, dtype, "large q, k, steep gate")
    shape = (1, 1, 160, 256, 64)
    q = torch.randn(shape, generator=gen) / 64
    k = torch.randn(shape, generator=gen).abs()
    v = torch.randn(shape, generator=gen).abs()
    g = torch.zeros(shape)
    q, k, v, g = (t.to(cast) for t in (q, k, v, g))
    _, s_final = oracle.gla_forward(q, k, v, g, 0, want_state=True)
    assert 2e4 < float(np.abs(s_final).max()) < 6.5e4
    for path in (0, 1):
        check(q, k, v, g, 0, dtype, "unit gate, growing state", path=path)


def test_unit_gate_long_sequence():
    """alpha = 1 over 16,384 tokens: the state only grows."""
    q, k, v, g = gla_inputs.make_inputs(1, 2, 128, 128, 64, 64, "f16", "ones", seed=6)
    check(q, k, v, g, 1, "f16", "ones 128x128")


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_state_beyond_the_fp16_range(dtype, path):
    """alpha = 1 with keys near 2 and values near 4 (positive means): every state entry grows by
    about 8 per token and passes 65504 halfway through 16,384 tokens, while queries near 1/256
    keep the outputs in range.  The state reaches the fp16 MFMA operands through an exact power
    of two, so it neither overflows there nor loses precision when small."""
    gen = torch.Generator().manual_seed(77)
    shape = (1, 2, 128, 128, 64)
    q = (torch.randn(shape, generator=gen) / 256).to(gla_inputs.TORCH_DTYPES[dtype])
    k = (2 + 0.1 * torch.randn(shape, generator=gen)).to(gla_inputs.TORCH_DTYPES[dtype])
    v = (4 + 0.1 * torch.randn(shape, generator=gen)).to(gla_inputs.TORCH_DTYPES[dtype])
    g = torch.zeros(shape, dtype=gla_inputs.TORCH_DTYPES[dtype])
    for d in (0, 3):
        e = check(q, k, v, g, d, dtype, f"state beyond fp16 range ({path})", path=PATHS[path])
        assert np.isfinite(e["err_raw"])
    s_end = oracle.gla_forward(q, k, v, g, 0, want_state=True)[1]
    assert np.abs(s_end).max() > 1e5  # the state did leave the fp16 range


# ---- head dims: 64-wide key blocks walked together, value blocks as sequences of their own,
#      narrower heads masked --------------------------------------------------------------

HEAD_DIMS = [(32, 32), (32, 64), (64, 32), (128, 64), (64, 128), (128, 128), (32, 128), (128, 32),
             (4, 8), (96, 76), (124, 4)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("dims", HEAD_DIMS, ids=lambda d: f"dk{d[0]}_dv{d[1]}")
def test_head_dims(dims, dtype):
    dk, dv = dims
    q, k, v, g = gla_inputs.make_inputs(2, 3, 9, 17, dk, dv, dtype, "light", seed=dk * 1000 + dv)
    # (path, chunks per segment); above 64 key dims the one-launch path keeps both key blocks
    runs = [(2, 1), (2, 3), (0, 0), (1, 2)] if dk <= 64 else [(2, 1), (1, 3), (0, 0), (1, 2)]
    for d in range(4):
        path, seg = runs[d % len(runs)]
        check(q, k, v, g, d, dtype, f"dk={dk} dv={dv}", path=path, chunks_per_segment=seg)


@pytest.mark.parametrize("dims", [(128, 64), (64, 128), (32, 96), (128, 128), (100, 36)],
                         ids=lambda d: f"dk{d[0]}_dv{d[1]}")
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_head_dims_state(dims, dtype):
    dk, dv = dims
    B, H, gh, gw = 1, 2, 11, 13
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, dk, dv, dtype, "light", seed=dk + dv)
    s0 = torch.randn(B, H, dk, dv, generator=torch.Generator().manual_seed(dk * dv)) * 0.5
    runs = [(2, 1), (2, 4), (1, 1), (1, 3)]
    for d, (path, seg) in zip(range(4), runs * 2):
        note(f"state dk={dk} dv={dv} dir={d} dtype={dtype} path={path} seg={seg}")
        y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=seg,
                        path=path)
        ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, dtype)["ok"]
        es = parity_errors(sf.double().cpu().numpy(), sref, "f32" if dtype == "f32" else "f16")
        assert es["ok"], es


@pytest.mark.parametrize("gate", ["const:-30", "mixed_extreme", "ones"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_extremes_wide_heads(gate, dtype):
    """The exact diagonal tiles of the second key block, and masked value columns."""
    q, k, v, g = gla_inputs.make_inputs(1, 2, 13, 11, 128, 96, dtype, gate, seed=21)
    for d, seg, path in ((1, 1, 2), (3, 2, 2), (0, 3, 1), (2, 1, 1)):
        check(q, k, v, g, d, dtype, f"wide gate={gate}", path=path, chunks_per_segment=seg)


@pytest.mark.parametrize("dims", [(128, 64), (96, 128)], ids=lambda d: f"dk{d[0]}_dv{d[1]}")
@pytest.mark.parametrize("dtype", DTYPES)
def test_wide_keys_one_launch_long(dims, dtype):
    """Two key blocks on the one-launch path over 4,096 tokens (22 to 64 segments, up to 8 fold
    blocks): both blocks' aggregates, decays and prefixes pass between workgroups; with s0 and
    s_final."""
    dk, dv = dims
    q, k, v, g = gla_inputs.make_inputs(1, 3, 64, 64, dk, dv, dtype, "light", seed=dk + 7 * dv)
    s0 = torch.randn(1, 3, dk, dv, generator=torch.Generator().manual_seed(dk)) * 0.5
    for d, seg in ((0, 3), (3, 1), (2, 2)):
        note(f"wide keys one launch dk={dk} dv={dv} dtype={dtype} dir={d} seg={seg}")
        y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=seg, path=1)
        ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, dtype)["ok"]
        assert parity_errors(sf.double().cpu().numpy(), sref, "f32" if dtype == "f32" else "f16")["ok"]


# ---- initial / final state -----------------------------------------------------------------

@pytest.mark.parametrize("seg", [1, 3])
@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("dtype", DTYPES)
def test_initial_and_final_state(dtype, path, seg):
    B, H, gh, gw = 1, 3, 11, 13
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, dtype, "light", seed=8)
    s0 = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(9)) * 0.5
    for d in range(4):
        note(f"state dir={d} dtype={dtype} seg={seg}")
        y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=seg,
                        path=PATHS[path])
        ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, dtype)["ok"]
        es = parity_errors(sf.double().cpu().numpy(), sref, "f32" if dtype == "f32" else "f16")
        assert es["ok"], es


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("grid", [(8, 8), (11, 13), (7, 9)], ids=lambda g: f"{g[0]}x{g[1]}")
def test_final_state_from_zero(grid, path):
    """Final state with no initial state, including a single segment."""
    gh, gw = grid
    q, k, v, g = gla_inputs.make_inputs(1, 2, gh, gw, 64, 64, "f16", "light", seed=12)
    for seg in (1, 3):
        note(f"final state {gh}x{gw} seg={seg} path={path}")
        y, sf = gpu_run(q, k, v, g, 1, want_state=True, chunks_per_segment=seg, path=PATHS[path])
        ref, sref = oracle.gla_forward(q, k, v, g, 1, want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, "f16")["ok"]
        assert parity_errors(sf.double().cpu().numpy(), sref, "f16")["ok"]


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("dtype", DTYPES)
def test_non_finite_inputs_stay_in_their_sequence(dtype, path):
    """Values outside the domain (NaN, infinities, a positive log-gate) in one head give an
    unspecified result for that head only: the call succeeds, the stream stays healthy, and
    the other heads match the oracle."""
    q, k, v, g = gla_inputs.make_inputs(1, 3, 13, 11, 64, 64, dtype, "light", seed=51)
    ref = oracle.gla_forward(q[:, :2], k[:, :2], v[:, :2], g[:, :2], 3)
    q[0, 2, 1, 2, 5] = float("nan")
    k[0, 2, 4, 4, 0] = float("inf")
    v[0, 2, 7, 1, 9] = float("-inf")
    g[0, 2, 3, 3, 3] = float("nan")
    g[0, 2, 9, 0, :] = 5.0  # alpha > 1
    g[0, 2, 10, 10, 7] = float("-inf")
    note(f"non-finite inputs dtype={dtype} path={path}")
    y = gpu_run(q, k, v, g, 3, path=PATHS[path], chunks_per_segment=1)
    gla.gtr_gla_stream_status()
    e = parity_errors(y[:, :2].double().cpu().numpy(), ref, dtype)
    assert e["ok"], e


@pytest.mark.parametrize("path", sorted(PATHS))
def test_empty_calls(path):
    """No tokens: out is empty and the final state is s0 (or zero); no sequences: nothing happens."""
    s0 = torch.randn(2, 3, 64, 64, generator=torch.Generator().manual_seed(14)).to(DEV)
    x = torch.empty(2, 3, 0, 5, 64, dtype=torch.float16, device=DEV)
    y, sf = gpu_run(x, x, x, x, 0, s0=s0, want_state=True, path=PATHS[path])
    assert y.shape == x.shape and torch.equal(sf, s0)
    y, sf = gpu_run(x, x, x, x, 2, want_state=True, path=PATHS[path])
    assert torch.count_nonzero(sf) == 0
    z = torch.empty(0, 3, 4, 5, 64, dtype=torch.float16, device=DEV)
    assert gpu_run(z, z, z, z, 1, path=PATHS[path]).shape == z.shape


def test_maximum_grid():
    """2^23 tokens (2048 x 4096): 1 GB per tensor, byte offsets up to 2^30.  Outputs depend only on
    earlier scan positions, so the first 4096 positions of every direction are checked against the
    oracle on the truncated grid those positions cover; every output must be finite, and carrying
    the state from the top half into the bottom half must give the whole call's final state."""
    gh, gw = 2048, 4096
    gen = torch.Generator(device=DEV).manual_seed(15)
    shape = (1, 1, gh, gw, 64)
    q = torch.randn(shape, generator=gen, device=DEV).half()
    k = (torch.randn(shape, generator=gen, device=DEV) / 8).half()
    v = torch.randn(shape, generator=gen, device=DEV).half()
    g = (torch.nn.functional.logsigmoid(torch.randn(shape, generator=gen, device=DEV)) / 16).half()
    views = {  # direction -> the grid slice its first 4096 scan positions cover
        0: (slice(0, 1), slice(None)), 1: (slice(gh - 1, gh), slice(None)),
        2: (slice(None), slice(0, 2)), 3: (slice(None), slice(gw - 2, gw)),
    }
    for d, (rs, cs) in views.items():
        note(f"maximum grid dir={d}")
        y = gpu_run(q, k, v, g, d)
        assert bool(torch.isfinite(y).all())
        part = [t[:, :, rs, cs].contiguous().cpu() for t in (q, k, v, g)]
        ref = oracle.gla_forward(*part, d)
        e = parity_errors(y[:, :, rs, cs].double().cpu().numpy(), ref, "f16")
        assert e["ok"], e
        del y
    half = gh // 2
    _, s_whole = gpu_run(q, k, v, g, 0, want_state=True)
    _, s_top = gpu_run(*[t[:, :, :half].contiguous() for t in (q, k, v, g)], 0, want_state=True)
    _, s_bot = gpu_run(*[t[:, :, half:].contiguous() for t in (q, k, v, g)], 0, s0=s_top,
                       want_state=True)
    err = (s_bot - s_whole).abs().max() / s_whole.pow(2).mean().sqrt()
    assert float(err) < 1e-4, float(err)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_maximum_sequence_count(path):
    """B*H = 2^20 sequences (1024 x 1024) of a 1x3 grid: a grid of 2^20 workgroups, and on the
    one-launch path a control line per sequence; sampled sequences are checked against the oracle.
    (The automatic choice takes three launches here: a sequence is one segment.)"""
    B = H = 1024
    gen = torch.Generator(device=DEV).manual_seed(17)
    shape = (B, H, 1, 3, 64)
    q = torch.randn(shape, generator=gen, device=DEV).half()
    k = (torch.randn(shape, generator=gen, device=DEV) / 8).half()
    v = torch.randn(shape, generator=gen, device=DEV).half()
    g = (torch.nn.functional.logsigmoid(torch.randn(shape, generator=gen, device=DEV)) / 16).half()
    assert gla.gtr_gla_plan(B, H, 1, 3, path=PATHS[path])["fused"] == (path == "fused")
    assert not gla.gtr_gla_plan(B, H, 1, 3)["fused"]
    note(f"2^20 sequences path={path}")
    y = gpu_run(q, k, v, g, 1, path=PATHS[path])
    gla.gtr_gla_stream_status()
    rows = torch.tensor([0, 1, 511, 777, 1023])
    part = [t[rows][:, rows].cpu() for t in (q, k, v, g)]  # 25 sequences spread over B and H
    ref = oracle.gla_forward(*part, 1)
    e = parity_errors(y[rows][:, rows].double().cpu().numpy(), ref, "f16")
    assert e["ok"], e
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("grid", [(80, 81), (150, 128), (200, 200)], ids=lambda g: f"{g[0]}x{g[1]}")
def test_long_boundary_scans(grid, path):
    """One-chunk segments on long sequences (102, 300 and 625 chunks): boundary scans of
    hundreds of steps, with s0 and s_final, in fp32.  On the one-launch path the segments form
    13 to 79 fold blocks of at most 8, and the state passes from block to block."""
    gh, gw = grid
    q, k, v, g = gla_inputs.make_inputs(1, 2, gh, gw, 64, 64, "f32", "light", seed=gh + gw)
    s0 = torch.randn(1, 2, 64, 64, generator=torch.Generator().manual_seed(gh)) * 0.5
    for d in (0, 3):
        note(f"long scan {gh}x{gw} dir={d} path={path}")
        y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=1,
                        path=PATHS[path])
        ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, "f32")["ok"]
        assert parity_errors(sf.double().cpu().numpy(), sref, "f32")["ok"]


@pytest.mark.parametrize("seg", [1, 2, 3])
def test_long_sequence_state_16bit_one_launch(seg):
    """The one-launch path at 16-bit I/O over 12,800 tokens (200 chunks: 67 to 200 segments,
    9 to 25 fold blocks) with s0 and s_final."""
    q, k, v, g = gla_inputs.make_inputs(1, 3, 100, 128, 64, 64, "f16", "light", seed=40 + seg)
    s0 = torch.randn(1, 3, 64, 64, generator=torch.Generator().manual_seed(seg)) * 0.5
    for d in (1, 2):
        note(f"one-launch state 100x128 seg={seg} dir={d}")
        y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=seg, path=1)
        ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
        assert parity_errors(y.double().cpu().numpy(), ref, "f16")["ok"]
        assert parity_errors(sf.double().cpu().numpy(), sref, "f16")["ok"]


def test_split_sequence_equals_whole():
    """Top rows then bottom rows with the state carried equals one L->R call."""
    B, H, gh, gw, r = 1, 2, 40, 40, 17
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, "f32", "light", seed=10)
    whole = gpu_run(q, k, v, g, 0)
    top, s_mid = gpu_run(q[:, :, :r].contiguous(), k[:, :, :r].contiguous(),
                         v[:, :, :r].contiguous(), g[:, :, :r].contiguous(), 0, want_state=True)
    bot = gpu_run(q[:, :, r:].contiguous(), k[:, :, r:].contiguous(), v[:, :, r:].contiguous(),
                  g[:, :, r:].contiguous(), 0, s0=s_mid)
    joined = torch.cat([top, bot], dim=2)
    ref = oracle.gla_forward(q, k, v, g, 0)
    assert parity_errors(joined.double().cpu().numpy(), ref, "f32")["ok"]
    assert parity_errors(whole.double().cpu().numpy(), ref, "f32")["ok"]


# ---- execution properties ------------------------------------------------------------------

@pytest.mark.parametrize("path", sorted(PATHS))
def test_deterministic_bitwise(path):
    q, k, v, g = (x.to(DEV) for x in gla_inputs.make_inputs(1, 4, 40, 40, 64, 64, "f16", "light",
                                                              seed=11))
    outs = [gla.gla_forward(q, k, v, g, 2, path=PATHS[path], chunks_per_segment=2)
            for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_deterministic_bitwise_wide_heads():
    """Two key blocks and two value blocks (d_k = 128, d_v = 96): repeated calls are bitwise equal."""
    q, k, v, g = (x.to(DEV) for x in gla_inputs.make_inputs(1, 3, 23, 29, 128, 96, "bf16", "light",
                                                              seed=22))
    outs = [gla.gla_forward(q, k, v, g, 3, chunks_per_segment=2) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_streams_run_concurrently_with_their_own_workspaces():
    """Calls in flight on two streams at once (each stream has its own workspace) give the results
    of the same calls made one after the other; no one-launch wait gives up."""
    w = gla_inputs.workload(3)
    ins = [[x.to(DEV) for x in gla_inputs.workload_inputs(w, layer)] for layer in range(2)]
    ref = [gla.gla_forward(*ins[i], w.directions[i], path=path) for i, path in ((0, 1), (1, 2))]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in ref]
    for rep in range(20):
        for i, path in ((0, 1), (1, 2)):
            with torch.cuda.stream(streams[i]):
                gla.gtr_gla_fwd_ex(*ins[i], outs[i], w.directions[i], path=path, stream=streams[i])
    for i in range(2):
        gla.gtr_gla_stream_status(streams[i])
        assert torch.equal(outs[i], ref[i])


def test_fused_repeated_calls_are_identical():
    """Many fused calls in a row (segments wait on each other's flags) give bitwise-equal results."""
    w = gla_inputs.workload(3)
    q, k, v, g = (x.to(DEV) for x in gla_inputs.workload_inputs(w, 0))
    first = gla.gla_forward(q, k, v, g, 2, path=1)
    torch.cuda.synchronize()
    ref = oracle.gla_forward(*gla_inputs.workload_inputs(w, 0), 2)
    assert parity_errors(first.double().cpu().numpy(), ref, "f16")["ok"]
    out = torch.empty_like(first)
    for i in range(60):
        gla.gtr_gla_fwd_ex(q, k, v, g, out, 2, path=1, chunks_per_segment=1 + i % 3)
        if i % 3 == 1:  # a different segmentation only reorders fp32 sums: compare to the oracle
            torch.cuda.synchronize()
            assert parity_errors(out.double().cpu().numpy(), ref, "f16")["ok"], i
    gla.gtr_gla_fwd_ex(q, k, v, g, out, 2, path=1)
    gla.gtr_gla_stream_status()  # no wait between workgroups gave up
    assert torch.equal(out, first)


@pytest.mark.parametrize("shape", [(1, 12, 64, 64, 2), (1, 12, 64, 64, 1), (1, 4, 64, 64, 3), (1, 6, 40, 40, 1),
                                   (1, 9, 40, 40, 2), (3, 1, 33, 31, 1)],
                         ids=lambda s: "B{}H{}_{}x{}_seg{}".format(*s))
def test_one_launch_with_fewer_batches_than_xcds(shape):
    """The one-launch path with fewer sequence batches than XCDs: an XCD without a batch of its
    own takes over, at launch, one whose XCD has not begun, and works it with all its workgroups.
    Whoever works a batch, the outputs match the oracle, no wait gives up, and a second call is
    bitwise the same."""
    B, H, gh, gw, seg = shape
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, "f16", "light", seed=H + gh + seg)
    ref = oracle.gla_forward(q, k, v, g, 3)
    note(f"few batches {shape}")
    y = gpu_run(q, k, v, g, 3, chunks_per_segment=seg, path=1)
    gla.gtr_gla_stream_status()
    assert parity_errors(y.double().cpu().numpy(), ref, "f16")["ok"]
    y2 = gpu_run(q, k, v, g, 3, chunks_per_segment=seg, path=1)
    gla.gtr_gla_stream_status()
    assert torch.equal(y, y2)


# (B, H, grid, dtype, the segment length the automatic choice takes for that type)
AUTO_SHAPES = [(4, 6, (24, 24), "f16", 1), (1, 16, (48, 48), "bf16", 2), (32, 6, (16, 16), "f16", 2),
               (16, 6, (32, 32), "f16", 3), (4, 6, (32, 32), "f32", 2), (1, 8, (40, 40), "f16", 1),
               (2, 8, (9, 13), "f16", 1), (16, 8, (8, 16), "bf16", 1)]  # 2 chunks, the first ragged


@pytest.mark.parametrize("case", AUTO_SHAPES, ids=lambda c: f"B{c[0]}H{c[1]}_{c[2][0]}x{c[2][1]}_{c[3]}")
def test_automatic_one_launch_shapes(case):
    """Shapes for which the automatic choice takes the one launch with 1-, 2- or 3-chunk segments:
    parity with the oracle, and bitwise the same as an explicit call with that plan."""
    B, H, (gh, gw), dtype, seg = case
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, dtype, "light", seed=B * H + gh)
    for direction in (0, 2):
        note(f"auto {case} dir={direction}")
        y = gpu_run(q, k, v, g, direction)
        ref = oracle.gla_forward(q, k, v, g, direction)
        e = parity_errors(y.double().cpu().numpy(), ref, dtype)
        assert e["ok"], (case, direction, e)
        explicit = gpu_run(q, k, v, g, direction, chunks_per_segment=seg, path=1)
        gla.gtr_gla_stream_status()
        assert torch.equal(y, explicit), case


def test_paths_agree_and_repeat_on_one_workspace():
    """Different shapes and both paths back to back on one stream reuse one workspace."""
    shapes = [(1, 6, 40, 40, 1), (2, 3, 17, 19, 3), (1, 6, 40, 40, 2), (1, 2, 64, 64, 1),
              (2, 3, 17, 19, 1)]
    for B, H, gh, gw, seg in shapes:
        q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, "f16", "light", seed=B + gh)
        ref = oracle.gla_forward(q, k, v, g, 1)
        for path in (1, 2, 1):
            note(f"reuse {B}x{H}x{gh}x{gw} seg={seg} path={path}")
            y = gpu_run(q, k, v, g, 1, chunks_per_segment=seg, path=path)
            assert parity_errors(y.double().cpu().numpy(), ref, "f16")["ok"]


def test_non_default_stream_and_graph_replay():
    w = gla_inputs.workload(2)
    ins = [[x.to(DEV) for x in gla_inputs.workload_inputs(w, l)] for l in range(4)]
    outs = [torch.empty_like(i[2]) for i in ins]
    s = torch.cuda.Stream()
    eager = []
    with torch.cuda.stream(s):
        for (q, k, v, g), d in zip(ins, w.directions):
            eager.append(gla.gla_forward(q, k, v, g, d, stream=s))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):  # warm the capture stream's workspace first
        for (q, k, v, g), d, o in zip(ins, w.directions, outs):
            gla.gtr_gla_fwd(q, k, v, g, o, d, stream=cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        for (q, k, v, g), d, o in zip(ins, w.directions, outs):
            gla.gtr_gla_fwd(q, k, v, g, o, d, stream=cap)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from eager"
        # unrelated eager work between replays
        gla.gla_forward(*ins[0], 0)
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", sorted(PATHS))
def test_graph_replays_after_workspace_growth(path):
    """A graph keeps the workspace it was captured with: a larger eager call on the same
    stream grows the workspace into new buffers, and the graph's still hold its data."""
    p = PATHS[path]
    small = [x.to(DEV) for x in gla_inputs.make_inputs(1, 6, 24, 24, 64, 64, "f16", "light", seed=21)]
    big = [x.to(DEV) for x in gla_inputs.make_inputs(4, 8, 40, 40, 64, 64, "f16", "light", seed=22)]
    out = torch.empty_like(small[2])
    cap = torch.cuda.Stream()
    note(f"graph after growth path={path}")
    with torch.cuda.stream(cap):
        gla.gtr_gla_fwd_ex(*small, out, 1, chunks_per_segment=1, path=p, stream=cap)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        gla.gtr_gla_fwd_ex(*small, out, 1, chunks_per_segment=1, path=p, stream=cap)
    for rep in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} before growth"
        # more segments and sequences than the capture: the workspace grows
        big_out = torch.empty_like(big[2])
        with torch.cuda.stream(cap):
            gla.gtr_gla_fwd_ex(*big, big_out, 1, chunks_per_segment=1, path=p, stream=cap)
        torch.cuda.synchronize()
        big = [torch.cat([x, x[:1]]) for x in big]  # one more batch row next time round
    out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager), "replay after growth"
    del graph
    gla.gtr_gla_release_workspaces()
    y = gla.gla_forward(*small, 1, chunks_per_segment=1, path=p, stream=cap)
    torch.cuda.synchronize()
    assert torch.equal(y, eager), "call after release"


@pytest.mark.parametrize("path", sorted(PATHS))
def test_workspace_allocation_failure(path, monkeypatch):
    """GTR_GLA_TEST_FAIL_ALLOC=1 makes every workspace allocation fail: the call returns
    GTR_ERR_ALLOC and runs nothing, and the stream's cached workspace stays usable."""
    p = PATHS[path]
    small = gla_inputs.make_inputs(1, 2, 20, 21, 64, 64, "f16", "light", seed=41)
    big = [x.to(DEV) for x in gla_inputs.make_inputs(2, 4, 30, 31, 64, 64, "f16", "light", seed=42)]
    ref = oracle.gla_forward(*small, 2)
    small = [x.to(DEV) for x in small]
    s = torch.cuda.Stream()  # no workspace yet
    note(f"allocation failure path={path}")

    def run(ins, out):
        gla.gtr_gla_fwd_ex(*ins, out, 2, chunks_per_segment=1, path=p, stream=s)
        torch.cuda.synchronize()

    out = torch.full_like(small[2], float("nan"))
    monkeypatch.setenv("GTR_GLA_TEST_FAIL_ALLOC", "1")
    with pytest.raises(gla.GlaError) as ex:
        run(small, out)
    assert ex.value.code == -7 and "hipMalloc" in str(ex.value)
    assert torch.isnan(out).all(), "a refused call ran"
    monkeypatch.delenv("GTR_GLA_TEST_FAIL_ALLOC")
    run(small, out)
    assert parity_errors(out.double().cpu().numpy(), ref, "f16")["ok"]
    first = out.clone()
    # growing fails, and the workspace the stream has keeps serving calls that fit it
    monkeypatch.setenv("GTR_GLA_TEST_FAIL_ALLOC", "1")
    big_out = torch.full_like(big[2], float("nan"))
    with pytest.raises(gla.GlaError) as ex:
        run(big, big_out)
    assert ex.value.code == -7 and torch.isnan(big_out).all()
    out.fill_(float("nan"))
    run(small, out)
    assert torch.equal(out, first)
    monkeypatch.delenv("GTR_GLA_TEST_FAIL_ALLOC")
    run(big, big_out)
    assert not torch.isnan(big_out).any()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the one launch is refused
def test_capture_refuses_workspace_growth():
    q, k, v, g = (x.to(DEV) for x in gla_inputs.make_inputs(1, 2, 30, 31, 64, 64, "f16", "light",
                                                              seed=12))
    out = torch.empty_like(v)
    fresh = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(graph, stream=fresh):
        try:
            gla.gtr_gla_fwd_ex(q, k, v, g, out, 0, chunks_per_segment=1, path=2, stream=fresh)
        except gla.GlaError as ex:
            err = ex
    assert err is not None and err.code == -8


def test_pointer_checks_on_gpu():
    """Host-side pointer checks, exercised through gtr_gla_check, which launches nothing."""
    L = gla.lib()
    q, k, v, g = (x.to(DEV) for x in gla_inputs.make_inputs(1, 1, 8, 8, 64, 64, "f16", "light",
                                                              seed=13))
    out = torch.empty_like(v)
    pinned = torch.empty_like(v, device="cpu").pin_memory()
    plain_host = np.zeros(8 * 8 * 64 + 16, dtype=np.float16)
    host_ptr = (plain_host.ctypes.data + 15) // 16 * 16

    def chk(o, gh=8, gw=8):
        return L.gtr_gla_check(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), o, 1, 1, gh,
                               gw, 64, 64, 0, 1, None, None, 0, 0)

    assert chk(out.data_ptr()) == 0
    assert chk(host_ptr) == -6
    assert chk(pinned.data_ptr()) == -6
    # an output allocation half the size the tensor needs (a raw hipMalloc, so that
    # no caching-allocator segment around it hides the shortfall)
    import ctypes
    hip = ctypes.CDLL(gla.hip_runtimes_mapped()[0])
    raw = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(raw), ctypes.c_size_t(4096)) == 0
    try:
        assert chk(raw.value) == -6
    finally:
        hip.hipFree(raw)
    torch.cuda.synchronize()


def test_profiling_counts_launches():
    q, k, v, g = (x.to(DEV) for x in gla_inputs.make_inputs(1, 2, 40, 40, 64, 64, "f16", "light",
                                                              seed=14))
    gla.gtr_gla_profile_begin()
    for _ in range(3):
        gla.gla_forward(q, k, v, g, 0, chunks_per_segment=5, path=2)
    for _ in range(2):
        gla.gla_forward(q, k, v, g, 0, chunks_per_segment=5, path=1)
    prof = gla.gtr_gla_profile_end()
    assert prof["gla_seg_out"][1] == 3 and prof["gla_seg_state"][1] == 3
    assert prof["gla_seg_scan"][1] == 3 and prof["gla_fused"][1] == 2
    assert all(ms > 0 for ms, n in prof.values() if n > 0)


def test_single_runtime_and_library_loaded():
    gla.lib()
    assert len(gla.hip_runtimes_mapped()) == 1
    with open("/proc/self/maps") as f:
        assert any("libgtr_gla.so" in ln for ln in f)


@pytest.mark.parametrize("dtype", DTYPES)
def test_boundary_scan_across_lanes(dtype, monkeypatch):
    """The boundary scan as a scan across the lanes of a wave (GTR_GLA_SCAN=lanes, off by
    default because it is slower): outputs and final states against the oracle, with and
    without an initial state, over several segment counts, in every direction."""
    monkeypatch.setenv("GTR_GLA_SCAN", "lanes")
    B, H, gh, gw = 1, 3, 23, 29
    q, k, v, g = gla_inputs.make_inputs(B, H, gh, gw, 64, 64, dtype, "light", seed=91)
    s0 = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(92)) * 0.5
    for seg in (1, 2, 5, 11):
        for d in range(4):
            note(f"lane scan seg={seg} dir={d} dtype={dtype}")
            y, sf = gpu_run(q, k, v, g, d, s0=s0.to(DEV), want_state=True, chunks_per_segment=seg,
                            path=PATHS["split"])
            ref, sref = oracle.gla_forward(q, k, v, g, d, s0=s0.double().numpy(), want_state=True)
            assert parity_errors(y.double().cpu().numpy(), ref, dtype)["ok"]
            es = parity_errors(sf.double().cpu().numpy(), sref, "f32" if dtype == "f32" else "f16")
            assert es["ok"], es
            y2 = gpu_run(q, k, v, g, d, chunks_per_segment=seg, path=PATHS["split"])
            assert parity_errors(y2.double().cpu().numpy(), oracle.gla_forward(q, k, v, g, d), dtype)["ok"]
