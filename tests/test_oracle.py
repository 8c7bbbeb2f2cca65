"""Pins for the fp64 oracle (CPU only).

The pages print no worked example for the operator, so every pin here comes
from mathematics that the pages' description fixes: the closed-form masked sum
of the recurrence, the reduction to causal linear attention when the gate is
one, flip/transpose identities between scan directions, independence from the
chunk size used to evaluate it, hand-derived tiny cases, causality and
linearity.  Each test is chosen so that a plausible slip in the oracle (current
token dropped, decay after the write, gate sign, gate on the value side, a
transposed operand, a wrong scan order) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def rand_inputs(rng, B, H, gh, gw, dk, dv, gate_scale=0.3):
    q = rng.standard_normal((B, H, gh, gw, dk))
    k = rng.standard_normal((B, H, gh, gw, dk)) / math.sqrt(dk)
    v = rng.standard_normal((B, H, gh, gw, dv))
    g = -gate_scale * rng.random((B, H, gh, gw, dk))  # log alpha in (-gate_scale, 0]
    return q, k, v, g


# ---- independent scan orders (numpy flips / transposes, not the C map) ----------

def order_np(gh, gw, direction):
    grid = np.arange(gh * gw).reshape(gh, gw)
    if direction == 0:
        return grid.reshape(-1)
    if direction == 1:
        return grid.reshape(-1)[::-1]
    if direction == 2:
        return grid.T.reshape(-1)
    if direction == 3:
        return grid.T.reshape(-1)[::-1]
    raise ValueError(direction)


def to_seq(x, order):
    """[..., gh, gw, d] -> [..., N, d] in scan order."""
    s = x.reshape(x.shape[:-3] + (-1, x.shape[-1]))
    return s[..., order, :]


def from_seq(y, order, gh, gw):
    out = np.empty_like(y)
    out[..., order, :] = y
    return out.reshape(y.shape[:-2] + (gh, gw, y.shape[-1]))


def closed_form(q, k, v, g, direction):
    """o_t = sum_{s<=t} sum_i q_ti k_si exp(G_ti - G_si) v_s, G = inclusive cumsum of log alpha."""
    B, H, gh, gw, dk = q.shape
    order = order_np(gh, gw, direction)
    qs, ks, vs, gs = (to_seq(x, order) for x in (q, k, v, g))
    G = np.cumsum(gs, axis=-2)
    N = gh * gw
    out = np.zeros(vs.shape)
    for t in range(N):
        for s in range(t + 1):
            w = np.sum(qs[..., t, :] * ks[..., s, :] * np.exp(G[..., t, :] - G[..., s, :]), axis=-1)
            out[..., t, :] += w[..., None] * vs[..., s, :]
    return from_seq(out, order, gh, gw)


# ---- scan orders -----------------------------------------------------------------

def read_golden_orders():
    rows = []
    with open(os.path.join(GOLDEN, "scan_orders.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, tail = line.split(":")
            gh, gw, d = (int(x) for x in head.split())
            rows.append((gh, gw, d, [int(x) for x in tail.split()]))
    return rows


def test_scan_orders_match_hand_written_fixture():
    rows = read_golden_orders()
    assert len(rows) >= 8
    for gh, gw, d, idx in rows:
        assert oracle.scan_order(gh, gw, d) == idx, (gh, gw, d)
        assert list(order_np(gh, gw, d)) == idx, (gh, gw, d)


@pytest.mark.parametrize("gh,gw", [(1, 1), (3, 5), (5, 3), (4, 4), (1, 7), (7, 1)])
@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_scan_order_is_a_permutation(gh, gw, d):
    o = oracle.scan_order(gh, gw, d)
    assert sorted(o) == list(range(gh * gw))
    assert oracle.scan_index(gh * gw, gh, gw, d) == -1
    assert oracle.scan_index(-1, gh, gw, d) == -1


# ---- (i) closed-form masked sum ------------------------------------------------------

@pytest.mark.parametrize("gh,gw", [(1, 1), (1, 7), (7, 1), (3, 5), (5, 3), (4, 4)])
@pytest.mark.parametrize("dk,dv", [(1, 1), (3, 2), (8, 8)])
@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_matches_closed_form(gh, gw, dk, dv, direction):
    rng = np.random.default_rng(100 * gh + 10 * gw + dk + direction)
    q, k, v, g = rand_inputs(rng, 1, 2, gh, gw, dk, dv, gate_scale=1.0)
    got = oracle.gla_forward(q, k, v, g, direction)
    ref = closed_form(q, k, v, g, direction)
    assert rel(got, ref) <= 1e-12


# ---- (ii) all-ones gate reduces to causal linear attention ----------------------------

@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_unit_gate_is_causal_linear_attention(direction):
    rng = np.random.default_rng(7 + direction)
    gh, gw, dk, dv = 6, 5, 8, 4
    q, k, v, _ = rand_inputs(rng, 2, 1, gh, gw, dk, dv)
    g = np.zeros_like(q)
    got = oracle.gla_forward(q, k, v, g, direction)
    order = order_np(gh, gw, direction)
    qs, ks, vs = (to_seq(x, order) for x in (q, k, v))
    scores = np.tril(qs @ np.swapaxes(ks, -1, -2))
    ref = from_seq(scores @ vs, order, gh, gw)
    assert rel(got, ref) <= 1e-12


# ---- (iii) directions are flips / transposes of each other ---------------------------

def rot180(x):
    return x[..., ::-1, ::-1, :].copy()


def transp(x):
    return np.ascontiguousarray(np.swapaxes(x, -3, -2))


@pytest.mark.parametrize("gh,gw", [(5, 7), (3, 8), (1, 6), (6, 1)])
def test_direction_identities(gh, gw):
    rng = np.random.default_rng(gh * 31 + gw)
    q, k, v, g = rand_inputs(rng, 1, 2, gh, gw, 4, 3)
    o = {d: oracle.gla_forward(q, k, v, g, d) for d in range(4)}
    lr_rot = oracle.gla_forward(rot180(q), rot180(k), rot180(v), rot180(g), 0)
    assert np.array_equal(o[1], rot180(lr_rot))
    lr_t = oracle.gla_forward(transp(q), transp(k), transp(v), transp(g), 0)
    assert np.array_equal(o[2], transp(lr_t))
    rl_t = oracle.gla_forward(transp(q), transp(k), transp(v), transp(g), 1)
    assert np.array_equal(o[3], transp(rl_t))


def test_reversal_reading_differs_from_row_mirror_reading():
    """Guard: full reversal (the reading used) and a per-row mirror are different layers."""
    rng = np.random.default_rng(3)
    gh, gw = 4, 5
    q, k, v, g = rand_inputs(rng, 1, 1, gh, gw, 4, 4)
    rl = oracle.gla_forward(q, k, v, g, 1)
    mirror = oracle.gla_forward(q[..., ::-1, :].copy(), k[..., ::-1, :].copy(),
                                v[..., ::-1, :].copy(), g[..., ::-1, :].copy(), 0)[..., ::-1, :]
    assert rel(rl, mirror) > 0.1


# ---- (iv) independence from chunk size: a chunked fp64 evaluation --------------------

def chunked(q, k, v, g, direction, C, sub=None):
    """Chunkwise evaluation in fp64.

    Per chunk: Gam = inclusive cumsum of log alpha from the chunk start;
    o = (q*e^Gam) S_prev + causal intra-chunk sum; S_next = diag(e^Gam_last) S_prev
    + (k*e^(Gam_last-Gam))^T V.  With ``sub`` the intra-chunk scores are formed
    per sub-block pair with bounded factors: queries referenced at their
    sub-block start, keys at their sub-block end, a per-key-dim factor between
    the two references, and the diagonal sub-blocks referenced at their
    midpoint.
    """
    B, H, gh, gw, dk = q.shape
    order = order_np(gh, gw, direction)
    qs, ks, vs, gs = (to_seq(x, order) for x in (q, k, v, g))
    N = gh * gw
    out = np.zeros(vs.shape)
    S = np.zeros((B, H, dk, vs.shape[-1]))
    for c0 in range(0, N, C):
        sl = slice(c0, min(c0 + C, N))
        Q, K, V, Gm = qs[..., sl, :], ks[..., sl, :], vs[..., sl, :], np.cumsum(gs[..., sl, :], axis=-2)
        L = Q.shape[-2]
        o = (Q * np.exp(Gm)) @ S
        if sub is None:
            A = np.einsum("bhti,bhsi,bhtsi->bhts", Q, K,
                          np.exp(np.minimum(Gm[..., :, None, :] - Gm[..., None, :, :], 0.0)))
            A = A * np.tril(np.ones((L, L)))
        else:
            A = np.zeros(Q.shape[:-2] + (L, L))
            starts = list(range(0, L, sub))
            ref_start = [Gm[..., s - 1, :] if s > 0 else np.zeros_like(Gm[..., 0, :]) for s in starts]
            ref_end = [Gm[..., min(s + sub, L) - 1, :] for s in starts]
            for a, sa in enumerate(starts):
                ta = slice(sa, min(sa + sub, L))
                Qa = Q[..., ta, :] * np.exp(Gm[..., ta, :] - ref_start[a][..., None, :])
                for b in range(a + 1):
                    sb = starts[b]
                    tb = slice(sb, min(sb + sub, L))
                    Kb = K[..., tb, :] * np.exp(ref_end[b][..., None, :] - Gm[..., tb, :])
                    if b < a:
                        c = np.exp(ref_start[a] - ref_end[b])        # <= 1
                        A[..., ta, tb] = (Qa * c[..., None, :]) @ np.swapaxes(Kb, -1, -2)
                    else:
                        h = np.exp(0.5 * (ref_start[a] - ref_end[a]))  # >= 1, midpoint
                        blk = (Qa * h[..., None, :]) @ np.swapaxes(Kb * h[..., None, :], -1, -2)
                        A[..., ta, tb] = np.tril(blk)
        o = o + A @ V
        out[..., sl, :] = o
        last = Gm[..., -1, :]
        S = np.exp(last)[..., :, None] * S + np.swapaxes(K * np.exp(last[..., None, :] - Gm), -1, -2) @ V
    return from_seq(out, order, gh, gw)


@pytest.mark.parametrize("C", [1, 3, 7, 8, 16, 64, 200])
@pytest.mark.parametrize("direction", [0, 3])
def test_chunk_size_independence(C, direction):
    rng = np.random.default_rng(C + 10 * direction)
    q, k, v, g = rand_inputs(rng, 1, 2, 10, 13, 8, 6, gate_scale=0.8)
    ref = oracle.gla_forward(q, k, v, g, direction)
    assert rel(chunked(q, k, v, g, direction, C), ref) <= 1e-12


@pytest.mark.parametrize("C,sub", [(64, 16), (64, 4), (16, 16), (64, 1), (64, 3), (7, 2), (128, 16)])
def test_sub_block_referenced_chunk_algebra(C, sub):
    """The bounded-factor form of the intra-chunk sum reaches the same result."""
    rng = np.random.default_rng(C * 7 + sub)
    q, k, v, g = rand_inputs(rng, 1, 1, 9, 17, 8, 8, gate_scale=0.6)
    ref = oracle.gla_forward(q, k, v, g, 2)
    assert rel(chunked(q, k, v, g, 2, C, sub=sub), ref) <= 1e-12


# ---- special cases --------------------------------------------------------------------

def test_hand_worked_scalar_example():
    """d_k = d_v = 1, two tokens, worked by hand from S_t = a_t S_{t-1} + k_t v_t, o_t = q_t S_t:
    o_0 = q_0 k_0 v_0 = 2*1*4 = 8;  o_1 = q_1 (a_1 k_0 v_0 + k_1 v_1) = 3*(0.25*4 - 5) = -12."""
    q = np.array([2.0, 3.0]).reshape(1, 1, 1, 2, 1)
    k = np.array([1.0, -1.0]).reshape(1, 1, 1, 2, 1)
    v = np.array([4.0, 5.0]).reshape(1, 1, 1, 2, 1)
    g = np.log(np.array([0.5, 0.25])).reshape(1, 1, 1, 2, 1)
    out = oracle.gla_forward(q, k, v, g, 0).reshape(-1)
    assert out[0] == pytest.approx(8.0, abs=1e-14)
    assert out[1] == pytest.approx(-12.0, abs=1e-14)
    # right-to-left visits token 1 first: o_1 = 3*(-1)*5 = -15, o_0 = 2*(0.5*(-5) + 4) = 3
    out = oracle.gla_forward(q, k, v, g, 1).reshape(-1)
    assert out[1] == pytest.approx(-15.0, abs=1e-14)
    assert out[0] == pytest.approx(3.0, abs=1e-14)


def test_single_token_is_qk_times_v():
    rng = np.random.default_rng(11)
    q, k, v, g = rand_inputs(rng, 2, 3, 1, 1, 5, 7)
    out = oracle.gla_forward(q, k, v, g, 2)
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    assert rel(out, ref) <= 1e-14


def test_vanishing_gate_keeps_only_current_token():
    rng = np.random.default_rng(12)
    q, k, v, _ = rand_inputs(rng, 1, 2, 4, 6, 8, 5)
    g = np.full_like(q, -80.0)
    out = oracle.gla_forward(q, k, v, g, 0)
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    assert rel(out, ref) <= 1e-15 * 1e3


def test_constant_gate_geometric_series():
    """Scalar state with log alpha = c: o_t = q_t * sum_{s<=t} e^{c (t-s)} k_s v_s."""
    rng = np.random.default_rng(13)
    N, c = 9, -0.37
    q = rng.standard_normal(N)
    k = rng.standard_normal(N)
    v = rng.standard_normal(N)
    out = oracle.gla_forward(q.reshape(1, 1, 1, N, 1), k.reshape(1, 1, 1, N, 1), v.reshape(1, 1, 1, N, 1),
                             np.full((1, 1, 1, N, 1), c), 0).reshape(-1)
    ref = [q[t] * sum(math.exp(c * (t - s)) * k[s] * v[s] for s in range(t + 1)) for t in range(N)]
    assert rel(out, ref) <= 1e-14


def test_gate_acts_on_key_dims_only():
    """Gate one key dim to zero: that dim keeps only the current token; other dims are untouched."""
    rng = np.random.default_rng(14)
    q, k, v, g = rand_inputs(rng, 1, 1, 3, 4, 3, 5)
    g = np.zeros_like(g)
    g[..., 0] = -200.0
    out = oracle.gla_forward(q, k, v, g, 0)
    qs, ks, vs = (to_seq(x, order_np(3, 4, 0))[0, 0] for x in (q, k, v))
    ref = np.zeros_like(vs)
    for t in range(12):
        ref[t] = qs[t, 0] * ks[t, 0] * vs[t] + (qs[t, 1:] @ (ks[: t + 1, 1:].T @ vs[: t + 1]))
    assert rel(out[0, 0].reshape(12, -1), ref) <= 1e-13


def test_causality_and_linearity():
    rng = np.random.default_rng(15)
    gh, gw = 5, 6
    q, k, v, g = rand_inputs(rng, 1, 1, gh, gw, 6, 6)
    for d in range(4):
        base = oracle.gla_forward(q, k, v, g, d)
        order = oracle.scan_order(gh, gw, d)
        t0 = 17
        n = order[t0]
        r, c = divmod(n, gw)
        k2, v2, g2 = k.copy(), v.copy(), g.copy()
        k2[0, 0, r, c] += 1.0
        v2[0, 0, r, c] -= 2.0
        g2[0, 0, r, c] -= 0.5
        pert = oracle.gla_forward(q, k2, v2, g2, d)
        for t in range(gh * gw):
            rr, cc = divmod(order[t], gw)
            same = np.array_equal(base[0, 0, rr, cc], pert[0, 0, rr, cc])
            assert same == (t < t0), (d, t)
    # linear in v and in q
    v_b = rng.standard_normal(v.shape)
    o1 = oracle.gla_forward(q, k, v, g, 2)
    o2 = oracle.gla_forward(q, k, v_b, g, 2)
    o12 = oracle.gla_forward(q, k, 2.0 * v - 3.0 * v_b, g, 2)
    assert rel(o12, 2.0 * o1 - 3.0 * o2) <= 1e-13
    o3 = oracle.gla_forward(-0.5 * q, k, v, g, 2)
    assert rel(o3, -0.5 * o1) <= 1e-14


def test_initial_and_final_state_split_the_sequence():
    """Running rows [0, r) then rows [r, gh) with the state carried equals one L->R pass."""
    rng = np.random.default_rng(16)
    gh, gw, r = 7, 5, 3
    q, k, v, g = rand_inputs(rng, 2, 2, gh, gw, 6, 4)
    full, s_full = oracle.gla_forward(q, k, v, g, 0, want_state=True)
    top, s_top = oracle.gla_forward(q[:, :, :r], k[:, :, :r], v[:, :, :r], g[:, :, :r], 0, want_state=True)
    bot, s_bot = oracle.gla_forward(q[:, :, r:], k[:, :, r:], v[:, :, r:], g[:, :, r:], 0, s0=s_top,
                                    want_state=True)
    assert rel(np.concatenate([top, bot], axis=2), full) <= 1e-13
    assert rel(s_bot, s_full) <= 1e-13
    # with k = 0 the initial state only decays: o_t = q_t diag(prod alpha) S_0
    k0 = np.zeros_like(k)
    s0 = rng.standard_normal(s_full.shape)
    out = oracle.gla_forward(q, k0, v, g, 0, s0=s0)
    G = np.cumsum(to_seq(g, order_np(gh, gw, 0)), axis=-2)
    ref = np.einsum("bhti,bhij->bhtj", to_seq(q, order_np(gh, gw, 0)) * np.exp(G), s0)
    assert rel(out.reshape(ref.shape), ref) <= 1e-13


def test_argument_errors():
    z = np.zeros((1, 1, 1, 1, 1))
    with pytest.raises(ValueError):
        oracle.gla_forward(z, z, z, z, 4)
    with pytest.raises(ValueError):
        oracle.gla_forward(z, z, z, np.zeros((1, 1, 1, 2, 1)), 0)
    out, threads = oracle.gla_forward(z, z, z, z, 0, return_threads=True)
    assert threads == 1 and out.shape == (1, 1, 1, 1, 1)
