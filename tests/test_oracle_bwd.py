"""Pins for the fp64 backward oracle (CPU only).

The backward pass is fixed by the forward recurrence, so its pins come from
that: central finite differences of the (separately pinned) forward oracle for
every input, including the initial state and a loss on the final state; the
identity dlog_gate_t = sum over later scan positions of (q dq - k dk), which the
oracle does not use; closed forms when the gate erases the state at every
step; and linearity in the output gradient.
"""
import numpy as np
import pytest

import oracle


def rand_problem(rng, B=1, H=2, gh=3, gw=4, dk=3, dv=2):
    q = rng.standard_normal((B, H, gh, gw, dk))
    k = rng.standard_normal((B, H, gh, gw, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, gh, gw, dv))
    g = -rng.random((B, H, gh, gw, dk))  # log alpha in (-1, 0]
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    dout = rng.standard_normal((B, H, gh, gw, dv))
    dsf = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, s0, dout, dsf


def loss(q, k, v, g, s0, dout, dsf, direction):
    out, sf = oracle.gla_forward(q, k, v, g, direction, s0=s0, want_state=True)
    return float(np.sum(out * dout) + np.sum(sf * dsf))


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_gradients_match_central_differences(direction):
    rng = np.random.default_rng(40 + direction)
    q, k, v, g, s0, dout, dsf = rand_problem(rng)
    dq, dk, dv, dg, ds0 = oracle.gla_backward(q, k, v, g, dout, direction, s0=s0, ds_final=dsf,
                                              want_ds0=True)
    args = [q, k, v, g, s0]
    grads = [dq, dk, dv, dg, ds0]
    eps = 1e-6
    for a, grad in zip(args, grads):
        num = np.zeros_like(a)
        flat = a.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + eps
            up = loss(*args, dout, dsf, direction)
            flat[idx] = old - eps
            down = loss(*args, dout, dsf, direction)
            flat[idx] = old
            num.reshape(-1)[idx] = (up - down) / (2 * eps)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), np.max(np.abs(grad - num))


@pytest.mark.parametrize("direction", [0, 3])
def test_gate_gradient_identity(direction):
    """dlog_gate_t = sum_{u >= t in scan order} (q_u dq_u - k_u dk_u) + rowsum(dS_final * S_final)."""
    rng = np.random.default_rng(50 + direction)
    q, k, v, g, s0, dout, dsf = rand_problem(rng, gh=4, gw=5, dk=4, dv=3)
    dq, dk, dv, dg = oracle.gla_backward(q, k, v, g, dout, direction, s0=s0, ds_final=dsf)
    _, sf = oracle.gla_forward(q, k, v, g, direction, s0=s0, want_state=True)
    B, H, gh, gw, _ = q.shape
    order = oracle.scan_order(gh, gw, direction)
    for b in range(B):
        for h in range(H):
            run = np.sum(dsf[b, h] * sf[b, h], axis=1)
            for t in reversed(range(gh * gw)):
                r, c = divmod(order[t], gw)
                run = run + q[b, h, r, c] * dq[b, h, r, c] - k[b, h, r, c] * dk[b, h, r, c]
                assert np.allclose(dg[b, h, r, c], run, rtol=1e-10, atol=1e-12)


def test_vanishing_gate_closed_forms():
    """alpha ~ 0 everywhere: every state is its own token's k^T v, so dq_t = k_t (v_t . dout_t),
    dk_t = q_t (v_t . dout_t) and dv_t = (q_t . k_t) dout_t."""
    rng = np.random.default_rng(6)
    q, k, v, g, s0, dout, _ = rand_problem(rng, gh=2, gw=5, dk=4, dv=3)
    g[:] = -80.0
    dq, dk, dv, _ = oracle.gla_backward(q, k, v, g, dout, 2)
    vd = np.sum(v * dout, axis=-1, keepdims=True)
    assert np.allclose(dq, k * vd, atol=1e-12)
    assert np.allclose(dk, q * vd, atol=1e-12)
    assert np.allclose(dv, np.sum(q * k, axis=-1, keepdims=True) * dout, atol=1e-12)


def test_linear_in_the_output_gradient():
    rng = np.random.default_rng(7)
    q, k, v, g, s0, d1, _ = rand_problem(rng)
    d2 = rng.standard_normal(d1.shape)
    a = oracle.gla_backward(q, k, v, g, d1, 1, s0=s0)
    b = oracle.gla_backward(q, k, v, g, d2, 1, s0=s0)
    c = oracle.gla_backward(q, k, v, g, d1 + 2.0 * d2, 1, s0=s0)
    for x, y, z in zip(a, b, c):
        assert np.allclose(z, x + 2.0 * y, atol=1e-12)
