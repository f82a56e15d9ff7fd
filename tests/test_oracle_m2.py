"""Pins of the oracle's Mamba-2 functions (CPU only).

Each test ties the oracle to something other than itself: a hand-worked
example, a closed form, an exact brute-force sum in rational arithmetic, or an
invariant the method states (replay = eager, commit interval does not change
the outputs, rollback + re-append reproduces the outputs).
"""
import json
import os
import random
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import replay
from brute import m2_unrolled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T, batch, H, G, P, N):
    x = rng.standard_normal((T, batch, H, P)) / np.sqrt(N)
    B = rng.standard_normal((T, batch, G, N)) / np.sqrt(N)
    C = rng.standard_normal((T, batch, G, N)) / np.sqrt(N)
    dt = np.logaddexp(0, rng.normal(-2, 0.5, (T, batch, H)))
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    h0 = rng.normal(0, 0.1, (batch, H, P, N))
    return A, D, x, B, C, dt, h0


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "m2_tiny_worked.json")))
    T = len(g["a"])
    a = np.array(g["a"]).reshape(T, 1, 1)
    dt = np.array(g["dt"]).reshape(T, 1, 1)
    x = np.array(g["x"]).reshape(T, 1, 1, 1)
    B = np.array(g["B"]).reshape(T, 1, 1, 2)
    C = np.array(g["C"]).reshape(T, 1, 1, 2)
    h = np.array(g["h0"]).reshape(1, 1, 1, 2)
    y = oracle.m2_recur(a, dt, x, B, C, np.array([g["D"]]), h)
    assert y.reshape(-1).tolist() == g["y"]
    assert h.reshape(1, 2).tolist() == g["h_final"]


def test_dt_zero_keeps_state():
    """dt = 0: a = exp(0) = 1 and no input term, so y_t = h0 C_t + D x_t."""
    rng = np.random.default_rng(1)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 6, 2, 4, 2, 8, 16)
    dt[:] = 0.0
    h = h0.copy()
    y = oracle.m2_eager(A, D, x, B, C, dt, h)
    np.testing.assert_array_equal(h, h0)
    g = np.arange(4) // 2
    for t in range(6):
        want = np.einsum("bhpn,bhn->bhp", h0, C[t][:, g]) + D[None, :, None] * x[t]
        np.testing.assert_allclose(y[t], want, rtol=0, atol=1e-15)


def test_constant_input_geometric_closed_form():
    """Constant a, dt, x, B: h_t = a^t h0 + dt x B^T (1 - a^t) / (1 - a)."""
    rng = np.random.default_rng(2)
    T, P, N = 9, 4, 5
    a0, dt0 = 0.7, 0.3
    x0 = rng.standard_normal(P)
    B0 = rng.standard_normal(N)
    h0 = rng.standard_normal((1, 1, P, N))
    C = rng.standard_normal((T, 1, 1, N))
    a = np.full((T, 1, 1), a0)
    dt = np.full((T, 1, 1), dt0)
    x = np.broadcast_to(x0, (T, 1, 1, P)).copy()
    B = np.broadcast_to(B0, (T, 1, 1, N)).copy()
    h = h0.copy()
    y = oracle.m2_recur(a, dt, x, B, C, np.array([0.25]), h)
    for t in range(1, T + 1):
        ht = a0 ** t * h0[0, 0] + dt0 * np.outer(x0, B0) * (1 - a0 ** t) / (1 - a0)
        np.testing.assert_allclose(y[t - 1, 0, 0], ht @ C[t - 1, 0, 0] + 0.25 * x0,
                                   rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(h[0, 0], ht, rtol=1e-13, atol=1e-14)


def test_decay_discretisation_special_values():
    """a = exp(dt A): dt A = -ln 2 gives 1/2, dt = 0 gives 1, dt A -> -inf gives 0."""
    A = np.array([-np.log(2.0), -4.0, -1e6])
    dt = np.array([[[1.0, 0.0, 1.0]]])
    a = oracle.m2_decays(A, dt)
    assert abs(a[0, 0, 0] - 0.5) < 1e-15
    assert a[0, 0, 1] == 1.0
    assert a[0, 0, 2] == 0.0


def _dyadic(rng, *shape, choices=(-1, -0.5, -0.25, 0.25, 0.5, 1)):
    return np.array(rng.choice(choices, size=shape), dtype=np.float64)


@pytest.mark.parametrize("G", [1, 2])
def test_bruteforce_unrolled_sum_exact(G):
    """Dyadic inputs: the fp64 eager recurrence equals the exact unrolled sum."""
    rng = np.random.default_rng(3 + G)
    T, batch, H, P, N = 5, 2, 4, 2, 3
    a = _dyadic(rng, T, batch, H, choices=(0.25, 0.5, 0.75, 1.0))
    dt = _dyadic(rng, T, batch, H, choices=(0.25, 0.5, 1.0))
    x = _dyadic(rng, T, batch, H, P)
    B = _dyadic(rng, T, batch, G, N)
    C = _dyadic(rng, T, batch, G, N)
    D = _dyadic(rng, H)
    h0 = _dyadic(rng, batch, H, P, N)
    h = h0.copy()
    y = oracle.m2_recur(a, dt, x, B, C, D, h)
    want = m2_unrolled(a.tolist(), dt.tolist(), x.tolist(), B.tolist(),
                       C.tolist(), D.tolist(), h0.tolist(), G)
    for t in range(T):
        for b in range(batch):
            for hh in range(H):
                for p in range(P):
                    assert Fr(y[t, b, hh, p]) == want[t][b][hh][p], (t, b, hh, p)


def test_ssd_quadratic_form():
    """Second independent form (SSD): for a chunk from checkpoint h0,
    Y = diag(Gamma_{1..k}) (C h0^T) + (M o (C B^T)) (dt o X) + D X,
    M[k,i] = prod_{i<j<=k} a_j for i <= k, else 0."""
    rng = np.random.default_rng(5)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 7, 1, 1, 1, 6, 8)
    h = h0.copy()
    y = oracle.m2_eager(A, D, x, B, C, dt, h)[:, 0, 0]
    a = np.exp(dt[:, 0, 0] * A[0])
    T = 7
    M = np.zeros((T, T))
    for k in range(T):
        for i in range(k + 1):
            M[k, i] = np.prod(a[i + 1:k + 1])
    Cm, Bm, X = C[:, 0, 0], B[:, 0, 0], x[:, 0, 0]
    gam = np.cumprod(a)
    Y = gam[:, None] * (Cm @ h0[0, 0].T) + (M * (Cm @ Bm.T)) @ (dt[:, 0, 0, None] * X) \
        + D[0] * X
    np.testing.assert_allclose(y, Y, rtol=1e-12, atol=1e-14)


def test_replay_form_equals_eager():
    rng = np.random.default_rng(6)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 8, 1, 1, 1, 16, 32)
    h = h0.copy()
    y = oracle.m2_eager(A, D, x, B, C, dt, h)
    for t in range(8):
        yr = replay.m2_output(h0[0, 0], x[:t + 1, 0, 0], B[:t + 1, 0, 0],
                              dt[:t + 1, 0, 0], C[t, 0, 0], A[0], D[0])
        np.testing.assert_allclose(yr, y[t, 0, 0], rtol=1e-12, atol=1e-14)
    hf = replay.m2_fold(h0[0, 0], x[:, 0, 0], B[:, 0, 0], dt[:, 0, 0], A[0])
    np.testing.assert_allclose(hf, h[0, 0], rtol=1e-12, atol=1e-14)


def test_replay_empty_buffer_and_commit_consistency():
    """No buffered entries: h_c C + D x.  After folding through t, the new
    checkpoint with an empty buffer reproduces y_t's state part."""
    rng = np.random.default_rng(7)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 4, 1, 1, 1, 8, 8)
    y0 = replay.m2_output_empty(h0[0, 0], C[0, 0, 0], x[0, 0, 0], D[0])
    np.testing.assert_allclose(y0, h0[0, 0] @ C[0, 0, 0] + D[0] * x[0, 0, 0])
    yt = replay.m2_output(h0[0, 0], x[:, 0, 0], B[:, 0, 0], dt[:, 0, 0], C[3, 0, 0],
                          A[0], D[0])
    hn = replay.m2_fold(h0[0, 0], x[:, 0, 0], B[:, 0, 0], dt[:, 0, 0], A[0])
    np.testing.assert_allclose(replay.m2_output_empty(hn, C[3, 0, 0], x[3, 0, 0], D[0]),
                               yt, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("interval", [1, 2, 4, 8, 16])
def test_interval_independence(interval):
    """Checkpoint + buffer replay with a commit every `interval` tokens gives
    the eager outputs whatever the interval (interval 1 is eager itself)."""
    rng = np.random.default_rng(8)
    T = 20
    A, D, x, B, C, dt, h0 = _rand_case(rng, T, 1, 1, 1, 8, 16)
    h = h0.copy()
    y_e = oracle.m2_eager(A, D, x, B, C, dt, h)[:, 0, 0]
    ck = h0[0, 0].copy()
    buf = []
    for t in range(T):
        buf.append(t)
        y = replay.m2_output(ck, x[buf, 0, 0], B[buf, 0, 0], dt[buf, 0, 0], C[t, 0, 0],
                             A[0], D[0])
        np.testing.assert_allclose(y, y_e[t], rtol=1e-12, atol=1e-14)
        if len(buf) == interval:
            ck = replay.m2_fold(ck, x[buf, 0, 0], B[buf, 0, 0], dt[buf, 0, 0], A[0])
            buf = []


def test_rollback_then_reappend_reproduces_outputs():
    """Drop the last k buffered entries (the checkpoint is untouched), append
    the same inputs again: identical outputs; append different ones: the
    outputs of an eager run that only ever saw the kept + new inputs."""
    rng = np.random.default_rng(9)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 6, 1, 1, 1, 4, 8)
    _, _, x2, B2, C2, dt2, _ = _rand_case(rng, 6, 1, 1, 1, 4, 8)
    ck = h0[0, 0]
    run = lambda xs, Bs, dts, Cq: replay.m2_output(ck, xs, Bs, dts, Cq, A[0], D[0])
    y_first = [run(x[:t + 1, 0, 0], B[:t + 1, 0, 0], dt[:t + 1, 0, 0], C[t, 0, 0])
               for t in range(6)]
    keep = 3   # roll back 3 of 6
    y_again = [run(x[:t + 1, 0, 0], B[:t + 1, 0, 0], dt[:t + 1, 0, 0], C[t, 0, 0])
               for t in range(keep, 6)]
    for a_, b_ in zip(y_first[keep:], y_again):
        np.testing.assert_array_equal(a_, b_)
    # different continuation after rollback == eager over the spliced history
    xs = np.concatenate([x[:keep], x2[keep:]])
    Bs = np.concatenate([B[:keep], B2[keep:]])
    Cs = np.concatenate([C[:keep], C2[keep:]])
    dts = np.concatenate([dt[:keep], dt2[keep:]])
    h = h0.copy()
    y_e = oracle.m2_eager(A, D, xs, Bs, Cs, dts, h)[:, 0, 0]
    for t in range(keep, 6):
        y = run(xs[:t + 1, 0, 0], Bs[:t + 1, 0, 0], dts[:t + 1, 0, 0], Cs[t, 0, 0])
        np.testing.assert_allclose(y, y_e[t], rtol=1e-12, atol=1e-14)


def test_units_are_independent_and_groups_map_in_blocks():
    """Running a sequence alone equals running it inside a batch, and head h
    reads group h // (H/G): permuting groups' inputs changes exactly the
    heads of that block."""
    rng = np.random.default_rng(10)
    A, D, x, B, C, dt, h0 = _rand_case(rng, 3, 3, 6, 3, 4, 8)
    h = h0.copy()
    y = oracle.m2_eager(A, D, x, B, C, dt, h)
    h1 = h0[1:2].copy()
    y1 = oracle.m2_eager(A, D, x[:, 1:2], B[:, 1:2], C[:, 1:2], dt[:, 1:2], h1)
    np.testing.assert_array_equal(y1[:, 0], y[:, 1])
    B2 = B.copy()
    B2[:, :, 1] *= 2.0     # only group 1 -> heads 2, 3
    h = h0.copy()
    y2 = oracle.m2_eager(A, D, x, B2, C, dt, h)
    changed = np.abs(y2 - y).max(axis=(0, 1, 3)) > 0
    assert changed.tolist() == [False, False, True, True, False, False]
