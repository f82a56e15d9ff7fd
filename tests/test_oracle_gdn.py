"""Pins of the oracle's Gated DeltaNet functions (CPU only).

Hand-worked example, closed forms of the delta rule (alpha = 0, beta = 0,
recall identity, orthonormal-key recall), exact brute force with explicit
dk x dk transition matrices, and the replay invariants (backward-carried query
= eager, forward-substitution fold = eager state, interval independence,
rollback + re-append).
"""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import replay
from brute import gdn_matrix_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, *shape):
    v = rng.standard_normal(shape)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _rand_case(rng, T, batch, H, dk, dv, s0=0.1):
    q = _unit(rng, T, batch, H, dk)
    k = _unit(rng, T, batch, H, dk)
    v = rng.standard_normal((T, batch, H, dv))
    al = np.exp(-np.logaddexp(0, rng.standard_normal((T, batch, H))))
    be = 1 / (1 + np.exp(-rng.standard_normal((T, batch, H))))
    S0 = rng.normal(0, s0, (batch, H, dv, dk))
    return q, k, v, al, be, S0


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "gdn_tiny_worked.json")))
    T = len(g["alpha"])
    sh = lambda a, *s: np.array(a, dtype=np.float64).reshape(*s)
    S = sh(g["S0"], 1, 1, 2, 2)
    o = oracle.gdn_eager(sh(g["q"], T, 1, 1, 2), sh(g["k"], T, 1, 1, 2),
                         sh(g["v"], T, 1, 1, 2), sh(g["alpha"], T, 1, 1),
                         sh(g["beta"], T, 1, 1), S)
    assert o.reshape(T, 2).tolist() == g["o"]
    assert S.reshape(2, 2).tolist() == g["S_final"]


def test_delta_rule_recall_identity():
    """beta = 1 and |k| = 1: S_t k_t = v_t for any history, so q_t = k_t reads v_t."""
    rng = np.random.default_rng(11)
    q, k, v, al, be, S0 = _rand_case(rng, 10, 2, 3, 16, 12, s0=1.0)
    be[:] = 1.0
    q[:] = k
    S = S0.copy()
    o = oracle.gdn_eager(q, k, v, al, be, S)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_orthonormal_keys_exact_recall():
    """alpha = beta = 1, orthonormal keys, S0 = 0: every stored value is
    recalled exactly by its key after all writes."""
    rng = np.random.default_rng(12)
    dk = dv = 8
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q.T[:6]                      # 6 orthonormal rows
    vals = rng.standard_normal((6, dv))
    T = 6
    k = keys.reshape(T, 1, 1, dk)
    v = vals.reshape(T, 1, 1, dv)
    one = np.ones((T, 1, 1))
    S = np.zeros((1, 1, dv, dk))
    oracle.gdn_eager(k, k, v, one, one, S)
    for j in range(6):
        np.testing.assert_allclose(S[0, 0] @ keys[j], vals[j], atol=1e-12)


def test_beta_zero_pure_decay():
    """beta = 0: S_t = (prod alpha) S_0, o_t = (prod alpha) S_0 q_t."""
    rng = np.random.default_rng(13)
    q, k, v, al, be, S0 = _rand_case(rng, 7, 2, 2, 8, 8, s0=1.0)
    be[:] = 0.0
    S = S0.copy()
    o = oracle.gdn_eager(q, k, v, al, be, S)
    decay = np.cumprod(al, axis=0)
    want = decay[..., None] * np.einsum("bhrc,tbhc->tbhr", S0, q)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-14)


def test_alpha_zero_forgets():
    """alpha = 0: S_t = beta v k^T, o_t = beta (k . q) v."""
    rng = np.random.default_rng(14)
    q, k, v, al, be, S0 = _rand_case(rng, 4, 1, 2, 8, 6, s0=1.0)
    al[:] = 0.0
    S = S0.copy()
    o = oracle.gdn_eager(q, k, v, al, be, S)
    kq = np.einsum("tbhc,tbhc->tbh", k, q)
    np.testing.assert_allclose(o, (be * kq)[..., None] * v, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S, be[-1][..., None, None] * np.einsum(
        "bhr,bhc->bhrc", v[-1], k[-1]), rtol=1e-13, atol=1e-15)


def test_bruteforce_matrix_form_exact():
    """Dyadic inputs (keys in {+-1/2}^4, unit norm; alpha, beta in {1/4,1/2,1}):
    fp64 eager == explicit-matrix form in exact rationals."""
    rng = np.random.default_rng(15)
    T, dk, dv = 5, 4, 4
    for unit in range(3):
        k = rng.choice([-0.5, 0.5], size=(T, dk))
        q = rng.choice([-0.5, 0.5, 0.25, 1.0], size=(T, dk))
        v = rng.choice([-1, -0.5, 0.5, 1, 2], size=(T, dv)).astype(float)
        al = rng.choice([0.25, 0.5, 1.0], size=T)
        be = rng.choice([0.25, 0.5, 1.0], size=T)
        S0 = rng.choice([-0.5, 0, 0.5, 1], size=(dv, dk)).astype(float)
        S = S0.reshape(1, 1, dv, dk).copy()
        o = oracle.gdn_eager(q.reshape(T, 1, 1, dk), k.reshape(T, 1, 1, dk),
                             v.reshape(T, 1, 1, dv), al.reshape(T, 1, 1),
                             be.reshape(T, 1, 1), S)
        want_o, want_S = gdn_matrix_form(q.tolist(), k.tolist(), v.tolist(),
                                         al.tolist(), be.tolist(), S0.tolist())
        for t in range(T):
            for r in range(dv):
                assert Fr(o[t, 0, 0, r]) == want_o[t][r], (unit, t, r)
        for r in range(dv):
            for c in range(dk):
                assert Fr(S[0, 0, r, c]) == want_S[r][c]


def test_backward_carried_query_equals_eager():
    rng = np.random.default_rng(16)
    q, k, v, al, be, S0 = _rand_case(rng, 9, 1, 1, 16, 12)
    S = S0.copy()
    o = oracle.gdn_eager(q, k, v, al, be, S)
    for t in range(9):
        ot = replay.gdn_output(S0[0, 0], q[t, 0, 0], k[:t + 1, 0, 0], v[:t + 1, 0, 0],
                               al[:t + 1, 0, 0], be[:t + 1, 0, 0])
        np.testing.assert_allclose(ot, o[t, 0, 0], rtol=1e-12, atol=1e-13)
    Sf = replay.gdn_fold(S0[0, 0], k[:, 0, 0], v[:, 0, 0], al[:, 0, 0], be[:, 0, 0])
    np.testing.assert_allclose(Sf, S[0, 0], rtol=1e-12, atol=1e-13)


def test_empty_carry_is_plain_matvec():
    rng = np.random.default_rng(17)
    S0 = rng.standard_normal((5, 7))
    q = rng.standard_normal(7)
    qt, s = replay.gdn_carry(q, np.zeros((0, 7)), np.zeros(0), np.zeros(0))
    np.testing.assert_array_equal(qt, q)
    np.testing.assert_array_equal(replay.gdn_output(S0, q, np.zeros((0, 7)),
                                                    np.zeros((0, 5)), np.zeros(0),
                                                    np.zeros(0)), S0 @ q)


@pytest.mark.parametrize("interval", [1, 2, 4, 8, 16])
def test_interval_independence(interval):
    rng = np.random.default_rng(18)
    T = 18
    q, k, v, al, be, S0 = _rand_case(rng, T, 1, 1, 8, 8)
    S = S0.copy()
    o_e = oracle.gdn_eager(q, k, v, al, be, S)[:, 0, 0]
    ck = S0[0, 0].copy()
    buf = []
    for t in range(T):
        buf.append(t)
        o = replay.gdn_output(ck, q[t, 0, 0], k[buf, 0, 0], v[buf, 0, 0],
                              al[buf, 0, 0], be[buf, 0, 0])
        np.testing.assert_allclose(o, o_e[t], rtol=1e-11, atol=1e-13)
        if len(buf) == interval:
            ck = replay.gdn_fold(ck, k[buf, 0, 0], v[buf, 0, 0], al[buf, 0, 0],
                                 be[buf, 0, 0])
            buf = []


def test_rollback_then_reappend_reproduces_outputs():
    rng = np.random.default_rng(19)
    q, k, v, al, be, S0 = _rand_case(rng, 6, 1, 1, 8, 8)
    ck = S0[0, 0]
    out = lambda t: replay.gdn_output(ck, q[t, 0, 0], k[:t + 1, 0, 0], v[:t + 1, 0, 0],
                                      al[:t + 1, 0, 0], be[:t + 1, 0, 0])
    first = [out(t) for t in range(6)]
    again = [out(t) for t in range(2, 6)]
    for a_, b_ in zip(first[2:], again):
        np.testing.assert_array_equal(a_, b_)
