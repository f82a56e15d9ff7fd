"""Pins of the oracle's prefill drivers (CPU only).

Prefill continues each selected sequence's state over its buffered entries and
then over a prompt, with the eager output of every prompt token.  The pins:
* closed forms: dt = 0 keeps the Mamba-2 state; constant inputs give
  h_n = a^n h_0 + dt x B^T (1 - a^n) / (1 - a) after n = ring + prompt steps;
  GDN with beta = 0 only decays; the delta-rule identity (beta = 1, unit keys,
  q_t = k_t) returns v_t at every prompt token whatever the history;
* ragged buffers: a sequence's buffered entries count exactly once, before the
  prompt, whatever the other sequences hold;
* a masked-out sequence keeps its state and gets no output.
"""
import numpy as np

from oracle import drivers

P, N, DK = 4, 8, 6


def _m2_case(rng, Lr, T, b, H, G):
    ring = dict(x=rng.standard_normal((Lr, b, H, P)) * 0.3,
                B=rng.standard_normal((Lr, b, G, N)) * 0.3,
                dt=rng.uniform(0.05, 0.4, (Lr, b, H)))
    prompt = dict(x=rng.standard_normal((T, b, H, P)) * 0.3,
                  B=rng.standard_normal((T, b, G, N)) * 0.3,
                  C=rng.standard_normal((T, b, G, N)) * 0.3,
                  dt=rng.uniform(0.05, 0.4, (T, b, H)))
    A = -np.exp(rng.uniform(0, np.log(4), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N)) * 0.3
    return A, D, ring, prompt, h0


def test_m2_dt_zero_keeps_state():
    rng = np.random.default_rng(300)
    A, D, ring, prompt, h0 = _m2_case(rng, 3, 5, 3, 4, 2)
    ring["dt"][:] = 0.0
    prompt["dt"][:] = 0.0
    h = h0.copy()
    y = drivers.m2_prefill(A, D, h, ring, np.array([0, 2, 3]), prompt)
    np.testing.assert_array_equal(h, h0)
    g = np.arange(4) // 2
    for t in range(5):
        want = np.einsum("bhpn,bhn->bhp", h0, prompt["C"][t][:, g]) + D[None, :, None] * prompt["x"][t]
        np.testing.assert_allclose(y[t], want, rtol=0, atol=1e-14)


def test_m2_constant_inputs_closed_form():
    """Every entry (buffered and prompt) has the same x, B, dt: after n steps
    h_n = a^n h_0 + dt x B^T (1 - a^n) / (1 - a), a = exp(dt A)."""
    rng = np.random.default_rng(301)
    Lr, T, b, H, G = 4, 7, 2, 2, 1
    A, D, ring, prompt, h0 = _m2_case(rng, Lr, T, b, H, G)
    xc = rng.standard_normal((b, H, P)) * 0.3
    Bc = rng.standard_normal((b, G, N)) * 0.3
    dtc = rng.uniform(0.05, 0.4, (b, H))
    for d, n in ((ring, Lr), (prompt, T)):
        d["x"][:] = xc
        d["B"][:] = Bc
        d["dt"][:] = dtc
    ring_len = np.array([Lr, 1])
    h = h0.copy()
    y = drivers.m2_prefill(A, D, h, ring, ring_len, prompt)
    for s in range(b):
        n = ring_len[s] + T
        a = np.exp(dtc[s] * A)                                       # [H]
        outer = dtc[s][:, None, None] * xc[s][:, :, None] * Bc[s][0][None, None, :]
        want = (a ** n)[:, None, None] * h0[s] + outer * ((1 - a ** n) / (1 - a))[:, None, None]
        np.testing.assert_allclose(h[s], want, rtol=1e-12, atol=1e-14)
        y_last = np.einsum("hpn,n->hp", want, prompt["C"][-1, s, 0]) + D[:, None] * xc[s]
        np.testing.assert_allclose(y[-1, s], y_last, rtol=1e-12, atol=1e-14)


def test_m2_ragged_ring_counts_once():
    """A sequence with r buffered entries equals the plain recurrence over
    those r entries followed by the prompt; its neighbours do not matter."""
    rng = np.random.default_rng(302)
    Lr, T, b, H, G = 5, 6, 3, 4, 2
    A, D, ring, prompt, h0 = _m2_case(rng, Lr, T, b, H, G)
    ring_len = np.array([0, 5, 2])
    h = h0.copy()
    y = drivers.m2_prefill(A, D, h, ring, ring_len, prompt)
    for s in range(b):
        r = ring_len[s]
        x = np.concatenate([ring["x"][:r, s:s + 1], prompt["x"][:, s:s + 1]])
        B = np.concatenate([ring["B"][:r, s:s + 1], prompt["B"][:, s:s + 1]])
        C = np.concatenate([np.zeros((r, 1, G, N)), prompt["C"][:, s:s + 1]])
        dt = np.concatenate([ring["dt"][:r, s:s + 1], prompt["dt"][:, s:s + 1]])
        hs = h0[s:s + 1].copy()
        ys = drivers.m2_eager(A, D, x, B, C, dt, hs)
        np.testing.assert_array_equal(y[:, s:s + 1], ys[r:])
        np.testing.assert_array_equal(h[s:s + 1], hs)


def test_m2_mask_leaves_sequence():
    rng = np.random.default_rng(303)
    A, D, ring, prompt, h0 = _m2_case(rng, 2, 3, 2, 2, 1)
    h = h0.copy()
    y = drivers.m2_prefill(A, D, h, ring, np.array([2, 2]), prompt, mask=np.array([1, 0]))
    np.testing.assert_array_equal(h[1], h0[1])
    assert np.isnan(y[:, 1]).all() and np.isfinite(y[:, 0]).all()
    assert not np.array_equal(h[0], h0[0])


def _unit(rng, shape):
    k = rng.standard_normal(shape)
    return k / np.linalg.norm(k, axis=-1, keepdims=True)


def _gdn_case(rng, Lr, T, b, H):
    ring = dict(k=_unit(rng, (Lr, b, H, DK)), v=rng.standard_normal((Lr, b, H, DK)),
                alpha=rng.uniform(0.3, 1.0, (Lr, b, H)), beta=rng.uniform(0.1, 1.0, (Lr, b, H)))
    prompt = dict(q=_unit(rng, (T, b, H, DK)), k=_unit(rng, (T, b, H, DK)),
                  v=rng.standard_normal((T, b, H, DK)),
                  alpha=rng.uniform(0.3, 1.0, (T, b, H)), beta=rng.uniform(0.1, 1.0, (T, b, H)))
    S0 = rng.standard_normal((b, H, DK, DK)) * 0.3
    return ring, prompt, S0


def test_gdn_delta_rule_identity():
    """beta = 1 and unit keys: S_t k_t = v_t after every update, so querying
    each prompt token with its own key returns its value exactly."""
    rng = np.random.default_rng(304)
    ring, prompt, S0 = _gdn_case(rng, 3, 6, 2, 3)
    prompt["beta"][:] = 1.0
    prompt["q"] = prompt["k"].copy()
    S = S0.copy()
    o = drivers.gdn_prefill(S, ring, np.array([3, 1]), prompt)
    np.testing.assert_allclose(o, prompt["v"], rtol=0, atol=1e-12)


def test_gdn_beta_zero_only_decays():
    """beta = 0: S_n = (prod of all alphas) S_0; o_t = (prod alphas so far) S_0 q_t."""
    rng = np.random.default_rng(305)
    Lr, T = 4, 5
    ring, prompt, S0 = _gdn_case(rng, Lr, T, 2, 2)
    ring["beta"][:] = 0.0
    prompt["beta"][:] = 0.0
    ring_len = np.array([4, 0])
    S = S0.copy()
    o = drivers.gdn_prefill(S, ring, ring_len, prompt)
    for s in range(2):
        g = np.prod(ring["alpha"][:ring_len[s], s], axis=0)         # [H]
        for t in range(T):
            g = g * prompt["alpha"][t, s]
            want = g[:, None] * np.einsum("hvk,hk->hv", S0[s], prompt["q"][t, s])
            np.testing.assert_allclose(o[t, s], want, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S[s], g[:, None, None] * S0[s], rtol=1e-12, atol=1e-14)
