"""Pins of three oracle drivers that the GPU tests lean on (CPU only).

* ``drivers.gdn_carry_batched`` supplies the carried query q~ from which the
  GPU tests form the one-quantisation bound of a dual GDN layer.  Pinned by the
  replay identity S_c q~ + sum_i s_i v_i = o_t of the eager recurrence run
  from S_c over the same entries (the backward-carried query of the explainer
  section "Compute outputs without eagerly updating the checkpoint"), with
  decays and write strengths away from 1, so that a dropped alpha or beta, or
  a carry taken oldest-first, changes the result; and by exact dyadic
  arithmetic against an explicit product of dk x dk transition matrices.
* ``drivers.gdn_tree_verify`` is the reference of GDN tree verification: a
  chain equals one eager continuation over the drafts, a star equals
  independent single steps from the same state, and a deeper tree's draft
  equals the eager run over exactly its root-to-node path.
* the ``ckpt`` snapshot of ``drivers.m2_decode`` / ``drivers.gdn_decode`` is
  the state at the last commit: checked against an eager run stopped at that
  step, and the outputs against one uninterrupted eager run.

Each pin is also run against planted mistakes in copies of the driver (never
in the driver itself) and must reject every one of them.
"""
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import drivers
from brute import gdn_matrix_form


def _unit(rng, *shape):
    v = rng.standard_normal(shape)
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _gdn_entries(rng, U, L, dk, dv):
    """Entries with alpha in [0.3, 0.9] and beta in [0.2, 0.8], far from 1."""
    q = _unit(rng, U, dk)
    ks = _unit(rng, U, L, dk)
    vs = rng.standard_normal((U, L, dv))
    al = rng.uniform(0.3, 0.9, (U, L))
    be = rng.uniform(0.2, 0.8, (U, L))
    Sc = rng.normal(0, 0.3, (U, dv, dk))
    return q, ks, vs, al, be, Sc


# ------------------------------------------------------ carried query ----

def _carry_pin_error(carry_fn, seed=60, U=12, L=7, dk=16, dv=10):
    """Largest |S_c q~ + sum_i s_i v_i - o_t| over U units, o_t from the eager
    recurrence (the C oracle) run from S_c over the L entries with q_t last."""
    rng = np.random.default_rng(seed)
    q, ks, vs, al, be, Sc = _gdn_entries(rng, U, L, dk, dv)
    qt, s = carry_fn(q, ks, al, be)
    o_replay = np.einsum("urc,uc->ur", Sc, qt) + np.einsum("ul,ulr->ur", s, vs)
    # eager: every entry's query is q_t; only the last step's output matters
    S = Sc.reshape(1, U, dv, dk).copy()
    qq = np.broadcast_to(q[None], (L, U, dk)).reshape(L, 1, U, dk)
    o = oracle.gdn_eager(qq, ks.transpose(1, 0, 2)[:, None], vs.transpose(1, 0, 2)[:, None],
                         al.T[:, None], be.T[:, None], S)
    return float(np.abs(o_replay - o[-1, 0]).max())


def _carry_no_alpha(q_t, ks, alphas, betas):
    return drivers.gdn_carry_batched(q_t, ks, np.ones_like(alphas), betas)


def _carry_no_beta(q_t, ks, alphas, betas):
    qt, s = drivers.gdn_carry_batched(q_t, ks, alphas, np.ones_like(betas))
    return qt, s * np.asarray(betas)


def _carry_oldest_first(q_t, ks, alphas, betas):
    ks = np.asarray(ks)[:, ::-1]
    qt, s = drivers.gdn_carry_batched(q_t, ks, np.asarray(alphas)[:, ::-1],
                                      np.asarray(betas)[:, ::-1])
    return qt, s[:, ::-1]


def _carry_last_alpha_dropped(q_t, ks, alphas, betas):
    """Off by one: the oldest entry's decay is not applied."""
    qt, s = drivers.gdn_carry_batched(q_t, ks, alphas, betas)
    return qt / np.asarray(alphas)[:, :1], s


def test_carry_batched_reproduces_eager_output():
    assert _carry_pin_error(drivers.gdn_carry_batched) < 1e-12


def test_carry_batched_one_entry_closed_form():
    """L = 1: s = beta (k . q) and q~ = alpha (q - s k), written out."""
    rng = np.random.default_rng(61)
    q, ks, _, al, be, _ = _gdn_entries(rng, 5, 1, 8, 4)
    qt, s = drivers.gdn_carry_batched(q, ks, al, be)
    kq = (ks[:, 0] * q).sum(-1)
    np.testing.assert_allclose(s[:, 0], be[:, 0] * kq, rtol=1e-14)
    np.testing.assert_allclose(qt, al[:, :1] * (q - (be[:, 0] * kq)[:, None] * ks[:, 0]),
                               rtol=1e-13, atol=1e-15)


def test_carry_batched_empty_buffer_is_identity():
    rng = np.random.default_rng(62)
    q = rng.standard_normal((3, 6))
    qt, s = drivers.gdn_carry_batched(q, np.zeros((3, 0, 6)), np.zeros((3, 0)),
                                      np.zeros((3, 0)))
    np.testing.assert_array_equal(qt, q)
    assert s.shape == (3, 0)


def test_carry_batched_exact_against_transition_matrices():
    """Dyadic inputs (k in {+-1/2}^4, alpha and beta in {1/4, 1/2, 1}): the
    fp64 result is exact, and equals o_t of the product of explicit
    transition matrices computed with Fractions."""
    rng = np.random.default_rng(63)
    dk = dv = 4
    for unit in range(6):
        L = int(rng.integers(1, 6))
        ks = rng.choice([-0.5, 0.5], (1, L, dk))
        vs = rng.choice([-1.0, -0.5, 0.5, 1.0], (1, L, dv))
        al = rng.choice([0.25, 0.5, 1.0], (1, L))
        be = rng.choice([0.25, 0.5, 1.0], (1, L))
        Sc = rng.choice([-0.5, 0.0, 0.5], (1, dv, dk))
        q = rng.choice([-0.5, 0.5], (1, dk))
        qt, s = drivers.gdn_carry_batched(q, ks, al, be)
        o = Sc[0] @ qt[0] + s[0] @ vs[0]
        qs = [q[0].tolist()] * L
        want_o, _ = gdn_matrix_form(qs, ks[0].tolist(), vs[0].tolist(), al[0].tolist(),
                                    be[0].tolist(), Sc[0].tolist())
        for r in range(dv):
            assert Fr(o[r]) == want_o[L - 1][r], (unit, r)


@pytest.mark.parametrize("mutant", [_carry_no_alpha, _carry_no_beta, _carry_oldest_first,
                                    _carry_last_alpha_dropped])
def test_carry_pin_rejects_planted_mistakes(mutant):
    assert _carry_pin_error(mutant) > 1e-3


def test_one_quantisation_bound_tightens_with_the_decays():
    """The bound's query weight |q~| shrinks with the product of the decays
    (|q~| <= prod alpha * |q| for unit keys and beta <= 1, since I - beta k k^T
    is a contraction): a dropped alpha would loosen the GPU gate by up to
    1 / prod alpha, and this inequality is what it would break."""
    rng = np.random.default_rng(64)
    q, ks, _, al, be, _ = _gdn_entries(rng, 40, 8, 16, 4)
    qt, _ = drivers.gdn_carry_batched(q, ks, al, be)
    lhs = np.linalg.norm(qt, axis=-1)
    rhs = np.prod(al, axis=-1) * np.linalg.norm(q, axis=-1)
    assert np.all(lhs <= rhs * (1 + 1e-12))
    qt_bad, _ = _carry_no_alpha(q, ks, al, be)
    assert np.any(np.linalg.norm(qt_bad, axis=-1) > rhs * 10)


# ------------------------------------------------------------ GDN trees ----

def _gdn_drafts(rng, n, b, H, dk, dv):
    return dict(q=_unit(rng, n, b, H, dk), k=_unit(rng, n, b, H, dk),
                v=rng.standard_normal((n, b, H, dv)),
                alpha=rng.uniform(0.3, 0.9, (n, b, H)), beta=rng.uniform(0.2, 0.8, (n, b, H)))


def _gdn_eager_path(S, dr, path):
    Ss = np.array(S, dtype=np.float64, copy=True)
    return oracle.gdn_eager(*(dr[s][path] for s in ("q", "k", "v", "alpha", "beta")), Ss)


def _tree_pin_error(tree_fn, seed=65):
    """Largest deviation of tree_fn from three pins: chain = one eager
    continuation, star = independent single steps, and a binary tree's draft =
    the eager run over its root-to-node path written out by hand."""
    rng = np.random.default_rng(seed)
    n, b, H, dk, dv = 7, 2, 3, 8, 6
    S = rng.normal(0, 0.3, (b, H, dv, dk))
    dr = _gdn_drafts(rng, n, b, H, dk, dv)
    err = 0.0
    chain = tree_fn(S, dr, [-1, 0, 1, 2, 3, 4, 5])
    err = max(err, float(np.abs(chain - _gdn_eager_path(S, dr, list(range(n)))).max()))
    star = tree_fn(S, dr, [-1] * n)
    for j in range(n):
        err = max(err, float(np.abs(star[j] - _gdn_eager_path(S, dr, [j])[0]).max()))
    tree = tree_fn(S, dr, [-1, 0, 0, 1, 1, 2, 2])
    paths = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 4], 5: [0, 2, 5],
             6: [0, 2, 6]}
    for j, path in paths.items():
        err = max(err, float(np.abs(tree[j] - _gdn_eager_path(S, dr, path)[-1]).max()))
    return err


def _tree_state_shared(S, drafts, parent):
    """Mistake: the drafts continue one shared state instead of a fresh copy."""
    q, k, v, al, be = (drafts[s] for s in ("q", "k", "v", "alpha", "beta"))
    Ss = np.array(S, dtype=np.float64, copy=True)
    o = np.empty(v.shape, np.float64)
    for j, path in enumerate(drivers.tree_paths(parent)):
        o[j] = oracle.gdn_eager(q[path[-1:]], k[path[-1:]], v[path[-1:]], al[path[-1:]],
                                be[path[-1:]], Ss)[-1]
    return o


def _tree_first_output(S, drafts, parent):
    """Mistake: the path's first output instead of its last."""
    q, k, v, al, be = (drafts[s] for s in ("q", "k", "v", "alpha", "beta"))
    o = np.empty(v.shape, np.float64)
    for j, path in enumerate(drivers.tree_paths(parent)):
        Ss = np.array(S, dtype=np.float64, copy=True)
        o[j] = oracle.gdn_eager(q[path], k[path], v[path], al[path], be[path], Ss)[0]
    return o


def _tree_own_query_only(S, drafts, parent):
    """Mistake: the ancestors' entries are skipped (only the node is applied)."""
    q, k, v, al, be = (drafts[s] for s in ("q", "k", "v", "alpha", "beta"))
    o = np.empty(v.shape, np.float64)
    for j in range(len(parent)):
        Ss = np.array(S, dtype=np.float64, copy=True)
        o[j] = oracle.gdn_eager(q[j:j + 1], k[j:j + 1], v[j:j + 1], al[j:j + 1],
                                be[j:j + 1], Ss)[0]
    return o


def test_gdn_tree_verify_chain_star_and_paths():
    assert _tree_pin_error(drivers.gdn_tree_verify) < 1e-13


def test_gdn_tree_verify_leaves_the_state_alone():
    rng = np.random.default_rng(66)
    S = rng.normal(0, 0.3, (1, 2, 4, 4))
    before = S.copy()
    drivers.gdn_tree_verify(S, _gdn_drafts(rng, 3, 1, 2, 4, 4), [-1, 0, 0])
    np.testing.assert_array_equal(S, before)


@pytest.mark.parametrize("mutant", [_tree_state_shared, _tree_first_output,
                                    _tree_own_query_only])
def test_gdn_tree_pin_rejects_planted_mistakes(mutant):
    assert _tree_pin_error(mutant) > 1e-3


# ------------------------------------------------- decode checkpoint snapshot --

def _m2_case(rng, T, b, H, G, P, N):
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    x = rng.standard_normal((T, b, H, P)) / np.sqrt(N)
    B = rng.standard_normal((T, b, G, N)) / np.sqrt(N)
    C = rng.standard_normal((T, b, G, N)) / np.sqrt(N)
    dt = np.logaddexp(0, rng.normal(-2, 0.5, (T, b, H)))
    h0 = rng.normal(0, 0.1, (b, H, P, N))
    return A, D, x, B, C, dt, h0


def _m2_decode_pin_error(decode_fn, T=21, interval=4):
    rng = np.random.default_rng(67)
    A, D, x, B, C, dt, h0 = _m2_case(rng, T, 2, 4, 2, 4, 8)
    res = decode_fn(A, D, x, B, C, dt, h0, interval, interval)
    last = max(t for t in range(T) if (t + 1) % interval == 0)
    h = h0.copy()
    y = oracle.m2_eager(A, D, x, B, C, dt, h)            # one uninterrupted run
    hc = h0.copy()
    oracle.m2_eager(A, D, x[:last + 1], B[:last + 1], C[:last + 1], dt[:last + 1], hc)
    err = float(np.abs(res["y"] - y).max())
    err = max(err, float(np.abs(res["ckpt"] - hc).max()))
    err = max(err, float(np.abs(res["state"] - h).max()))
    assert list(np.nonzero(res["committed"])[0]) == [t for t in range(T) if (t + 1) % interval == 0]
    return err


def _gdn_decode_pin_error(decode_fn, T=21, interval=4):
    rng = np.random.default_rng(68)
    b, H, d = 2, 3, 6
    q, k = _unit(rng, T, b, H, d), _unit(rng, T, b, H, d)
    v = rng.standard_normal((T, b, H, d))
    al = rng.uniform(0.3, 0.9, (T, b, H))
    be = rng.uniform(0.2, 0.8, (T, b, H))
    S0 = rng.normal(0, 0.3, (b, H, d, d))
    res = decode_fn(q, k, v, al, be, S0, interval, interval)
    last = max(t for t in range(T) if (t + 1) % interval == 0)
    S = S0.copy()
    o = oracle.gdn_eager(q, k, v, al, be, S)
    Sc = S0.copy()
    oracle.gdn_eager(q[:last + 1], k[:last + 1], v[:last + 1], al[:last + 1], be[:last + 1], Sc)
    err = float(np.abs(res["o"] - o).max())
    err = max(err, float(np.abs(res["ckpt"] - Sc).max()))
    err = max(err, float(np.abs(res["state"] - S).max()))
    return err


def _m2_ckpt_one_late(A, D, x, B, C, dt, h0, interval, cap):
    """Mistake: the snapshot is taken one step after the commit."""
    res = drivers.m2_decode(A, D, x, B, C, dt, h0, interval, cap)
    last = int(np.nonzero(res["committed"])[0][-1])
    h = np.array(h0, dtype=np.float64, copy=True)
    oracle.m2_eager(A, D, x[:last + 2], B[:last + 2], C[:last + 2], dt[:last + 2], h)
    return dict(res, ckpt=h)


def _m2_ckpt_first_commit(A, D, x, B, C, dt, h0, interval, cap):
    """Mistake: the snapshot of the first commit is kept."""
    res = drivers.m2_decode(A, D, x, B, C, dt, h0, interval, cap)
    h = np.array(h0, dtype=np.float64, copy=True)
    oracle.m2_eager(A, D, x[:interval], B[:interval], C[:interval], dt[:interval], h)
    return dict(res, ckpt=h)


def _gdn_ckpt_initial(q, k, v, al, be, S0, interval, cap):
    """Mistake: the snapshot is never refreshed."""
    res = drivers.gdn_decode(q, k, v, al, be, S0, interval, cap)
    return dict(res, ckpt=np.array(S0, dtype=np.float64))


def _gdn_ckpt_one_early(q, k, v, al, be, S0, interval, cap):
    res = drivers.gdn_decode(q, k, v, al, be, S0, interval, cap)
    last = int(np.nonzero(res["committed"])[0][-1])
    S = np.array(S0, dtype=np.float64, copy=True)
    oracle.gdn_eager(q[:last], k[:last], v[:last], al[:last], be[:last], S)
    return dict(res, ckpt=S)


def test_m2_decode_checkpoint_and_outputs():
    assert _m2_decode_pin_error(drivers.m2_decode) < 1e-13


def test_gdn_decode_checkpoint_and_outputs():
    assert _gdn_decode_pin_error(drivers.gdn_decode) < 1e-13


@pytest.mark.parametrize("mutant", [_m2_ckpt_one_late, _m2_ckpt_first_commit])
def test_m2_decode_pin_rejects_planted_mistakes(mutant):
    assert _m2_decode_pin_error(mutant) > 1e-4


@pytest.mark.parametrize("mutant", [_gdn_ckpt_initial, _gdn_ckpt_one_early])
def test_gdn_decode_pin_rejects_planted_mistakes(mutant):
    assert _gdn_decode_pin_error(mutant) > 1e-4


def test_decode_without_commit_keeps_the_initial_checkpoint():
    rng = np.random.default_rng(69)
    A, D, x, B, C, dt, h0 = _m2_case(rng, 3, 1, 2, 1, 4, 8)
    res = drivers.m2_decode(A, D, x, B, C, dt, h0, 8, 8)
    np.testing.assert_array_equal(res["ckpt"], h0)
    assert not res["committed"].any()
