"""Pins of the oracle's index model and workload drivers (CPU only).

Index model: a hand-worked trace, the conservation invariant under random
operations, and the two error conditions.  Drivers: speculative rounds agree
with a plain decode that only ever saw the accepted tokens; the dual
low-precision emulation obeys the one-quantisation error bound at every step
and the shared one does not improve on it; quantisation idempotence.
"""
import numpy as np
import pytest

import oracle
from oracle import drivers, replay
from oracle.index_model import (IndexModel, STATUS_OVERFLOW, STATUS_ROLLBACK)


def test_hand_trace():
    im = IndexModel(1, 4)
    im.append(3)
    assert (im.pos[0], im.len[0]) == (0, 3)
    assert [im.slot(0, j) for j in range(3)] == [0, 1, 2]
    im.rollback([2])
    assert im.len[0] == 1 and im.status == 0
    im.append(3)
    assert im.len[0] == 4
    ok = im.append(1)                       # 5 > cap: refused, unchanged
    assert not ok[0] and im.len[0] == 4 and im.status & STATUS_OVERFLOW
    im.commit()
    assert (im.pos[0], im.len[0]) == (4, 0)
    assert im.slot(0, 0) == 0 and im.slot(0, 3) == 3
    im.append(2)
    im.commit(min_len=3)                    # len 2 < 3: no commit
    assert (im.pos[0], im.len[0]) == (4, 2)
    assert [im.slot(0, j) for j in range(2)] == [0, 1]
    im.status = 0
    ok = im.rollback([3])                   # past the checkpoint: refused
    assert not ok[0] and im.len[0] == 2 and im.status == STATUS_ROLLBACK
    ok = im.rollback([-1])
    assert not ok[0] and im.len[0] == 2


def test_conservation_under_random_ops():
    rng = np.random.default_rng(30)
    b, cap = 16, 12
    im = IndexModel(b, cap)
    net = np.zeros(b, np.int64)
    for _ in range(400):
        op = rng.integers(3)
        if op == 0:
            n = int(rng.integers(1, 5))
            ok = im.append(n)
            net[ok] += n
        elif op == 1:
            k = rng.integers(-1, 6, size=b)
            ok = im.rollback(k)
            net[ok] -= k[ok]
        else:
            im.commit(mask=rng.integers(0, 2, size=b).astype(bool),
                      min_len=int(rng.integers(0, 9)))
        assert np.all((im.len >= 0) & (im.len <= cap))
        np.testing.assert_array_equal(im.pos + im.len, net)


def test_decode_trace_commit_every_interval():
    pos, ln, com = drivers.decode_trace(3, 20, 8, 8)
    assert np.nonzero(com)[0].tolist() == [7, 15]
    assert ln[:, 0].tolist() == [1, 2, 3, 4, 5, 6, 7, 0] * 2 + [1, 2, 3, 4]
    assert pos[:, 0].tolist() == [0] * 7 + [8] * 8 + [16] * 5


def _m2_case(rng, T, batch, H=2, G=1, P=4, N=8):
    x = rng.standard_normal((T, batch, H, P)) / np.sqrt(N)
    B = rng.standard_normal((T, batch, G, N)) / np.sqrt(N)
    C = rng.standard_normal((T, batch, G, N)) / np.sqrt(N)
    dt = np.logaddexp(0, rng.normal(-2, 0.5, (T, batch, H)))
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.standard_normal(H)
    h0 = rng.normal(0, 0.1, (batch, H, P, N))
    return A, D, dict(x=x, B=B, C=C, dt=dt), h0


def test_spec_rounds_match_decode_of_accepted_tokens():
    """The draft outputs at accepted positions equal the outputs of a plain
    decode whose history is exactly the accepted tokens; the final state too."""
    rng = np.random.default_rng(31)
    R, n, batch = 12, 4, 5
    A, D, d, h0 = _m2_case(rng, R * n, batch)
    drafts = {k: v.reshape((R, n) + v.shape[1:]) for k, v in d.items()}
    accept = rng.integers(0, n + 1, size=(R, batch))
    res = drivers.m2_spec_rounds(A, D, h0, drafts, accept, cap=12, commit_len=8)
    assert res["status"] == 0
    for b in range(batch):
        keep = [(r, j) for r in range(R) for j in range(accept[r, b])]
        if not keep:
            continue
        sel = lambda a: np.stack([a[r, j, b] for r, j in keep])[:, None]
        h = h0[b:b + 1].copy()
        y = oracle.m2_eager(A, D, sel(drafts["x"]), sel(drafts["B"]), sel(drafts["C"]),
                            sel(drafts["dt"]), h)
        for i, (r, j) in enumerate(keep):
            np.testing.assert_allclose(res["y"][r, j, b], y[i, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(res["state"][b], h[0], rtol=1e-12, atol=1e-14)
    # index trace: conservation and commit rule
    tot = accept.cumsum(axis=0)
    np.testing.assert_array_equal(res["pos"] + res["len"], tot)
    assert np.all(res["len"] < 8)


def test_gdn_spec_rounds_match_decode_of_accepted_tokens():
    rng = np.random.default_rng(32)
    R, n, batch, H, dk, dv = 6, 4, 3, 2, 8, 8
    T = R * n
    q = rng.standard_normal((T, batch, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, batch, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, batch, H, dv))
    al = np.exp(-np.logaddexp(0, rng.standard_normal((T, batch, H))))
    be = 1 / (1 + np.exp(-rng.standard_normal((T, batch, H))))
    d = dict(q=q, k=k, v=v, alpha=al, beta=be)
    drafts = {kk: vv.reshape((R, n) + vv.shape[1:]) for kk, vv in d.items()}
    S0 = rng.normal(0, 0.1, (batch, H, dv, dk))
    accept = rng.integers(0, n + 1, size=(R, batch))
    res = drivers.gdn_spec_rounds(S0, drafts, accept, cap=12, commit_len=8)
    for b in range(batch):
        keep = [(r, j) for r in range(R) for j in range(accept[r, b])]
        if not keep:
            continue
        sel = lambda a: np.stack([a[r, j, b] for r, j in keep])[:, None]
        S = S0[b:b + 1].copy()
        o = oracle.gdn_eager(*(sel(drafts[s]) for s in ("q", "k", "v", "alpha", "beta")), S)
        for i, (r, j) in enumerate(keep):
            np.testing.assert_allclose(res["o"][r, j, b], o[i, 0], rtol=1e-12, atol=1e-13)


def _gdn_case(rng, T, batch, H, d, slow=False):
    q = rng.standard_normal((T, batch, H, d)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, batch, H, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, batch, H, d))
    mu = -5.0 if slow else 0.0
    al = np.exp(-np.logaddexp(0, rng.normal(mu, 1.0, (T, batch, H))))
    be = 1 / (1 + np.exp(-rng.standard_normal((T, batch, H))))
    return q, k, v, al, be


def _one_quant_bound(res, q, k, al, be, interval, lp):
    """Per-element bound: |o - o_exact| <= sum_j delta(S_c[r,j]) |q~_j| + 1e-9 |o|inf,
    delta = half an lp ulp at the exact checkpoint S_c of the last commit."""
    T, batch, H, d = q.shape
    ok = True
    ck = None
    ckpts = {}
    # rebuild the exact checkpoint after each commit by an eager run
    S = np.zeros((batch, H, d, d))
    for t in range(T):
        if t % interval == 0:
            ckpts[t] = S.copy()
        oracle.gdn_eager(q[t:t + 1], k[t:t + 1], res["v"][t:t + 1], al[t:t + 1],
                         be[t:t + 1], S)
    worst = 0.0
    for t in range(T):
        c0 = (t // interval) * interval
        Sc = ckpts[c0]
        U = batch * H
        qt, _ = drivers.gdn_carry_batched(
            q[t].reshape(U, d), k[c0:t + 1].transpose(1, 2, 0, 3).reshape(U, -1, d),
            al[c0:t + 1].transpose(1, 2, 0).reshape(U, -1),
            be[c0:t + 1].transpose(1, 2, 0).reshape(U, -1))
        if lp == "bf16":
            delta = 2.0 ** -8 * np.abs(Sc)
        else:
            amax = np.abs(Sc).reshape(batch, H, -1).max(-1)
            sc = np.where(amax > 0, amax / 448.0, 1.0)[..., None, None]
            delta = np.maximum(2.0 ** -4 * np.abs(Sc), 2.0 ** -10 * sc)
        bound = np.einsum("bhrc,bhc->bhr", delta, np.abs(qt.reshape(batch, H, d)))
        err = np.abs(res["o_emul"][t] - res["o_exact"][t])
        scale = np.abs(res["o_exact"][t]).max()
        worst = max(worst, float((err - bound).max() / scale))
        ok &= bool(np.all(err <= bound * (1 + 1e-6) + 1e-9 * scale))
    return ok, worst


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
def test_dual_emulation_obeys_one_quantisation_bound(lp):
    rng = np.random.default_rng(33)
    T, batch, H, d, interval = 40, 2, 2, 16, 8
    q, k, v, al, be = _gdn_case(rng, T, batch, H, d, slow=True)
    res = drivers.gdn_lowprec(q, k, v, al, be, np.zeros((batch, H, d, d)),
                              interval, "dual", lp)
    res["v"] = v
    # the exact path is the eager recurrence itself
    S = np.zeros((batch, H, d, d))
    np.testing.assert_allclose(res["o_exact"], oracle.gdn_eager(q, k, v, al, be, S),
                               rtol=0, atol=0)
    ok, worst = _one_quant_bound(res, q, k, al, be, interval, lp)
    assert ok, worst
    # shared feeds its own rounding back: it is never better by much and
    # with slow decay it is worse on average
    sh = drivers.gdn_lowprec(q, k, v, al, be, np.zeros((batch, H, d, d)),
                             interval, "shared", lp)
    e_dual = np.abs(res["o_emul"] - res["o_exact"]).mean()
    e_sh = np.abs(sh["o_emul"] - sh["o_exact"]).mean()
    assert e_sh > e_dual


def test_quantise_is_idempotent_on_its_own_output():
    rng = np.random.default_rng(34)
    s = rng.standard_normal((2, 3, 8, 8)).astype(np.float32)
    for lp in ("bf16", "e4m3"):
        c1, sc1, v1 = drivers.quantize(s, lp)
        c2, sc2, v2 = drivers.quantize(v1.astype(np.float32), lp)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(v1, v2)


def test_tree_paths():
    from oracle.drivers import tree_paths
    assert tree_paths([-1, 0, 0, 1, -1]) == [[0], [0, 1], [0, 2], [0, 1, 3], [4]]
    import pytest as _pt
    with _pt.raises(ValueError):
        tree_paths([-1, 2, 0])


def test_tree_verify_chain_equals_speculative_outputs():
    """A chain (parent[j] = j - 1) is linear verification: outputs equal the
    eager continuation over the drafts; a star (all parents -1) gives every
    draft the one-step output from the same state."""
    import numpy as np
    import oracle
    from oracle import drivers
    rng = np.random.default_rng(7)
    n, b, H, G, P, N = 4, 2, 4, 2, 4, 8
    A = -np.exp(rng.uniform(0, 2, H)); D = rng.standard_normal(H)
    h = rng.standard_normal((b, H, P, N))
    dr = dict(x=rng.standard_normal((n, b, H, P)), B=rng.standard_normal((n, b, G, N)),
              C=rng.standard_normal((n, b, G, N)), dt=rng.uniform(0.05, 0.3, (n, b, H)))
    chain = drivers.m2_tree_verify(A, D, h, dr, [-1, 0, 1, 2])
    want = oracle.m2_eager(A, D, dr["x"], dr["B"], dr["C"], dr["dt"], h.copy())
    np.testing.assert_array_equal(chain, want)
    star = drivers.m2_tree_verify(A, D, h, dr, [-1, -1, -1, -1])
    for j in range(n):
        one = oracle.m2_eager(A, D, dr["x"][j:j + 1], dr["B"][j:j + 1], dr["C"][j:j + 1],
                              dr["dt"][j:j + 1], h.copy())
        np.testing.assert_array_equal(star[j], one[0])
