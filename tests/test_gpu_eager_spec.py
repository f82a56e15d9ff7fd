"""The eager speculative comparator on the GPU (rssm_eager_spec_round /
rssm_eager_spec_accept) against the fp64 oracle.

Rounds of n drafts with random accept counts: every draft output equals the
oracle's speculative-round outputs (the eager recurrence continued over the
drafts from the accepted state) within the fp32 tolerance, and after the
rounds the current slot of every sequence holds the oracle's accepted state
(1e-5).  An out-of-range accept count raises RSSM_STATUS_ROLLBACK and leaves
the slot index unchanged.
"""
import numpy as np
import pytest

from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N, DK = 64, 128, 128


def _run(L, slots, cur, drafts, accept, names, n):
    t_ = gu.torch()
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out_name = "x" if "x" in names else "v"
    ys = []
    for r in range(accept.shape[0]):
        out = t_.empty_like(dd[out_name][r])
        R.rssm_eager_spec_round(L, n, {k: dd[k][r] for k in names}, out, slots, cur)
        R.rssm_eager_spec_accept(L, n, cur, gu.dev(accept[r]))
        ys.append(gu.host(out))
    return np.stack(ys)


def _current(slots, cur):
    s, c = gu.host(slots), gu.host(cur)
    return np.stack([s[c[b], b] for b in range(len(c))])


def test_m2_eager_spec_rounds():
    rounds, n, b, H, G = 5, 4, 3, 10, 5
    A, D = syn.m2_params(210, H)
    h0 = syn.m2_state0(210, b, H, P, N)
    drafts = syn.stack_rounds(syn.m2_steps(210, 0, rounds * n, b, H, G, P, N), rounds, n)
    accept = syn.accept_counts(210, rounds, b, n)
    L = gu.m2_layer(A, D, h0, G, 16)
    t_ = gu.torch()
    slots = t_.zeros((n + 1, b, H, P, N), dtype=t_.float32, device="cuda")
    slots[2].copy_(gu.dev(h0))                 # any starting slot
    cur = gu.dev(np.full(b, 2, np.int32))
    y = _run(L, slots, cur, drafts, accept, ("x", "B", "C", "dt"), n)
    ref = drivers.m2_spec_rounds(A, D, h0, drafts, accept, 64, 1 << 20)
    for r in range(rounds):
        gu.check_m2_outputs(y[r], ref["y"][r], drafts["x"][r], D)
    assert gu.vec_rel_err(_current(slots, cur), ref["state"]) <= 1e-5
    np.testing.assert_array_equal(gu.host(cur), (2 + accept.sum(0)) % (n + 1))
    assert R.rssm_status(L) == 0


def test_gdn_eager_spec_rounds():
    rounds, n, b, H = 5, 3, 3, 4
    S0 = syn.gdn_state0(211, b, H, DK, DK, std=0.1)
    drafts = syn.stack_rounds(syn.gdn_steps(211, 0, rounds * n, b, H, DK, DK), rounds, n)
    accept = syn.accept_counts(211, rounds, b, n)
    L = gu.gdn_layer(S0, 16)
    t_ = gu.torch()
    slots = t_.zeros((n + 1, b, H, DK, DK), dtype=t_.float32, device="cuda")
    slots[0].copy_(gu.dev(S0))
    cur = gu.dev(np.zeros(b, np.int32))
    o = _run(L, slots, cur, drafts, accept, ("q", "k", "v", "alpha", "beta"), n)
    ref = drivers.gdn_spec_rounds(S0, drafts, accept, 64, 1 << 20)
    assert gu.vec_rel_err(o, ref["o"]) <= gu.TOL_F32
    assert gu.vec_rel_err(_current(slots, cur), ref["state"]) <= 1e-5
    assert R.rssm_status(L) == 0


def test_eager_spec_bad_accept_leaves_sequence():
    n, b, H, G = 2, 3, 10, 5
    A, D = syn.m2_params(212, H)
    L = gu.m2_layer(A, D, syn.m2_state0(212, b, H, P, N), G, 16)
    cur = gu.dev(np.array([0, 1, 2], np.int32))
    R.rssm_eager_spec_accept(L, n, cur, gu.dev(np.array([1, 3, -1], np.int32)))
    assert gu.host(cur).tolist() == [1, 1, 2]
    assert R.rssm_status(L) == R.STATUS_ROLLBACK
