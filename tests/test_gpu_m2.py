"""Mamba-2 parity: HIP path (through the C ABI) vs the fp64 oracle.

Outputs: max over output vectors of ||y - y_oracle||_inf / ||y_oracle||_inf
<= 1e-4, for y and for its state part y - D x (which is ~60x smaller than D x
at these distributions, so a check on y alone would hide replay errors).
Indices (checkpoint position, buffer length): bit-exact.
"""
import numpy as np
import pytest

import oracle
from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _case(seed, T, b, H, G, P=64, N=128):
    A, D = syn.m2_params(seed, H)
    h0 = syn.m2_state0(seed, b, H, P, N)
    st = syn.m2_steps(seed, 0, T, b, H, G, P, N)
    return A, D, h0, st


_check_outputs = gu.check_m2_outputs


@pytest.mark.parametrize("fused", [False, True], ids=["standalone_commit", "fused_commit"])
def test_decode_small(fused):
    """batch 4, 8 heads, 1 group, 64 steps, commit interval 16, ring 16."""
    T, b, H, G, interval, cap = 64, 4, 8, 1, 16, 16
    A, D, h0, st = _case(0, T, b, H, G)
    L = gu.m2_layer(A, D, h0, G, cap)
    y, pos, ln = gu.m2_decode(L, {k: gu.dev(v) for k, v in st.items()}, interval, fused)
    ref = drivers.m2_decode(A, D, st["x"], st["B"], st["C"], st["dt"], h0, interval, cap)
    _check_outputs(gu.host(y), ref["y"], st["x"], D)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    ck = gu.host(L.ckpt)
    assert gu.vec_rel_err(ck, ref["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("fused", [False, True], ids=["standalone_commit", "fused_commit"])
def test_decode_ragged(fused):
    """batch 3 x 10 heads (30 tiles: not a multiple of the 8 XCDs), 5 groups
    of 2 heads, ring 5, interval 5, 23 steps (ends mid-interval)."""
    T, b, H, G, interval, cap = 23, 3, 10, 5, 5, 5
    A, D, h0, st = _case(1, T, b, H, G)
    L = gu.m2_layer(A, D, h0, G, cap)
    y, pos, ln = gu.m2_decode(L, {k: gu.dev(v) for k, v in st.items()}, interval, fused)
    ref = drivers.m2_decode(A, D, st["x"], st["B"], st["C"], st["dt"], h0, interval, cap)
    _check_outputs(gu.host(y), ref["y"], st["x"], D)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])


def test_eager_small():
    T, b, H, G = 64, 4, 8, 1
    A, D, h0, st = _case(2, T, b, H, G)
    L = gu.m2_layer(A, D, h0, G, 16)
    t_ = gu.torch()
    d = {k: gu.dev(v) for k, v in st.items()}
    y = t_.empty_like(d["x"])
    for t in range(T):
        R.rssm_eager_step(L, dict(x=d["x"][t], B=d["B"][t], C=d["C"][t], dt=d["dt"][t]), y[t])
    h = h0.astype(np.float64)
    want = oracle.m2_eager(A, D, st["x"], st["B"], st["C"], st["dt"], h)
    _check_outputs(gu.host(y), want, st["x"], D)
    assert gu.vec_rel_err(gu.host(L.ckpt), h) <= 1e-5


def test_serving_shape_sampled():
    """batch 256, 80 heads, 8 groups, interval 8 = ring 8, fused commit (the
    configuration the benchmark times); 64 steps; the oracle recomputes three
    whole sequences (all heads)."""
    T, b, H, G, interval, cap = 64, 256, 80, 8, 8, 8
    A, D, h0, st = _case(3, T, b, H, G)
    L = gu.m2_layer(A, D, h0, G, cap)
    d = {k: gu.dev(v) for k, v in st.items()}
    y, _, _ = gu.m2_decode(L, d, interval, fused=True, record=False)
    sel = [0, 137, 255]
    yh = gu.host(y[:, sel])
    pos, ln = gu.indices(L)
    sub = {k: np.ascontiguousarray(v[:, sel]) for k, v in st.items()}
    ref = drivers.m2_decode(A, D, sub["x"], sub["B"], sub["C"], sub["dt"], h0[sel],
                            interval, cap)
    _check_outputs(yh, ref["y"], sub["x"], D)
    assert (pos == T).all() and (ln == 0).all()
    assert gu.vec_rel_err(gu.host(L.ckpt[sel]), ref["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0


def test_overflow_sets_status_and_leaves_sequence_unchanged():
    T, b, H, G, cap = 5, 2, 8, 1, 4
    A, D, h0, st = _case(4, T, b, H, G)
    L = gu.m2_layer(A, D, h0, G, cap)
    d = {k: gu.dev(v) for k, v in st.items()}
    t_ = gu.torch()
    y = t_.zeros_like(d["x"])
    for t in range(T):    # never commit: the 5th append overflows the 4-slot ring
        R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y[t])
    pos, ln = gu.indices(L)
    assert (ln == cap).all() and (pos == 0).all()
    yh = gu.host(y)
    assert np.isnan(yh[4]).all() and np.isfinite(yh[:4]).all()
    assert R.rssm_status(L) == R.STATUS_OVERFLOW
    assert R.rssm_status(L) == 0     # cleared by the read


# ------------------------------------------------------ verify / rollback --

def _spec_inputs(seed, rounds, n, b, H, G, pool=None):
    T = rounds * n if pool is None else pool
    st = syn.m2_steps(seed, 0, T, b, H, G, 64, 128)
    if pool is not None:
        idx = np.arange(rounds * n) % pool
        st = {k: v[idx] for k, v in st.items()}
    return syn.stack_rounds(st, rounds, n)


def _run_spec_gpu(L, drafts_dev, accept, n, commit_len, sel=None):
    """Verify / rollback / commit rounds.  Returns (outputs of the selected
    sequences [R,n,len(sel),H,P], pos [R,b], len [R,b])."""
    t_ = gu.torch()
    Rn = accept.shape[0]
    out = t_.empty_like(drafts_dev["x"][0])
    ys, pos, ln = [], [], []
    for r in range(Rn):
        R.rssm_verify(L, n, dict(x=drafts_dev["x"][r], B=drafts_dev["B"][r],
                                 C=drafts_dev["C"][r], dt=drafts_dev["dt"][r]), out)
        nrej = gu.dev((n - accept[r]).astype(np.int32))
        R.rssm_rollback(L, nrej)
        R.rssm_commit(L, None, commit_len)
        ys.append(gu.host(out if sel is None else out[:, sel]))
        p, l = gu.indices(L)
        pos.append(p)
        ln.append(l)
    return np.array(ys), np.array(pos), np.array(ln)


def test_verify_rollback_small():
    rounds, n, b, H, G, cap, commit_len = 40, 4, 8, 8, 2, 12, 8
    A, D = syn.m2_params(5, H)
    h0 = syn.m2_state0(5, b, H, 64, 128)
    drafts = _spec_inputs(5, rounds, n, b, H, G)
    accept = syn.accept_counts(5, rounds, b, n)
    L = gu.m2_layer(A, D, h0, G, cap)
    y, pos, ln = _run_spec_gpu(L, {k: gu.dev(v) for k, v in drafts.items()}, accept, n,
                               commit_len)
    ref = drivers.m2_spec_rounds(A, D, h0, drafts, accept, cap, commit_len)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    _check_outputs(y, ref["y"], drafts["x"], D)
    assert R.rssm_status(L) == 0


def test_rollback_past_checkpoint_is_refused():
    b, H, G = 4, 8, 1
    A, D, h0, st = _case(6, 3, b, H, G)
    L = gu.m2_layer(A, D, h0, G, 8)
    d = {k: gu.dev(v) for k, v in st.items()}
    y = gu.torch().empty_like(d["x"])
    for t in range(3):
        R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y[t])
    R.rssm_rollback(L, gu.dev(np.array([1, 4, -1, 3], np.int32)))
    _, ln = gu.indices(L)
    assert ln.tolist() == [2, 3, 3, 0]
    assert R.rssm_status(L) == R.STATUS_ROLLBACK


def test_rollback_reappend_and_rerun_are_bitwise_identical():
    """Roll back k entries and append the same inputs again: outputs, ring
    and checkpoint are bitwise those of the first pass; a rerun from the same
    state is bitwise identical too."""
    T, b, H, G, cap = 7, 4, 8, 2, 8
    A, D, h0, st = _case(7, T, b, H, G)
    d = {k: gu.dev(v) for k, v in st.items()}

    def run(L, ts):
        ys = []
        for t in ts:
            y = gu.torch().empty_like(d["x"][0])
            R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y)
            ys.append(gu.host(y))
        return ys

    L = gu.m2_layer(A, D, h0, G, cap)
    first = run(L, range(T))
    R.rssm_rollback(L, gu.dev(np.full(b, 3, np.int32)))
    again = run(L, range(T - 3, T))
    for a_, b_ in zip(first[T - 3:], again):
        np.testing.assert_array_equal(a_, b_)
    L2 = gu.m2_layer(A, D, h0, G, cap)
    rerun = run(L2, range(T))
    for a_, b_ in zip(first, rerun):
        np.testing.assert_array_equal(a_, b_)
    for r1, r2 in zip(L.rings, L2.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
    np.testing.assert_array_equal(gu.host(L.ckpt), gu.host(L2.ckpt))


def test_speculative_serving_shape():
    """batch 256, 80 heads, 8 groups, ring 12, 4 drafts per round, accepted
    counts uniform in 0..4, commit when the buffer reaches 8; 512 rounds.
    Index traces of all 256 sequences are compared bit-exactly; draft outputs
    of two whole sequences against the oracle.  Draft inputs cycle through a
    pool of 64 distinct steps."""
    rounds, n, b, H, G, cap, commit_len = 512, 4, 256, 80, 8, 12, 8
    A, D = syn.m2_params(8, H)
    h0 = syn.m2_state0(8, b, H, 64, 128)
    accept = syn.accept_counts(8, rounds, b, n)
    pool = syn.m2_steps(8, 0, 64, b, H, G, 64, 128)
    pool_dev = {k: gu.dev(v) for k, v in pool.items()}
    idx = (np.arange(rounds * n) % 64).reshape(rounds, n)
    t_ = gu.torch()
    L = gu.m2_layer(A, D, h0, G, cap)
    sel = [3, 200]
    out = t_.empty((n, b, H, 64), dtype=t_.float32, device="cuda")
    ys, pos, ln = [], [], []
    for r in range(rounds):
        j0 = int(idx[r, 0])      # 64 % n == 0: every round is a contiguous window
        dr = {k: v[j0:j0 + n] for k, v in pool_dev.items()}
        R.rssm_verify(L, n, dict(x=dr["x"], B=dr["B"], C=dr["C"], dt=dr["dt"]), out)
        R.rssm_rollback(L, gu.dev((n - accept[r]).astype(np.int32)))
        R.rssm_commit(L, None, commit_len)
        ys.append(gu.host(out[:, sel]))
        p, l = gu.indices(L)
        pos.append(p)
        ln.append(l)
    from oracle.index_model import IndexModel
    im = IndexModel(b, cap)
    for r in range(rounds):
        im.append(n)
        im.rollback(n - accept[r])
        im.commit(min_len=commit_len)
        np.testing.assert_array_equal(pos[r], im.pos)
        np.testing.assert_array_equal(ln[r], im.len)
    assert im.status == 0
    sub = {k: np.ascontiguousarray(v[:, sel][idx.reshape(-1)]) for k, v in pool.items()}
    sub = syn.stack_rounds(sub, rounds, n)
    ref = drivers.m2_spec_rounds(A, D, h0[sel], sub, accept[:, sel], cap, commit_len)
    _check_outputs(np.array(ys), ref["y"], sub["x"], D)
    assert R.rssm_status(L) == 0
