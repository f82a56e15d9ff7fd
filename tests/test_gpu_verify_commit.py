"""rssm_verify_commit (Mamba-2, fp32 checkpoint): draft verification that
first folds a full buffer into the checkpoint from the same state read.

Pinned against the fp64 oracle: draft outputs of speculative rounds are the
eager recurrence's (the explainer's "Cheap speculative decoding rollback";
when the commit happens does not change them), the index trace equals the
integer model's commit-then-append at every verify, bit-exactly, and the
checkpoint after a final commit is the oracle state after every accepted
token.  Against the standalone path on the GPU: the folded checkpoint is
bitwise that of rssm_commit (same arithmetic, same order), indices equal.
"""
import numpy as np
import pytest

from oracle import drivers
from oracle.index_model import IndexModel
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu


def _drafts(seed, rounds, n, b, H, G):
    st = syn.m2_steps(seed, 0, rounds * n, b, H, G, 64, 128)
    return syn.stack_rounds(st, rounds, n)


def _tile_rel(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = np.abs(got - want).max(axis=(-2, -1))
    den = np.abs(want).max(axis=(-2, -1))
    return float((num / den).max())


def test_spec_rounds_against_oracle():
    # ring 16: a buffer of up to 11 entries waits for the next verify's fold
    # while that verify's 4 drafts take their slots
    rounds, n, b, H, G, cap, commit_len = 40, 4, 8, 8, 2, 16, 8
    A, D = syn.m2_params(31, H)
    h0 = syn.m2_state0(31, b, H, 64, 128)
    drafts = _drafts(31, rounds, n, b, H, G)
    accept = syn.accept_counts(31, rounds, b, n)
    d = {k: gu.dev(v) for k, v in drafts.items()}
    L = gu.m2_layer(A, D, h0, G, cap)
    out = gu.torch().empty_like(d["x"][0])
    im = IndexModel(b, cap)
    ys = []
    for r in range(rounds):
        R.rssm_verify_commit(L, n, dict(x=d["x"][r], B=d["B"][r], C=d["C"][r], dt=d["dt"][r]),
                             out, commit_len)
        im.commit(min_len=commit_len)
        assert im.append(n).all()
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        ys.append(gu.host(out))
        R.rssm_rollback(L, gu.dev((n - accept[r]).astype(np.int32)))
        im.rollback(n - accept[r])
    ref = drivers.m2_spec_rounds(A, D, h0, drafts, accept, cap, commit_len)
    gu.check_m2_outputs(np.array(ys), ref["y"], drafts["x"], D)
    R.rssm_commit(L, None, 1)    # fold what is left: the state after every accepted token
    assert _tile_rel(gu.host(L.ckpt), ref["state"]) <= 1e-4
    assert R.rssm_status(L) == 0


def test_fold_matches_standalone_commit_bitwise():
    """Two layers with the same ragged buffers: rssm_commit + rssm_verify on
    one, rssm_verify_commit on the other.  Checkpoints bitwise equal, indices
    equal, draft outputs within the fp32 tolerance of each other."""
    b, H, G, cap, n, min_len = 6, 8, 2, 16, 3, 5
    A, D = syn.m2_params(32, H)
    h0 = syn.m2_state0(32, b, H, 64, 128)
    st = syn.m2_steps(32, 0, 9, b, H, G, 64, 128)
    dr = syn.m2_steps(32, 9, n, b, H, G, 64, 128)
    d = {k: gu.dev(v) for k, v in st.items()}
    dd = {k: gu.dev(v) for k, v in dr.items()}
    nrej = gu.dev(np.array([0, 2, 4, 5, 8, 9], np.int32))   # lens 9, 7, 5, 4, 1, 0

    def prepare():
        L = gu.m2_layer(A, D, h0, G, cap)
        y = gu.torch().empty_like(d["x"][0])
        for t in range(9):
            R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y)
        R.rssm_rollback(L, nrej)
        return L

    L1, L2 = prepare(), prepare()
    o1 = gu.torch().empty_like(dd["x"])
    o2 = gu.torch().empty_like(dd["x"])
    inp = dict(x=dd["x"], B=dd["B"], C=dd["C"], dt=dd["dt"])
    R.rssm_commit(L1, None, min_len)
    R.rssm_verify(L1, n, inp, o1)
    R.rssm_verify_commit(L2, n, inp, o2, min_len)
    np.testing.assert_array_equal(gu.host(L1.ckpt), gu.host(L2.ckpt))
    for a_, b_ in zip(gu.indices(L1), gu.indices(L2)):
        np.testing.assert_array_equal(a_, b_)
    assert gu.vec_rel_err(gu.host(o2), gu.host(o1)) <= gu.TOL_F32
    pos, ln = gu.indices(L2)
    assert ln.tolist() == [n, n, n, 4 + n, 1 + n, n] and pos.tolist() == [9, 7, 5, 0, 0, 0]
    for r1, r2 in zip(L1.rings, L2.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
    assert R.rssm_status(L1) == 0 and R.rssm_status(L2) == 0


def test_no_sequence_due_equals_plain_verify():
    """min_len above every buffer: bitwise rssm_verify, checkpoint untouched."""
    b, H, G, cap, n = 4, 8, 1, 16, 4
    A, D = syn.m2_params(33, H)
    h0 = syn.m2_state0(33, b, H, 64, 128)
    st = syn.m2_steps(33, 0, 3, b, H, G, 64, 128)
    dr = syn.m2_steps(33, 3, n, b, H, G, 64, 128)
    d = {k: gu.dev(v) for k, v in st.items()}
    dd = {k: gu.dev(v) for k, v in dr.items()}
    outs = []
    layers = []
    for fused in (False, True):
        L = gu.m2_layer(A, D, h0, G, cap)
        y = gu.torch().empty_like(d["x"][0])
        for t in range(3):
            R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y)
        o = gu.torch().empty_like(dd["x"])
        inp = dict(x=dd["x"], B=dd["B"], C=dd["C"], dt=dd["dt"])
        if fused:
            R.rssm_verify_commit(L, n, inp, o, 4)
        else:
            R.rssm_verify(L, n, inp, o)
        outs.append(gu.host(o))
        layers.append(L)
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(gu.host(layers[1].ckpt), h0.astype(np.float32))
    for a_, b_ in zip(gu.indices(layers[0]), gu.indices(layers[1])):
        np.testing.assert_array_equal(a_, b_)


def test_overflowing_sequence_is_neither_folded_nor_appended():
    b, H, G, cap, n = 3, 8, 2, 8, 4
    A, D = syn.m2_params(34, H)
    h0 = syn.m2_state0(34, b, H, 64, 128)
    st = syn.m2_steps(34, 0, 6, b, H, G, 64, 128)
    dr = syn.m2_steps(34, 6, n, b, H, G, 64, 128)
    d = {k: gu.dev(v) for k, v in st.items()}
    dd = {k: gu.dev(v) for k, v in dr.items()}
    L = gu.m2_layer(A, D, h0, G, cap)
    y = gu.torch().empty_like(d["x"][0])
    for t in range(6):
        R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t], d["dt"][t], y)
    R.rssm_rollback(L, gu.dev(np.array([0, 2, 6], np.int32)))     # lens 6, 4, 0
    rings = [gu.host(r).copy() for r in L.rings]
    o = gu.torch().empty_like(dd["x"])
    R.rssm_verify_commit(L, n, dict(x=dd["x"], B=dd["B"], C=dd["C"], dt=dd["dt"]), o, 4)
    pos, ln = gu.indices(L)
    assert pos.tolist() == [0, 4, 0] and ln.tolist() == [6, n, n]
    oh = gu.host(o)
    assert np.isnan(oh[:, 0]).all() and np.isfinite(oh[:, 1:]).all()
    ck = gu.host(L.ckpt)
    np.testing.assert_array_equal(ck[0], h0[0].astype(np.float32))   # sequence 0 untouched
    assert not np.array_equal(ck[1], h0[1].astype(np.float32))       # sequence 1 folded
    for r0, r1 in zip(rings, L.rings):   # sequence 0's ring untouched
        np.testing.assert_array_equal(r0[0], gu.host(r1)[0])
    assert R.rssm_status(L) == R.STATUS_OVERFLOW


@pytest.mark.parametrize("one_launch", [False, True])
def test_serving_shape_spec_rounds(one_launch):
    """batch 256 x 80 heads x 8 groups, 4 drafts, commit of buffers of 8+ at
    the next verify, ring 16; 128 rounds.  Index trace of every sequence
    bit-exact against the integer model; draft outputs of two sequences
    against the oracle.  one_launch: each round's rollback is passed to the
    next round's verify (rssm_rollback_verify_commit)."""
    rounds, n, b, H, G, cap, commit_len = 128, 4, 256, 80, 8, 16, 8
    A, D = syn.m2_params(35, H)
    h0 = syn.m2_state0(35, b, H, 64, 128)
    accept = syn.accept_counts(35, rounds, b, n)
    pool = syn.m2_steps(35, 0, 64, b, H, G, 64, 128)
    pool_dev = {k: gu.dev(v) for k, v in pool.items()}
    idx = (np.arange(rounds * n) % 64).reshape(rounds, n)
    t_ = gu.torch()
    L = gu.m2_layer(A, D, h0, G, cap)
    sel = [5, 250]
    out = t_.empty((n, b, H, 64), dtype=t_.float32, device="cuda")
    im = IndexModel(b, cap)
    ys = []
    nrej = [gu.dev((n - accept[r]).astype(np.int32)) for r in range(rounds)]
    for r in range(rounds):
        j0 = int(idx[r, 0])
        dr = {k: v[j0:j0 + n] for k, v in pool_dev.items()}
        inp = dict(x=dr["x"], B=dr["B"], C=dr["C"], dt=dr["dt"])
        if one_launch and r > 0:
            R.rssm_rollback_verify_commit(L, nrej[r - 1], n, inp, out, commit_len)
            im.rollback(n - accept[r - 1])
        else:
            R.rssm_verify_commit(L, n, inp, out, commit_len)
        im.commit(min_len=commit_len)
        assert im.append(n).all()
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        ys.append(gu.host(out[:, sel]))
        if not one_launch:
            R.rssm_rollback(L, nrej[r])
            im.rollback(n - accept[r])
    sub = {k: np.ascontiguousarray(v[:, sel][idx.reshape(-1)]) for k, v in pool.items()}
    sub = syn.stack_rounds(sub, rounds, n)
    ref = drivers.m2_spec_rounds(A, D, h0[sel], sub, accept[:, sel], cap, commit_len)
    gu.check_m2_outputs(np.array(ys), ref["y"], sub["x"], D)
    assert R.rssm_status(L) == 0


# ------------------------------------------------------- Gated DeltaNet --

_GDN = ("q", "k", "v", "alpha", "beta")


def test_gdn_spec_rounds_against_oracle():
    rounds, n, b, H, cap, commit_len = 30, 4, 6, 4, 16, 8
    S0 = syn.gdn_state0(36, b, H, 128, 128, std=0.1)
    st = syn.gdn_steps(36, 0, rounds * n, b, H, 128, 128)
    drafts = syn.stack_rounds(st, rounds, n)
    accept = syn.accept_counts(36, rounds, b, n)
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    L = gu.gdn_layer(S0, cap)
    out = gu.torch().empty_like(dd["v"][0])
    im = IndexModel(b, cap)
    os_ = []
    for r in range(rounds):
        R.rssm_verify_commit(L, n, {k: dd[k][r] for k in _GDN}, out, commit_len)
        im.commit(min_len=commit_len)
        assert im.append(n).all()
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        os_.append(gu.host(out))
        R.rssm_rollback(L, gu.dev((n - accept[r]).astype(np.int32)))
        im.rollback(n - accept[r])
    ref = drivers.gdn_spec_rounds(S0, drafts, accept, cap, commit_len)
    assert gu.vec_rel_err(np.array(os_), ref["o"]) <= gu.TOL_F32
    R.rssm_commit(L, None, 1)
    assert _tile_rel(gu.host(L.ckpt), ref["state"]) <= 1e-4
    assert R.rssm_status(L) == 0


def test_gdn_fold_matches_standalone_commit():
    """rssm_commit + rssm_verify against rssm_verify_commit on ragged buffers:
    indices and rings equal, checkpoints equal to fp32 rounding (the two
    kernels split the rows over different workgroup shapes), outputs within
    the fp32 tolerance."""
    b, H, cap, n, min_len = 6, 4, 16, 3, 5
    S0 = syn.gdn_state0(37, b, H, 128, 128, std=0.1)
    st = syn.gdn_steps(37, 0, 9, b, H, 128, 128)
    dr = syn.gdn_steps(37, 9, n, b, H, 128, 128)
    d = {k: gu.dev(v) for k, v in st.items()}
    dd = {k: gu.dev(v) for k, v in dr.items()}
    nrej = gu.dev(np.array([0, 2, 4, 5, 8, 9], np.int32))

    def prepare():
        L = gu.gdn_layer(S0, cap)
        o = gu.torch().empty_like(d["v"][0])
        for t in range(9):
            R.rssm_gdn_step(L, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t], o)
        R.rssm_rollback(L, nrej)
        return L

    L1, L2 = prepare(), prepare()
    o1 = gu.torch().empty_like(dd["v"])
    o2 = gu.torch().empty_like(dd["v"])
    inp = {k: dd[k] for k in _GDN}
    R.rssm_commit(L1, None, min_len)
    R.rssm_verify(L1, n, inp, o1)
    R.rssm_verify_commit(L2, n, inp, o2, min_len)
    assert _tile_rel(gu.host(L2.ckpt), gu.host(L1.ckpt)) <= 1e-5
    for a_, b_ in zip(gu.indices(L1), gu.indices(L2)):
        np.testing.assert_array_equal(a_, b_)
    assert gu.vec_rel_err(gu.host(o2), gu.host(o1)) <= gu.TOL_F32
    for r1, r2 in zip(L1.rings, L2.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
    assert R.rssm_status(L1) == 0 and R.rssm_status(L2) == 0


@pytest.mark.parametrize("one_launch", [False, True])
def test_gdn_serving_shape_spec_rounds(one_launch):
    """batch 256 x 32 heads (d 128), 4 drafts, commit of buffers of 8+ at the
    next verify, ring 16; 96 rounds.  Index trace of every sequence bit-exact
    against the integer model; draft outputs of two sequences against the
    oracle.  one_launch: each round's rollback is passed to the next round's
    verify (rssm_rollback_verify_commit)."""
    rounds, n, b, H, cap, commit_len = 96, 4, 256, 32, 16, 8
    S0 = syn.gdn_state0(38, b, H, 128, 128)
    accept = syn.accept_counts(38, rounds, b, n)
    pool = syn.gdn_steps(38, 0, 64, b, H, 128, 128)
    pool_dev = {k: gu.dev(v) for k, v in pool.items()}
    idx = (np.arange(rounds * n) % 64).reshape(rounds, n)
    t_ = gu.torch()
    L = gu.gdn_layer(S0, cap)
    sel = [7, 201]
    out = t_.empty((n, b, H, 128), dtype=t_.float32, device="cuda")
    im = IndexModel(b, cap)
    os_ = []
    nrej = [gu.dev((n - accept[r]).astype(np.int32)) for r in range(rounds)]
    for r in range(rounds):
        j0 = int(idx[r, 0])
        inp = {k: pool_dev[k][j0:j0 + n] for k in _GDN}
        if one_launch and r > 0:
            R.rssm_rollback_verify_commit(L, nrej[r - 1], n, inp, out, commit_len)
            im.rollback(n - accept[r - 1])
        else:
            R.rssm_verify_commit(L, n, inp, out, commit_len)
        im.commit(min_len=commit_len)
        assert im.append(n).all()
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        os_.append(gu.host(out[:, sel]))
        if not one_launch:
            R.rssm_rollback(L, nrej[r])
            im.rollback(n - accept[r])
    sub = {k: np.ascontiguousarray(v[:, sel][idx.reshape(-1)]) for k, v in pool.items()}
    sub = syn.stack_rounds(sub, rounds, n)
    ref = drivers.gdn_spec_rounds(S0[sel], sub, accept[:, sel], cap, commit_len)
    assert gu.vec_rel_err(np.array(os_), ref["o"]) <= gu.TOL_F32
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("n", [1, 2, 5, 8])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_every_draft_width_matches_commit_then_verify(kind, n):
    """Every instantiated draft width (1, 2, 4 and 8 slots) of the fused
    kernels against rssm_commit + rssm_verify on ragged buffers (lens 8, 6, 5,
    3, 0 with min_len 5): indices and rings equal, checkpoints bitwise
    (Mamba-2) or within fp32 rounding (GDN), outputs within the tolerance."""
    b, H, cap, min_len, T = 5, 8, 16, 5, 8
    nrej = gu.dev(np.array([0, 2, 3, 5, 8], np.int32))
    t_ = gu.torch()
    if kind == "mamba2":
        G = 2
        A, D = syn.m2_params(39, H)
        h0 = syn.m2_state0(39, b, H, 64, 128)
        st = {k: gu.dev(v) for k, v in syn.m2_steps(39, 0, T, b, H, G, 64, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.m2_steps(39, T, n, b, H, G, 64, 128).items()}

        def prepare():
            L = gu.m2_layer(A, D, h0, G, cap)
            y = t_.empty_like(st["x"][0])
            for t in range(T):
                R.rssm_mamba2_step(L, st["x"][t], st["B"][t], st["C"][t], st["dt"][t], y)
            R.rssm_rollback(L, nrej)
            return L
        inp = dict(x=dr["x"], B=dr["B"], C=dr["C"], dt=dr["dt"])
        out_like = dr["x"]
    else:
        S0 = syn.gdn_state0(39, b, H, 128, 128, std=0.1)
        st = {k: gu.dev(v) for k, v in syn.gdn_steps(39, 0, T, b, H, 128, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.gdn_steps(39, T, n, b, H, 128, 128).items()}

        def prepare():
            L = gu.gdn_layer(S0, cap)
            o = t_.empty_like(st["v"][0])
            for t in range(T):
                R.rssm_gdn_step(L, *(st[k][t] for k in _GDN), o)
            R.rssm_rollback(L, nrej)
            return L
        inp = {k: dr[k] for k in _GDN}
        out_like = dr["v"]
    L1, L2 = prepare(), prepare()
    o1, o2 = t_.empty_like(out_like), t_.empty_like(out_like)
    R.rssm_commit(L1, None, min_len)
    R.rssm_verify(L1, n, inp, o1)
    R.rssm_verify_commit(L2, n, inp, o2, min_len)
    for a_, b_ in zip(gu.indices(L1), gu.indices(L2)):
        np.testing.assert_array_equal(a_, b_)
    pos, ln = gu.indices(L2)
    assert pos.tolist() == [8, 6, 5, 0, 0] and ln.tolist() == [n, n, n, 3 + n, n]
    if kind == "mamba2":
        np.testing.assert_array_equal(gu.host(L1.ckpt), gu.host(L2.ckpt))
    else:
        assert _tile_rel(gu.host(L2.ckpt), gu.host(L1.ckpt)) <= 1e-5
    assert gu.vec_rel_err(gu.host(o2), gu.host(o1)) <= gu.TOL_F32
    for r1, r2 in zip(L1.rings, L2.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
    assert R.rssm_status(L1) == 0 and R.rssm_status(L2) == 0


# ------------------------------------------------------------ draft trees --

@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_tree_commit_matches_commit_then_tree(kind):
    """rssm_verify_tree_commit against rssm_commit + rssm_verify_tree on
    ragged buffers (lens 9, 6, 5, 3, 0; min_len 5) with a binary tree of 7
    drafts: indices equal (nothing appended; folded sequences end with len
    0), checkpoints bitwise (Mamba-2) or within fp32 rounding (GDN), outputs
    within the tolerance."""
    b, H, cap, min_len, T = 5, 8, 16, 5, 9
    parent = [-1, 0, 0, 1, 1, 2, 2]
    n = len(parent)
    nrej = gu.dev(np.array([0, 3, 4, 6, 9], np.int32))
    t_ = gu.torch()
    if kind == "mamba2":
        G = 2
        A, D = syn.m2_params(42, H)
        h0 = syn.m2_state0(42, b, H, 64, 128)
        st = {k: gu.dev(v) for k, v in syn.m2_steps(42, 0, T, b, H, G, 64, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.m2_steps(42, T, n, b, H, G, 64, 128).items()}

        def prepare():
            L = gu.m2_layer(A, D, h0, G, cap)
            y = t_.empty_like(st["x"][0])
            for t in range(T):
                R.rssm_mamba2_step(L, st["x"][t], st["B"][t], st["C"][t], st["dt"][t], y)
            R.rssm_rollback(L, nrej)
            return L
        inp = dict(x=dr["x"], B=dr["B"], C=dr["C"], dt=dr["dt"])
        out_like = dr["x"]
    else:
        S0 = syn.gdn_state0(42, b, H, 128, 128, std=0.1)
        st = {k: gu.dev(v) for k, v in syn.gdn_steps(42, 0, T, b, H, 128, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.gdn_steps(42, T, n, b, H, 128, 128).items()}

        def prepare():
            L = gu.gdn_layer(S0, cap)
            o = t_.empty_like(st["v"][0])
            for t in range(T):
                R.rssm_gdn_step(L, *(st[k][t] for k in _GDN), o)
            R.rssm_rollback(L, nrej)
            return L
        inp = {k: dr[k] for k in _GDN}
        out_like = dr["v"]
    L1, L2 = prepare(), prepare()
    o1, o2 = t_.empty_like(out_like), t_.empty_like(out_like)
    R.rssm_commit(L1, None, min_len)
    R.rssm_verify_tree(L1, parent, inp, o1)
    R.rssm_verify_tree_commit(L2, parent, inp, o2, min_len)
    for a_, b_ in zip(gu.indices(L1), gu.indices(L2)):
        np.testing.assert_array_equal(a_, b_)
    pos, ln = gu.indices(L2)
    assert pos.tolist() == [9, 6, 5, 0, 0] and ln.tolist() == [0, 0, 0, 3, 0]
    if kind == "mamba2":
        np.testing.assert_array_equal(gu.host(L1.ckpt), gu.host(L2.ckpt))
    else:
        assert _tile_rel(gu.host(L2.ckpt), gu.host(L1.ckpt)) <= 1e-5
    assert gu.vec_rel_err(gu.host(o2), gu.host(o1)) <= gu.TOL_F32
    assert R.rssm_status(L1) == 0 and R.rssm_status(L2) == 0


def test_chain_as_tree_appends_only_accepted_drafts():
    """A speculative loop that writes only accepted drafts to the ring: each
    round verifies 4 drafts as a chain-shaped tree, folding a buffer of 8+
    from the same state read (rssm_verify_tree_commit), then appends the
    accepted prefix (rssm_append_path); no rollback.  Index trace bit-exact
    against the integer model, draft outputs against the oracle."""
    rounds, n, b, H, G, cap, commit_len = 40, 4, 8, 8, 2, 16, 8
    A, D = syn.m2_params(43, H)
    h0 = syn.m2_state0(43, b, H, 64, 128)
    drafts = _drafts(43, rounds, n, b, H, G)
    accept = syn.accept_counts(43, rounds, b, n)
    d = {k: gu.dev(v) for k, v in drafts.items()}
    L = gu.m2_layer(A, D, h0, G, cap)
    out = gu.torch().empty_like(d["x"][0])
    path = gu.dev(np.tile(np.arange(n, dtype=np.int32), (b, 1)))
    im = IndexModel(b, cap)
    ys = []
    for r in range(rounds):
        inp = dict(x=d["x"][r], B=d["B"][r], C=d["C"][r], dt=d["dt"][r])
        R.rssm_verify_tree_commit(L, list(range(-1, n - 1)), inp, out, commit_len)
        R.rssm_append_path(L, n, path, gu.dev(accept[r].astype(np.int32)), inp)
        im.commit(min_len=commit_len)
        im.append(n)
        im.rollback(n - accept[r])
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        ys.append(gu.host(out))
    ref = drivers.m2_spec_rounds(A, D, h0, drafts, accept, cap, commit_len)
    gu.check_m2_outputs(np.array(ys), ref["y"], drafts["x"], D)
    R.rssm_commit(L, None, 1)
    assert _tile_rel(gu.host(L.ckpt), ref["state"]) <= 1e-4
    assert R.rssm_status(L) == 0


# ------------------------------------------- rollback fused into the verify --

def _spec_setup(kind, seed, rounds, n, b, H, cap):
    """A layer and stacked draft rounds for either layer type."""
    if kind == "mamba2":
        G = 2
        A, D = syn.m2_params(seed, H)
        h0 = syn.m2_state0(seed, b, H, 64, 128)
        drafts = _drafts(seed, rounds, n, b, H, G)
        L = gu.m2_layer(A, D, h0, G, cap)
        keys, like = ("x", "B", "C", "dt"), "x"

        def ref(acc, commit_len):
            return drivers.m2_spec_rounds(A, D, h0, drafts, acc, cap, commit_len)

        def check(ys, want):
            gu.check_m2_outputs(ys, want["y"], drafts["x"], D)
    else:
        S0 = syn.gdn_state0(seed, b, H, 128, 128, std=0.1)
        drafts = syn.stack_rounds(syn.gdn_steps(seed, 0, rounds * n, b, H, 128, 128), rounds, n)
        L = gu.gdn_layer(S0, cap)
        keys, like = _GDN, "v"

        def ref(acc, commit_len):
            return drivers.gdn_spec_rounds(S0, drafts, acc, cap, commit_len)

        def check(os_, want):
            assert gu.vec_rel_err(os_, want["o"]) <= gu.TOL_F32
    return L, drafts, keys, like, ref, check


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_rollback_fused_into_next_verify_against_oracle(kind):
    """Speculative rounds in which each round's rejections go to the next
    round's verify (rssm_rollback_verify_commit): the draft outputs are the
    eager recurrence's, the indices follow the integer model's rollback, then
    commit, then append at every call, and the state after the last round is
    the oracle's (explainer, "Cheap speculative decoding rollback")."""
    rounds, n, b, H, cap, commit_len = 30, 4, 6, 8 if kind == "mamba2" else 4, 16, 8
    L, drafts, keys, like, ref, check = _spec_setup(kind, 41, rounds, n, b, H, cap)
    accept = syn.accept_counts(41, rounds, b, n)
    d = {k: gu.dev(v) for k, v in drafts.items()}
    out = gu.torch().empty_like(d[like][0])
    nrej = [gu.dev((n - accept[r]).astype(np.int32)) for r in range(rounds)]
    im = IndexModel(b, cap)
    outs = []
    for r in range(rounds):
        inp = {k: d[k][r] for k in keys}
        if r == 0:
            R.rssm_verify_commit(L, n, inp, out, commit_len)
        else:
            R.rssm_rollback_verify_commit(L, nrej[r - 1], n, inp, out, commit_len)
            im.rollback(n - accept[r - 1])
        im.commit(min_len=commit_len)
        assert im.append(n).all()
        pos, ln = gu.indices(L)
        np.testing.assert_array_equal(pos, im.pos)
        np.testing.assert_array_equal(ln, im.len)
        outs.append(gu.host(out))
    R.rssm_rollback(L, nrej[-1])
    want = ref(accept, commit_len)
    check(np.array(outs), want)
    R.rssm_commit(L, None, 1)
    assert _tile_rel(gu.host(L.ckpt), want["state"]) <= 1e-4
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_rollback_fused_equals_rollback_then_verify_commit(kind):
    """One launch against the two calls it replaces, on full buffers (14 of 16
    slots) and every case at once: overflow without and with a rollback (the
    rollback stands), a plain append, a fold, and counts below zero and above
    len (refused, the bit raised, the sequence verified on its old length).
    Outputs (NaN where refused), indices, rings, checkpoints and status bits
    bitwise equal; the indices also equal the integer model's."""
    b, H, cap, n, min_len, T = 6, 8 if kind == "mamba2" else 4, 16, 4, 8, 14
    nrej_h = np.array([0, 1, 9, -1, 15, 6], np.int32)
    t_ = gu.torch()
    if kind == "mamba2":
        G = 2
        A, D = syn.m2_params(43, H)
        h0 = syn.m2_state0(43, b, H, 64, 128)
        st = {k: gu.dev(v) for k, v in syn.m2_steps(43, 0, T, b, H, G, 64, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.m2_steps(43, T, n, b, H, G, 64, 128).items()}

        def prepare():
            L = gu.m2_layer(A, D, h0, G, cap)
            y = t_.empty_like(st["x"][0])
            for t in range(T):
                R.rssm_mamba2_step(L, st["x"][t], st["B"][t], st["C"][t], st["dt"][t], y)
            return L
        inp = dict(x=dr["x"], B=dr["B"], C=dr["C"], dt=dr["dt"])
        like = dr["x"]
    else:
        S0 = syn.gdn_state0(43, b, H, 128, 128, std=0.1)
        st = {k: gu.dev(v) for k, v in syn.gdn_steps(43, 0, T, b, H, 128, 128).items()}
        dr = {k: gu.dev(v) for k, v in syn.gdn_steps(43, T, n, b, H, 128, 128).items()}

        def prepare():
            L = gu.gdn_layer(S0, cap)
            o = t_.empty_like(st["v"][0])
            for t in range(T):
                R.rssm_gdn_step(L, *(st[k][t] for k in _GDN), o)
            return L
        inp = {k: dr[k] for k in _GDN}
        like = dr["v"]
    nrej = gu.dev(nrej_h)
    L1, L2 = prepare(), prepare()
    o1, o2 = t_.empty_like(like), t_.empty_like(like)
    R.rssm_rollback(L1, nrej)
    R.rssm_verify_commit(L1, n, inp, o1, min_len)
    R.rssm_rollback_verify_commit(L2, nrej, n, inp, o2, min_len)
    s1, s2 = R.rssm_status(L1), R.rssm_status(L2)
    assert s1 == s2 == (R.STATUS_ROLLBACK | R.STATUS_OVERFLOW)
    im = IndexModel(b, cap)
    im.append(T)
    im.rollback(nrej_h)
    ok = im.len + n <= cap
    fold = ok & (im.len >= min_len)
    im.pos[fold] += im.len[fold]
    im.len[fold] = 0
    im.len[ok] += n
    for got, want in zip(gu.indices(L2), (im.pos, im.len)):
        np.testing.assert_array_equal(got, want)
    assert gu.indices(L2)[1].tolist() == [14, 13, 9, 14, 14, 4]
    for a_, b_ in zip(gu.indices(L1), gu.indices(L2)):
        np.testing.assert_array_equal(a_, b_)
    np.testing.assert_array_equal(gu.host(o1), gu.host(o2))   # NaN where refused, on both
    assert np.isnan(gu.host(o2)[:, [0, 1, 3, 4]]).all() and np.isfinite(gu.host(o2)[:, [2, 5]]).all()
    np.testing.assert_array_equal(gu.host(L1.ckpt), gu.host(L2.ckpt))
    for r1, r2 in zip(L1.rings, L2.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
