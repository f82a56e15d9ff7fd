"""Edge cases of the HIP path against the fp64 oracle, through the C ABI.

Draft counts that hit every verify instantiation (1, 2, 4 and 8 padded
positions, with ragged counts in between); verify served from low-precision
checkpoints; commits restricted by mask and min_len; a one-slot ring; an empty
batch; error status of Gated DeltaNet; non-finite state at E4M3 quantisation.
Tolerances as in the Mamba-2 and GDN parity tests: 1e-4 max vector relative
error for fp32 outputs, bit-exact indices and codes.
"""
import numpy as np
import pytest

import oracle
from oracle import drivers
from oracle.index_model import IndexModel, STATUS_NONFINITE
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N = 64, 128
DK = DV = 128
GDN_NAMES = ("q", "k", "v", "alpha", "beta")
M2_NAMES = ("x", "B", "C", "dt")


def _spec_gpu(L, drafts_dev, names, accept, n, commit_len, out_shape_like):
    """Verify / rollback / (commit) rounds; returns outputs [R,n,...], pos, len."""
    t_ = gu.torch()
    out = t_.empty_like(out_shape_like)
    ys, pos, ln = [], [], []
    for r in range(accept.shape[0]):
        R.rssm_verify(L, n, {nm: drafts_dev[nm][r] for nm in names}, out)
        R.rssm_rollback(L, gu.dev((n - accept[r]).astype(np.int32)))
        if commit_len is not None:
            R.rssm_commit(L, None, commit_len)
        ys.append(gu.host(out))
        p, l = gu.indices(L)
        pos.append(p)
        ln.append(l)
    return np.array(ys), np.array(pos), np.array(ln)


# ------------------------------------------------------------ draft counts --

@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_m2_verify_draft_counts(n):
    """batch 3 x 10 heads in 5 groups, ring 16, commit at 8 buffered entries."""
    rounds, b, H, G, cap, commit_len = 10, 3, 10, 5, 16, 8
    seed = 30 + n
    A, D = syn.m2_params(seed, H)
    h0 = syn.m2_state0(seed, b, H, P, N)
    drafts = syn.stack_rounds(syn.m2_steps(seed, 0, rounds * n, b, H, G, P, N), rounds, n)
    accept = syn.accept_counts(seed, rounds, b, n)
    L = gu.m2_layer(A, D, h0, G, cap)
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    y, pos, ln = _spec_gpu(L, dd, M2_NAMES, accept, n, commit_len, dd["x"][0])
    ref = drivers.m2_spec_rounds(A, D, h0, drafts, accept, cap, commit_len)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    gu.check_m2_outputs(y, ref["y"], drafts["x"], D)
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("n", [1, 3, 8])
def test_gdn_verify_draft_counts(n):
    rounds, b, H, cap, commit_len = 10, 3, 5, 16, 8
    seed = 40 + n
    S0 = syn.gdn_state0(seed, b, H, DV, DK, std=0.1)
    drafts = syn.stack_rounds(syn.gdn_steps(seed, 0, rounds * n, b, H, DK, DV), rounds, n)
    accept = syn.accept_counts(seed, rounds, b, n)
    L = gu.gdn_layer(S0, cap)
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    o, pos, ln = _spec_gpu(L, dd, GDN_NAMES, accept, n, commit_len, dd["v"][0])
    ref = drivers.gdn_spec_rounds(S0, drafts, accept, cap, commit_len)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    assert gu.vec_rel_err(o, ref["o"]) <= gu.TOL_F32
    assert R.rssm_status(L) == 0


# ------------------------------------------------- low-precision verify --

def _lp_checkpoint(rng, b, H, lp):
    """Host-made low-precision checkpoint: (codes, scale or None, exact value)."""
    if lp == R.RSSM_E4M3:
        codes = rng.integers(0, 256, size=(b, H, DV, DK)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x05                 # no NaN codes
        scale = rng.uniform(1e-4, 4e-4, size=(b, H)).astype(np.float32)
        exact = oracle.e4m3_dequant_heads(scale, codes.reshape(b, H, -1)).reshape(codes.shape)
        return codes, scale, exact
    f = (rng.standard_normal((b, H, DV, DK)) * 0.1).astype(np.float32)
    codes = oracle.bf16_encode(f)
    return codes, None, oracle.bf16_decode(codes)


@pytest.mark.parametrize("scheme", [R.RSSM_DUAL, R.RSSM_SHARED], ids=["dual", "shared"])
@pytest.mark.parametrize("lp", [R.RSSM_BF16, R.RSSM_E4M3], ids=["bf16", "e4m3"])
def test_gdn_verify_low_precision(scheme, lp):
    """Verify rounds served from a low-precision checkpoint (no commit in
    between): the outputs are the exact recurrence from the decoded copy."""
    rounds, n, b, H, cap = 5, 3, 3, 4, 16
    rng = np.random.default_rng(50 + scheme * 4 + lp)
    codes, scale, exact = _lp_checkpoint(rng, b, H, lp)
    drafts = syn.stack_rounds(syn.gdn_steps(51, 0, rounds * n, b, H, DK, DV), rounds, n)
    accept = syn.accept_counts(51, rounds, b, 2)   # <= 2 kept per round: ring never fills
    L = gu.gdn_layer(np.zeros((b, H, DV, DK), np.float32), cap, scheme=scheme, lp=lp)
    t_ = gu.torch()
    L.ckpt_lp.copy_(t_.from_numpy(codes.view(np.int16) if lp == R.RSSM_BF16 else codes))
    if scale is not None:
        L.lp_scale.copy_(gu.dev(scale))
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    o, pos, ln = _spec_gpu(L, dd, GDN_NAMES, accept, n, None, dd["v"][0])
    ref = drivers.gdn_spec_rounds(exact, drafts, accept, cap, cap + 1)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    assert gu.vec_rel_err(o, ref["o"]) <= gu.TOL_F32
    assert R.rssm_status(L) == 0


# ----------------------------------------------------- commit mask / min_len --

def _masked_commits(L, b, cap, T, step, seed):
    """Run T steps; after each, commit a random subset of sequences with a
    random min_len (sequences whose ring is full are always selected).
    Returns (index traces from the device, from the index model)."""
    g = np.random.default_rng(seed)
    im = IndexModel(b, cap)
    got, want = [], []
    for t in range(T):
        step(t)
        im.append(1)
        mask = (g.random(b) < 0.4) | (im.len >= cap)
        min_len = int(g.integers(0, 5))
        R.rssm_commit(L, gu.dev(mask.astype(np.uint8)), min_len)
        im.commit(mask, min_len)
        got.append(gu.indices(L))
        want.append(im.snapshot())
    return got, want


def test_m2_commit_mask_and_min_len():
    """Outputs do not depend on when each sequence commits: every step equals
    the eager recurrence, whatever subset of sequences folded before it."""
    T, b, H, G, cap = 40, 6, 8, 2, 8
    A, D = syn.m2_params(60, H)
    h0 = syn.m2_state0(60, b, H, P, N)
    st = syn.m2_steps(60, 0, T, b, H, G, P, N)
    L = gu.m2_layer(A, D, h0, G, cap)
    d = {k: gu.dev(v) for k, v in st.items()}
    y = gu.torch().empty_like(d["x"])
    got, want = _masked_commits(
        L, b, cap, T, lambda t: R.rssm_mamba2_step(L, d["x"][t], d["B"][t], d["C"][t],
                                                   d["dt"][t], y[t]), 61)
    for (gp, gl), (wp, wl) in zip(got, want):
        np.testing.assert_array_equal(gp, wp)
        np.testing.assert_array_equal(gl, wl)
    assert len(set(map(tuple, np.array([w[0] for w in want]).T))) > 1   # traces differ
    h = h0.astype(np.float64)
    y_ref = oracle.m2_eager(A, D, st["x"], st["B"], st["C"], st["dt"], h)
    gu.check_m2_outputs(gu.host(y), y_ref, st["x"], D)
    R.rssm_commit(L, None, 0)
    assert gu.vec_rel_err(gu.host(L.ckpt), h) <= 1e-5
    assert (gu.indices(L)[0] == T).all()
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("scheme", [R.RSSM_F32, R.RSSM_DUAL], ids=["f32", "dual_e4m3"])
def test_gdn_commit_mask_and_min_len(scheme):
    T, b, H, cap = 40, 6, 4, 8
    S0 = syn.gdn_state0(62, b, H, DV, DK, std=0.1)
    st = syn.gdn_steps(62, 0, T, b, H, DK, DV)
    lp = R.RSSM_E4M3 if scheme == R.RSSM_DUAL else R.RSSM_LP_NONE
    L = gu.gdn_layer(S0, cap, scheme=scheme, lp=lp)
    if scheme == R.RSSM_DUAL:
        R.rssm_commit(L, None, 0)
    d = {k: gu.dev(v) for k, v in st.items()}
    o = gu.torch().empty_like(d["v"])
    got, want = _masked_commits(
        L, b, cap, T, lambda t: R.rssm_gdn_step(L, *(d[nm][t] for nm in GDN_NAMES), o[t]), 63)
    for (gp, gl), (wp, wl) in zip(got, want):
        np.testing.assert_array_equal(gp, wp)
        np.testing.assert_array_equal(gl, wl)
    S = S0.astype(np.float64)
    o_ref = oracle.gdn_eager(*(st[nm] for nm in GDN_NAMES), S)
    if scheme == R.RSSM_F32:
        assert gu.vec_rel_err(gu.host(o), o_ref) <= gu.TOL_F32
    else:
        assert np.isfinite(gu.host(o)).all()
    R.rssm_commit(L, None, 0)
    assert gu.vec_rel_err(gu.host(L.ckpt), S) <= 1e-5
    if scheme == R.RSSM_DUAL:
        # the copy of the final commit is the E4M3 image of the exact state
        # (rounded to fp32): codes equal or one step apart, rarely unequal
        scale, codes = oracle.e4m3_quant_heads(S.astype(np.float32).reshape(b, H, -1))
        assert np.abs(gu.host(L.lp_scale) / scale - 1).max() <= 1e-5
        g = gu.host(L.ckpt_lp).reshape(b, H, -1).astype(np.int64)
        w = codes.astype(np.int64)
        same_sign = (g & 0x80) == (w & 0x80)
        adjacent = (g == w) | ((np.abs(g - w) == 1) & same_sign) | (((g | w) & 0x7F) <= 1)
        assert adjacent.all() and (g != w).mean() <= 1e-3
    assert R.rssm_status(L) == 0


# ------------------------------------------------------------ one-slot ring --

@pytest.mark.parametrize("fused", [False, True], ids=["standalone_commit", "fused_commit"])
def test_capacity_one(fused):
    """Ring of one slot, commit after every step: replay degenerates to the
    eager recurrence with the state written every step."""
    T, b, H, G = 12, 2, 8, 2
    A, D = syn.m2_params(70, H)
    h0 = syn.m2_state0(70, b, H, P, N)
    st = syn.m2_steps(70, 0, T, b, H, G, P, N)
    L = gu.m2_layer(A, D, h0, G, 1)
    y, pos, ln = gu.m2_decode(L, {k: gu.dev(v) for k, v in st.items()}, 1, fused)
    ref = drivers.m2_decode(A, D, st["x"], st["B"], st["C"], st["dt"], h0, 1, 1)
    gu.check_m2_outputs(gu.host(y), ref["y"], st["x"], D)
    np.testing.assert_array_equal(pos, ref["pos"])
    np.testing.assert_array_equal(ln, ref["len"])
    assert gu.vec_rel_err(gu.host(L.ckpt), ref["ckpt"]) <= 1e-5

    S0 = syn.gdn_state0(71, b, H, DV, DK, std=0.1)
    sg = syn.gdn_steps(71, 0, T, b, H, DK, DV)
    Lg = gu.gdn_layer(S0, 1)
    o, pos, ln = gu.gdn_decode(Lg, {k: gu.dev(v) for k, v in sg.items()}, 1, fused)
    refg = drivers.gdn_decode(*(sg[nm] for nm in GDN_NAMES), S0, 1, 1)
    assert gu.vec_rel_err(gu.host(o), refg["o"]) <= gu.TOL_F32
    np.testing.assert_array_equal(pos, refg["pos"])
    np.testing.assert_array_equal(ln, refg["len"])
    assert gu.vec_rel_err(gu.host(Lg.ckpt), refg["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0 and R.rssm_status(Lg) == 0


# -------------------------------------------------------------- empty batch --

def test_empty_batch_launches_nothing():
    t_ = gu.torch()
    L = R.Layer.mamba2(0, 8, 2, P, N, 4)
    e = t_.empty((0, 8, P), device="cuda")
    eb = t_.empty((0, 2, N), device="cuda")
    R.rssm_mamba2_step(L, e, eb, eb, t_.empty((0, 8), device="cuda"), e, commit_after=True)
    R.rssm_commit(L, None, 0)
    R.rssm_rollback(L, t_.empty(0, dtype=t_.int32, device="cuda"))
    for scheme, lp in ((R.RSSM_F32, R.RSSM_LP_NONE), (R.RSSM_DUAL, R.RSSM_E4M3),
                       (R.RSSM_SHARED, R.RSSM_BF16)):
        Lg = R.Layer.gdn(0, 4, DK, DV, 4, scheme=scheme, lp_dtype=lp)
        z = t_.empty((3, 0, 4, DK), device="cuda")
        zs = t_.empty((3, 0, 4), device="cuda")
        R.rssm_verify(Lg, 3, dict(q=z, k=z, v=z, alpha=zs, beta=zs), z)
        R.rssm_commit(Lg, None, 0)
        assert R.rssm_status(Lg) == 0
    assert R.rssm_status(L) == 0


# ------------------------------------------------------ GDN error status --

def test_gdn_overflow_and_rollback_status():
    T, b, H, cap = 5, 2, 4, 4
    S0 = syn.gdn_state0(80, b, H, DV, DK, std=0.1)
    st = syn.gdn_steps(80, 0, T, b, H, DK, DV)
    L = gu.gdn_layer(S0, cap)
    d = {k: gu.dev(v) for k, v in st.items()}
    o = gu.torch().zeros_like(d["v"])
    for t in range(T):    # the 5th append overflows the 4-slot ring
        R.rssm_gdn_step(L, *(d[nm][t] for nm in GDN_NAMES), o[t])
    pos, ln = gu.indices(L)
    assert (ln == cap).all() and (pos == 0).all()
    oh = gu.host(o)
    assert np.isnan(oh[4]).all() and np.isfinite(oh[:4]).all()
    ref = drivers.gdn_decode(*(st[nm][:4] for nm in GDN_NAMES), S0, 99, cap)
    assert gu.vec_rel_err(oh[:4], ref["o"]) <= gu.TOL_F32
    assert R.rssm_status(L) == R.STATUS_OVERFLOW
    R.rssm_rollback(L, gu.dev(np.array([5, -1], np.int32)))
    assert gu.indices(L)[1].tolist() == [cap, cap]
    assert R.rssm_status(L) == R.STATUS_ROLLBACK
    R.rssm_rollback(L, gu.dev(np.array([1, 4], np.int32)))
    assert gu.indices(L)[1].tolist() == [3, 0]
    assert R.rssm_status(L) == 0


def test_nonfinite_state_at_e4m3_quantisation():
    """A DUAL commit that meets inf / NaN in a head raises the status bit, gives
    that head scale 1 and encodes its values unscaled; other heads are exact."""
    b, H = 2, 4
    S = syn.gdn_state0(81, b, H, DV, DK, std=0.1)
    S[0, 1, 5, 9] = np.inf
    S[1, 2, 100, 0] = np.nan
    S[1, 2, 3, 3] = -np.inf
    L = gu.gdn_layer(S, 4, scheme=R.RSSM_DUAL, lp=R.RSSM_E4M3)
    R.rssm_commit(L, None, 0)
    scale, codes, bad = oracle.e4m3_quant_heads(S.reshape(b, H, -1), return_nonfinite=True)
    assert bad == 2
    np.testing.assert_array_equal(gu.host(L.lp_scale), scale)
    got = gu.host(L.ckpt_lp).reshape(b, H, -1)
    nan = (codes & 0x7F) == 0x7F
    np.testing.assert_array_equal(got[~nan], codes[~nan])
    assert ((got[nan] & 0x7F) == 0x7F).all()      # NaN stays NaN
    assert R.rssm_status(L) == STATUS_NONFINITE
    assert R.rssm_status(L) == 0


# ------------------------------------------------------ unusable indices --

def _bad_indices(L, cap):
    """Sequences 0-2 get indices no call of the library writes (len -1, len
    cap + 1, ckpt_pos -3); sequence 3 stays at (0, 0)."""
    t_ = gu.torch()
    L.len.copy_(t_.tensor([-1, cap + 1, 0, 0], dtype=t_.int32))
    L.ckpt_pos.copy_(t_.tensor([0, 0, -3, 0], dtype=t_.int64))


def _check_refused(L, cap):
    pos, ln = gu.indices(L)
    assert ln.tolist() == [-1, cap + 1, 0, 0] and pos.tolist() == [0, 0, -3, 0]
    assert not gu.host(L.arrive).any(), "arrival counters must return to zero"
    assert R.rssm_status(L) == R.STATUS_INDEX


@pytest.mark.parametrize("kind", ["m2", "gdn"])
def test_unusable_indices_are_refused(kind):
    """Every call that reads a sequence's indices refuses one whose len is
    negative or above the capacity, or whose checkpoint position is negative:
    it leaves the sequence as it is, writes NaN outputs (step, verify), raises
    RSSM_STATUS_INDEX, and the arrival counters still return to zero, so that
    the next calls on the repaired sequences are exact."""
    t_ = gu.torch()
    b, cap, n = 4, 4, 2
    if kind == "m2":
        H, G = 8, 2
        A, D = syn.m2_params(90, H)
        h0 = syn.m2_state0(90, b, H, P, N)
        st = syn.m2_steps(90, 0, 3, b, H, G, P, N)
        L = gu.m2_layer(A, D, h0, G, cap)
        names = M2_NAMES
        d = {k: gu.dev(v) for k, v in st.items()}
        out = t_.zeros_like(d["x"])
        step = lambda t: R.rssm_mamba2_step(L, *(d[nm][t] for nm in names), out[t])
        one = lambda t, h: drivers.m2_decode(A, D, *(st[nm][t:t + 1] for nm in names), h, 99, cap)["y"][0]
        ref_state = h0
    else:
        H = 4
        S0 = syn.gdn_state0(90, b, H, DV, DK, std=0.1)
        st = syn.gdn_steps(90, 0, 3, b, H, DK, DV)
        L = gu.gdn_layer(S0, cap)
        names = GDN_NAMES
        d = {k: gu.dev(v) for k, v in st.items()}
        out = t_.zeros_like(d["v"])
        step = lambda t: R.rssm_gdn_step(L, *(d[nm][t] for nm in names), out[t])
        one = lambda t, S: drivers.gdn_decode(*(st[nm][t:t + 1] for nm in names), S, 99, cap)["o"][0]
        ref_state = S0
    drafts = {nm: d[nm][:n] for nm in names}

    _bad_indices(L, cap)
    step(0)                                        # replay step
    oh = gu.host(out[0])
    assert np.isnan(oh[:3]).all()
    assert gu.vec_rel_err(oh[3], one(0, ref_state)[3]) <= gu.TOL_F32
    assert gu.indices(L)[1][3] == 1
    L.len[3] = 0
    _check_refused(L, cap)

    vo = t_.zeros((n,) + tuple(out.shape[1:]), dtype=t_.float32, device="cuda")
    R.rssm_verify(L, n, drafts, vo)                # verification
    assert np.isnan(gu.host(vo)[:, :3]).all() and np.isfinite(gu.host(vo)[:, 3]).all()
    L.len[3] = 0
    _check_refused(L, cap)

    R.rssm_append_path(L, n, gu.dev(np.zeros((b, 1), np.int32)),
                       gu.dev(np.ones(b, np.int32)), drafts)   # accepted-path append
    L.len[3] = 0
    _check_refused(L, cap)

    R.rssm_commit(L, None, 0)                      # commit: nothing read or written
    _check_refused(L, cap)

    R.rssm_rollback(L, gu.dev(np.zeros(b, np.int32)))
    _check_refused(L, cap)

    po = t_.full((1,) + tuple(out.shape[1:]), 7.0, dtype=t_.float32, device="cuda")
    before = gu.host(L.ckpt).copy()
    R.rssm_prefill(L, 1, {nm: d[nm][:1] for nm in names}, po)
    assert (gu.host(po)[:, :3] == 7.0).all()
    np.testing.assert_array_equal(gu.host(L.ckpt)[:3], before[:3])
    pos, ln = gu.indices(L)
    assert ln.tolist() == [-1, cap + 1, 0, 0] and pos.tolist() == [0, 0, -3, 1]
    assert not gu.host(L.arrive).any()
    assert R.rssm_status(L) == R.STATUS_INDEX

    # repaired: every sequence steps exactly from its (unchanged) checkpoint
    L.len.zero_()
    L.ckpt_pos.zero_()
    L.ckpt[3].copy_(gu.dev(ref_state[3]))
    step(1)
    want = one(1, ref_state)
    assert gu.vec_rel_err(gu.host(out[1]), want) <= gu.TOL_F32
    assert gu.indices(L)[1].tolist() == [1] * b
    assert not gu.host(L.arrive).any()
    assert R.rssm_status(L) == 0


# ------------------------------------------- E4M3 quotients near code ties --

def _tiles_near_ties(rng, b, H, rows, cols):
    """fp32 tiles with scales from subnormal to 1e28 whose values lie within
    two ulps of t x scale for every E4M3 rounding tie t (the midpoints between
    neighbouring codes, subnormal ones included), so that each code depends on
    the last bit of the quotient v / scale; plus signed zeros and values whose
    quotient underflows.  Element [0, 0] holds the tile's amax."""
    vals = np.array([oracle.e4m3_decode(np.array([c], np.uint8))[0] for c in range(0x7F)])
    ties = (vals[:-1] + vals[1:]) / 2
    amaxes = np.array([1e-40, 3.3e-38, 2.0 ** -100, 1e-20, 0.037, 1.0, 3.0, 448.0, 5e3,
                       7.7e10, 1e28], np.float32)
    S = np.zeros((b, H, rows, cols), np.float32)
    for u in range(b * H):
        amax = amaxes[u % len(amaxes)] * np.float32(1.0 + 0.37 * rng.random())
        scale = np.float32(amax) / np.float32(448.0)
        base = (ties * np.float64(scale)).astype(np.float32)
        near = [base]
        for d in (1, 2):
            near.append(np.nextafter(base, np.float32(np.inf), dtype=np.float32))
            near.append(np.nextafter(base, np.float32(0), dtype=np.float32))
            base = near[-2]
        pool = np.concatenate(near + [np.array([0.0, -0.0], np.float32),
                                      (rng.standard_normal(64) * 1e-30 * scale).astype(np.float32)])
        pool = pool[np.abs(pool) <= amax]
        t = rng.choice(pool, size=rows * cols) * rng.choice([-1, 1], size=rows * cols)
        t = t.astype(np.float32)
        t[0] = amax
        S.reshape(b * H, rows * cols)[u] = t
    return S


@pytest.mark.parametrize("kind", ["m2", "gdn"])
def test_e4m3_codes_at_ties_bit_exact(kind):
    """A DUAL commit with empty buffers re-encodes the fp32 checkpoint: for
    tiles whose quotients sit at E4M3 rounding ties, the codes and scales equal
    the oracle's IEEE-division encoder bit for bit (the kernels form the
    quotient with a reciprocal and one correction step)."""
    rng = np.random.default_rng(91)
    b = 2
    if kind == "m2":
        H, G = 12, 1
        S = _tiles_near_ties(rng, b, H, P, N)
        A, D = syn.m2_params(91, H)
        L = gu.m2_layer(A, D, S, G, 4)
        L2 = R.Layer.mamba2(b, H, G, P, N, 4, scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_E4M3)
        L2.ckpt.copy_(L.ckpt)
        L = L2
    else:
        H = 12
        S = _tiles_near_ties(rng, b, H, DV, DK)
        L = gu.gdn_layer(S, 4, scheme=R.RSSM_DUAL, lp=R.RSSM_E4M3)
    R.rssm_commit(L, None, 0)
    scale, want = oracle.e4m3_quant_heads(S.reshape(b, H, -1))
    np.testing.assert_array_equal(gu.host(L.lp_scale), scale)
    got = gu.host(L.ckpt_lp).reshape(b, H, -1)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])
    assert R.rssm_status(L) == 0
