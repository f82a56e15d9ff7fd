"""Draft trees on the GPU: rssm_verify_tree outputs every draft of a tree from
one checkpoint read, and rssm_append_path appends the accepted path, against
the fp64 oracle (outputs within the fp32 tolerance, indices bit-exact).

Tree shapes: a chain (equals linear verification), a star (every draft one
step after the buffer tail), a binary tree and a forest of two subtrees.
Each test first decodes a few plain steps so that the drafts hang below a
non-empty buffer, and after the append continues plain decoding: the outputs
must be those of plain decoding along buffer + accepted path + new steps.
"""
import numpy as np
import pytest

import oracle
from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N, DK = 64, 128, 128
TREES = {
    "chain": [-1, 0, 1, 2],
    "star": [-1, -1, -1, -1, -1],
    "binary": [-1, 0, 0, 1, 1, 2, 2],
    "forest": [-1, 0, -1, 2, 0, 4, 1, 6],
}
M2_NAMES = ("x", "B", "C", "dt")
GDN_NAMES = ("q", "k", "v", "alpha", "beta")


def _accepted_paths(parent, b, rng):
    """Per sequence, the path to a random draft (or nothing), root first."""
    paths = drivers.tree_paths(parent)
    out = []
    for s in range(b):
        j = int(rng.integers(-1, len(parent)))
        out.append([] if j < 0 else paths[j])
    depth = max(1, max(len(p) for p in out))
    arr = np.zeros((b, depth), np.int32)
    for s, p in enumerate(out):
        arr[s, :len(p)] = p
    return out, arr, np.array([len(p) for p in out], np.int32)


@pytest.mark.parametrize("tree", list(TREES), ids=list(TREES))
def test_m2_tree_verify_and_append(tree):
    parent = TREES[tree]
    n, b, H, G, cap, pre, post = len(parent), 3, 10, 5, 16, 3, 2
    seed = 130 + len(tree)
    A, D = syn.m2_params(seed, H)
    h0 = syn.m2_state0(seed, b, H, P, N)
    st = syn.m2_steps(seed, 0, pre + n + post, b, H, G, P, N)
    pre_st = {k: v[:pre] for k, v in st.items()}
    drafts = {k: np.ascontiguousarray(v[pre:pre + n]) for k, v in st.items()}
    post_st = {k: np.ascontiguousarray(v[pre + n:]) for k, v in st.items()}
    L = gu.m2_layer(A, D, h0, G, cap)
    gu.m2_decode(L, {k: gu.dev(v) for k, v in pre_st.items()}, 1 << 20, False)
    h = h0.astype(np.float64)
    oracle.m2_eager(A, D, pre_st["x"], pre_st["B"], pre_st["C"], pre_st["dt"], h)

    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out = gu.torch().empty_like(dd["x"])
    R.rssm_verify_tree(L, parent, dd, out)
    want = drivers.m2_tree_verify(A, D, h, drafts, parent)
    gu.check_m2_outputs(gu.host(out), want, drafts["x"], D)
    assert (gu.indices(L)[1] == pre).all()

    paths, arr, plen = _accepted_paths(parent, b, np.random.default_rng(seed))
    R.rssm_append_path(L, n, gu.dev(arr), gu.dev(plen), dd)
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen)
    y, _, _ = gu.m2_decode(L, {k: gu.dev(v) for k, v in post_st.items()}, 1 << 20, False)
    yh = gu.host(y)
    for s in range(b):
        hs = h[s:s + 1].copy()
        p = paths[s]
        if p:
            oracle.m2_eager(A, D, drafts["x"][p][:, s:s + 1], drafts["B"][p][:, s:s + 1],
                            drafts["C"][p][:, s:s + 1], drafts["dt"][p][:, s:s + 1], hs)
        ys = oracle.m2_eager(A, D, post_st["x"][:, s:s + 1], post_st["B"][:, s:s + 1],
                             post_st["C"][:, s:s + 1], post_st["dt"][:, s:s + 1], hs)
        gu.check_m2_outputs(yh[:, s:s + 1], ys, post_st["x"][:, s:s + 1], D)
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen + post)
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("tree", ["chain", "binary", "forest"])
def test_gdn_tree_verify_and_append(tree):
    parent = TREES[tree]
    n, b, H, cap, pre, post = len(parent), 3, 5, 16, 3, 2
    seed = 140 + len(tree)
    S0 = syn.gdn_state0(seed, b, H, DK, DK, std=0.1)
    st = syn.gdn_steps(seed, 0, pre + n + post, b, H, DK, DK)
    pre_st = {k: v[:pre] for k, v in st.items()}
    drafts = {k: np.ascontiguousarray(v[pre:pre + n]) for k, v in st.items()}
    post_st = {k: np.ascontiguousarray(v[pre + n:]) for k, v in st.items()}
    L = gu.gdn_layer(S0, cap)
    gu.gdn_decode(L, {k: gu.dev(v) for k, v in pre_st.items()}, 1 << 20, False)
    S = S0.astype(np.float64)
    oracle.gdn_eager(*(pre_st[nm] for nm in GDN_NAMES), S)

    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out = gu.torch().empty_like(dd["v"])
    R.rssm_verify_tree(L, parent, dd, out)
    want = drivers.gdn_tree_verify(S, drafts, parent)
    assert gu.vec_rel_err(gu.host(out), want) <= gu.TOL_F32

    paths, arr, plen = _accepted_paths(parent, b, np.random.default_rng(seed))
    R.rssm_append_path(L, n, gu.dev(arr), gu.dev(plen), dd)
    o, _, _ = gu.gdn_decode(L, {k: gu.dev(v) for k, v in post_st.items()}, 1 << 20, False)
    oh = gu.host(o)
    for s in range(b):
        Ss = S[s:s + 1].copy()
        p = paths[s]
        if p:
            oracle.gdn_eager(*(drafts[nm][p][:, s:s + 1] for nm in GDN_NAMES), Ss)
        os_ = oracle.gdn_eager(*(post_st[nm][:, s:s + 1] for nm in GDN_NAMES), Ss)
        assert gu.vec_rel_err(oh[:, s:s + 1], os_) <= gu.TOL_F32
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen + post)
    assert R.rssm_status(L) == 0


@pytest.mark.parametrize("lp", ["e4m3", "bf16"])
@pytest.mark.parametrize("kind", ["m2", "gdn"])
def test_tree_from_low_precision_copy(kind, lp):
    """A DUAL layer verifies its tree from the low-precision copy: outputs
    equal the exact tree outputs from the decoded copy (empty buffer)."""
    parent = TREES["binary"]
    n, b, H, cap = len(parent), 2, 4, 16
    rng = np.random.default_rng(150)
    shape = (b, H, P if kind == "m2" else DK, N if kind == "m2" else DK)
    if lp == "e4m3":
        codes = rng.integers(0, 0x7F, size=shape)
        codes = (codes | (rng.integers(0, 2, size=codes.shape) << 7)).astype(np.uint8)
        scale = rng.uniform(1e-4, 4e-4, size=(b, H)).astype(np.float32)
        exact = oracle.e4m3_dequant_heads(scale, codes.reshape(b, H, -1)).reshape(codes.shape)
    else:
        codes = oracle.bf16_encode((rng.standard_normal(shape) * 0.1).astype(np.float32))
        scale = None
        exact = oracle.bf16_decode(codes)
    lpc = R.RSSM_E4M3 if lp == "e4m3" else R.RSSM_BF16
    t_ = gu.torch()
    if kind == "m2":
        G = 2
        A, D = syn.m2_params(150, H)
        drafts = syn.m2_steps(150, 0, n, b, H, G, P, N)
        L = R.Layer.mamba2(b, H, G, P, N, cap, scheme=R.RSSM_DUAL, lp_dtype=lpc)
        L.A.copy_(gu.dev(A))
        L.D.copy_(gu.dev(D))
    else:
        drafts = syn.gdn_steps(150, 0, n, b, H, DK, DK)
        L = R.Layer.gdn(b, H, DK, DK, cap, scheme=R.RSSM_DUAL, lp_dtype=lpc)
    L.ckpt_lp.copy_(t_.from_numpy(codes.view(np.int16) if lp == "bf16" else codes))
    if scale is not None:
        L.lp_scale.copy_(gu.dev(scale))
    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out = t_.empty_like(dd["x"] if kind == "m2" else dd["v"])
    R.rssm_verify_tree(L, parent, dd, out)
    if kind == "m2":
        want = drivers.m2_tree_verify(A, D, exact, drafts, parent)
        gu.check_m2_outputs(gu.host(out), want, drafts["x"], D)
    else:
        want = drivers.gdn_tree_verify(exact, drafts, parent)
        assert gu.vec_rel_err(gu.host(out), want) <= gu.TOL_F32
    assert R.rssm_status(L) == 0


def test_append_path_overflow_and_bad_index_leave_sequences_unchanged():
    parent = TREES["chain"]
    n, b, H, G, cap = len(parent), 3, 10, 5, 4
    A, D = syn.m2_params(160, H)
    h0 = syn.m2_state0(160, b, H, P, N)
    st = syn.m2_steps(160, 0, 2 + n, b, H, G, P, N)
    L = gu.m2_layer(A, D, h0, G, cap)
    gu.m2_decode(L, {k: gu.dev(v[:2]) for k, v in st.items()}, 1 << 20, False)
    dd = {k: gu.dev(np.ascontiguousarray(v[2:])) for k, v in st.items()}
    # seq 0: 3 more entries overflow the 4-slot ring (len 2); seq 1: draft 7 does
    # not exist; seq 2: a valid path of two
    path = np.array([[0, 1, 2], [0, 7, 0], [0, 1, 0]], np.int32)
    plen = np.array([3, 2, 2], np.int32)
    R.rssm_append_path(L, n, gu.dev(path), gu.dev(plen), dd)
    assert gu.indices(L)[1].tolist() == [2, 2, 4]
    assert R.rssm_status(L) == R.STATUS_OVERFLOW


SEL = [0, 77, 160, 255]   # sequences the oracle follows at the serving shapes


def _sub(st):
    return {k: np.ascontiguousarray(v[:, SEL]) for k, v in st.items()}


def test_m2_binary_tree_serving_shape():
    """The benchmark's tree workload: batch 256 x 80 heads (8 groups), a
    binary tree of 7 drafts below a buffer of 5 entries (ring 16), then an
    accepted path per sequence and two plain steps.  Outputs of four sampled
    sequences (every head, every draft) against the oracle; indices of all
    256 sequences bit-exact."""
    parent = TREES["binary"]
    n, b, H, G, cap, pre, post = len(parent), 256, 80, 8, 16, 5, 2
    seed = 171
    A, D = syn.m2_params(seed, H)
    h0 = syn.m2_state0(seed, b, H, P, N)
    st = syn.m2_steps(seed, 0, pre + n + post, b, H, G, P, N)
    pre_st = {k: v[:pre] for k, v in st.items()}
    drafts = {k: np.ascontiguousarray(v[pre:pre + n]) for k, v in st.items()}
    post_st = {k: np.ascontiguousarray(v[pre + n:]) for k, v in st.items()}
    L = gu.m2_layer(A, D, h0, G, cap)
    gu.m2_decode(L, {k: gu.dev(v) for k, v in pre_st.items()}, 1 << 20, False)
    h = h0[SEL].astype(np.float64)
    ps = _sub(pre_st)
    oracle.m2_eager(A, D, ps["x"], ps["B"], ps["C"], ps["dt"], h)

    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out = gu.torch().empty_like(dd["x"])
    R.rssm_verify_tree(L, parent, dd, out)
    ds = _sub(drafts)
    want = drivers.m2_tree_verify(A, D, h, ds, parent)
    gu.check_m2_outputs(gu.host(out)[:, SEL], want, ds["x"], D)
    assert (gu.indices(L)[1] == pre).all()

    paths, arr, plen = _accepted_paths(parent, b, np.random.default_rng(seed))
    R.rssm_append_path(L, n, gu.dev(arr), gu.dev(plen), dd)
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen)
    y, _, _ = gu.m2_decode(L, {k: gu.dev(v) for k, v in post_st.items()}, 1 << 20, False)
    yh = gu.host(y)
    for i, s in enumerate(SEL):
        hs = h[i:i + 1].copy()
        p = paths[s]
        if p:
            oracle.m2_eager(A, D, drafts["x"][p][:, s:s + 1], drafts["B"][p][:, s:s + 1],
                            drafts["C"][p][:, s:s + 1], drafts["dt"][p][:, s:s + 1], hs)
        ys = oracle.m2_eager(A, D, post_st["x"][:, s:s + 1], post_st["B"][:, s:s + 1],
                             post_st["C"][:, s:s + 1], post_st["dt"][:, s:s + 1], hs)
        gu.check_m2_outputs(yh[:, s:s + 1], ys, post_st["x"][:, s:s + 1], D)
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen + post)
    assert R.rssm_status(L) == 0


def test_gdn_binary_tree_serving_shape():
    """As above for GDN at batch 256 x 32 heads (d 128)."""
    parent = TREES["binary"]
    n, b, H, cap, pre, post = len(parent), 256, 32, 16, 5, 2
    seed = 172
    S0 = syn.gdn_state0(seed, b, H, DK, DK, std=0.1)
    st = syn.gdn_steps(seed, 0, pre + n + post, b, H, DK, DK)
    pre_st = {k: v[:pre] for k, v in st.items()}
    drafts = {k: np.ascontiguousarray(v[pre:pre + n]) for k, v in st.items()}
    post_st = {k: np.ascontiguousarray(v[pre + n:]) for k, v in st.items()}
    L = gu.gdn_layer(S0, cap)
    gu.gdn_decode(L, {k: gu.dev(v) for k, v in pre_st.items()}, 1 << 20, False)
    S = S0[SEL].astype(np.float64)
    ps = _sub(pre_st)
    oracle.gdn_eager(*(ps[nm] for nm in GDN_NAMES), S)

    dd = {k: gu.dev(v) for k, v in drafts.items()}
    out = gu.torch().empty_like(dd["v"])
    R.rssm_verify_tree(L, parent, dd, out)
    want = drivers.gdn_tree_verify(S, _sub(drafts), parent)
    assert gu.vec_rel_err(gu.host(out)[:, SEL], want) <= gu.TOL_F32
    assert (gu.indices(L)[1] == pre).all()

    paths, arr, plen = _accepted_paths(parent, b, np.random.default_rng(seed))
    R.rssm_append_path(L, n, gu.dev(arr), gu.dev(plen), dd)
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen)
    o, _, _ = gu.gdn_decode(L, {k: gu.dev(v) for k, v in post_st.items()}, 1 << 20, False)
    oh = gu.host(o)
    for i, s in enumerate(SEL):
        Ss = S[i:i + 1].copy()
        p = paths[s]
        if p:
            oracle.gdn_eager(*(drafts[nm][p][:, s:s + 1] for nm in GDN_NAMES), Ss)
        os_ = oracle.gdn_eager(*(post_st[nm][:, s:s + 1] for nm in GDN_NAMES), Ss)
        assert gu.vec_rel_err(oh[:, s:s + 1], os_) <= gu.TOL_F32
    np.testing.assert_array_equal(gu.indices(L)[1], pre + plen + post)
    assert R.rssm_status(L) == 0
