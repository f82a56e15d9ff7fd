"""The commit fused into the step that fills the interval, for DUAL layers
(explainer, "Separate precisions for serving vs updating state": the fp32
checkpoint alone takes the folds, the low-precision copy serves the outputs).

The fused step reads the fp32 checkpoint, which it folds anyway, serves its
own output from it and then writes the low-precision image of the folded
state.  Pinned against the oracle's fused dual emulation
(drivers.*_lowprec(..., fused=True)): the boundary steps' outputs within the
fp32 tolerance of the exact ones, the copy's codes equal or adjacent to the
emulation's, the fp32 state within 1e-5.  Against the standalone path on the
GPU (a low-precision step, then rssm_commit): every other step's output and
the final checkpoint and copy are bitwise equal for Mamba-2 (same fold
arithmetic) and equal to fp32 rounding for GDN."""
import numpy as np
import pytest

from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu

LPS = [R.RSSM_BF16, R.RSSM_E4M3]
LP_IDS = ["bf16", "e4m3"]
LP_NAME = {R.RSSM_BF16: "bf16", R.RSSM_E4M3: "e4m3"}
GDN = ("q", "k", "v", "alpha", "beta")


def _m2_run(A, D, h0, G, interval, lp, st, fused):
    b, H = h0.shape[:2]
    L = R.Layer.mamba2(b, H, G, 64, 128, interval, scheme=R.RSSM_DUAL, lp_dtype=lp)
    L.A.copy_(gu.dev(A))
    L.D.copy_(gu.dev(D))
    L.ckpt.copy_(gu.dev(h0))
    R.rssm_commit(L, None, 0)                      # the copy starts as Q(h_0)
    d = {k: gu.dev(v) for k, v in st.items()}
    y, _, _ = gu.m2_decode(L, d, interval, fused, record=False)
    return L, gu.host(y)


def _gdn_run(S0, interval, lp, st, fused):
    L = gu.gdn_layer(S0, interval, scheme=R.RSSM_DUAL, lp=lp)
    R.rssm_commit(L, None, 0)
    o, _, _ = gu.gdn_decode(L, {k: gu.dev(v) for k, v in st.items()}, interval, fused,
                            record=False)
    return L, gu.host(o)


def _boundary(T, interval):
    m = np.zeros(T, bool)
    m[interval - 1::interval] = True
    return m


@pytest.mark.parametrize("lp", LPS, ids=LP_IDS)
def test_mamba2_dual_fused_commit(lp):
    T, b, H, G, interval = 40, 4, 8, 2, 8
    A, D = syn.m2_params(130, H)
    h0 = syn.m2_state0(130, b, H, 64, 128)
    st = syn.m2_steps(130, 0, T, b, H, G, 64, 128)
    Lf, yf = _m2_run(A, D, h0, G, interval, lp, st, True)
    Ls, ys = _m2_run(A, D, h0, G, interval, lp, st, False)
    ref = drivers.m2_lowprec(A, D, st["x"], st["B"], st["C"], st["dt"], h0, interval, "dual",
                             LP_NAME[lp], fused=True)
    bd = _boundary(T, interval)
    gu.check_m2_outputs(yf[bd], ref["o_emul"][bd], st["x"][bd], D)   # = the exact outputs
    np.testing.assert_array_equal(yf[~bd], ys[~bd])
    np.testing.assert_array_equal(gu.host(Lf.ckpt), gu.host(Ls.ckpt))
    np.testing.assert_array_equal(gu.host(Lf.ckpt_lp), gu.host(Ls.ckpt_lp))
    ok, frac = gu.codes_close(gu.host(Lf.ckpt_lp), ref["codes"], lp == R.RSSM_BF16,
                              None if Lf.lp_scale is None else gu.host(Lf.lp_scale), ref["scale"])
    assert ok and frac <= 1e-3, frac
    assert gu.vec_rel_err(gu.host(Lf.ckpt), ref["state"]) <= 1e-5
    for a_, b_ in zip(gu.indices(Lf), gu.indices(Ls)):
        np.testing.assert_array_equal(a_, b_)
    assert R.rssm_status(Lf) == 0


@pytest.mark.parametrize("lp", LPS, ids=LP_IDS)
def test_gdn_dual_fused_commit(lp):
    T, b, H, interval = 40, 4, 8, 8
    S0 = syn.gdn_state0(131, b, H, 128, 128, std=0.1)
    st = syn.gdn_steps(131, 0, T, b, H, 128, 128)
    Lf, of = _gdn_run(S0, interval, lp, st, True)
    Ls, os_ = _gdn_run(S0, interval, lp, st, False)
    ref = drivers.gdn_lowprec(*(st[k] for k in GDN), S0, interval, "dual", LP_NAME[lp],
                              fused=True)
    bd = _boundary(T, interval)
    assert gu.vec_rel_err(of[bd], ref["o_emul"][bd]) <= gu.TOL_F32
    assert gu.vec_rel_err(gu.host(Lf.ckpt), gu.host(Ls.ckpt)) <= 1e-6
    other = gu.host(Ls.ckpt_lp)
    other = other.view(np.uint16) if lp == R.RSSM_BF16 else other
    ok, frac = gu.codes_close(gu.host(Lf.ckpt_lp), other, lp == R.RSSM_BF16,
                              None if Lf.lp_scale is None else gu.host(Lf.lp_scale),
                              None if Ls.lp_scale is None else gu.host(Ls.lp_scale))
    assert ok and frac <= 1e-3, frac
    # off the boundary both serve their copy: equal up to the copies' code flips
    assert gu.vec_rel_err(of[~bd], os_[~bd]) <= (2e-2 if lp == R.RSSM_BF16 else 0.25)
    ok, frac = gu.codes_close(gu.host(Lf.ckpt_lp), ref["codes"], lp == R.RSSM_BF16,
                              None if Lf.lp_scale is None else gu.host(Lf.lp_scale), ref["scale"])
    assert ok and frac <= 1e-3, frac
    assert gu.vec_rel_err(gu.host(Lf.ckpt), ref["state"]) <= 1e-5
    for a_, b_ in zip(gu.indices(Lf), gu.indices(Ls)):
        np.testing.assert_array_equal(a_, b_)
    assert R.rssm_status(Lf) == 0
