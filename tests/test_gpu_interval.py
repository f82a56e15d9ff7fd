"""Commit-interval independence on the GPU: with an fp32 checkpoint the outputs
do not depend on when the buffer is folded, so plain decode with intervals
1, 2, 4, 8 and 16 (ring = interval, fused and standalone commits; Mamba-2 also
20 and 32, the rings of more than 16 slots that its fp32 step and commit
serve) must match the fp64 oracle's eager recurrence within the fp32
tolerance, and the checkpoint after a final commit must match the eager
state.  Interval 1 commits after every step (the state is written every
step, as in the eager kernel)."""
import numpy as np
import pytest

import oracle
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N, D_ = 64, 128, 128
INTERVALS = (1, 2, 4, 8, 16)
M2_INTERVALS = INTERVALS + (20, 32)


@pytest.mark.parametrize("fused", [False, True], ids=["standalone_commit", "fused_commit"])
def test_m2_interval_independence(fused):
    T, b, H, G = 70, 3, 10, 5
    A, D = syn.m2_params(90, H)
    h0 = syn.m2_state0(90, b, H, P, N)
    st = syn.m2_steps(90, 0, T, b, H, G, P, N)
    h = h0.astype(np.float64)
    y_ref = oracle.m2_eager(A, D, st["x"], st["B"], st["C"], st["dt"], h)
    d = {k: gu.dev(v) for k, v in st.items()}
    for interval in M2_INTERVALS:
        L = gu.m2_layer(A, D, h0, G, interval)
        y, pos, ln = gu.m2_decode(L, d, interval, fused)
        gu.check_m2_outputs(gu.host(y), y_ref, st["x"], D)
        R.rssm_commit(L, None, 0)
        assert gu.vec_rel_err(gu.host(L.ckpt), h) <= 1e-5, interval
        assert (gu.indices(L)[0] == T).all() and R.rssm_status(L) == 0


@pytest.mark.parametrize("fused", [False, True], ids=["standalone_commit", "fused_commit"])
def test_gdn_interval_independence(fused):
    T, b, H = 32, 3, 5
    S0 = syn.gdn_state0(91, b, H, D_, D_, std=0.1)
    st = syn.gdn_steps(91, 0, T, b, H, D_, D_)
    names = ("q", "k", "v", "alpha", "beta")
    S = S0.astype(np.float64)
    o_ref = oracle.gdn_eager(*(st[n] for n in names), S)
    d = {k: gu.dev(v) for k, v in st.items()}
    for interval in INTERVALS:
        L = gu.gdn_layer(S0, interval)
        o, pos, ln = gu.gdn_decode(L, d, interval, fused)
        assert gu.vec_rel_err(gu.host(o), o_ref) <= gu.TOL_F32, interval
        R.rssm_commit(L, None, 0)
        assert gu.vec_rel_err(gu.host(L.ckpt), S) <= 1e-5, interval
        assert (gu.indices(L)[0] == T).all() and R.rssm_status(L) == 0
