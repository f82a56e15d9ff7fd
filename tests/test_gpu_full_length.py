"""Parity at the serving configurations' full length: 1024 decode steps at
batch 256 with the commit fused into every 8th step (ring 8), Mamba-2 (80
heads, P 64, N 128, 8 groups) and Gated DeltaNet (32 heads, d 128, S_0 = 0).
Step inputs cycle through a pool of 64 distinct seeded steps, as in the
benchmark; the fp64 oracle recomputes three whole sequences (every head, every
step) on the same cycled inputs.  Outputs within 1e-4 per vector (Mamba-2:
also the state part y - D x), final checkpoints within 1e-5, indices exact."""
import numpy as np
import pytest

from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu

T, POOL, SEL = 1024, 64, [2, 129, 253]


def test_mamba2_serving_shape_1024_steps():
    b, H, G, P, N, interval = 256, 80, 8, 64, 128, 8
    A, D = syn.m2_params(40, H)
    h0 = syn.m2_state0(40, b, H, P, N)
    pool = syn.m2_steps(40, 0, POOL, b, H, G, P, N)
    pd = {k: gu.dev(v) for k, v in pool.items()}
    L = gu.m2_layer(A, D, h0, G, interval)
    t_ = gu.torch()
    y = t_.empty((T, len(SEL), H, P), dtype=t_.float32, device="cuda")
    out = t_.empty((b, H, P), dtype=t_.float32, device="cuda")
    sel = t_.tensor(SEL, device="cuda")
    for t in range(T):
        j = t % POOL
        R.rssm_mamba2_step(L, pd["x"][j], pd["B"][j], pd["C"][j], pd["dt"][j], out,
                           commit_after=(t + 1) % interval == 0)
        y[t] = out.index_select(0, sel)
    idx = np.arange(T) % POOL
    sub = {k: np.ascontiguousarray(v[:, SEL][idx]) for k, v in pool.items()}
    ref = drivers.m2_decode(A, D, sub["x"], sub["B"], sub["C"], sub["dt"], h0[SEL], interval,
                            interval)
    gu.check_m2_outputs(gu.host(y), ref["y"], sub["x"], D)
    pos, ln = gu.indices(L)
    assert (pos == T).all() and (ln == 0).all()
    assert gu.vec_rel_err(gu.host(L.ckpt[SEL]), ref["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0


def test_gdn_serving_shape_1024_steps():
    b, H, d, interval = 256, 32, 128, 8
    S0 = syn.gdn_state0(41, b, H, d, d)
    pool = syn.gdn_steps(41, 0, POOL, b, H, d, d)
    names = ("q", "k", "v", "alpha", "beta")
    pd = {k: gu.dev(v) for k, v in pool.items()}
    L = gu.gdn_layer(S0, interval)
    t_ = gu.torch()
    o = t_.empty((T, len(SEL), H, d), dtype=t_.float32, device="cuda")
    out = t_.empty((b, H, d), dtype=t_.float32, device="cuda")
    sel = t_.tensor(SEL, device="cuda")
    for t in range(T):
        j = t % POOL
        R.rssm_gdn_step(L, *(pd[k][j] for k in names), out,
                        commit_after=(t + 1) % interval == 0)
        o[t] = out.index_select(0, sel)
    idx = np.arange(T) % POOL
    sub = {k: np.ascontiguousarray(v[:, SEL][idx]) for k, v in pool.items()}
    ref = drivers.gdn_decode(*(sub[k] for k in names), S0[SEL], interval, interval)
    assert gu.vec_rel_err(gu.host(o), ref["o"]) <= gu.TOL_F32
    pos, ln = gu.indices(L)
    assert (pos == T).all() and (ln == 0).all()
    assert gu.vec_rel_err(gu.host(L.ckpt[SEL]), ref["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0
