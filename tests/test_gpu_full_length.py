"""Parity at the serving configurations' full length: 1024 decode steps at
batch 256 with the commit fused into every 8th step (ring 8), Mamba-2 (80
heads, P 64, N 128, 8 groups) and Gated DeltaNet (32 heads, d 128, S_0 = 0).
Step inputs cycle through a pool of 64 distinct seeded steps, as in the
benchmark.  The fp64 oracle recomputes every one of the 256 Mamba-2 sequences
(every head, every step; in blocks of 16 sequences) and 32 of the 256 GDN
sequences (every eighth) on the same cycled inputs.  Outputs within 1e-4 per
vector (Mamba-2: also the state part y - D x), final checkpoints within 1e-5,
indices exact."""
import numpy as np
import pytest

from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu

T, POOL = 1024, 64
GDN_SEL = list(range(3, 256, 8))          # 32 sequences spread over the batch


def test_mamba2_serving_shape_1024_steps():
    b, H, G, P, N, interval, blk = 256, 80, 8, 64, 128, 8, 16
    A, D = syn.m2_params(40, H)
    h0 = syn.m2_state0(40, b, H, P, N)
    pool = syn.m2_steps(40, 0, POOL, b, H, G, P, N)
    pd = {k: gu.dev(v) for k, v in pool.items()}
    L = gu.m2_layer(A, D, h0, G, interval)
    t_ = gu.torch()
    y = t_.empty((T, b, H, P), dtype=t_.float32, device="cuda")      # every output, 5.4 GB
    for t in range(T):
        j = t % POOL
        R.rssm_mamba2_step(L, pd["x"][j], pd["B"][j], pd["C"][j], pd["dt"][j], y[t],
                           commit_after=(t + 1) % interval == 0)
    t_.cuda.synchronize()
    pos, ln = gu.indices(L)
    assert (pos == T).all() and (ln == 0).all()
    assert R.rssm_status(L) == 0
    idx = np.arange(T) % POOL
    ck = gu.host(L.ckpt)
    for s0 in range(0, b, blk):
        sel = slice(s0, s0 + blk)
        sub = {k: np.ascontiguousarray(v[:, sel][idx]) for k, v in pool.items()}
        ref = drivers.m2_decode(A, D, sub["x"], sub["B"], sub["C"], sub["dt"], h0[sel],
                                interval, interval)
        gu.check_m2_outputs(gu.host(y[:, sel]), ref["y"], sub["x"], D)
        assert gu.vec_rel_err(ck[sel], ref["ckpt"]) <= 1e-5, s0


def test_gdn_serving_shape_1024_steps():
    b, H, d, interval = 256, 32, 128, 8
    S0 = syn.gdn_state0(41, b, H, d, d)
    pool = syn.gdn_steps(41, 0, POOL, b, H, d, d)
    names = ("q", "k", "v", "alpha", "beta")
    pd = {k: gu.dev(v) for k, v in pool.items()}
    L = gu.gdn_layer(S0, interval)
    t_ = gu.torch()
    o = t_.empty((T, len(GDN_SEL), H, d), dtype=t_.float32, device="cuda")
    out = t_.empty((b, H, d), dtype=t_.float32, device="cuda")
    sel = t_.tensor(GDN_SEL, device="cuda")
    for t in range(T):
        j = t % POOL
        R.rssm_gdn_step(L, *(pd[k][j] for k in names), out,
                        commit_after=(t + 1) % interval == 0)
        o[t] = out.index_select(0, sel)
    idx = np.arange(T) % POOL
    sub = {k: np.ascontiguousarray(v[:, GDN_SEL][idx]) for k, v in pool.items()}
    ref = drivers.gdn_decode(*(sub[k] for k in names), S0[GDN_SEL], interval, interval)
    assert gu.vec_rel_err(gu.host(o), ref["o"]) <= gu.TOL_F32
    pos, ln = gu.indices(L)
    assert (pos == T).all() and (ln == 0).all()
    assert gu.vec_rel_err(gu.host(L.ckpt[GDN_SEL]), ref["ckpt"]) <= 1e-5
    assert R.rssm_status(L) == 0
