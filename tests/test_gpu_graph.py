"""The decode path under HIP graph capture.

Every call of the step / commit path is a kernel launch on the caller's stream
(no allocation, no memset, no host synchronisation), so one commit interval of
steps can be captured once and replayed, each replay continuing from the state
that the previous one left.  The fold is captured both ways: fused into the
interval's last step, and as the standalone commit after it.

The test captures an 8-step interval, then replays it several times.  Before
each replay, the next 8 steps' inputs are copied into the captured input
buffers.  Between replays the program does eager work of its own and
synchronises.  A second layer is driven through the same calls without a graph.
Every replay's outputs, checkpoints (fp32 and low precision, with the E4M3
scales), rings and indices must equal the eager layer's bit for bit; the
kernels are deterministic, so any difference is a capture problem.

The same holds for a speculative round: verification of 4 drafts that folds a
due buffer (min_len 8, ring 16) followed by the rollback of the rejected
drafts, whose counts the caller writes into the captured device buffer before
each replay."""
import numpy as np
import pytest

from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu

INTERVAL, REPLAYS = 8, 3


def _same(a, b, what):
    if a is None:
        assert b is None, what
        return
    assert gu.torch().equal(a, b), what


def _compare(Lg, Le, outg, oute, r):
    _same(outg, oute, f"outputs, replay {r}")
    for name in ("ckpt", "ckpt_lp", "lp_scale", "ckpt_pos", "len"):
        _same(getattr(Lg, name), getattr(Le, name), f"{name}, replay {r}")
    for i, (a, b) in enumerate(zip(Lg.rings, Le.rings)):
        _same(a, b, f"ring {i}, replay {r}")
    assert R.rssm_status(Lg) == 0 and R.rssm_status(Le) == 0


def _drive(make_layer, pool, step, fused):
    """pool: dict of numpy [REPLAYS * INTERVAL, ...] step inputs."""
    t_ = gu.torch()
    Lg, Le = make_layer(), make_layer()
    names = list(pool)
    stat = {s: gu.dev(pool[s][:INTERVAL]) for s in names}    # the captured input buffers
    out_shape = step.out_shape
    outg = t_.empty((INTERVAL,) + out_shape, dtype=t_.float32, device="cuda")
    oute = t_.empty_like(outg)

    def interval(L, out):
        for t in range(INTERVAL):
            last = t == INTERVAL - 1
            step(L, {s: stat[s][t] for s in names}, out[t], fused and last)
            if last and not fused:
                R.rssm_commit(L, None, 0)

    t_.cuda.synchronize()
    g = t_.cuda.CUDAGraph()
    with t_.cuda.graph(g):
        interval(Lg, outg)
    t_.cuda.synchronize()
    for r in range(REPLAYS):
        for s in names:
            stat[s].copy_(gu.dev(pool[s][r * INTERVAL:(r + 1) * INTERVAL]))
        t_.cuda.synchronize()
        g.replay()
        junk = t_.randn(1 << 18, device="cuda").abs().sum()   # eager work between replays
        t_.cuda.synchronize()
        interval(Le, oute)
        t_.cuda.synchronize()
        assert float(junk) > 0
        _compare(Lg, Le, outg, oute, r)
        pos, ln = gu.indices(Lg)
        assert (pos == (r + 1) * INTERVAL).all() and (ln == 0).all()
    del g


class _M2Step:
    def __init__(self, b, H, P):
        self.out_shape = (b, H, P)

    def __call__(self, L, inp, out, commit_after):
        R.rssm_mamba2_step(L, inp["x"], inp["B"], inp["C"], inp["dt"], out,
                           commit_after=commit_after)


class _GdnStep:
    def __init__(self, b, H, dv):
        self.out_shape = (b, H, dv)

    def __call__(self, L, inp, out, commit_after):
        R.rssm_gdn_step(L, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], out,
                        commit_after=commit_after)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "standalone"])
@pytest.mark.parametrize("scheme", ["f32", "dual_bf16", "dual_e4m3"])
def test_mamba2_interval_graph_replays_equal_eager(scheme, fused):
    b, H, G, P, N = 6, 16, 2, 64, 128
    A, D = syn.m2_params(70, H)
    h0 = syn.m2_state0(70, b, H, P, N)
    pool = syn.m2_steps(70, 0, REPLAYS * INTERVAL, b, H, G, P, N)
    lp = {"f32": None, "dual_bf16": R.RSSM_BF16, "dual_e4m3": R.RSSM_E4M3}[scheme]

    def make():
        if lp is None:
            return gu.m2_layer(A, D, h0, G, INTERVAL)
        L = R.Layer.mamba2(b, H, G, P, N, INTERVAL, scheme=R.RSSM_DUAL, lp_dtype=lp)
        L.A.copy_(gu.dev(A))
        L.D.copy_(gu.dev(D))
        L.ckpt.copy_(gu.dev(h0))
        R.rssm_commit(L, None, 0)      # the serving copy from the fp32 checkpoint
        return L

    _drive(make, pool, _M2Step(b, H, P), fused)


@pytest.mark.parametrize("scheme,fused", [
    ("f32", True), ("f32", False), ("dual_bf16", True), ("dual_bf16", False),
    ("dual_e4m3", True), ("dual_e4m3", False),
    ("shared_e4m3", False)])   # a SHARED layer has no fp32 checkpoint to fold in the step
def test_gdn_interval_graph_replays_equal_eager(scheme, fused):
    b, H, d = 5, 6, 128
    S0 = syn.gdn_state0(71, b, H, d, d, std=0.1)
    pool = syn.gdn_steps(71, 0, REPLAYS * INTERVAL, b, H, d, d)
    sch, lp = {"f32": (R.RSSM_F32, R.RSSM_LP_NONE), "dual_bf16": (R.RSSM_DUAL, R.RSSM_BF16),
               "dual_e4m3": (R.RSSM_DUAL, R.RSSM_E4M3),
               "shared_e4m3": (R.RSSM_SHARED, R.RSSM_E4M3)}[scheme]

    def make():
        L = gu.gdn_layer(S0, INTERVAL, scheme=sch, lp=lp)
        if sch != R.RSSM_F32:
            R.rssm_commit(L, None, 0)
        return L

    _drive(make, pool, _GdnStep(b, H, d), fused)


# ------------------------------------------------------- speculative round --

def _drive_spec(L_make, drafts, accept, verify, n, min_len, one_launch=False):
    """drafts: dict of numpy [rounds, n, ...]; accept: [rounds, b] accepted counts.
    one_launch: each round is rssm_rollback_verify_commit with the previous
    round's rejections (none before the first); the last round's rollback is
    applied after the loop."""
    t_ = gu.torch()
    Lg, Le = L_make(), L_make()
    names = list(drafts)
    rounds = accept.shape[0]
    stat = {s: gu.dev(drafts[s][0]) for s in names}
    nrej = gu.dev((n - accept[0]).astype(np.int32))
    outg = t_.empty((n,) + tuple(stat[names[0]].shape[1:3]) + (verify.dv,), dtype=t_.float32,
                    device="cuda")
    oute = t_.empty_like(outg)

    def round_(L, out):
        if one_launch:
            R.rssm_rollback_verify_commit(L, nrej, n, {s: stat[s] for s in names}, out, min_len)
        else:
            R.rssm_verify_commit(L, n, {s: stat[s] for s in names}, out, min_len)
            R.rssm_rollback(L, nrej)

    t_.cuda.synchronize()
    g = t_.cuda.CUDAGraph()
    with t_.cuda.graph(g):
        round_(Lg, outg)
    t_.cuda.synchronize()
    for r in range(rounds):
        for s in names:
            stat[s].copy_(gu.dev(drafts[s][r]))
        if one_launch:
            prev = n - accept[r - 1] if r > 0 else np.zeros_like(accept[0])
            nrej.copy_(gu.dev(prev.astype(np.int32)))
        else:
            nrej.copy_(gu.dev((n - accept[r]).astype(np.int32)))
        t_.cuda.synchronize()
        g.replay()
        junk = t_.randn(1 << 16, device="cuda").abs().sum()
        t_.cuda.synchronize()
        round_(Le, oute)
        t_.cuda.synchronize()
        assert float(junk) > 0
        _compare(Lg, Le, outg, oute, r)
    if one_launch:
        last = gu.dev((n - accept[-1]).astype(np.int32))
        R.rssm_rollback(Lg, last)
        R.rssm_rollback(Le, last)
        _compare(Lg, Le, outg, oute, rounds)
    pos, ln = gu.indices(Lg)
    assert (pos + ln == accept.sum(axis=0)).all()
    del g


class _Dv:
    def __init__(self, dv):
        self.dv = dv


@pytest.mark.parametrize("one_launch", [False, True])
def test_mamba2_spec_round_graph_replays_equal_eager(one_launch):
    rounds, n, b, H, G, P, N, cap, min_len = 12, 4, 6, 16, 2, 64, 128, 16, 8
    A, D = syn.m2_params(72, H)
    h0 = syn.m2_state0(72, b, H, P, N)
    drafts = syn.stack_rounds(syn.m2_steps(72, 0, rounds * n, b, H, G, P, N), rounds, n)
    accept = syn.accept_counts(72, rounds, b, n)
    _drive_spec(lambda: gu.m2_layer(A, D, h0, G, cap), drafts, accept, _Dv(P), n, min_len,
                one_launch)


@pytest.mark.parametrize("one_launch", [False, True])
def test_gdn_spec_round_graph_replays_equal_eager(one_launch):
    rounds, n, b, H, d, cap, min_len = 12, 4, 5, 6, 128, 16, 8
    S0 = syn.gdn_state0(73, b, H, d, d, std=0.1)
    drafts = syn.stack_rounds(syn.gdn_steps(73, 0, rounds * n, b, H, d, d), rounds, n)
    accept = syn.accept_counts(73, rounds, b, n)
    _drive_spec(lambda: gu.gdn_layer(S0, cap), drafts, accept, _Dv(d), n, min_len, one_launch)
