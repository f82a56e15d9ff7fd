"""One set of buffer indices shared by the layers of a stack (explainer, "How
to think about using it": per-layer or shared buffers), through the C ABI.

Three layers with their own states, rings and inputs share one ckpt_pos / len
pair: the first two carry RSSM_LAYER_INDEX_READONLY and no arrival counters,
the third moves the indices after the others have run, on the same stream.
Against three layers with indices of their own, driven by the same calls,
every output, checkpoint and ring slot must be equal bit for bit (the kernels
are the same; only who writes the indices differs) and the shared indices
must equal each independent layer's.  Covered: plain steps with fused and
standalone commits, speculative rounds (verify, rollback, commit at a
minimum length) and one-launch rounds (rssm_rollback_verify_commit: a
read-only layer applies the rejections to the indices it reads, the owner
writes them) for both layer types."""
import numpy as np
import pytest

from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N, D_ = 64, 128, 128
NL = 3


def _stack(make, shared):
    Ls = [make(layer) for layer in range(NL)]
    if shared:
        for L in Ls[:-1]:
            L.share_indices(Ls[-1], readonly=True)
            L.desc.arrive = None          # a read-only layer needs no counters
    return Ls


def _compare(A, B):
    for La, Lb in zip(A, B):
        np.testing.assert_array_equal(gu.host(La.ckpt), gu.host(Lb.ckpt))
        for ra, rb in zip(La.rings, Lb.rings):
            np.testing.assert_array_equal(gu.host(ra), gu.host(rb))
        np.testing.assert_array_equal(gu.host(La.len), gu.host(Lb.len))
        np.testing.assert_array_equal(gu.host(La.ckpt_pos), gu.host(Lb.ckpt_pos))


@pytest.mark.parametrize("kind", ["m2", "gdn"])
def test_shared_indices_equal_per_layer_indices(kind):
    t_ = gu.torch()
    b, cap, interval, T, n = 6, 12, 8, 20, 3
    if kind == "m2":
        H, G = 8, 2
        names = ("x", "B", "C", "dt")

        def make(layer):
            A, D = syn.m2_params(140 + layer, H)
            return gu.m2_layer(A, D, syn.m2_state0(140 + layer, b, H, P, N), G, cap)
        steps = [syn.m2_steps(140 + layer, 0, T + n * 6, b, H, G, P, N) for layer in range(NL)]
        step = R.rssm_mamba2_step
        out_of = "x"
    else:
        H = 4
        names = ("q", "k", "v", "alpha", "beta")

        def make(layer):
            return gu.gdn_layer(syn.gdn_state0(150 + layer, b, H, D_, D_, std=0.1), cap)
        steps = [syn.gdn_steps(150 + layer, 0, T + n * 6, b, H, D_, D_) for layer in range(NL)]
        step = R.rssm_gdn_step
        out_of = "v"
    dev = [{k: gu.dev(v) for k, v in st.items()} for st in steps]
    own, shr = _stack(make, False), _stack(make, True)
    outs = {}
    for tag, Ls in (("own", own), ("shared", shr)):
        ys = []
        for t in range(T):                      # plain decode: fused, then standalone commits
            last = (t + 1) % interval == 0
            for layer, L in enumerate(Ls):
                y = t_.empty_like(dev[layer][out_of][0])
                step(L, *(dev[layer][k][t] for k in names), y,
                     commit_after=last and t < interval)
                ys.append(gu.host(y))
            if last and t >= interval:
                for L in Ls:
                    R.rssm_commit(L, None, 0)
        accept = syn.accept_counts(141, 3, b, n)
        for r in range(3):                      # speculative rounds
            for layer, L in enumerate(Ls):
                sl = slice(T + r * n, T + (r + 1) * n)
                out = t_.empty_like(dev[layer][out_of][sl])
                R.rssm_verify(L, n, {k: dev[layer][k][sl] for k in names}, out)
                ys.append(gu.host(out))
            for L in Ls:
                R.rssm_rollback(L, gu.dev((n - accept[r]).astype(np.int32)))
            for L in Ls:
                R.rssm_commit(L, None, 6)
        # one launch per round: each round's rejections go with the next
        # round's drafts; a read-only layer applies them to the indices it
        # reads, the owner writes them
        acc2 = syn.accept_counts(142, 3, b, n)
        for r in range(3):
            prev = np.zeros(b, np.int32) if r == 0 else (n - acc2[r - 1]).astype(np.int32)
            for layer, L in enumerate(Ls):
                sl = slice(T + (3 + r) * n, T + (4 + r) * n)
                out = t_.empty_like(dev[layer][out_of][sl])
                R.rssm_rollback_verify_commit(L, gu.dev(prev), n,
                                              {k: dev[layer][k][sl] for k in names}, out, 6)
                ys.append(gu.host(out))
        for L in Ls:
            R.rssm_rollback(L, gu.dev((n - acc2[2]).astype(np.int32)))
        t_.cuda.synchronize()
        outs[tag] = ys
        for L in Ls:
            assert R.rssm_status(L) == 0
    for a, c in zip(outs["own"], outs["shared"]):
        np.testing.assert_array_equal(a, c)
    _compare(own, shr)
    for L in shr[:-1]:
        assert not gu.host(L.arrive).any()
    assert gu.host(shr[-1].len).max() > 0 and gu.host(shr[-1].ckpt_pos).min() > 0
