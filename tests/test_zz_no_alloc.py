"""rssm_mamba2_step_noalloc against rssm_mamba2_step, through the C ABI (GPU).

The no-allocation variant keeps the arrival counters in the library's own
device array instead of the caller's `arrive` buffer.  Two layers start from
the same state and receive the same inputs; one is driven by
rssm_mamba2_step, the other by rssm_mamba2_step_noalloc with no arrival
buffer in its descriptor.  Outputs, checkpoints, rings and indices must be
equal bit for bit (the same kernels run), over plain steps and a fused
commit, on two calls in a row of which the second has a smaller batch; the
second layer's outputs are also held to the oracle's 1e-4 bar.
"""
import numpy as np
import pytest

from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu
P, N = 64, 128
NAMES = ("x", "B", "C", "dt")


def _run(seed, b, H, G, steps, interval):
    A, D = syn.m2_params(seed, H)
    h0 = syn.m2_state0(seed, b, H, P, N)
    st = syn.m2_steps(seed, 0, steps, b, H, G, P, N)
    d = {k: gu.dev(v) for k, v in st.items()}
    ref = gu.m2_layer(A, D, h0, G, interval)
    new = gu.m2_layer(A, D, h0, G, interval)
    new.desc.arrive = None                      # the variant brings its own counters
    t_ = gu.torch()
    y_ref = t_.empty_like(d["x"])
    y_new = t_.empty_like(d["x"])
    for t in range(steps):
        commit = (t + 1) % interval == 0
        R.rssm_mamba2_step(ref, *(d[k][t] for k in NAMES), y_ref[t], commit_after=commit)
        R.rssm_mamba2_step_noalloc(new, *(d[k][t] for k in NAMES), y_new[t], commit_after=commit)
        t_.cuda.synchronize()
        np.testing.assert_array_equal(gu.host(ref.len), gu.host(new.len))
        np.testing.assert_array_equal(gu.host(ref.ckpt_pos), gu.host(new.ckpt_pos))
    np.testing.assert_array_equal(gu.host(y_ref), gu.host(y_new))
    np.testing.assert_array_equal(gu.host(ref.ckpt), gu.host(new.ckpt))
    for r1, r2 in zip(ref.rings, new.rings):
        np.testing.assert_array_equal(gu.host(r1), gu.host(r2))
    assert not gu.host(new.arrive).any()        # the caller's buffer was never touched
    assert R.rssm_status(ref) == 0 and R.rssm_status(new) == 0
    want = drivers.m2_decode(A, D, *(st[k] for k in NAMES), h0, interval, interval)
    gu.check_m2_outputs(gu.host(y_new), want["y"], st["x"], D)


def test_noalloc_step_equals_step_on_two_calls_the_second_smaller():
    _run(seed=120, b=12, H=16, G=2, steps=10, interval=4)
    _run(seed=121, b=5, H=8, G=1, steps=9, interval=3)


def test_noalloc_step_refuses_a_batch_beyond_its_counters():
    L = R.Layer.mamba2(1, 8, 1, P, N, 4)
    L.batch = R.RSSM_NOALLOC_MAX_BATCH + 1
    desc = L.refresh()
    desc.batch = R.RSSM_NOALLOC_MAX_BATCH + 1
    t_ = gu.torch()
    z = t_.zeros(16, dtype=t_.float32, device="cuda")
    rc = R.rssm_mamba2_step_noalloc(desc, z, z, z, z, z, 0, check=False)
    assert rc == R.RSSM_ERANGE
