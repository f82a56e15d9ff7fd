"""The streaming probe on the GPU: the copy reproduces its source, and the
read-only pass writes the XOR of every wave's words (checked on the host)."""
import numpy as np
import pytest

from linear_attention_decode_replayssm_amd import rssm as R
import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_probe_copy_and_read():
    t_ = gu.torch()
    nbytes = 64 * 32768
    rng = np.random.default_rng(220)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = gu.dev(words.view(np.float32))
    dst = t_.empty_like(src)
    sink = t_.empty(nbytes // 8192, dtype=t_.float32, device="cuda")
    R.rssm_probe_stream(src, dst, sink, nbytes)
    np.testing.assert_array_equal(gu.host(dst).view(np.uint32), words)
    R.rssm_probe_stream(src, None, sink, nbytes)
    got = gu.host(sink).view(np.uint32)
    # wave w of workgroup t reads lanes 64w..64w+63 of every 256-chunk row
    chunks = words.reshape(64, 8, 256, 4)            # tile, k, thread, word
    want = np.bitwise_xor.reduce(chunks.reshape(64, 8, 4, 64, 4), axis=(1, 3, 4)).reshape(-1)
    np.testing.assert_array_equal(got, want)
