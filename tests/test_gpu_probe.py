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


@pytest.mark.parametrize("tile", [4096, 32768])
def test_probe_tiles_copy_and_read(tile):
    t_ = gu.torch()
    nbytes = 16 * 32768
    rng = np.random.default_rng(221)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = gu.dev(words.view(np.float32))
    dst = t_.empty_like(src)
    sink = t_.empty(nbytes // (tile // 4), dtype=t_.float32, device="cuda")
    R.rssm_probe_stream_tiles(src, dst, sink, nbytes, tile)
    np.testing.assert_array_equal(gu.host(dst).view(np.uint32), words)
    R.rssm_probe_stream_tiles(src, None, sink, nbytes, tile)
    got = gu.host(sink).view(np.uint32)
    per = tile // 4096                                # loads per thread
    chunks = words.reshape(nbytes // tile, per, 4, 64, 4)   # tile, k, wave, lane, word
    want = np.bitwise_xor.reduce(chunks, axis=(1, 3, 4)).reshape(-1)
    np.testing.assert_array_equal(got, want)


def test_probe_timing_mode_writes_only_the_key():
    """write_all=False: a wave writes its fold only when it equals the key."""
    t_ = gu.torch()
    nbytes = 8 * 32768
    rng = np.random.default_rng(222)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = gu.dev(words.view(np.float32))
    sink = t_.zeros(nbytes // 1024, dtype=t_.float32, device="cuda")
    R.rssm_probe_stream_tiles(src, None, sink, nbytes, 4096, write_all=False)
    got = gu.host(sink).view(np.uint32)
    assert np.all((got == 0) | (got == 0x9E3779B9))
