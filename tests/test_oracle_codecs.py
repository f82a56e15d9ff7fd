"""Pins of the oracle's low-precision codecs (CPU only).

The expected values come from the formats' definitions, written here
independently of oracle.c: bfloat16 is the upper half of a binary32 with
round-to-nearest-even; OCP FP8 E4M3 has 1 sign, 4 exponent (bias 7) and 3
fraction bits, no infinities, S.1111.111 = NaN and largest finite 448.
Encoding is checked against an exhaustive nearest-value search over the
decoded code table, with ties to the even code.
"""
import math
import struct

import numpy as np
import pytest

import oracle


def _e4m3_value(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


def _e4m3_nearest(v):
    """Nearest finite E4M3 code (ties to even code), saturating at 448."""
    if math.isnan(v):
        return 0x7F | (0x80 if math.copysign(1, v) < 0 else 0)
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    best, bestd = None, None
    for c in range(0x7F):            # non-negative finite codes 0x00..0x7E
        d = abs(_e4m3_value(c) - a)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return sign | best


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    for c in range(256):
        want = _e4m3_value(c)
        if math.isnan(want):
            assert math.isnan(got[c]), c
        else:
            assert got[c] == want, (c, got[c], want)


@pytest.mark.parametrize("value,code", [
    (448.0, 0x7E), (-448.0, 0xFE), (464.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
    (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (-0.0, 0x80), (0.0, 0x00),
    (2.0 ** -6, 0x08), (240.0, 0x77), (256.0, 0x78),
    # E4M3 has no infinity; the saturating conversion maps it to the largest finite
    (math.inf, 0x7E), (-math.inf, 0xFE),
])
def test_e4m3_spec_values(value, code):
    assert int(oracle.e4m3_encode(np.array([value], np.float32))[0]) == code


def test_e4m3_nan():
    c = int(oracle.e4m3_encode(np.array([np.nan], np.float32))[0])
    assert c & 0x7F == 0x7F


def test_e4m3_encode_matches_exhaustive_search():
    rng = np.random.default_rng(20)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0,
        rng.standard_normal(1000) * 0.01,
        rng.uniform(-500, 500, 500),
    ]).astype(np.float32)
    # every midpoint between neighbouring finite codes (exact ties)
    pos = sorted(_e4m3_value(c) for c in range(0x7F))
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    vals = np.concatenate([vals, np.array(mids + [-m for m in mids], np.float32)])
    got = oracle.e4m3_encode(vals)
    for v, c in zip(vals.tolist(), got.tolist()):
        assert c == _e4m3_nearest(v), (v, c, _e4m3_nearest(v))


def _bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def _bf16_nearest(f):
    """Nearest bf16 by comparing the two candidates that bracket f."""
    u = _bits(f)
    lo = u >> 16
    cands = [lo, lo + 1]
    def val(c):
        return struct.unpack("<f", struct.pack("<I", (c & 0xFFFF) << 16))[0] \
            if (c & 0x7F80) != 0x7F80 else math.copysign(math.inf, f)
    best = None
    for c in cands:
        d = abs(val(c) - f)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0] & 0xFFFF


@pytest.mark.parametrize("value,code", [
    (1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
    (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    # 3e38 = 1.7632 * 2^127: fraction 0.7632*128 = 97.69 -> 98 = 0x62, exponent 254
    (3.0e38, 0x7F62),
    (3.4028234663852886e38, 0x7F80),
    # subnormal: 2^-130 = 8 * 2^-133 (bf16 subnormal spacing 2^-133) -> fraction 8
    (2.0 ** -130, 0x0008),
])
def test_bf16_spec_values(value, code):
    assert int(oracle.bf16_encode(np.array([value], np.float32))[0]) == code


def test_bf16_encode_matches_bracketing_search_and_decode_roundtrip():
    rng = np.random.default_rng(21)
    vals = np.concatenate([rng.standard_normal(5000) * 3,
                           rng.standard_normal(1000) * 1e-38,
                           rng.standard_normal(1000) * 1e30]).astype(np.float32)
    got = oracle.bf16_encode(vals)
    for v, c in zip(vals.tolist(), got.tolist()):
        assert c == _bf16_nearest(v), (v, hex(c))
    dec = oracle.bf16_decode(got)
    # decode is the upper-half reinterpretation
    want = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(dec, want)
    # half-ulp error bound for normal values: |q - v| <= 2^-8 |v|
    nz = np.abs(vals) > 1e-37
    assert np.all(np.abs(dec[nz] - vals[nz]) <= 2.0 ** -8 * np.abs(vals[nz]))


def test_e4m3_per_head_scale():
    rng = np.random.default_rng(22)
    tiles = rng.standard_normal((3, 64)).astype(np.float32)
    tiles[1] = 0.0
    scale, codes = oracle.e4m3_quant_heads(tiles)
    assert scale[1] == 1.0 and np.all(codes[1] == 0)
    for h in (0, 2):
        amax = np.abs(tiles[h]).max()
        assert scale[h] == np.float32(amax) / np.float32(448.0)
        i = int(np.argmax(np.abs(tiles[h])))
        assert codes[h, i] & 0x7F == 0x7E          # the max maps to +-448
        deq = oracle.e4m3_dequant_heads(scale[h:h + 1], codes[h:h + 1])[0]
        err = np.abs(deq - tiles[h])
        bound = np.maximum(2.0 ** -4 * np.abs(tiles[h]), 2.0 ** -10 * scale[h]) * 1.0001
        assert np.all(err <= bound)


def test_e4m3_nonfinite_tile_is_encoded_unscaled():
    """A tile holding NaN or an infinity has no usable amax: scale 1, every
    value encoded as it is (saturating), NaN kept; other tiles unaffected."""
    rng = np.random.default_rng(23)
    tiles = (rng.standard_normal((4, 64)) * 1000).astype(np.float32)
    tiles[1, 7] = np.nan
    tiles[2, 3] = -np.inf
    scale, codes, bad = oracle.e4m3_quant_heads(tiles, return_nonfinite=True)
    assert bad == 2
    assert scale[1] == 1.0 and scale[2] == 1.0
    for h in (1, 2):
        for v, c in zip(tiles[h].tolist(), codes[h].tolist()):
            if math.isnan(v):
                assert c & 0x7F == 0x7F
            else:
                assert c == _e4m3_nearest(max(-448.0, min(448.0, v))), (v, c)
    s_ok, c_ok = oracle.e4m3_quant_heads(tiles[[0, 3]])
    np.testing.assert_array_equal(scale[[0, 3]], s_ok)
    np.testing.assert_array_equal(codes[[0, 3]], c_ok)


def test_e4m3_scale_that_underflows_is_one():
    """amax / 448 rounds to 0 in fp32 when amax < 448 x 2^-150: the tile is
    encoded with scale 1, as an all-zero tile is, and every code is +-0 (the
    values are far below the smallest E4M3 step); a slightly larger amax gives
    a subnormal scale and the usual encoding, the max mapping to +-448."""
    tiles = np.zeros((2, 8), np.float32)
    tiles[0, :4] = np.array([1e-43, -1e-43, 0.0, -0.0], np.float32)
    tiles[1, :3] = np.array([1e-40, -5e-41, 0.0], np.float32)
    scale, codes = oracle.e4m3_quant_heads(tiles)
    assert np.float32(1e-43) / np.float32(448.0) == 0.0
    assert scale[0] == 1.0
    assert codes[0].tolist() == [0x00, 0x80, 0x00, 0x80, 0, 0, 0, 0]
    assert 0.0 < scale[1] < np.finfo(np.float32).tiny
    assert codes[1, 0] == 0x7E and codes[1, 1] & 0x80
