"""fp64 CPU oracle for the ReplaySSM decode-time state engine.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path (``linear_attention_decode_replayssm_amd``) and never
imports it; the two meet only through the seeded inputs the caller hands to
both.

Modules:
  * this file      -- ctypes binding of ``oracle.c`` (eager recurrences, codecs)
  * ``replay``     -- the unrolled (checkpoint + buffer) forms, fp64 numpy
  * ``index_model``-- the exact integer model of checkpoint position / buffer length
  * ``drivers``    -- plain decode, speculative rounds and low-precision
                      emulation built from the pieces above

Pins (what ties each function to something other than itself) are listed in
the test files ``tests/test_oracle_*.py``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_fp = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i = ctypes.c_int
_l = ctypes.c_long


def lib():
    """Load liboracle.so, building it with gcc if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_max_threads.restype = _i
        L.orc_set_threads.argtypes = [_i]
        L.orc_m2_decays.argtypes = [_i, _i, _i, _dp, _dp, _dp]
        L.orc_m2_recur.argtypes = [_i] * 6 + [_dp] * 8
        L.orc_gdn_recur.argtypes = [_i] * 5 + [_dp] * 7
        L.orc_bf16_encode.argtypes = [_l, _fp, _u16p]
        L.orc_bf16_decode.argtypes = [_l, _u16p, _dp]
        L.orc_e4m3_encode.argtypes = [_l, _fp, _u8p]
        L.orc_e4m3_decode.argtypes = [_l, _u8p, _dp]
        L.orc_e4m3_quant_heads.argtypes = [_l, _l, _fp, _fp, _u8p]
        L.orc_e4m3_quant_heads.restype = _l
        _lib = L
    return _lib


def max_threads() -> int:
    return lib().orc_max_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def _d(a):
    """Exact widening to a contiguous float64 array."""
    return np.ascontiguousarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Mamba-2
# --------------------------------------------------------------------------

def m2_decays(A, dt):
    """a[t,b,h] = exp(dt[t,b,h] * A[h]) -- the scalar Mamba-2 (SSD) decay."""
    dt = _d(dt)
    A = _d(A)
    T, batch, H = dt.shape
    assert A.shape == (H,)
    a = np.empty_like(dt)
    lib().orc_m2_decays(T, batch, H, A, dt, a)
    return a


def m2_recur(a, dt, x, B, C, D, h):
    """T eager Mamba-2 steps with the decays given directly.

    a, dt: [T,b,H]; x: [T,b,H,P]; B, C: [T,b,G,N]; D: [H];
    h: float64 [b,H,P,N], updated in place.  Returns y float64 [T,b,H,P].
    """
    a, dt, x, B, C, D = map(_d, (a, dt, x, B, C, D))
    assert h.dtype == np.float64 and h.flags["C_CONTIGUOUS"]
    T, batch, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert a.shape == dt.shape == (T, batch, H)
    assert B.shape == C.shape == (T, batch, G, N)
    assert h.shape == (batch, H, P, N) and D.shape == (H,)
    assert H % G == 0
    y = np.empty((T, batch, H, P), dtype=np.float64)
    if T and batch:
        lib().orc_m2_recur(T, batch, H, G, P, N, a, dt, x, B, C, D, h, y)
    return y


def m2_eager(A, D, x, B, C, dt, h):
    """T eager Mamba-2 steps: a = exp(dt*A); h = a*h + dt*x B^T; y = h C + D x."""
    return m2_recur(m2_decays(A, dt), dt, x, B, C, D, h)


# --------------------------------------------------------------------------
# Gated DeltaNet
# --------------------------------------------------------------------------

def gdn_eager(q, k, v, alpha, beta, S):
    """T eager GDN steps: S = alpha S (I - beta k k^T) + beta v k^T; o = S q.

    q, k: [T,b,H,dk]; v: [T,b,H,dv]; alpha, beta: [T,b,H];
    S: float64 [b,H,dv,dk], updated in place.  Returns o float64 [T,b,H,dv].
    """
    q, k, v, alpha, beta = map(_d, (q, k, v, alpha, beta))
    assert S.dtype == np.float64 and S.flags["C_CONTIGUOUS"]
    T, batch, H, DK = q.shape
    DV = v.shape[3]
    assert k.shape == q.shape and v.shape == (T, batch, H, DV)
    assert alpha.shape == beta.shape == (T, batch, H)
    assert S.shape == (batch, H, DV, DK)
    o = np.empty((T, batch, H, DV), dtype=np.float64)
    if T and batch:
        lib().orc_gdn_recur(T, batch, H, DK, DV, q, k, v, alpha, beta, S, o)
    return o


# --------------------------------------------------------------------------
# Number formats (decisions taken on fp32 values)
# --------------------------------------------------------------------------

def bf16_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_encode(x.size, x.reshape(-1), out.reshape(-1))
    return out


def bf16_decode(c):
    c = np.ascontiguousarray(c, dtype=np.uint16)
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_bf16_decode(c.size, c.reshape(-1), out.reshape(-1))
    return out


def e4m3_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3_encode(x.size, x.reshape(-1), out.reshape(-1))
    return out


def e4m3_decode(c):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_e4m3_decode(c.size, c.reshape(-1), out.reshape(-1))
    return out


def e4m3_quant_heads(tiles, return_nonfinite=False):
    """Per-head scaled E4M3: tiles [..., per_head] fp32 -> (scale[...], codes).

    scale = amax/448 (fp32; 1 if amax == 0), code = E4M3(s / scale).  A tile
    holding a NaN or an infinity gets scale 1 and is encoded as it is.  With
    return_nonfinite, also returns the number of such tiles.
    """
    tiles = np.ascontiguousarray(tiles, dtype=np.float32)
    lead = tiles.shape[:-1]
    per = tiles.shape[-1]
    nh = int(np.prod(lead)) if lead else 1
    scale = np.empty(lead, dtype=np.float32)
    codes = np.empty(tiles.shape, dtype=np.uint8)
    bad = lib().orc_e4m3_quant_heads(nh, per, tiles.reshape(-1), scale.reshape(-1),
                                     codes.reshape(-1))
    return (scale, codes, int(bad)) if return_nonfinite else (scale, codes)


def e4m3_dequant_heads(scale, codes):
    """Exact value of a scaled E4M3 tile: decode(code) * scale, in fp64.

    The product of a 4-significant-bit code and an fp32 scale is exact in fp64.
    """
    vals = e4m3_decode(codes)
    return vals * np.asarray(scale, dtype=np.float64)[..., None]
