"""C ABI host tests (CPU only, no kernel launches).

librssm.so must load without a GPU, export every function include/rssm.h
declares, and reject bad arguments on the host before launching anything.
Every call here either fails validation or has batch == 0, which returns
before any launch, so no device is touched.
"""
import ctypes
import os
import re

import pytest

from linear_attention_decode_replayssm_amd import rssm as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rssm.h")

FAKE = 0x10000          # 16-byte aligned stand-in address (never dereferenced)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0   # counts devices without initialising them
    except Exception:
        return False


# The stand-in addresses are only safe where nothing can be launched: should a
# validation ever let one of these calls through, a visible GPU would receive
# a kernel with bogus pointers.  On a machine with a GPU these host tests are
# skipped (the GPU tests cover the same entry points with real buffers).
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only tests with stand-in pointers")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(rssm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for f in ("rssm_mamba2_step", "rssm_gdn_step", "rssm_commit", "rssm_verify",
              "rssm_rollback", "rssm_eager_step", "rssm_status", "rssm_strerror",
              "rssm_abi_version"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = R.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    # exported dynamic symbols of the shared object, read from its ELF table
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(rssm_\w+)$", out, re.M))
    assert set(_declared()) <= exported


def test_version_and_strerror():
    assert R.rssm_abi_version() == R.RSSM_ABI_VERSION == 11
    for code in (0, -1, -2, -3, -4, -5):
        assert R.rssm_strerror(code)
    assert "unknown" in R.rssm_strerror(12345)


def _m2_desc(**kw):
    d = dict(kind=R.RSSM_MAMBA2, scheme=R.RSSM_F32, lp_dtype=0, batch=0, nheads=8,
             ngroups=1, dim_v=64, dim_k=128, capacity=16, flags=0)
    d.update(kw)
    L = R.rssm_layer(d["kind"], d["scheme"], d["lp_dtype"], d["batch"], d["nheads"],
                     d["ngroups"], d["dim_v"], d["dim_k"], d["capacity"], d["flags"])
    L.ckpt = kw.get("ckpt", FAKE)
    L.A = FAKE
    L.D = FAKE
    for i in range(3):
        L.ring[i] = FAKE
    L.ckpt_pos = L.len = L.arrive = L.status = FAKE
    return L


def _gdn_desc(**kw):
    d = dict(kind=R.RSSM_GDN, scheme=R.RSSM_F32, lp_dtype=0, batch=0, nheads=4,
             ngroups=1, dim_v=128, dim_k=128, capacity=8)
    d.update(kw)
    L = R.rssm_layer(d["kind"], d["scheme"], d["lp_dtype"], d["batch"], d["nheads"],
                     d["ngroups"], d["dim_v"], d["dim_k"], d["capacity"], 0)
    L.ckpt = FAKE
    if d["scheme"] != R.RSSM_F32:
        L.ckpt_lp = FAKE
        L.lp_scale = FAKE
    for i in range(4):
        L.ring[i] = FAKE
    L.ckpt_pos = L.len = L.arrive = L.status = FAKE
    return L


def _step(L, **kw):
    a = dict(x=FAKE, B=FAKE, C=FAKE, dt=FAKE, y=FAKE)
    a.update(kw)
    return R.rssm_mamba2_step(L, a["x"], a["B"], a["C"], a["dt"], a["y"], 0, stream=0,
                              check=False)


def test_empty_batch_is_ok_without_launch():
    assert _step(_m2_desc(batch=0)) == R.RSSM_OK
    assert R.rssm_commit(_m2_desc(batch=0), None, 0, stream=0, check=False) == R.RSSM_OK
    assert R.rssm_rollback(_m2_desc(batch=0), FAKE, stream=0, check=False) == R.RSSM_OK
    L = _gdn_desc(batch=0)
    assert R.rssm_gdn_step(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, stream=0,
                           check=False) == R.RSSM_OK


def test_empty_batch_accepts_null_arrays():
    """At batch 0 every per-sequence array holds no elements: NULL is
    accepted everywhere, while enums, dims and counts are still validated."""
    def bare(kind, scheme=R.RSSM_F32, lp=0):
        m2 = kind == R.RSSM_MAMBA2
        return R.rssm_layer(kind, scheme, lp, 0, 8 if m2 else 4, 1, 64 if m2 else 128, 128,
                            8, 0)
    m2, gdn = bare(R.RSSM_MAMBA2), bare(R.RSSM_GDN, R.RSSM_DUAL, R.RSSM_E4M3)
    none = R.make_inputs()
    for L in (m2, gdn):
        assert R.rssm_commit(L, None, 0, stream=0, check=False) == R.RSSM_OK
        assert R.rssm_rollback(L, None, stream=0, check=False) == R.RSSM_OK
        assert R.rssm_verify(L, 3, none, None, stream=0, check=False) == R.RSSM_OK
        assert R.rssm_eager_step(L, none, None, stream=0, check=False) == R.RSSM_OK
        assert R.rssm_verify(L, 9, none, None, stream=0, check=False) == R.RSSM_ERANGE
        assert R.rssm_commit(L, None, -1, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_mamba2_step(m2, None, None, None, None, None, 1, stream=0,
                              check=False) == R.RSSM_OK
    assert R.rssm_gdn_step(gdn, None, None, None, None, None, None, 0, stream=0,
                           check=False) == R.RSSM_OK
    assert R.rssm_gdn_step(gdn, None, None, None, None, None, None, 1, stream=0,
                           check=False) == R.RSSM_OK           # DUAL: fused commit allowed
    assert R.rssm_mamba2_step(gdn, None, None, None, None, None, 0, stream=0,
                              check=False) == R.RSSM_EINVAL
    shared = bare(R.RSSM_GDN, R.RSSM_SHARED, R.RSSM_BF16)
    assert R.rssm_eager_step(shared, none, None, stream=0, check=False) == R.RSSM_OK
    assert R.rssm_gdn_step(shared, None, None, None, None, None, None, 1, stream=0,
                           check=False) == R.RSSM_EUNSUPPORTED   # SHARED: no fused commit


def test_null_layer():
    lib = R.lib()
    assert lib.rssm_mamba2_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0) == R.RSSM_EINVAL
    assert lib.rssm_commit(None, None, 0, 0) == R.RSSM_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(kind=7), R.RSSM_EINVAL),
    (dict(scheme=9), R.RSSM_EINVAL),
    (dict(nheads=0), R.RSSM_EINVAL),
    (dict(batch=-1), R.RSSM_EINVAL),
    (dict(ngroups=3), R.RSSM_EINVAL),               # 8 % 3 != 0
    (dict(dim_v=32), R.RSSM_EUNSUPPORTED),
    (dict(dim_k=64), R.RSSM_EUNSUPPORTED),
    (dict(capacity=33), R.RSSM_EUNSUPPORTED),
    (dict(capacity=17, scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16), R.RSSM_EUNSUPPORTED),
    (dict(flags=2), R.RSSM_EINVAL),
    (dict(capacity=0), R.RSSM_EINVAL),
    (dict(batch=2 ** 27, nheads=8), R.RSSM_EUNSUPPORTED),   # batch * nheads = 2^30
    (dict(batch=2 ** 24, nheads=64, ngroups=8), R.RSSM_EUNSUPPORTED),
    (dict(scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16), R.RSSM_EINVAL),   # ckpt_lp missing
    (dict(scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_LP_NONE), R.RSSM_EINVAL),
    (dict(ckpt=FAKE + 4), R.RSSM_EALIGN),
    (dict(ckpt=0), R.RSSM_EINVAL),
])
def test_m2_layer_validation(kw, code):
    args = dict(batch=4)
    args.update(kw)
    assert _step(_m2_desc(**args)) == code


def test_m2_pointer_validation():
    assert _step(_m2_desc(batch=4), x=None) == R.RSSM_EINVAL
    assert _step(_m2_desc(batch=4), C=FAKE + 8) == R.RSSM_EALIGN
    L = _m2_desc(batch=4)
    L.ring[1] = None
    assert _step(L) == R.RSSM_EINVAL
    L = _m2_desc(batch=4)
    L.arrive = None
    assert _step(L) == R.RSSM_EINVAL
    L = _m2_desc(batch=4)
    L.ring[0] = FAKE + 4
    assert _step(L) == R.RSSM_EALIGN
    # wrong layer kind for the entry point
    assert R.rssm_gdn_step(_m2_desc(batch=4), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                           stream=0, check=False) == R.RSSM_EINVAL


def test_commit_verify_rollback_ranges():
    L = _m2_desc(batch=4, capacity=12)
    assert R.rssm_commit(L, None, -1, stream=0, check=False) == R.RSSM_ERANGE
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    assert R.rssm_verify(L, 0, inp, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_verify(L, 9, inp, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    L4 = _m2_desc(batch=4, capacity=4)
    assert R.rssm_verify(L4, 5, inp, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_verify(L, 4, R.make_inputs(x=FAKE, B=FAKE, C=FAKE), FAKE, stream=0,
                         check=False) == R.RSSM_EINVAL
    assert R.rssm_rollback(L, None, stream=0, check=False) == R.RSSM_EINVAL


def test_rollback_verify_commit_validates_on_host():
    """The fused rollback + verify refuses, before any launch, what either of
    the two calls it replaces refuses, and a missing rejection array."""
    L = _m2_desc(batch=4, capacity=12)
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    rvc = R.rssm_rollback_verify_commit
    assert rvc(L, None, 4, inp, FAKE, 8, stream=0, check=False) == R.RSSM_EINVAL
    assert rvc(L, FAKE, 4, inp, FAKE, 0, stream=0, check=False) == R.RSSM_ERANGE
    assert rvc(L, FAKE, 0, inp, FAKE, 8, stream=0, check=False) == R.RSSM_ERANGE
    assert rvc(L, FAKE, 9, inp, FAKE, 8, stream=0, check=False) == R.RSSM_ERANGE
    assert rvc(L, FAKE, 4, R.make_inputs(x=FAKE, B=FAKE, C=FAKE), FAKE, 8, stream=0,
               check=False) == R.RSSM_EINVAL
    dual = _m2_desc(batch=4, capacity=12, scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16)
    dual.ckpt_lp = FAKE
    assert rvc(dual, FAKE, 4, inp, FAKE, 8, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert rvc(_m2_desc(batch=0), FAKE, 4, inp, FAKE, 8, stream=0, check=False) == R.RSSM_OK


def test_gdn_validation():
    L = _gdn_desc(batch=2, ngroups=2)
    assert R.rssm_gdn_step(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0,
                           check=False) == R.RSSM_EINVAL
    L = _gdn_desc(batch=2, dim_k=64)
    assert R.rssm_gdn_step(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0,
                           check=False) == R.RSSM_EUNSUPPORTED
    L = _gdn_desc(batch=2, scheme=R.RSSM_SHARED, lp_dtype=R.RSSM_BF16)
    assert R.rssm_gdn_step(L, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, stream=0,
                           check=False) == R.RSSM_EUNSUPPORTED       # fused: F32 or DUAL
    L = _gdn_desc(batch=2, scheme=R.RSSM_DUAL, lp_dtype=0)
    assert R.rssm_commit(L, None, 0, stream=0, check=False) == R.RSSM_EINVAL
    L = _gdn_desc(batch=2, scheme=R.RSSM_SHARED, lp_dtype=R.RSSM_E4M3)
    L.lp_scale = None
    assert R.rssm_commit(L, None, 0, stream=0, check=False) == R.RSSM_EINVAL
    L = _gdn_desc(batch=2, scheme=R.RSSM_SHARED, lp_dtype=R.RSSM_BF16)
    L.ckpt = None
    L.ckpt_lp = None                  # the eager comparator of SHARED needs the copy
    inp = R.make_inputs(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE)
    assert R.rssm_eager_step(L, inp, FAKE, stream=0, check=False) == R.RSSM_EINVAL
    L = _gdn_desc(batch=2)
    L.ring[3] = None
    assert R.rssm_commit(L, None, 0, stream=0, check=False) == R.RSSM_EINVAL


def test_status_rejects_null():
    assert R.lib().rssm_status(None, None, None) == R.RSSM_EINVAL


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(R, "_lib", None)
    monkeypatch.setattr(R, "LIB_PATH", "/nonexistent/librssm.so")
    with pytest.raises(RuntimeError, match="missing"):
        R.lib()


def test_tree_entry_points_validate_on_host():
    L = _m2_desc(batch=4, capacity=12)
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    assert R.rssm_verify_tree(L, [-1, 1], inp, FAKE, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_verify_tree(L, [-1, -2], inp, FAKE, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_verify_tree(L, [-1] * 9, inp, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_verify_tree(_m2_desc(batch=0), [-1, 0], inp, FAKE, stream=0,
                              check=False) == R.RSSM_OK
    lib = R.lib()
    assert lib.rssm_verify_tree(ctypes.byref(L), 2, None, ctypes.byref(inp), FAKE, None) == R.RSSM_EINVAL
    assert lib.rssm_append_path(ctypes.byref(L), 4, FAKE, FAKE, 5, ctypes.byref(inp), None) == R.RSSM_ERANGE
    assert lib.rssm_append_path(ctypes.byref(L), 9, FAKE, FAKE, 1, ctypes.byref(inp), None) == R.RSSM_ERANGE
    assert lib.rssm_append_path(ctypes.byref(L), 4, None, FAKE, 2, ctypes.byref(inp), None) == R.RSSM_EINVAL
    L0 = _m2_desc(batch=0)
    assert lib.rssm_append_path(ctypes.byref(L0), 4, None, None, 2, ctypes.byref(inp), None) == R.RSSM_OK
    bad = R.make_inputs(x=FAKE + 4, B=FAKE, C=FAKE, dt=FAKE)
    assert lib.rssm_append_path(ctypes.byref(L), 4, FAKE, FAKE, 2, ctypes.byref(bad), None) == R.RSSM_EALIGN
    G = _gdn_desc(batch=4, capacity=12)
    badg = R.make_inputs(q=FAKE, k=FAKE, v=FAKE + 8, alpha=FAKE, beta=FAKE)
    assert lib.rssm_append_path(ctypes.byref(G), 4, FAKE, FAKE, 2, ctypes.byref(badg), None) == R.RSSM_EALIGN


def test_prefill_validates_on_host():
    L = _m2_desc(batch=4, capacity=8)
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    assert R.rssm_prefill(L, 0, inp, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_prefill(L, 5, R.make_inputs(x=FAKE, B=FAKE, dt=FAKE), FAKE, stream=0,
                          check=False) == R.RSSM_EINVAL            # outputs need C
    assert R.rssm_prefill(L, 5, R.make_inputs(x=FAKE, B=FAKE, C=FAKE), None, stream=0,
                          check=False) == R.RSSM_EINVAL            # dt missing
    assert R.rssm_prefill(L, 5, inp, FAKE + 8, stream=0, check=False) == R.RSSM_EALIGN
    assert R.rssm_prefill(_m2_desc(batch=0), 5, R.make_inputs(), None, stream=0,
                          check=False) == R.RSSM_OK
    assert R.lib().rssm_prefill(None, 5, ctypes.byref(inp), FAKE, None, None) == R.RSSM_EINVAL


def test_eager_spec_validates_on_host():
    L = _m2_desc(batch=4, capacity=8)
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    assert R.rssm_eager_spec_round(L, 0, inp, FAKE, FAKE, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_eager_spec_round(L, 9, inp, FAKE, FAKE, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_eager_spec_round(L, 4, inp, FAKE, None, FAKE, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_eager_spec_round(L, 4, inp, FAKE, FAKE + 8, FAKE, stream=0,
                                   check=False) == R.RSSM_EALIGN
    D = _m2_desc(batch=4, scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16, ckpt_lp=FAKE)
    assert R.rssm_eager_spec_round(D, 4, inp, FAKE, FAKE, FAKE, stream=0,
                                   check=False) == R.RSSM_EUNSUPPORTED
    assert R.rssm_eager_spec_accept(L, 0, FAKE, FAKE, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_eager_spec_accept(L, 4, None, FAKE, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_eager_spec_accept(_m2_desc(batch=0), 4, None, None, stream=0,
                                    check=False) == R.RSSM_OK


def test_verify_commit_validates_on_host():
    L = _m2_desc()
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    V = R.rssm_verify_commit
    assert V(L, 4, inp, FAKE, 0, stream=0, check=False) == R.RSSM_ERANGE
    assert V(L, 0, inp, FAKE, 8, stream=0, check=False) == R.RSSM_ERANGE
    assert V(_gdn_desc(scheme=R.RSSM_SHARED, lp_dtype=R.RSSM_E4M3), 4,
             R.make_inputs(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE),
             FAKE, 8, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert V(_m2_desc(scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16), 4, inp, FAKE, 8, stream=0,
             check=False) == R.RSSM_EUNSUPPORTED
    assert V(_m2_desc(batch=1), 4, inp, FAKE + 4, 8, stream=0, check=False) == R.RSSM_EALIGN


def test_verify_tree_commit_validates_on_host():
    L = _m2_desc()
    inp = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    V = R.rssm_verify_tree_commit
    assert V(L, [-1, 0], inp, FAKE, 0, stream=0, check=False) == R.RSSM_ERANGE
    assert V(L, [-1, 1], inp, FAKE, 8, stream=0, check=False) == R.RSSM_EINVAL
    assert V(_m2_desc(scheme=R.RSSM_DUAL, lp_dtype=R.RSSM_BF16), [-1, 0], inp, FAKE, 8, stream=0,
             check=False) == R.RSSM_EUNSUPPORTED
    assert V(L, [-1, 0], inp, FAKE, 8, stream=0, check=False) == R.RSSM_OK       # batch 0


def test_probe_validates_on_host():
    lib = R.lib()
    assert R.rssm_probe_stream(None, None, FAKE, 32768, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_probe_stream(FAKE, None, None, 32768, stream=0, check=False) == R.RSSM_EINVAL
    assert R.rssm_probe_stream(FAKE + 4, None, FAKE, 32768, stream=0, check=False) == R.RSSM_EALIGN
    assert R.rssm_probe_stream(FAKE, None, FAKE, 1000, stream=0, check=False) == R.RSSM_ERANGE
    assert R.rssm_probe_stream(FAKE, None, FAKE, 0, stream=0, check=False) == R.RSSM_ERANGE
    T = R.rssm_probe_stream_tiles
    assert T(None, None, FAKE, 4096, 4096, stream=0, check=False) == R.RSSM_EINVAL
    assert T(FAKE, None, FAKE, 32768, 8192, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert T(FAKE + 4, None, FAKE, 4096, 4096, stream=0, check=False) == R.RSSM_EALIGN
    assert T(FAKE, FAKE + 8, None, 4096, 4096, stream=0, check=False) == R.RSSM_EALIGN
    assert T(FAKE, None, FAKE, 6144, 4096, stream=0, check=False) == R.RSSM_ERANGE
    assert T(FAKE, None, FAKE, 4096, 32768, stream=0, check=False) == R.RSSM_ERANGE


def test_noalloc_step_validation():
    """rssm_mamba2_step_noalloc validates as rssm_mamba2_step does, ignores the
    descriptor's arrival counters, and refuses a batch above its counters'
    room before launching anything."""
    f = lambda L, commit=0: R.rssm_mamba2_step_noalloc(L, FAKE, FAKE, FAKE, FAKE, FAKE, commit,
                                                       stream=0, check=False)
    assert f(_m2_desc(batch=0)) == R.RSSM_OK
    big = _m2_desc(batch=R.RSSM_NOALLOC_MAX_BATCH + 1)
    big.arrive = None
    assert f(big) == R.RSSM_ERANGE
    assert f(_gdn_desc(batch=2)) == R.RSSM_EINVAL
    assert f(_m2_desc(batch=2, scheme=R.RSSM_SHARED, lp_dtype=R.RSSM_BF16), 1) == R.RSSM_EUNSUPPORTED
    L = _m2_desc(batch=2)
    L.len = None
    assert f(L) == R.RSSM_EINVAL
    assert R.rssm_mamba2_step_noalloc(_m2_desc(batch=2), FAKE + 4, FAKE, FAKE, FAKE, FAKE, 0,
                                      stream=0, check=False) == R.RSSM_EALIGN


def test_capacity_above_16_only_for_plain_mamba2_decode():
    """Rings of 17..32 slots serve the fp32 Mamba-2 step, commit and rollback;
    every other call refuses them before launching."""
    L = _m2_desc(batch=4, capacity=20)
    ins = R.make_inputs(x=FAKE, B=FAKE, C=FAKE, dt=FAKE)
    assert R.rssm_verify(L, 2, ins, FAKE, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert R.rssm_prefill(L, 2, ins, FAKE, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert R.rssm_eager_step(L, ins, FAKE, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    G = _gdn_desc(batch=4, capacity=20)
    assert R.rssm_gdn_step(G, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0,
                           check=False) == R.RSSM_EUNSUPPORTED
    assert R.rssm_commit(G, None, 0, stream=0, check=False) == R.RSSM_EUNSUPPORTED
    assert R.rssm_rollback(G, FAKE, stream=0, check=False) == R.RSSM_EUNSUPPORTED


def test_readonly_indices_need_no_counters_and_rollback_is_a_no_op():
    L = _m2_desc(batch=4, flags=R.RSSM_LAYER_INDEX_READONLY)
    L.arrive = None
    assert R.rssm_rollback(L, FAKE, stream=0, check=False) == R.RSSM_OK   # nothing launched
    assert R.rssm_rollback(L, None, stream=0, check=False) == R.RSSM_EINVAL
    L2 = _m2_desc(batch=4)
    L2.arrive = None
    assert _step(L2) == R.RSSM_EINVAL                  # an updating layer needs its counters
