"""Pins of the oracle's low-precision emulations (Mamba-2 dual/shared serving
checkpoint, and the eager recurrence whose state is stored in low precision).

* Lossless cases: states that bf16 / scaled E4M3 represent exactly make every
  emulated output equal the exact one, bit for bit.
* A closed form: with x = 0 and a decay of exactly 1/2 per step the state is
  h_0 / 2^t; halving is exact in both formats (E4M3: the codes stay, the
  per-head scale halves), so the eager-in-low-precision path reproduces the
  exact outputs and its codes never change.
* A property: the dual scheme's error obeys the one-quantisation bound
  |y - y_exact| <= Gamma * sum_n delta(h_c[p, n]) |C_n| at every step.
"""
import numpy as np
import pytest

import oracle
from oracle import drivers

P, N = 4, 8


def _lossless_state(rng, lp, b, H):
    if lp == "bf16":
        f = (rng.standard_normal((b, H, P, N)) * 0.3).astype(np.float32)
        return oracle.bf16_decode(oracle.bf16_encode(f))
    codes = rng.integers(0, 0x7F, size=(b, H, P * N)).astype(np.uint8)
    codes[..., 0] = 0x7E                         # amax = 448 * 2^-10: scale 2^-10 exactly
    signs = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    scale = np.full((b, H), 2.0 ** -10)
    return oracle.e4m3_dequant_heads(scale, codes | signs).reshape(b, H, P, N)


def _inputs(rng, T, b, H, G, zero_dt=False):
    x = (rng.standard_normal((T, b, H, P)) * 0.2).astype(np.float32)
    B = (rng.standard_normal((T, b, G, N)) * 0.2).astype(np.float32)
    C = (rng.standard_normal((T, b, G, N)) * 0.2).astype(np.float32)
    dt = np.zeros((T, b, H), np.float32) if zero_dt else rng.uniform(0.05, 0.3, (T, b, H)).astype(np.float32)
    return x, B, C, dt


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
@pytest.mark.parametrize("scheme", ["dual", "shared"])
def test_lossless_state_serves_exactly(lp, scheme):
    """dt = 0: the state never changes and is exactly representable."""
    rng = np.random.default_rng(100)
    T, b, H, G = 6, 2, 2, 1
    h0 = _lossless_state(rng, lp, b, H)
    A = np.array([-1.0, -3.0])
    D = np.array([0.5, -0.25])
    x, B, C, dt = _inputs(rng, T, b, H, G, zero_dt=True)
    r = drivers.m2_lowprec(A, D, x, B, C, dt, h0, 2, scheme, lp)
    np.testing.assert_array_equal(r["o_emul"], r["o_exact"])
    e = drivers.m2_eager_lowprec(A, D, x, B, C, dt, h0, lp)
    np.testing.assert_array_equal(e["o"], e["o_exact"])


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
def test_halving_closed_form(lp):
    """x = 0, a = exp(-ln 2) = 1/2: h_t = h_0 / 2^t and y_t = h_t C_t exactly."""
    rng = np.random.default_rng(101)
    T, b, H, G = 5, 1, 2, 1
    h0 = _lossless_state(rng, lp, b, H)
    A = np.full(H, -np.log(2.0))
    D = np.zeros(H)
    x, B, C, _ = _inputs(rng, T, b, H, G)
    x[:] = 0.0
    dt = np.ones((T, b, H), np.float32)
    e = drivers.m2_eager_lowprec(A, D, x, B, C, dt, h0, lp)
    want = np.stack([np.einsum("bhpn,bn->bhp", h0 / 2.0 ** (t + 1), C[t, :, 0].astype(np.float64))
                     for t in range(T)])
    np.testing.assert_array_equal(e["o"], want)
    c0, s0, _ = drivers.quantize(h0.astype(np.float32), lp)
    if lp == "e4m3":   # the codes never change, the scale halves every step
        np.testing.assert_array_equal(e["codes"], c0)
        np.testing.assert_array_equal(e["scale"], s0 / np.float32(2.0 ** T))
    else:
        np.testing.assert_array_equal(e["codes"], oracle.bf16_encode((h0 / 2.0 ** T).astype(np.float32)))


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
def test_dual_one_quantisation_bound(lp):
    rng = np.random.default_rng(102)
    T, b, H, G, interval = 24, 2, 4, 2, 6
    A = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N)) * 0.3
    x, B, C, dt = _inputs(rng, T, b, H, G)
    r = drivers.m2_lowprec(A, D, x, B, C, dt, h0, interval, "dual", lp)
    g = np.arange(H) * G // H
    h = h0.copy()
    for t in range(T):
        c0 = (t // interval) * interval
        if t == c0:
            hc = h.copy()
        gam = np.exp(A[None, :] * dt[c0:t + 1].astype(np.float64).sum(0))          # [b,H]
        if lp == "bf16":
            delta = 2.0 ** -8 * np.abs(hc)
        else:
            amax = np.abs(hc.astype(np.float32)).reshape(b, H, -1).max(-1).astype(np.float64)
            delta = np.maximum(2.0 ** -4 * np.abs(hc), 2.0 ** -10 * (amax / 448.0)[..., None, None])
        Ct = np.abs(C[t][:, g].astype(np.float64))                                     # [b,H,N]
        bound = gam[..., None] * np.einsum("bhpn,bhn->bhp", delta, Ct)
        err = np.abs(r["o_emul"][t] - r["o_exact"][t])
        assert np.all(err <= bound * (1 + 1e-4) + 1e-12), t
        oracle.m2_eager(A, D, x[t:t + 1], B[t:t + 1], C[t:t + 1], dt[t:t + 1], h)


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
@pytest.mark.parametrize("scheme", ["dual", "shared"])
def test_error_is_the_decayed_checkpoint_rounding(lp, scheme):
    """The recurrence is linear in the state, so between two commits the served
    output differs from the exact one by Gamma (h_served - h_c) C_t exactly,
    with h_served the codec image of the checkpoint the scheme encodes (the
    exact state for dual, the previous served state folded for shared)."""
    rng = np.random.default_rng(103)
    T, b, H, G, interval = 12, 2, 2, 1, 4
    A = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N)) * 0.3
    x, B, C, dt = _inputs(rng, T, b, H, G)
    r = drivers.m2_lowprec(A, D, x, B, C, dt, h0, interval, scheme, lp)
    g = np.arange(H) * G // H
    exact, served = h0.copy(), None
    for t in range(T):
        c0 = (t // interval) * interval
        if t == c0:
            src = exact if (scheme == "dual" or served is None) else served
            codes, scale, val = drivers.quantize(src.astype(np.float32), lp)
            served_c = val.copy()
            exact_c = exact.copy()
            served = val.copy()
        gam = np.exp(A[None, :] * dt[c0:t + 1].astype(np.float64).sum(0))
        want = gam[..., None] * np.einsum("bhpn,bhn->bhp", served_c - exact_c,
                                          C[t][:, g].astype(np.float64))
        got = r["o_emul"][t] - r["o_exact"][t]
        assert np.abs(want).max() > 0
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-12 * np.abs(r["o_exact"][t]).max())
        oracle.m2_eager(A, D, x[t:t + 1], B[t:t + 1], C[t:t + 1], dt[t:t + 1], exact)
        oracle.m2_eager(A, D, x[t:t + 1], B[t:t + 1], C[t:t + 1], dt[t:t + 1], served)


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
def test_eager_lowprec_first_step_error(lp):
    """One eager step from the stored copy: the output differs from the exact
    one by a_0 (h_stored - h_0) C_0, and the stored copy afterwards is the
    codec image of that step's fp32-rounded state."""
    rng = np.random.default_rng(104)
    T, b, H, G = 1, 2, 2, 1
    A = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N)) * 0.3
    x, B, C, dt = _inputs(rng, T, b, H, G)
    e = drivers.m2_eager_lowprec(A, D, x, B, C, dt, h0, lp)
    _, _, stored = drivers.quantize(h0.astype(np.float32), lp)
    a0 = np.exp(A[None, :] * dt[0].astype(np.float64))
    want = a0[..., None] * np.einsum("bhpn,bn->bhp", stored - h0, C[0, :, 0].astype(np.float64))
    np.testing.assert_allclose(e["o"][0] - e["o_exact"][0], want, rtol=1e-6, atol=1e-15)
    h1 = stored.copy()
    oracle.m2_eager(A, D, x, B, C, dt, h1)
    codes, scale, _ = drivers.quantize(h1.astype(np.float32), lp)
    np.testing.assert_array_equal(e["codes"], codes)


@pytest.mark.parametrize("lp", ["bf16", "e4m3"])
def test_fused_dual_commit_serves_the_boundary_step_exactly(lp):
    """With the commit fused into the step that fills the interval, that step
    reads the fp32-class state and its output is the exact one; every other
    step and the serving copy are those of the standalone commit.  Closed
    form on the boundary step: a lossless state keeps everything exact, and
    the unfused emulation already agrees with the fused one off the
    boundary; the fused error at the boundary is exactly zero."""
    rng = np.random.default_rng(104)
    T, b, H, G, interval = 18, 2, 4, 2, 6
    A = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N)) * 0.3
    x, B, C, dt = _inputs(rng, T, b, H, G)
    plain = drivers.m2_lowprec(A, D, x, B, C, dt, h0, interval, "dual", lp)
    fused = drivers.m2_lowprec(A, D, x, B, C, dt, h0, interval, "dual", lp, fused=True)
    boundary = np.zeros(T, bool)
    boundary[interval - 1::interval] = True
    np.testing.assert_array_equal(fused["o_emul"][~boundary], plain["o_emul"][~boundary])
    np.testing.assert_array_equal(fused["o_emul"][boundary], fused["o_exact"][boundary])
    assert np.abs(plain["o_emul"][boundary] - plain["o_exact"][boundary]).max() > 0
    np.testing.assert_array_equal(fused["codes"], plain["codes"])
    with pytest.raises(ValueError):
        drivers.m2_lowprec(A, D, x, B, C, dt, h0, interval, "shared", lp, fused=True)
