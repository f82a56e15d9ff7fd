"""Seeded synthetic inputs for the decode workloads.

This module holds only random-number generation and the value distributions
of the workloads; it contains none of the state engine's arithmetic, and both
the HIP path's tests and the oracle consume the arrays it returns.

Every array is drawn in float64 from ``numpy.random.Generator(PCG64)`` seeded
by ``SeedSequence([seed, stream, layer, purpose, chunk])`` and then rounded
once to float32, so any window of steps can be regenerated on its own.

Distributions (normal laws are given as (mean, standard deviation)):

Mamba-2 decode
    x, B, C ~ N(0, 1) / sqrt(N)   dt = softplus(N(-2, 0.5))
    A_h = -exp(U(ln 1, ln 16))    D_h ~ N(0, 1)      h_0 ~ N(0, 0.1)
Gated DeltaNet decode
    q, k = v / ||v||_2 with v ~ N(0, 1)^dk          v ~ N(0, 1)
    alpha = exp(-softplus(N(0, 1)))                  beta = sigmoid(N(0, 1))
    S_0 = 0 (or N(0, s0_std) when asked for)
Speculative acceptance
    accepted count per (round, sequence) ~ U{0, ..., n_drafts}
"""
import numpy as np

CHUNK = 16          # steps per independently seeded chunk

M2_STREAM = 1
GDN_STREAM = 2
ACCEPT_STREAM = 3

_P_PARAMS, _P_STATE, _P_STEPS = 0, 1, 2


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _softplus(z):
    return np.logaddexp(0.0, z)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ------------------------------------------------------------------ Mamba-2 --

def m2_params(seed, H, layer=0):
    """Per-head A (negative decay rate) and D (skip), float32 [H]."""
    g = _rng(seed, M2_STREAM, layer, _P_PARAMS)
    A = -np.exp(g.uniform(np.log(1.0), np.log(16.0), size=H))
    D = g.standard_normal(H)
    return _f32(A), _f32(D)


def m2_state0(seed, batch, H, P, N, layer=0, std=0.1):
    g = _rng(seed, M2_STREAM, layer, _P_STATE)
    return _f32(g.normal(0.0, std, size=(batch, H, P, N)))


def m2_steps(seed, t0, T, batch, H, G, P, N, layer=0):
    """Inputs of steps t0 .. t0+T-1: dict x [T,b,H,P], B, C [T,b,G,N], dt [T,b,H]."""
    out = dict(x=np.empty((T, batch, H, P), np.float32),
               B=np.empty((T, batch, G, N), np.float32),
               C=np.empty((T, batch, G, N), np.float32),
               dt=np.empty((T, batch, H), np.float32))
    t = t0
    while t < t0 + T:
        c = t // CHUNK
        g = _rng(seed, M2_STREAM, layer, _P_STEPS, c)
        inv = 1.0 / np.sqrt(N)
        x = g.standard_normal((CHUNK, batch, H, P)) * inv
        B = g.standard_normal((CHUNK, batch, G, N)) * inv
        C = g.standard_normal((CHUNK, batch, G, N)) * inv
        dt = _softplus(g.normal(-2.0, 0.5, size=(CHUNK, batch, H)))
        lo = t - c * CHUNK
        hi = min(CHUNK, t0 + T - c * CHUNK)
        d0, d1 = t - t0, t - t0 + (hi - lo)
        out["x"][d0:d1] = x[lo:hi]
        out["B"][d0:d1] = B[lo:hi]
        out["C"][d0:d1] = C[lo:hi]
        out["dt"][d0:d1] = dt[lo:hi]
        t += hi - lo
    return out


# ------------------------------------------------------------ Gated DeltaNet --

def gdn_state0(seed, batch, H, dv, dk, layer=0, std=0.0):
    if std == 0.0:
        return np.zeros((batch, H, dv, dk), np.float32)
    g = _rng(seed, GDN_STREAM, layer, _P_STATE)
    return _f32(g.normal(0.0, std, size=(batch, H, dv, dk)))


def gdn_steps(seed, t0, T, batch, H, dk, dv, layer=0):
    """Inputs of steps t0 .. t0+T-1: q, k [T,b,H,dk], v [T,b,H,dv], alpha, beta [T,b,H]."""
    out = dict(q=np.empty((T, batch, H, dk), np.float32),
               k=np.empty((T, batch, H, dk), np.float32),
               v=np.empty((T, batch, H, dv), np.float32),
               alpha=np.empty((T, batch, H), np.float32),
               beta=np.empty((T, batch, H), np.float32))
    t = t0
    while t < t0 + T:
        c = t // CHUNK
        g = _rng(seed, GDN_STREAM, layer, _P_STEPS, c)
        q = g.standard_normal((CHUNK, batch, H, dk))
        k = g.standard_normal((CHUNK, batch, H, dk))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = g.standard_normal((CHUNK, batch, H, dv))
        alpha = np.exp(-_softplus(g.standard_normal((CHUNK, batch, H))))
        beta = 1.0 / (1.0 + np.exp(-g.standard_normal((CHUNK, batch, H))))
        lo = t - c * CHUNK
        hi = min(CHUNK, t0 + T - c * CHUNK)
        d0, d1 = t - t0, t - t0 + (hi - lo)
        for name, arr in (("q", q), ("k", k), ("v", v), ("alpha", alpha),
                          ("beta", beta)):
            out[name][d0:d1] = arr[lo:hi]
        t += hi - lo
    return out


# ------------------------------------------------------------- acceptance --

def accept_counts(seed, rounds, batch, n_drafts):
    """Accepted drafts per (round, sequence), uniform in {0..n_drafts},
    drawn round-major then sequence from one stream."""
    g = _rng(seed, ACCEPT_STREAM, 0, 0)
    return g.integers(0, n_drafts + 1, size=(rounds, batch)).astype(np.int32)


def stack_rounds(steps, rounds, n):
    """Reshape a [rounds*n, ...] step dict into [rounds, n, ...] drafts."""
    return {k: v.reshape((rounds, n) + v.shape[1:]) for k, v in steps.items()}
