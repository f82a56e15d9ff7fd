"""Unrolled (checkpoint + buffer) forms of the two recurrences, fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

ReplaySSM represents the state as a checkpoint plus a buffer of recent SSM
inputs and computes each output from the checkpoint and a replay over the
buffered inputs, without writing intermediate states ("ReplaySSM: Cache SSM
Inputs, Not State", Abstract (arXiv); explainer section "Compute outputs without
eagerly updating the checkpoint").  The explicit formulas are not printed on
the pages; they follow by unrolling the textbook recurrences:

Mamba-2, checkpoint h_c at position c, buffer entries i = c+1..t (the last one
is the current token), Gamma_{m..n} = exp(A * sum_{j=m..n} dt_j):

    y_t   = Gamma_{c+1..t} h_c C_t + sum_i Gamma_{i+1..t} dt_i (B_i . C_t) x_i + D x_t
    h_new = Gamma_{c+1..t} h_c + sum_i Gamma_{i+1..t} dt_i x_i B_i^T

Gated DeltaNet, A_i = alpha_i (I - beta_i k_i k_i^T), S_i = S_{i-1} A_i + beta_i v_i k_i^T:

    carry q <- q_t;  for i = t..c+1:  s_i = beta_i (k_i . q);  q <- alpha_i (q - s_i k_i)
    o_t   = S_c q + sum_i s_i v_i

and the fold, with u_i = beta_i (v_i - alpha_i S_{i-1} k_i) and
S_{i-1} k_i = G_{c+1..i-1} S_c k_i + sum_{m<i} G_{m+1..i-1} (k_m . k_i) u_m:

    S_new = G_{c+1..t} S_c + sum_i G_{i+1..t} u_i k_i^T        (G = products of alpha)

These functions are used by the oracle's invariant tests (replay = eager) and to
supply the carried query for the low-precision error bound.  They are written
one unit at a time, with Python loops over buffer entries.
"""
import numpy as np


def _f(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- Mamba-2 --

def m2_output(h_c, xs, Bs, dts, C_t, A, D):
    """Output of one head from checkpoint h_c [P,N] and L >= 1 buffer entries.

    xs [L,P], Bs [L,N], dts [L]: entries oldest first, the last is the current
    token.  C_t [N] is the current token's C; A, D scalars of the head.
    """
    h_c, xs, Bs, dts, C_t = map(_f, (h_c, xs, Bs, dts, C_t))
    L = xs.shape[0]
    gamma_all = np.exp(A * dts.sum())
    y = gamma_all * (h_c @ C_t)
    for i in range(L):
        gamma_after = np.exp(A * dts[i + 1:].sum())
        y = y + gamma_after * dts[i] * (Bs[i] @ C_t) * xs[i]
    return y + D * xs[L - 1]


def m2_output_empty(h_c, C_t, x_t, D):
    """Degenerate case with no buffered entries: h_c C + D x."""
    return _f(h_c) @ _f(C_t) + D * _f(x_t)


def m2_fold(h_c, xs, Bs, dts, A):
    """New checkpoint after folding L entries into h_c [P,N]."""
    h_c, xs, Bs, dts = map(_f, (h_c, xs, Bs, dts))
    h = np.exp(A * dts.sum()) * h_c
    for i in range(xs.shape[0]):
        h = h + np.exp(A * dts[i + 1:].sum()) * dts[i] * np.outer(xs[i], Bs[i])
    return h


# ---------------------------------------------------------- Gated DeltaNet --

def gdn_carry(q_t, ks, alphas, betas):
    """Backward-carried query.  ks [L,dk] oldest first; returns (q_tilde, s[L])."""
    q = _f(q_t).copy()
    ks, alphas, betas = map(_f, (ks, alphas, betas))
    L = ks.shape[0]
    s = np.zeros(L)
    for i in range(L - 1, -1, -1):
        s[i] = betas[i] * (ks[i] @ q)
        q = alphas[i] * (q - s[i] * ks[i])
    return q, s


def gdn_output(S_c, q_t, ks, vs, alphas, betas):
    """o_t = S_c q_tilde + sum_i s_i v_i.  S_c [dv,dk], vs [L,dv]."""
    qt, s = gdn_carry(q_t, ks, alphas, betas)
    S_c = _f(S_c)
    return S_c @ qt + s @ _f(vs).reshape(len(s), S_c.shape[0])


def gdn_fold(S_c, ks, vs, alphas, betas):
    """New checkpoint by forward substitution for u_i, then one rank-L update."""
    S_c, ks, vs, alphas, betas = map(_f, (S_c, ks, vs, alphas, betas))
    L = ks.shape[0]
    dv = S_c.shape[0]
    W = S_c @ ks.T                       # [dv, L]:  S_c k_i
    gram = ks @ ks.T                     # [L, L]:   k_m . k_i
    U = np.zeros((dv, L))

    def G(m, n):                          # prod alpha_m..alpha_n (empty -> 1)
        return float(np.prod(alphas[m:n + 1])) if n >= m else 1.0

    for i in range(L):
        sk = G(0, i - 1) * W[:, i]
        for m in range(i):
            sk = sk + G(m + 1, i - 1) * gram[m, i] * U[:, m]
        U[:, i] = betas[i] * (vs[i] - alphas[i] * sk)
    S = G(0, L - 1) * S_c
    for i in range(L):
        S = S + G(i + 1, L - 1) * np.outer(U[:, i], ks[i])
    return S
