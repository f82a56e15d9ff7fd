"""Exact brute-force forms of the recurrences, in pure Python ``Fraction``s.

Used only as pins for the oracle: they are written in a different form from
the oracle's code (explicit unrolled sums and explicit matrix products instead
of the in-place rank-one eager update), so a dropped term, a wrong sign or a
transposed operand in either one makes the two disagree.  With dyadic inputs
every intermediate of the oracle's fp64 arithmetic is exact, so the comparison
is equality.
"""
from fractions import Fraction as Fr


def m2_unrolled(a, dt, x, B, C, D, h0, groups):
    """Mamba-2 outputs from the explicit unrolled sum.

    a, dt: [T][b][H]; x: [T][b][H][P]; B, C: [T][b][G][N]; D: [H];
    h0: [b][H][P][N]; groups: G.  Head h reads group h // (H // G).
      y_t[p] = (prod_{j<=t} a_j) h0[p,:].C_t
               + sum_{i<=t} (prod_{i<j<=t} a_j) dt_i x_i[p] (B_i . C_t) + D x_t[p]
    """
    T = len(a)
    nb = len(a[0])
    H = len(a[0][0])
    P = len(x[0][0][0])
    N = len(B[0][0][0])
    per = H // groups
    y = [[[[None] * P for _ in range(H)] for _ in range(nb)] for _ in range(T)]
    for b in range(nb):
        for h in range(H):
            g = h // per
            for t in range(T):
                Ct = [Fr(c) for c in C[t][b][g]]
                for p in range(P):
                    dec = Fr(1)
                    for j in range(t + 1):
                        dec *= Fr(a[j][b][h])
                    acc = dec * sum(Fr(h0[b][h][p][n]) * Ct[n] for n in range(N))
                    for i in range(t + 1):
                        w = Fr(1)
                        for j in range(i + 1, t + 1):
                            w *= Fr(a[j][b][h])
                        bc = sum(Fr(B[i][b][g][n]) * Ct[n] for n in range(N))
                        acc += w * Fr(dt[i][b][h]) * Fr(x[i][b][h][p]) * bc
                    y[t][b][h][p] = acc + Fr(D[h]) * Fr(x[t][b][h][p])
    return y


def _matmul(X, Y):
    return [[sum(X[i][k] * Y[k][j] for k in range(len(Y))) for j in range(len(Y[0]))]
            for i in range(len(X))]


def gdn_matrix_form(q, k, v, alpha, beta, S0):
    """Gated DeltaNet for one head, with explicit dk x dk transition matrices.

    S_t = S_{t-1} M_t + beta_t v_t k_t^T,  M_t = alpha_t (I - beta_t k_t k_t^T),
    o_t = S_t q_t.  q, k: [T][dk]; v: [T][dv]; S0: [dv][dk].
    Returns (o [T][dv], S_T).
    """
    T = len(q)
    dk = len(q[0])
    S = [[Fr(s) for s in row] for row in S0]
    outs = []
    for t in range(T):
        al, be = Fr(alpha[t]), Fr(beta[t])
        kt = [Fr(c) for c in k[t]]
        M = [[al * ((1 if i == j else 0) - be * kt[i] * kt[j]) for j in range(dk)]
             for i in range(dk)]
        S = _matmul(S, M)
        S = [[S[r][c] + be * Fr(v[t][r]) * kt[c] for c in range(dk)]
             for r in range(len(S))]
        outs.append([sum(S[r][c] * Fr(q[t][c]) for c in range(dk))
                     for r in range(len(S))])
    return outs, S
