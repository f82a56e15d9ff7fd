"""Oracle-side runs of whole workloads, built from the eager recurrences.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* plain decode: eager outputs for every step plus the exact index trace of a
  commit every ``interval`` tokens (explainer, "Periodically commit a new
  checkpoint");
* speculative rounds: each round appends n drafts, the outputs at all n draft
  positions come from a scratch continuation of the accepted state, then the
  rejected suffix is dropped and a commit folds any sequence whose buffer has
  reached ``commit_len`` (explainer, "Cheap speculative decoding rollback";
  Abstract: rolling back only moves a pointer into the buffer, and drafts
  are verified from their outputs without storing intermediate states);
* low-precision emulation: a low-precision checkpoint serves the outputs and
  is refreshed at each commit either from the high-precision state ("dual") or
  from itself ("shared") (Abstract: the low-precision copy serves the outputs
  on most steps and only the high-precision checkpoint takes the recurrent
  updates; explainer, "Separate precisions for serving vs updating state");
* the eager recurrence with its state stored in low precision, re-encoded
  after every step (explainer, "What ReplaySSM is solving": rounding fed back
  into every later update);
* prefill: the buffered entries and a whole prompt folded into the state, with
  the eager output of every prompt token (the pages are silent on prefill; it
  is read as a commit over a long buffer).

Because the eager recurrence started from any state S and run over the buffered
inputs equals the replay from checkpoint S over the same inputs, serving from
a checkpoint is emulated by a second eager state that is reset to the
checkpoint's exact value at every commit.
"""
import numpy as np

from . import (m2_eager, m2_recur, m2_decays, gdn_eager, bf16_encode,
               bf16_decode, e4m3_quant_heads, e4m3_dequant_heads)
from .index_model import IndexModel


# ------------------------------------------------------------- plain decode --

def decode_trace(batch, steps, interval, cap, t0_len=0):
    """Index trace of plain decode: after each step, (pos, len) of every
    sequence, with a commit right after the step that brings len to interval.
    Returns (pos[T,b], len[T,b], committed[T] bool)."""
    im = IndexModel(batch, cap)
    im.len[:] = t0_len
    pos = np.zeros((steps, batch), np.int64)
    ln = np.zeros((steps, batch), np.int32)
    com = np.zeros(steps, bool)
    for t in range(steps):
        im.append(1)
        if (im.len >= interval).all():
            im.commit()
            com[t] = True
        pos[t], ln[t] = im.snapshot()
    return pos, ln, com


def m2_decode(A, D, x, B, C, dt, h0, interval, cap):
    """Plain Mamba-2 decode.  Returns dict(y, pos, len, committed, ckpt) where
    ckpt is the exact state at the last commit (h0 if none)."""
    h = np.array(h0, dtype=np.float64, copy=True)
    T = x.shape[0]
    pos, ln, com = decode_trace(x.shape[1], T, interval, cap)
    y = np.empty(x.shape, np.float64)
    ckpt = h.copy()
    start = 0
    for t in range(T):
        if com[t] or t == T - 1:
            y[start:t + 1] = m2_eager(A, D, x[start:t + 1], B[start:t + 1],
                                      C[start:t + 1], dt[start:t + 1], h)
            start = t + 1
            if com[t]:
                ckpt = h.copy()
    return dict(y=y, pos=pos, len=ln, committed=com, ckpt=ckpt, state=h)


def gdn_decode(q, k, v, alpha, beta, S0, interval, cap):
    """Plain GDN decode; same return layout as m2_decode (o instead of y)."""
    S = np.array(S0, dtype=np.float64, copy=True)
    T = q.shape[0]
    pos, ln, com = decode_trace(q.shape[1], T, interval, cap)
    o = np.empty(v.shape, np.float64)
    ckpt = S.copy()
    start = 0
    for t in range(T):
        if com[t] or t == T - 1:
            o[start:t + 1] = gdn_eager(q[start:t + 1], k[start:t + 1],
                                       v[start:t + 1], alpha[start:t + 1],
                                       beta[start:t + 1], S)
            start = t + 1
            if com[t]:
                ckpt = S.copy()
    return dict(o=o, pos=pos, len=ln, committed=com, ckpt=ckpt, state=S)


# ------------------------------------------------------- speculative rounds --

def m2_spec_rounds(A, D, h0, drafts, accept, cap, commit_len):
    """Speculative verify / rollback rounds on Mamba-2.

    drafts: dict x [R,n,b,H,P], B/C [R,n,b,G,N], dt [R,n,b,H]
    accept: int [R,b], number of leading drafts kept in each round.
    Returns dict(y [R,n,b,H,P], pos [R,b], len [R,b], committed [R,b],
    status, state) -- indices after each round's commit.
    """
    x, B, C, dt = drafts["x"], drafts["B"], drafts["C"], drafts["dt"]
    R, n, batch = x.shape[0], x.shape[1], x.shape[2]
    h = np.array(h0, dtype=np.float64, copy=True)
    im = IndexModel(batch, cap)
    y = np.empty(x.shape, np.float64)
    pos = np.zeros((R, batch), np.int64)
    ln = np.zeros((R, batch), np.int32)
    com = np.zeros((R, batch), bool)
    for r in range(R):
        ok = im.append(n)
        if not ok.all():
            raise ValueError("speculative round would overflow the ring")
        # outputs at every draft position from a scratch copy of the state
        scratch = h.copy()
        y[r] = m2_eager(A, D, x[r], B[r], C[r], dt[r], scratch)
        # keep the accepted prefix: advance the real state per accept count
        acc = np.asarray(accept[r])
        for a in range(1, n + 1):
            sel = np.nonzero(acc == a)[0]
            if sel.size == 0:
                continue
            hs = np.ascontiguousarray(h[sel])
            m2_eager(A, D, x[r, :a][:, sel], B[r, :a][:, sel], C[r, :a][:, sel],
                     dt[r, :a][:, sel], hs)
            h[sel] = hs
        im.rollback(n - acc)
        com[r] = im.commit(min_len=commit_len)
        pos[r], ln[r] = im.snapshot()
    return dict(y=y, pos=pos, len=ln, committed=com, status=im.status, state=h)


def gdn_spec_rounds(h0, drafts, accept, cap, commit_len):
    """Speculative rounds on Gated DeltaNet; drafts: q,k [R,n,b,H,dk], v
    [R,n,b,H,dv], alpha/beta [R,n,b,H].  Same return layout as m2_spec_rounds
    with the outputs under "o"."""
    q, k, v, al, be = (drafts[s] for s in ("q", "k", "v", "alpha", "beta"))
    R, n, batch = q.shape[0], q.shape[1], q.shape[2]
    S = np.array(h0, dtype=np.float64, copy=True)
    im = IndexModel(batch, cap)
    o = np.empty(v.shape, np.float64)
    pos = np.zeros((R, batch), np.int64)
    ln = np.zeros((R, batch), np.int32)
    com = np.zeros((R, batch), bool)
    for r in range(R):
        ok = im.append(n)
        if not ok.all():
            raise ValueError("speculative round would overflow the ring")
        scratch = S.copy()
        o[r] = gdn_eager(q[r], k[r], v[r], al[r], be[r], scratch)
        acc = np.asarray(accept[r])
        for a in range(1, n + 1):
            sel = np.nonzero(acc == a)[0]
            if sel.size == 0:
                continue
            Ss = np.ascontiguousarray(S[sel])
            gdn_eager(q[r, :a][:, sel], k[r, :a][:, sel], v[r, :a][:, sel],
                      al[r, :a][:, sel], be[r, :a][:, sel], Ss)
            S[sel] = Ss
        im.rollback(n - acc)
        com[r] = im.commit(min_len=commit_len)
        pos[r], ln[r] = im.snapshot()
    return dict(o=o, pos=pos, len=ln, committed=com, status=im.status, state=S)


# ------------------------------------------------------------- draft trees --

def tree_paths(parent):
    """Root-first list of the drafts on each draft's path (itself last)."""
    paths = []
    for j, p in enumerate(parent):
        if not (-1 <= p < j):
            raise ValueError("parents must come first")
        paths.append((paths[p] if p >= 0 else []) + [j])
    return paths


def m2_tree_verify(A, D, h, drafts, parent):
    """Outputs of every draft of a tree (explainer, "Why this matters for
    agentic systems now": replay from one checkpoint along different input
    buffers): draft j's output is the eager recurrence continued from state h
    over the drafts on its path, root first.  drafts: x [n,b,H,P], B/C
    [n,b,G,N], dt [n,b,H].  h is not modified.  Returns y [n,b,H,P]."""
    x, B, C, dt = drafts["x"], drafts["B"], drafts["C"], drafts["dt"]
    y = np.empty(x.shape, np.float64)
    for j, path in enumerate(tree_paths(parent)):
        hs = np.array(h, dtype=np.float64, copy=True)
        out = m2_eager(A, D, x[path], B[path], C[path], dt[path], hs)
        y[j] = out[-1]
    return y


def gdn_tree_verify(S, drafts, parent):
    """As m2_tree_verify for Gated DeltaNet; drafts q, k [n,b,H,dk], v
    [n,b,H,dv], alpha/beta [n,b,H].  Returns o [n,b,H,dv]."""
    q, k, v, al, be = (drafts[s] for s in ("q", "k", "v", "alpha", "beta"))
    o = np.empty(v.shape, np.float64)
    for j, path in enumerate(tree_paths(parent)):
        Ss = np.array(S, dtype=np.float64, copy=True)
        out = gdn_eager(q[path], k[path], v[path], al[path], be[path], Ss)
        o[j] = out[-1]
    return o


# ------------------------------------------------------------------ prefill --

def _ragged_ring(ring, ring_len, s):
    """Sequence s's buffered entries, oldest first: [ring_len[s], 1, ...]."""
    n = int(ring_len[s])
    return {k: v[:n, s:s + 1] for k, v in ring.items()}


def m2_prefill(A, D, h, ring, ring_len, prompt, mask=None):
    """Prefill of a prompt into the checkpoint (a fold over a long buffer,
    explainer "Periodically commit a new checkpoint", applied to a whole
    prompt).  Per selected sequence: the state continues from h over its
    ring_len[s] buffered entries (ring x [Lr,b,H,P], B [Lr,b,G,N], dt [Lr,b,H];
    oldest first; their outputs are not formed), then over the prompt (x
    [T,b,H,P], B/C [T,b,G,N], dt [T,b,H]) with the eager output of every prompt
    token.  h [b,H,P,N] fp64 is updated in place for selected sequences.
    Returns y [T,b,H,P] (NaN for unselected sequences)."""
    x, B, C, dt = prompt["x"], prompt["B"], prompt["C"], prompt["dt"]
    y = np.full(x.shape, np.nan)
    for s in range(x.shape[1]):
        if mask is not None and not mask[s]:
            continue
        hs = np.array(h[s:s + 1], dtype=np.float64, copy=True)
        r = _ragged_ring(ring, ring_len, s)
        if r["x"].shape[0]:
            zc = np.zeros(r["B"].shape, np.float32)   # no output: C does not matter
            m2_eager(A, D, r["x"], r["B"], zc, r["dt"], hs)
        y[:, s:s + 1] = m2_eager(A, D, x[:, s:s + 1], B[:, s:s + 1], C[:, s:s + 1],
                                 dt[:, s:s + 1], hs)
        h[s:s + 1] = hs
    return y


def gdn_prefill(S, ring, ring_len, prompt, mask=None):
    """As m2_prefill for Gated DeltaNet: ring k [Lr,b,H,dk], v [Lr,b,H,dv],
    alpha/beta [Lr,b,H]; prompt q, k [T,b,H,dk], v [T,b,H,dv], alpha/beta
    [T,b,H].  S [b,H,dv,dk] fp64 updated in place.  Returns o [T,b,H,dv]."""
    q, k, v, al, be = (prompt[n] for n in ("q", "k", "v", "alpha", "beta"))
    o = np.full(v.shape, np.nan)
    for s in range(q.shape[1]):
        if mask is not None and not mask[s]:
            continue
        Ss = np.array(S[s:s + 1], dtype=np.float64, copy=True)
        r = _ragged_ring(ring, ring_len, s)
        if r["k"].shape[0]:
            gdn_eager(np.zeros(r["k"].shape, np.float32), r["k"], r["v"], r["alpha"],
                      r["beta"], Ss)
        o[:, s:s + 1] = gdn_eager(q[:, s:s + 1], k[:, s:s + 1], v[:, s:s + 1],
                                  al[:, s:s + 1], be[:, s:s + 1], Ss)
        S[s:s + 1] = Ss
    return o


# ------------------------------------------------- low-precision emulation --

def quantize(state_f32, lp):
    """Quantise fp32 state tiles [..., R, C] to the low-precision copy.

    Returns (codes, scale or None, exact fp64 value of the copy).
    bf16: round-to-nearest-even per element.  e4m3: per-tile scale
    amax/448 then E4M3(s/scale), saturating (OCP FP8 E4M3)."""
    s = np.ascontiguousarray(state_f32, dtype=np.float32)
    if lp == "bf16":
        codes = bf16_encode(s)
        return codes, None, bf16_decode(codes)
    if lp == "e4m3":
        lead, (r, c) = s.shape[:-2], s.shape[-2:]
        scale, codes = e4m3_quant_heads(s.reshape(lead + (r * c,)))
        val = e4m3_dequant_heads(scale, codes).reshape(s.shape)
        return codes.reshape(s.shape), scale, val
    raise ValueError(lp)


def _lowprec(run, state0, T, out_shape, interval, scheme, lp, fused=False):
    """Plain decode with a low-precision serving checkpoint; `run(sl, state)`
    runs the eager recurrence over steps `sl` from `state` (fp64, updated in
    place) and returns their outputs.

    scheme "dual": an fp32-class state receives every update; at each commit
    the low-precision copy is re-quantised from it.  scheme "shared": the
    low-precision copy is the only checkpoint; each commit folds the buffer
    into its exact value and re-quantises the result.  In both, every step's
    output is served from the low-precision copy plus the buffered inputs
    (commit happens after the output of the step that fills the interval).
    The state that is quantised is first rounded to fp32, the precision in
    which a kernel holds it.

    fused (dual only): the step that fills the interval reads the fp32-class
    state for its fold and serves its own output from it, so that output is
    the exact one; the other steps and the copy are unchanged."""
    if fused and scheme != "dual":
        raise ValueError("a fused commit serves from the fp32 state: dual only")
    exact = np.array(state0, dtype=np.float64, copy=True)
    codes, scale, val = quantize(exact.astype(np.float32), lp)
    serve = val.copy()
    o_emul = np.empty(out_shape, np.float64)
    o_exact = np.empty(out_shape, np.float64)
    ckpt_exact = exact.copy()
    commits = []
    start = 0
    for t in range(T):
        if (t + 1 - start) == interval or t == T - 1:
            sl = slice(start, t + 1)
            o_exact[sl] = run(sl, exact)
            o_emul[sl] = run(sl, serve)
            if (t + 1 - start) == interval:
                if fused:
                    o_emul[t] = o_exact[t]
                src = exact if scheme == "dual" else serve
                codes, scale, val = quantize(src.astype(np.float32), lp)
                serve = val.copy()
                ckpt_exact = exact.copy()
                commits.append(t)
            start = t + 1
    return dict(o_emul=o_emul, o_exact=o_exact, ckpt_exact=ckpt_exact,
                codes=codes, scale=scale, commits=commits, state=exact,
                serve=serve)


def gdn_lowprec(q, k, v, alpha, beta, S0, interval, scheme, lp, fused=False):
    """GDN plain decode with a low-precision serving checkpoint (see _lowprec).

    Returns dict(o_emul, o_exact, ckpt_exact [b,H,dv,dk] at the last commit,
    codes, scale (last commit), commits (step indices))."""
    def run(sl, S):
        return gdn_eager(q[sl], k[sl], v[sl], alpha[sl], beta[sl], S)
    return _lowprec(run, S0, q.shape[0], v.shape, interval, scheme, lp, fused)


def m2_lowprec(A, D, x, B, C, dt, h0, interval, scheme, lp, fused=False):
    """Mamba-2 plain decode with a low-precision serving checkpoint (see
    _lowprec); outputs under "o_emul" / "o_exact", shape of x."""
    def run(sl, h):
        return m2_eager(A, D, x[sl], B[sl], C[sl], dt[sl], h)
    return _lowprec(run, h0, x.shape[0], x.shape, interval, scheme, lp, fused)


def _eager_lowprec(run, state0, T, out_shape, lp):
    """Eager recurrence whose state lives in low precision only (explainer,
    "What ReplaySSM is solving": storing the recurrent state in low precision
    feeds its rounding back into every later update).  Each step decodes the
    stored copy, runs one exact step from it, takes the output from the
    updated state, rounds that state to fp32 (the precision a kernel holds it
    in) and re-encodes it.  Returns dict(o, o_exact, codes, scale, state)."""
    exact = np.array(state0, dtype=np.float64, copy=True)
    codes, scale, val = quantize(exact.astype(np.float32), lp)
    o = np.empty(out_shape, np.float64)
    o_exact = np.empty(out_shape, np.float64)
    for t in range(T):
        sl = slice(t, t + 1)
        o_exact[sl] = run(sl, exact)
        cur = val.copy()
        o[sl] = run(sl, cur)
        codes, scale, val = quantize(cur.astype(np.float32), lp)
    return dict(o=o, o_exact=o_exact, codes=codes, scale=scale, state=exact, serve=val)


def m2_eager_lowprec(A, D, x, B, C, dt, h0, lp):
    def run(sl, h):
        return m2_eager(A, D, x[sl], B[sl], C[sl], dt[sl], h)
    return _eager_lowprec(run, h0, x.shape[0], x.shape, lp)


def gdn_eager_lowprec(q, k, v, alpha, beta, S0, lp):
    def run(sl, S):
        return gdn_eager(q[sl], k[sl], v[sl], alpha[sl], beta[sl], S)
    return _eager_lowprec(run, S0, q.shape[0], v.shape, lp)


def gdn_carry_batched(q_t, ks, alphas, betas):
    """Backward-carried query for many units at once.

    q_t [U,dk]; ks [U,L,dk]; alphas, betas [U,L].  Returns (q_tilde [U,dk],
    s [U,L]).  Same arithmetic as replay.gdn_carry, vectorised over units."""
    q = np.array(q_t, dtype=np.float64, copy=True)
    ks = np.asarray(ks, np.float64)
    al = np.asarray(alphas, np.float64)
    be = np.asarray(betas, np.float64)
    L = ks.shape[1]
    s = np.zeros(al.shape)
    for i in range(L - 1, -1, -1):
        s[:, i] = be[:, i] * np.einsum("ud,ud->u", ks[:, i], q)
        q = al[:, i, None] * (q - s[:, i, None] * ks[:, i])
    return q, s


__all__ = ["decode_trace", "m2_decode", "gdn_decode", "m2_spec_rounds",
           "gdn_spec_rounds", "quantize", "gdn_lowprec", "gdn_carry_batched",
           "m2_recur", "m2_decays"]
