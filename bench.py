#!/usr/bin/env python3
"""Benchmark of the ReplaySSM decode-time state engine on one MI355X.

Headline workload: Mamba-2 serving-shape decode, one layer, batch 256, 80
heads, headdim 64, dstate 128, 8 groups, fp32 checkpoint, commit every 8
tokens (fused into the 8th step), ring of 8.  One benchmark step = one decode
token for all 256 sequences: append + replay output (+ the fused commit every
8th step).  Inputs cycle through a pool of 64 distinct seeded steps that is
resident in HBM before timing starts.

Printed (one JSON line): seq-tokens/s of the replay path (value), the eager
read-modify-write kernel's seq-tokens/s on the same GPU and the speedup, the
HBM roofline of the dominant kernel (the replay step without commit), the
oracle timed on the host cores on a bounded sample, and secondary figures for
the Gated DeltaNet decode, speculative verify/rollback rounds, the
dual-precision GDN stack (with the eager comparator that keeps the state in
low precision), a sweep of the Mamba-2 commit interval, the Mamba-2 layer
with a low-precision checkpoint, and draft-tree speculation rounds.

Usage: python bench.py [--gpus 1] [--steps 1024] [--warmup 64] [--no-secondary]
       [--no-cpu]
"""
import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
REPEATS = 5   # extra repetitions of the headline's timed region, for its spread
METRIC = "seq-tokens/s per SSM layer at batch 256 + HBM GB/s vs peak; speedup vs eager"
COUNTERS = os.path.join(ROOT, "profiles", "m2_step_counters.json")
CALIB_COPY_BYTES = 671088640
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_decode_replayssm_amd", "csrc", f)
                  for f in ("m2_kernels.hip", "common.hpp", "lp_codec.hpp", "launch.hpp")] + [
                      os.path.join(ROOT, "linear_attention_decode_replayssm_amd", "build.py")]


def _spread(v):
    return {"median": round(float(np.median(v)), 1), "min": round(float(np.min(v)), 1),
            "max": round(float(np.max(v)), 1)}


def _round1(d):
    """Round every number of a (nested) dict to one decimal."""
    return {k: _round1(v) if isinstance(v, dict) else round(v, 1) for k, v in d.items()}


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ bytes --
# Algorithmic bytes (what the method must move; 4 bytes per fp32 element).
def m2_bytes(b, H, G, P, N):
    S = b * H * P * N * 4
    inputs = (b * H * P + 2 * b * G * N + b * H) * 4       # x, B, C, dt
    entry = (b * H * P + b * G * N + b * H) * 4            # one buffered (x, B, dt)
    out = b * H * P * 4
    idx = b * (8 + 4) * 2                                   # read + write pos/len
    return S, inputs, entry, out, idx


def m2_step_bytes(b, H, G, P, N, length):
    """Replay step with `length` previously buffered entries: checkpoint read,
    current inputs, the buffered entries, the appended entry, the output."""
    S, inputs, entry, out, idx = m2_bytes(b, H, G, P, N)
    return S + inputs + length * entry + entry + out + idx


def m2_fused_bytes(b, H, G, P, N, length):
    """Boundary step with fused commit: as a step, minus the append, plus the
    checkpoint write."""
    S, inputs, entry, out, idx = m2_bytes(b, H, G, P, N)
    return S + inputs + length * entry + out + S + idx


def m2_eager_bytes(b, H, G, P, N):
    S, inputs, entry, out, idx = m2_bytes(b, H, G, P, N)
    return 2 * S + inputs + out


def gdn_bytes(b, H, d, s_ck=4):
    S = b * H * d * d * s_ck
    inputs = (3 * b * H * d + 2 * b * H) * 4
    entry = (2 * b * H * d + 2 * b * H) * 4
    out = b * H * d * 4
    return S, inputs, entry, out


# ------------------------------------------------------------------ timing --
def _dev_state(torch, h):
    """An initial state uploaded once, then copied on the device into each
    layer a workload sets up.  Pageable uploads of hundreds of MB just before
    a timed loop were seen to stall the host thread for tens of milliseconds
    inside the timed region (at the first launches of the loop)."""
    t = torch.from_numpy(h).to("cuda")
    torch.cuda.synchronize()
    return t


def run_m2(torch, R, syn, steps, warmup, seed=0, pool_n=64):
    b, H, G, P, N, interval, cap = 256, 80, 8, 64, 128, 8, 8
    A, D = syn.m2_params(seed, H)
    h0 = _dev_state(torch, syn.m2_state0(seed, b, H, P, N))
    pool = syn.m2_steps(seed, 0, pool_n, b, H, G, P, N)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    L = R.Layer.mamba2(b, H, G, P, N, cap)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(h0)
    y = torch.empty((b, H, P), dtype=torch.float32, device="cuda")
    t = 0

    def step(ev=None):
        nonlocal t
        j = t % pool_n
        commit = (t + 1) % interval == 0
        if ev is not None:
            ev[0].record()
        R.rssm_mamba2_step(L, dev["x"][j], dev["B"][j], dev["C"][j], dev["dt"][j], y,
                           commit_after=commit)
        if ev is not None:
            ev[1].record()
        t += 1
        return commit

    for _ in range(warmup):
        step()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region 1 (value): K steps bracketed by two events, nothing between launches
    lens1 = [(t + i) % interval for i in range(steps)]
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    pass1_bytes = sum(m2_fused_bytes(b, H, G, P, N, l) if l == interval - 1 else
                      m2_step_bytes(b, H, G, P, N, l) for l in lens1)
    # timed region 2 (roofline): whole commit intervals after region 1, on the
    # stream the kernels run on.  One event pair brackets the interval's
    # interval-1 plain steps, launched back to back (their average launch
    # duration, gaps between them included, with the events' own cost spread
    # over them), and another its fused-commit step.
    while t % interval:
        step()
    groups = max(1, steps // interval)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(groups)]
    torch.cuda.synchronize()
    for g in range(groups):
        evs[g][0].record()
        for _ in range(interval - 1):
            step()
        evs[g][1].record()
        step()
        evs[g][2].record()
    torch.cuda.synchronize()
    assert R.rssm_status(L) == 0
    plain_us = np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3 / (interval - 1)
    fused_us = np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
    # the spread: the timed region of `value` repeated REPEATS times
    rep_ms = []
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            step()
        end.record()
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(end))
    assert R.rssm_status(L) == 0
    plain_bytes = np.array([m2_step_bytes(b, H, G, P, N, l) for l in range(interval - 1)])
    res = dict(total_ms=total_ms, seq_tok_s=b * steps / (total_ms * 1e-3),
               rep_seq_tok_s=[b * steps / (ms * 1e-3) for ms in rep_ms],
               step_us=float(plain_us),
               step_bytes=float(plain_bytes.mean()),
               fused_us=float(fused_us),
               fused_bytes=float(m2_fused_bytes(b, H, G, P, N, interval - 1)),
               all_bytes=float(pass1_bytes),
               # steady state: every step reads the checkpoint, one step in
               # `interval` also writes it (the fused commit)
               ckpt_bytes_per_step=(b * H * P * N * 4) * (interval + 1) / interval)
    # eager comparator on the same shapes, same pool
    L.ckpt.copy_(h0)
    inputs = [R.make_inputs(x=dev["x"][j], B=dev["B"][j], C=dev["C"][j], dt=dev["dt"][j])
              for j in range(pool_n)]
    for i in range(warmup):
        R.rssm_eager_step(L, inputs[i % pool_n], y)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        R.rssm_eager_step(L, inputs[i % pool_n], y)
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end)
    eager_rep = []
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            R.rssm_eager_step(L, inputs[i % pool_n], y)
        end.record()
        torch.cuda.synchronize()
        eager_rep.append(b * steps / (start.elapsed_time(end) * 1e-3))
    res["eager_rep_seq_tok_s"] = eager_rep
    res["eager_seq_tok_s"] = b * steps / (eager_ms * 1e-3)
    res["eager_us"] = eager_ms * 1e3 / steps
    res["eager_gbps"] = m2_eager_bytes(b, H, G, P, N) / (res["eager_us"] * 1e-6) / 1e9
    res["eager_ckpt_bytes_per_step"] = 2 * b * H * P * N * 4
    res["shape"] = dict(b=b, H=H, G=G, P=P, N=N, interval=interval, cap=cap)
    del L, dev
    torch.cuda.empty_cache()
    return res


def run_gdn(torch, R, syn, steps, warmup, seed=0, pool_n=16):
    b, H, d, interval, cap = 256, 32, 128, 8, 8
    pool = syn.gdn_steps(seed, 0, pool_n, b, H, d, d)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    L = R.Layer.gdn(b, H, d, d, cap)
    o = torch.empty((b, H, d), dtype=torch.float32, device="cuda")
    names = ("q", "k", "v", "alpha", "beta")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def replay(n, t0):
        for t in range(t0, t0 + n):
            j = t % pool_n
            R.rssm_gdn_step(L, *(dev[s][j] for s in names), o,
                            commit_after=(t + 1) % interval == 0)

    replay(warmup, 0)
    torch.cuda.synchronize()
    start.record()
    replay(steps, warmup)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    inputs = [R.make_inputs(**{s: dev[s][j] for s in names}) for j in range(pool_n)]
    for i in range(warmup):
        R.rssm_eager_step(L, inputs[i % pool_n], o)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        R.rssm_eager_step(L, inputs[i % pool_n], o)
    end.record()
    torch.cuda.synchronize()
    ems = start.elapsed_time(end)
    S, inp, entry, out = gdn_bytes(b, H, d)
    tot = 0   # algorithmic bytes of the timed replay steps (len = t mod interval)
    for t in range(warmup, warmup + steps):
        ln = t % interval
        if (t + 1) % interval == 0:   # fused commit: state read and written
            tot += 2 * S + inp + ln * entry + out
        else:                         # replay: state read, entry appended
            tot += S + inp + ln * entry + entry + out
    res = dict(seq_tok_s=b * steps / (ms * 1e-3), eager_seq_tok_s=b * steps / (ems * 1e-3),
               us_per_step=ms * 1e3 / steps, eager_us=ems * 1e3 / steps,
               hbm_gbps=tot / (ms * 1e-3) / 1e9, hbm_frac=tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               eager_gbps=(2 * S + inp + out) / (ems * 1e-3 / steps) / 1e9)
    res["speedup_vs_eager"] = res["seq_tok_s"] / res["eager_seq_tok_s"]
    del L, dev
    torch.cuda.empty_cache()
    return res


def _sweep_time(torch, run, n):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run(n)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def run_m2_interval_sweep(torch, R, syn, steps, seed=0, pool_n=16,
                          intervals=(1, 2, 4, 8, 16, 32)):
    """Replay cost vs state traffic (explainer, "How to think about using it":
    the commit interval trades replay work against state writes): the headline
    Mamba-2 shape with a commit every `interval` tokens (ring = interval),
    fused into the interval's last step ("fused") or as a standalone
    rssm_commit after it ("standalone").  Interval 1 writes the state every
    step, like the eager kernel."""
    b, H, G, P, N = 256, 80, 8, 64, 128
    A, D = syn.m2_params(seed, H)
    pool = syn.m2_steps(seed, 0, pool_n, b, H, G, P, N)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    h0 = _dev_state(torch, syn.m2_state0(seed, b, H, P, N))
    y = torch.empty((b, H, P), dtype=torch.float32, device="cuda")
    S, _, entry, _, idx = m2_bytes(b, H, G, P, N)
    res = {}
    for interval in intervals:
        L = R.Layer.mamba2(b, H, G, P, N, interval)
        L.A.copy_(torch.from_numpy(A))
        L.D.copy_(torch.from_numpy(D))
        L.ckpt.copy_(h0)
        n = max(1, steps // interval) * interval
        row = {}
        for mode in ("fused", "standalone"):
            def run(m):
                for t in range(m):
                    j = t % pool_n
                    last = (t + 1) % interval == 0
                    R.rssm_mamba2_step(L, dev["x"][j], dev["B"][j], dev["C"][j], dev["dt"][j], y,
                                       commit_after=last and mode == "fused")
                    if last and mode == "standalone":
                        R.rssm_commit(L, None, 0)

            run(2 * interval)                  # whole cycles: the timed run starts at len 0
            ms = _sweep_time(torch, run, n)
            assert R.rssm_status(L) == 0
            if mode == "fused":
                byt = sum(m2_fused_bytes(b, H, G, P, N, l) if l == interval - 1 else
                          m2_step_bytes(b, H, G, P, N, l) for l in (t % interval for t in range(n)))
            else:   # every step appends; each commit reads and writes the state, reads the ring
                byt = sum(m2_step_bytes(b, H, G, P, N, t % interval) for t in range(n)) + \
                    (n // interval) * (2 * S + interval * entry + idx)
            row[mode] = dict(seq_tok_s=round(b * n / (ms * 1e-3), 1), bytes_per_step=round(byt / n),
                             hbm_gbps=round(byt / (ms * 1e-3) / 1e9, 1))
        res[str(interval)] = row
        del L
        torch.cuda.empty_cache()
    del dev
    return res


def run_gdn_interval_sweep(torch, R, syn, steps, seed=0, pool_n=16, intervals=(1, 2, 4, 8, 16)):
    """The same trade-off for Gated DeltaNet at batch 256 x 32 heads (d 128),
    commit fused into the interval's last step (ring = interval)."""
    b, H, d = 256, 32, 128
    pool = syn.gdn_steps(seed, 0, pool_n, b, H, d, d)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    names = ("q", "k", "v", "alpha", "beta")
    o = torch.empty((b, H, d), dtype=torch.float32, device="cuda")
    S, inp, entry, out = gdn_bytes(b, H, d)
    res = {}
    for interval in intervals:
        L = R.Layer.gdn(b, H, d, d, interval)

        def run(m):
            for t in range(m):
                j = t % pool_n
                R.rssm_gdn_step(L, *(dev[s][j] for s in names), o,
                                commit_after=(t + 1) % interval == 0)

        n = max(1, steps // interval) * interval
        run(2 * interval)
        ms = _sweep_time(torch, run, n)
        assert R.rssm_status(L) == 0
        byt = 0
        for t in range(n):
            ln = t % interval
            byt += (2 * S + inp + ln * entry + out) if ln == interval - 1 else \
                (S + inp + ln * entry + entry + out)
        res[str(interval)] = dict(seq_tok_s=round(b * n / (ms * 1e-3), 1),
                                  bytes_per_step=round(byt / n),
                                  hbm_gbps=round(byt / (ms * 1e-3) / 1e9, 1))
        del L
        torch.cuda.empty_cache()
    del dev
    return res


def run_spec(torch, R, syn, rounds, seed=0, pool_n=16):
    """Mamba-2 speculative rounds at the serving shape: verify 4 drafts,
    roll back the rejected ones, commit at 8 buffered entries; ring 12.  Then
    the same rounds with the eager comparator (state read once, written after
    every draft)."""
    b, H, G, P, N, cap, n, commit_len = 256, 80, 8, 64, 128, 12, 4, 8
    A, D = syn.m2_params(seed, H)
    pool = syn.m2_steps(seed, 0, pool_n, b, H, G, P, N)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    accept = syn.accept_counts(seed, rounds, b, n)
    nrej = torch.from_numpy((n - accept).astype(np.int32)).to("cuda")
    h0 = _dev_state(torch, syn.m2_state0(seed, b, H, P, N))
    L = R.Layer.mamba2(b, H, G, P, N, cap)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(h0)
    out = torch.empty((n, b, H, P), dtype=torch.float32, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        j = (r * n) % pool_n
        R.rssm_verify(L, n, R.make_inputs(x=dev["x"][j:j + n], B=dev["B"][j:j + n],
                                          C=dev["C"][j:j + n], dt=dev["dt"][j:j + n]), out)
        R.rssm_rollback(L, nrej[r])
        R.rssm_commit(L, None, commit_len)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    # algorithmic bytes of the whole run from the per-sequence length trace
    S, inputs, entry, out_b, _ = m2_bytes(1, H, G, P, N)   # per sequence
    ln = np.zeros(b, np.int64)
    total = 0
    for r in range(rounds):
        total += b * (S + n * (inputs + out_b + entry)) + entry * int(ln.sum())   # verify
        ln += accept[r]                                          # append n, roll back n - a
        com = ln >= commit_len
        total += int(com.sum()) * 2 * S + entry * int(ln[com].sum())             # commit
        ln[com] = 0
    res = dict(rounds_per_s=rounds / (ms * 1e-3),
               accepted_seq_tok_s=float(accept.sum()) / (ms * 1e-3),
               us_per_round=ms * 1e3 / rounds,
               bytes_per_round=total / rounds,
               hbm_gbps=total / (ms * 1e-3) / 1e9)
    del L   # the next phase reuses the same cached blocks

    # the same rounds with the commit folded into the next verify
    # (rssm_verify_commit): a due buffer waits for the next round's state read,
    # so the ring holds up to 11 entries plus the 4 drafts (16 slots)
    L = R.Layer.mamba2(b, H, G, P, N, 16)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(h0)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        j = (r * n) % pool_n
        R.rssm_verify_commit(L, n, R.make_inputs(x=dev["x"][j:j + n], B=dev["B"][j:j + n],
                                                 C=dev["C"][j:j + n], dt=dev["dt"][j:j + n]),
                             out, commit_len)
        R.rssm_rollback(L, nrej[r])
    end.record()
    torch.cuda.synchronize()
    fms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    ln = np.zeros(b, np.int64)
    ftotal = 0
    for r in range(rounds):
        com = ln >= commit_len
        ftotal += b * (S + n * (inputs + out_b + entry)) + entry * int(ln.sum())   # verify
        ftotal += int(com.sum()) * S                                              # fold write
        ln[com] = 0
        ln += accept[r]
    # the same rounds with each round's rollback passed to the next round's
    # verify (rssm_rollback_verify_commit): one launch per round
    del L   # the next phase reuses the same cached blocks
    L = R.Layer.mamba2(b, H, G, P, N, 16)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(h0)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        j = (r * n) % pool_n
        inp = R.make_inputs(x=dev["x"][j:j + n], B=dev["B"][j:j + n], C=dev["C"][j:j + n],
                            dt=dev["dt"][j:j + n])
        if r == 0:
            R.rssm_verify_commit(L, n, inp, out, commit_len)
        else:
            R.rssm_rollback_verify_commit(L, nrej[r - 1], n, inp, out, commit_len)
    R.rssm_rollback(L, nrej[rounds - 1])
    end.record()
    torch.cuda.synchronize()
    rms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    # the same rounds appending only the accepted drafts: the drafts verified
    # as a chain-shaped tree (nothing appended, a due buffer folded from the
    # same state read), then the accepted prefix appended; no rollback
    del L   # the next phase reuses the same cached blocks
    L = R.Layer.mamba2(b, H, G, P, N, 16)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(h0)
    path = torch.arange(n, dtype=torch.int32, device="cuda").repeat(b, 1)
    acc_d = torch.from_numpy(accept.astype(np.int32)).to("cuda")
    chain = list(range(-1, n - 1))
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        j = (r * n) % pool_n
        inp = R.make_inputs(x=dev["x"][j:j + n], B=dev["B"][j:j + n], C=dev["C"][j:j + n],
                            dt=dev["dt"][j:j + n])
        R.rssm_verify_tree_commit(L, chain, inp, out, commit_len)
        R.rssm_append_path(L, n, path, acc_d[r], inp)
    end.record()
    torch.cuda.synchronize()
    ams = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    del L   # the next phase reuses the same cached blocks
    res["accepted_only"] = dict(rounds_per_s=rounds / (ams * 1e-3),
                                accepted_seq_tok_s=float(accept.sum()) / (ams * 1e-3),
                                us_per_round=ams * 1e3 / rounds,
                                speedup_vs_standalone_commit=ms / ams)
    res["fused_commit"] = dict(rounds_per_s=rounds / (fms * 1e-3),
                               accepted_seq_tok_s=float(accept.sum()) / (fms * 1e-3),
                               us_per_round=fms * 1e3 / rounds,
                               bytes_per_round=ftotal / rounds,
                               hbm_gbps=ftotal / (fms * 1e-3) / 1e9,
                               speedup_vs_standalone_commit=ms / fms)
    res["fused_commit"]["rollback_in_verify"] = dict(
        rounds_per_s=rounds / (rms * 1e-3),
        accepted_seq_tok_s=float(accept.sum()) / (rms * 1e-3),
        us_per_round=rms * 1e3 / rounds,
        hbm_gbps=ftotal / (rms * 1e-3) / 1e9)

    # the eager comparator on the same rounds: the state read once per round
    # and written after every draft (n + 1 state slots, accept = slot move)
    L = R.Layer.mamba2(b, H, G, P, N, cap)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    slots = torch.empty((n + 1, b, H, P, N), dtype=torch.float32, device="cuda")
    slots[0].copy_(h0)
    cur = torch.zeros(b, dtype=torch.int32, device="cuda")
    acc_d = torch.from_numpy(accept.astype(np.int32)).to("cuda")
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        j = (r * n) % pool_n
        R.rssm_eager_spec_round(L, n, R.make_inputs(x=dev["x"][j:j + n], B=dev["B"][j:j + n],
                                                    C=dev["C"][j:j + n], dt=dev["dt"][j:j + n]),
                                out, slots, cur)
        R.rssm_eager_spec_accept(L, n, cur, acc_d[r])
    end.record()
    torch.cuda.synchronize()
    ems = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    ebytes = b * ((1 + n) * S + n * (inputs + out_b))
    res["eager_rounds_per_s"] = rounds / (ems * 1e-3)
    res["eager_bytes_per_round"] = float(ebytes)
    res["eager_hbm_gbps"] = ebytes * rounds / (ems * 1e-3) / 1e9
    res["speedup_vs_eager_spec"] = ems / ms
    del L, dev, slots, h0
    torch.cuda.empty_cache()
    return res


def stream_ceilings(torch, R, nbytes=671088640, reps=10):
    """Context for the roofline fraction: what the library's streaming probe
    moves over a buffer the size of the headline checkpoint, far above the
    256 MB Infinity Cache: read-only, and a copy (bytes read + written per
    second).  Two workgroup shapes (rssm_probe_stream_tiles): the replay
    step's own (32 KiB per 256-thread workgroup, eight 16-byte nontemporal
    loads per thread, nothing else), and 4 KiB per workgroup with one load per
    thread (`*_4k`), the fastest pure-stream shape measured on this GPU."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(nbytes // 1024, dtype=torch.float32, device="cuda")
    res = {}
    for name, d, moved, tile in (("read_gbps", None, nbytes, 32768),
                                 ("copy_gbps", dst, 2 * nbytes, 32768),
                                 ("read_gbps_4k", None, nbytes, 4096),
                                 ("copy_gbps_4k", dst, 2 * nbytes, 4096)):
        R.rssm_probe_stream_tiles(src, d, sink, nbytes, tile, write_all=False)
        ev = []
        for i in range(reps):
            a_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            R.rssm_probe_stream_tiles(src, d, sink, nbytes, tile, write_all=False)
            e_.record()
            ev.append((a_, e_))
        torch.cuda.synchronize()
        ms = float(np.median([a_.elapsed_time(e_) for a_, e_ in ev]))
        res[name] = round(moved / (ms * 1e-3) / 1e9, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    return res


def run_gdn_spec(torch, R, syn, rounds, seed=0, pool_n=16):
    """GDN speculative rounds at the GDN serving shape (batch 256 x 32 heads,
    d 128): verify 4 drafts, roll back the rejected ones, commit at 8; ring
    12.  Then the same rounds with the commit folded into the next verify
    (rssm_verify_commit, ring 16), and with the eager comparator."""
    b, H, d, cap, n, commit_len = 256, 32, 128, 12, 4, 8
    names = ("q", "k", "v", "alpha", "beta")
    pool = syn.gdn_steps(seed, 0, pool_n, b, H, d, d)
    dev = {k: torch.from_numpy(pool[k]).to("cuda") for k in names}
    accept = syn.accept_counts(seed, rounds, b, n)
    nrej = torch.from_numpy((n - accept).astype(np.int32)).to("cuda")
    acc_d = torch.from_numpy(accept.astype(np.int32)).to("cuda")
    out = torch.empty((n, b, H, d), dtype=torch.float32, device="cuda")
    inp = [R.make_inputs(**{k: dev[k][(r * n) % pool_n:(r * n) % pool_n + n] for k in names})
           for r in range(pool_n // n)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    L = R.Layer.gdn(b, H, d, d, cap)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        R.rssm_verify(L, n, inp[r % len(inp)], out)
        R.rssm_rollback(L, nrej[r])
        R.rssm_commit(L, None, commit_len)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    del L   # the next phase reuses the same cached blocks
    # the commit folded into the next verify (ring 16, as for Mamba-2)
    L = R.Layer.gdn(b, H, d, d, 16)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        R.rssm_verify_commit(L, n, inp[r % len(inp)], out, commit_len)
        R.rssm_rollback(L, nrej[r])
    end.record()
    torch.cuda.synchronize()
    fms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    del L   # the next phase reuses the same cached blocks
    # each round's rollback passed to the next round's verify: one launch per round
    L = R.Layer.gdn(b, H, d, d, 16)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        if r == 0:
            R.rssm_verify_commit(L, n, inp[0], out, commit_len)
        else:
            R.rssm_rollback_verify_commit(L, nrej[r - 1], n, inp[r % len(inp)], out, commit_len)
    R.rssm_rollback(L, nrej[rounds - 1])
    end.record()
    torch.cuda.synchronize()
    rms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    del L   # the next phase reuses the same cached blocks
    L = R.Layer.gdn(b, H, d, d, cap)
    slots = torch.zeros((n + 1, b, H, d, d), dtype=torch.float32, device="cuda")
    cur = torch.zeros(b, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        R.rssm_eager_spec_round(L, n, inp[r % len(inp)], out, slots, cur)
        R.rssm_eager_spec_accept(L, n, cur, acc_d[r])
    end.record()
    torch.cuda.synchronize()
    ems = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    res = dict(rounds_per_s=rounds / (ms * 1e-3),
               accepted_seq_tok_s=float(accept.sum()) / (ms * 1e-3),
               us_per_round=ms * 1e3 / rounds,
               fused_commit=dict(rounds_per_s=rounds / (fms * 1e-3),
                                 accepted_seq_tok_s=float(accept.sum()) / (fms * 1e-3),
                                 us_per_round=fms * 1e3 / rounds,
                                 speedup_vs_standalone_commit=ms / fms,
                                 rollback_in_verify=dict(
                                     rounds_per_s=rounds / (rms * 1e-3),
                                     accepted_seq_tok_s=float(accept.sum()) / (rms * 1e-3),
                                     us_per_round=rms * 1e3 / rounds)),
               eager_rounds_per_s=rounds / (ems * 1e-3),
               speedup_vs_eager_spec=ems / ms)
    del L, dev, slots
    torch.cuda.empty_cache()
    return res


def run_tree_rounds(torch, R, syn, rounds, seed=0):
    """Mamba-2 headline shape, tree speculation: each round verifies a binary
    tree of 7 drafts (depth 3) from one checkpoint read, appends a random
    root-to-node path per sequence (0..3 drafts) and commits sequences whose
    buffer reached 8; ring 16 (up to 7 buffered + 7 drafts in flight).  Then
    the same rounds with the commit folded into the tree verify."""
    b, H, G, P, N, cap, commit_len = 256, 80, 8, 64, 128, 16, 8
    parent = [-1, 0, 0, 1, 1, 2, 2]
    paths = [[0], [0, 1], [0, 2], [0, 1, 3], [0, 1, 4], [0, 2, 5], [0, 2, 6]]
    n, depth = len(parent), 3
    A, D = syn.m2_params(seed, H)
    pool = syn.m2_steps(seed, 0, n, b, H, G, P, N)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    inp = R.make_inputs(x=dev["x"], B=dev["B"], C=dev["C"], dt=dev["dt"])
    g = np.random.default_rng(seed)
    pick = g.integers(-1, n, size=(rounds, b))
    arr = np.zeros((rounds, b, depth), np.int32)
    plen = np.zeros((rounds, b), np.int32)
    for r in range(rounds):
        for s_ in range(b):
            if pick[r, s_] >= 0:
                p = paths[pick[r, s_]]
                arr[r, s_, :len(p)] = p
                plen[r, s_] = len(p)
    arr_d = torch.from_numpy(arr).to("cuda")
    plen_d = torch.from_numpy(plen).to("cuda")
    L = R.Layer.mamba2(b, H, G, P, N, cap)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(_dev_state(torch, syn.m2_state0(seed, b, H, P, N)))
    out = torch.empty((n, b, H, P), dtype=torch.float32, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        R.rssm_verify_tree(L, parent, inp, out)
        R.rssm_append_path(L, n, arr_d[r], plen_d[r], inp)
        R.rssm_commit(L, None, commit_len)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    res = dict(rounds_per_s=rounds / (ms * 1e-3),
               accepted_seq_tok_s=float(plen.sum()) / (ms * 1e-3),
               us_per_round=ms * 1e3 / rounds, drafts_per_round=n)
    # the same rounds with the commit folded into the tree verify
    # (rssm_verify_tree_commit).  A buffer that waits one round longer must
    # still leave room for the 7 drafts: folding at 7 entries, a sequence holds
    # at most 6 + 3 = 9 before a verify, and 9 + 7 = 16 slots
    fold_len = 7
    del L
    L = R.Layer.mamba2(b, H, G, P, N, cap)
    L.A.copy_(torch.from_numpy(A))
    L.D.copy_(torch.from_numpy(D))
    L.ckpt.copy_(_dev_state(torch, syn.m2_state0(seed, b, H, P, N)))
    torch.cuda.synchronize()
    start.record()
    for r in range(rounds):
        R.rssm_verify_tree_commit(L, parent, inp, out, fold_len)
        R.rssm_append_path(L, n, arr_d[r], plen_d[r], inp)
    end.record()
    torch.cuda.synchronize()
    fms = start.elapsed_time(end)
    assert R.rssm_status(L) == 0
    res["fused_commit_at_7"] = dict(rounds_per_s=rounds / (fms * 1e-3),
                                    accepted_seq_tok_s=float(plen.sum()) / (fms * 1e-3),
                                    us_per_round=fms * 1e3 / rounds)
    del L, dev
    torch.cuda.empty_cache()
    return res


def run_gdn_tree_rounds(torch, R, syn, rounds, seed=0):
    """The tree rounds of run_tree_rounds at the GDN serving shape (batch 256 x
    32 heads, d 128): a binary tree of 7 drafts verified from one checkpoint
    read, a random root-to-node path appended, commit at 8 (standalone); then
    with the commit folded into the tree verify at 7 entries."""
    b, H, d, cap, commit_len = 256, 32, 128, 16, 8
    parent = [-1, 0, 0, 1, 1, 2, 2]
    paths = [[0], [0, 1], [0, 2], [0, 1, 3], [0, 1, 4], [0, 2, 5], [0, 2, 6]]
    n, depth = len(parent), 3
    names = ("q", "k", "v", "alpha", "beta")
    pool = syn.gdn_steps(seed, 0, n, b, H, d, d)
    dev = {k: torch.from_numpy(pool[k]).to("cuda") for k in names}
    inp = R.make_inputs(**dev)
    g = np.random.default_rng(seed)
    pick = g.integers(-1, n, size=(rounds, b))
    arr = np.zeros((rounds, b, depth), np.int32)
    plen = np.zeros((rounds, b), np.int32)
    for r in range(rounds):
        for s_ in range(b):
            if pick[r, s_] >= 0:
                p = paths[pick[r, s_]]
                arr[r, s_, :len(p)] = p
                plen[r, s_] = len(p)
    arr_d = torch.from_numpy(arr).to("cuda")
    plen_d = torch.from_numpy(plen).to("cuda")
    out = torch.empty((n, b, H, d), dtype=torch.float32, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for fused in (False, True):
        L = R.Layer.gdn(b, H, d, d, cap)
        torch.cuda.synchronize()
        start.record()
        for r in range(rounds):
            if fused:
                R.rssm_verify_tree_commit(L, parent, inp, out, commit_len - 1)
            else:
                R.rssm_verify_tree(L, parent, inp, out)
            R.rssm_append_path(L, n, arr_d[r], plen_d[r], inp)
            if not fused:
                R.rssm_commit(L, None, commit_len)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        assert R.rssm_status(L) == 0
        del L
        r_ = dict(rounds_per_s=rounds / (ms * 1e-3),
                  accepted_seq_tok_s=float(plen.sum()) / (ms * 1e-3),
                  us_per_round=ms * 1e3 / rounds)
        if fused:
            res["fused_commit_at_7"] = r_
        else:
            res.update(r_, drafts_per_round=n)
    del dev
    torch.cuda.empty_cache()
    return res


# MFMA work of one 16-token prefill chunk of one head (fp32 16x16x4 products as
# executed): Mamba-2 C B^T, outputs h C^T + W X, fold X^T B; GDN K K^T, Q K^T,
# S K^T, S Q^T, T z, M u, fold.
PREFILL_CHUNK_FLOP = {
    "mamba2": 2 * 16 * 16 * 128 + 2 * 16 * 64 * 128 + 2 * 16 * 64 * 16 + 2 * 64 * 128 * 16,
    "gdn": 2 * (2 * 16 * 16 * 128) + 2 * (2 * 16 * 128 * 128) + 2 * (2 * 16 * 16 * 128)
           + 2 * 128 * 128 * 16,
}
MFMA_F32_PEAK_TFLOPS = 157.3


def run_prefill(torch, R, syn, kind, T=512, reps=5, seed=0, pool_n=64):
    """Prefill of a T-token prompt into every sequence's checkpoint at the
    headline decode shape of the layer type, every prompt token's output
    written.  Inputs: a device pool of pool_n synthetic tokens repeated to T
    (the kernels' cost does not depend on the values).  Per-launch HIP events;
    median of `reps` launches after one warmup."""
    b = 256
    if kind == "mamba2":
        H, G, P, N = 80, 8, 64, 128
        A, D = syn.m2_params(seed, H)
        pool = syn.m2_steps(seed, 0, pool_n, b, H, G, P, N)
        L = R.Layer.mamba2(b, H, G, P, N, 8)
        L.A.copy_(torch.from_numpy(A))
        L.D.copy_(torch.from_numpy(D))
        L.ckpt.copy_(_dev_state(torch, syn.m2_state0(seed, b, H, P, N)))
        names, out_name, dv, state_bytes = ("x", "B", "C", "dt"), "x", P, b * H * P * N * 4
    else:
        H, dk = 32, 128
        pool = syn.gdn_steps(seed, 0, pool_n, b, H, dk, dk)
        L = R.Layer.gdn(b, H, dk, dk, 8)
        names, out_name, dv, state_bytes = ("q", "k", "v", "alpha", "beta"), "v", dk, b * H * dk * dk * 4
    reps_t = T // pool_n
    dev = {k: torch.from_numpy(pool[k]).to("cuda").repeat((reps_t,) + (1,) * (pool[k].ndim - 1))
           for k in names}
    out = torch.empty_like(dev[out_name])
    inp = R.make_inputs(**dev)
    ev = []
    for i in range(reps + 1):
        a_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        R.rssm_prefill(L, T, inp, out)
        e_.record()
        ev.append((a_, e_))
    torch.cuda.synchronize()
    assert R.rssm_status(L) == 0
    ms = float(np.median([a_.elapsed_time(e_) for a_, e_ in ev[1:]]))
    flop = PREFILL_CHUNK_FLOP[kind] * (T // 16) * b * H
    in_bytes = sum(int(v.numel()) * 4 for v in dev.values())
    hbm = 2 * state_bytes + in_bytes + int(out.numel()) * 4
    tflops = flop / (ms * 1e-3) / 1e12
    res = dict(prompt_tokens=T, us_per_prefill=round(ms * 1e3, 1),
               seq_tok_s=round(b * T / (ms * 1e-3), 1),
               tflops=round(tflops, 1), mfma_f32_peak_tflops=MFMA_F32_PEAK_TFLOPS,
               mfma_frac=round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
               flop_per_launch=flop, hbm_bytes_per_launch=hbm,
               hbm_gbps=round(hbm / (ms * 1e-3) / 1e9, 1))
    del L, dev, out
    torch.cuda.empty_cache()
    return res


def run_dual_stack(torch, R, syn, steps, seed=0, layers=12, pool_n=8):
    """12 GDN layers at batch 256 with a low-precision serving checkpoint,
    commit every 8 steps; seq-tokens/s through the whole stack.  DUAL layers
    fold in the step that fills the interval (commit_after; that step reads
    fp32), also measured with the standalone commit (`*_standalone`) and with
    one set of buffer indices shared by the 12 layers (`*_shared_indices`:
    11 read-only layers, the last one moves the indices); SHARED layers commit
    standalone (the fused commit needs the fp32 checkpoint)."""
    b, H, d, interval, cap = 256, 32, 128, 8, 8
    pool = syn.gdn_steps(seed, 0, pool_n, b, H, d, d)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    names = ("q", "k", "v", "alpha", "beta")
    o = torch.empty((b, H, d), dtype=torch.float32, device="cuda")
    res = {}
    inputs = [R.make_inputs(**{s: dev[s][j] for s in names}) for j in range(pool_n)]
    for scheme, sname, fused in ((R.RSSM_DUAL, "dual", True),
                                 (R.RSSM_DUAL, "dual_shared_indices", True),
                                 (R.RSSM_DUAL, "dual_standalone", False),
                                 (R.RSSM_SHARED, "shared", False), (None, "eager_lp", False)):
        for lp, lname in ((R.RSSM_BF16, "bf16"), (R.RSSM_E4M3, "e4m3")):
            Ls = [R.Layer.gdn(b, H, d, d, cap, lp_dtype=lp,
                              scheme=R.RSSM_SHARED if scheme is None else scheme)
                  for _ in range(layers)]
            if scheme is not None:
                for L in Ls:
                    R.rssm_commit(L, None, 0)
            if sname == "dual_shared_indices":
                for L in Ls[:-1]:
                    L.share_indices(Ls[-1], readonly=True)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for t in range(steps):
                j = t % pool_n
                for L in Ls:
                    if scheme is None:        # eager comparator: the state lives in low precision
                        R.rssm_eager_step(L, inputs[j], o)
                        continue
                    boundary = (t + 1) % interval == 0
                    R.rssm_gdn_step(L, *(dev[s][j] for s in names), o,
                                    commit_after=fused and boundary)
                    if boundary and not fused:
                        R.rssm_commit(L, None, 0)
            end.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(end)
            for L in Ls:
                assert R.rssm_status(L) == 0
            key = {"dual_standalone": f"dual_{lname}_standalone",
                   "dual_shared_indices": f"dual_{lname}_shared_indices"}.get(sname,
                                                                          f"{sname}_{lname}")
            res[key] = b * steps / (ms * 1e-3)
            del Ls
            torch.cuda.empty_cache()
    return res


def eager_lp_rooflines(torch, R, syn, reps=20, seed=0):
    """Per-launch time and HBM fraction of the eager comparators that keep the
    state in low precision only (decode, update in fp32, re-encode every step)
    at the serving shapes.  Their arithmetic per state element (decode,
    update, the block maximum of the E4M3 scale, encode) is issued by the
    vector ALUs against one or two bytes of traffic, so they are bound by
    VALU issue, not by HBM: reported beside the dual/eager-lp throughputs so
    that those ratios can be read against comparators that are not at the
    memory roofline."""
    out = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for kind in ("gdn", "mamba2"):
        if kind == "gdn":
            b, H, d = 256, 32, 128
            st = syn.gdn_steps(seed, 0, 1, b, H, d, d)
            names, S, ins, outb = ("q", "k", "v", "alpha", "beta"), b * H * d * d, \
                (3 * b * H * d + 2 * b * H) * 4, b * H * d * 4
        else:
            b, H, G, P, N = 256, 80, 8, 64, 128
            st = syn.m2_steps(seed, 0, 1, b, H, G, P, N)
            names, S, ins, outb = ("x", "B", "C", "dt"), b * H * P * N, \
                (b * H * P + 2 * b * G * N + b * H) * 4, b * H * P * 4
        dev = {k: torch.from_numpy(v[0]).to("cuda") for k, v in st.items()}
        inp = R.make_inputs(**{k: dev[k] for k in names})
        for lp, lname, eb in ((R.RSSM_BF16, "bf16", 2), (R.RSSM_E4M3, "e4m3", 1)):
            if kind == "gdn":
                L = R.Layer.gdn(b, H, d, d, 8, scheme=R.RSSM_SHARED, lp_dtype=lp)
                o = torch.empty((b, H, d), dtype=torch.float32, device="cuda")
            else:
                L = R.Layer.mamba2(b, H, G, P, N, 8, scheme=R.RSSM_SHARED, lp_dtype=lp)
                o = torch.empty((b, H, P), dtype=torch.float32, device="cuda")
            for _ in range(3):
                R.rssm_eager_step(L, inp, o)
            torch.cuda.synchronize()
            ev[0].record()
            for _ in range(reps):
                R.rssm_eager_step(L, inp, o)
            ev[1].record()
            torch.cuda.synchronize()
            us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
            byt = 2 * S * eb + ins + outb + (2 * b * H * 4 if lp == R.RSSM_E4M3 else 0)
            out[f"{kind}_{lname}"] = dict(us_per_launch=round(us, 2), bytes_per_launch=byt,
                                          hbm_frac=round(byt / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 3))
            del L
        del dev
        torch.cuda.empty_cache()
    out["bound"] = "valu"
    out["note"] = ("eager comparators with the state in low precision only: VALU-bound (decode, "
                   "update, block amax, encode per state element), not tuned to the HBM roofline")
    return out


def run_m2_lowprec(torch, R, syn, steps, seed=0, pool_n=16):
    """Mamba-2 headline shape with a low-precision serving checkpoint (dual:
    fp32 receives the commits; shared: the copy is the only state) and the
    eager comparator whose state is stored in low precision; seq-tokens/s of
    one layer, commit every 8 steps (fused into the step for DUAL, also
    measured standalone; standalone for SHARED)."""
    b, H, G, P, N, interval = 256, 80, 8, 64, 128, 8
    A, D = syn.m2_params(seed, H)
    pool = syn.m2_steps(seed, 0, pool_n, b, H, G, P, N)
    dev = {k: torch.from_numpy(v).to("cuda") for k, v in pool.items()}
    h0 = _dev_state(torch, syn.m2_state0(seed, b, H, P, N))
    y = torch.empty((b, H, P), dtype=torch.float32, device="cuda")
    res = {}
    for scheme, sname, fused in ((R.RSSM_DUAL, "dual", True),
                                 (R.RSSM_DUAL, "dual_standalone", False),
                                 (R.RSSM_SHARED, "shared", False), (None, "eager_lp", False)):
        for lp, lname in ((R.RSSM_BF16, "bf16"), (R.RSSM_E4M3, "e4m3")):
            L = R.Layer.mamba2(b, H, G, P, N, interval,
                               scheme=R.RSSM_SHARED if scheme is None else scheme, lp_dtype=lp)
            L.A.copy_(torch.from_numpy(A))
            L.D.copy_(torch.from_numpy(D))
            if L.ckpt is not None:
                L.ckpt.copy_(h0)
                R.rssm_commit(L, None, 0)
            inputs = [R.make_inputs(x=dev["x"][j], B=dev["B"][j], C=dev["C"][j], dt=dev["dt"][j])
                      for j in range(pool_n)]

            def run(n):
                for t in range(n):
                    j = t % pool_n
                    if scheme is None:
                        R.rssm_eager_step(L, inputs[j], y)
                    else:
                        boundary = (t + 1) % interval == 0
                        R.rssm_mamba2_step(L, dev["x"][j], dev["B"][j], dev["C"][j], dev["dt"][j], y,
                                           commit_after=fused and boundary)
                        if boundary and not fused:
                            R.rssm_commit(L, None, 0)

            run(2 * interval)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = (steps // interval) * interval
            torch.cuda.synchronize()
            start.record()
            run(n)
            end.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(end)
            assert R.rssm_status(L) == 0
            key = {"dual_standalone": f"dual_{lname}_standalone",
                   "dual_shared_indices": f"dual_{lname}_shared_indices"}.get(sname,
                                                                          f"{sname}_{lname}")
            res[key] = round(b * n / (ms * 1e-3), 1)
            del L
            torch.cuda.empty_cache()
    del dev
    return res


def cpu_baseline(syn, target_s=12.0, seed=0):
    """The fp64 oracle's eager recurrence on a bounded sample of the headline
    workload: the full batch of 256 sequences x 80 heads, inputs cycling
    through 16 seeded steps, as many steps as fit in about target_s seconds."""
    import oracle
    b, H, G, P, N, pool = 256, 80, 8, 64, 128, 16
    A, D = syn.m2_params(seed, H)
    h = syn.m2_state0(seed, b, H, P, N).astype(np.float64)
    st = syn.m2_steps(seed, 0, pool, b, H, G, P, N)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.m2_eager(A, D, st["x"][:2], st["B"][:2], st["C"][:2], st["dt"][:2], h)
    per = (time.perf_counter() - t0) / 2
    n = int(max(pool, min(16384, target_s / max(per, 1e-9))))
    n = max(pool, (n // pool) * pool)     # whole passes over the input pool
    t0 = time.perf_counter()
    for _ in range(n // pool):
        oracle.m2_eager(A, D, st["x"], st["B"], st["C"], st["dt"], h)
    el = time.perf_counter() - t0
    # one host thread, for context: 2 sequences x 80 heads x 64 steps
    oracle.set_threads(1)
    h1 = h[:2].copy()
    sub = {k: np.ascontiguousarray(v[:, :2]) for k, v in st.items()}
    t1 = time.perf_counter()
    for _ in range(4):
        oracle.m2_eager(A, D, sub["x"], sub["B"], sub["C"], sub["dt"], h1)
    el1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    return {"value": round(b * n / el, 1), "unit": "seq-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 eager Mamba-2 recurrence (the oracle, OpenMP over units), "
                      f"{b} sequences x {H} heads x {n} steps of the batch-256 serving shape "
                      f"(P=64, N=128, G=8); {el:.1f} s on {threads} host threads",
            "value_1thread": round(2 * 4 * pool / el1, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated subset of the secondary workloads to run (gdn, spec, "
                         "gdn_spec, stack, sweep, lowprec, tree, prefill); default: all")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain device copy of 671,088,640 bytes (counter "
                         "calibration for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every (sequence, head) unit of the state engine is "
              "independent and the library drives one device, so this benchmark runs and reports "
              "a single MI355X only "
              "(--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_decode_replayssm_amd import rssm as R
    from linear_attention_decode_replayssm_amd import synthetic as syn
    R.lib()                                   # fail loudly if the HIP library is missing
    torch.cuda.init()
    # Python's cyclic collector stays off while anything is timed (as timeit
    # does): with torch loaded a full collection takes tens of milliseconds,
    # and one was seen to land inside a timed loop of short launches.  Cycles
    # are collected explicitly between workloads instead.
    gc.collect()
    gc.disable()

    if args.calib_copy:
        n = CALIB_COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    m2 = run_m2(torch, R, syn, args.steps, args.warmup)
    step_gbps = m2["step_bytes"] / (m2["step_us"] * 1e-6) / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        c = json.load(open(COUNTERS))
        if c.get("kernel_source_sha") == kernel_source_sha():
            traffic = c.get("hbm_bytes_per_launch")
    out = {
        "metric": METRIC,
        "value": round(m2["seq_tok_s"], 1),
        "unit": "seq-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m2["total_ms"] / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mamba2-decode-replay: 1 layer, batch 256, 80 heads, headdim 64, "
                               "dstate 128, 8 groups, fp32 checkpoint, commit every 8 tokens "
                               "(fused), ring 8",
                   "global_batch": 256, "seq_len": args.steps, "parallelism": "single-gpu"},
        "hbm_gbps": round(m2["all_bytes"] / (m2["total_ms"] * 1e-3) / 1e9, 1),
        "hbm_frac": round(m2["all_bytes"] / (m2["total_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "eager": {"value": round(m2["eager_seq_tok_s"], 1), "unit": "seq-tokens/s",
                  "us_per_step": round(m2["eager_us"], 2),
                  "hbm_gbps": round(m2["eager_gbps"], 1)},
        "speedup_vs_eager": round(m2["seq_tok_s"] / m2["eager_seq_tok_s"], 4),
        # `value` is the first timed region; the same K steps timed REPEATS more times
        "repeats": {"n": REPEATS,
                    "value": _spread(m2["rep_seq_tok_s"]),
                    "eager": _spread(m2["eager_rep_seq_tok_s"]),
                    "speedup_vs_eager_median": round(float(np.median(m2["rep_seq_tok_s"])) /
                                                     float(np.median(m2["eager_rep_seq_tok_s"])),
                                                     4)},
        "ckpt_bytes_per_step_vs_eager": round(m2["ckpt_bytes_per_step"] /
                                              m2["eager_ckpt_bytes_per_step"], 4),
        # what the pages report, end to end inside a serving engine on hardware
        # they do not name: context for the per-layer figures, not a target
        "pages_context": {
            "standard_decoding_vs_tuned_vllm_batch256": "1.20-1.47x (four hybrid models)",
            "vs_vllm_speculative_decoding": "~1.8x (two 120B-class models)"},
        "roofline": {"bound": "hbm", "kernel": "m2_step_kernel<4, false, 1, 0> (replay step, no commit)",
                     "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(step_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "avg_launch_us": round(m2["step_us"], 3),
                     "bytes_per_launch": int(m2["step_bytes"]),
                     "fused_commit_launch_us": round(m2["fused_us"], 3),
                     "timing": "hipEvents on the kernels' stream around the 7 back-to-back "
                               "plain steps of each commit interval, averaged per launch"},
    }
    out["stream_ceilings"] = stream_ceilings(torch, R)
    if not args.no_secondary:
        only = set(filter(None, args.only.split(",")))

        def want(name):
            gc.collect()   # between workloads, outside every timed region
            return not only or name in only
        sec = {}
        sec_steps = max(64, min(args.steps, 256))
        g = None
        if want("gdn"):
            g = run_gdn(torch, R, syn, sec_steps, 16)
            sec["gdn_decode_b256_h32_d128"] = {k: round(v, 2) for k, v in g.items()}
        if want("spec"):
            sec["mamba2_spec_rounds_b256_4drafts"] = _round1(run_spec(torch, R, syn, 128))
        if want("gdn_spec"):
            sec["gdn_spec_rounds_b256_4drafts"] = _round1(run_gdn_spec(torch, R, syn, 128))
        if want("stack"):
            du = run_dual_stack(torch, R, syn, 32)
            sec["gdn_12layer_stack_seq_tok_s"] = {k: round(v, 1) for k, v in du.items()}
            sec["eager_lp_comparators"] = eager_lp_rooflines(torch, R, syn)
        if want("sweep"):
            sec["mamba2_commit_interval_sweep"] = run_m2_interval_sweep(torch, R, syn, 256)
            sec["gdn_commit_interval_sweep"] = run_gdn_interval_sweep(torch, R, syn, 256)
        if want("lowprec"):
            sec["mamba2_lowprec_seq_tok_s"] = run_m2_lowprec(torch, R, syn, 128)
        if want("tree"):
            tr = run_tree_rounds(torch, R, syn, 128)
            sec["mamba2_tree_rounds_b256_7drafts"] = _round1(tr)
            gc.collect()
            sec["gdn_tree_rounds_b256_7drafts"] = _round1(run_gdn_tree_rounds(torch, R, syn, 128))
        if want("prefill"):
            pm = run_prefill(torch, R, syn, "mamba2")
            pg = run_prefill(torch, R, syn, "gdn")
            pm["speedup_vs_decode_steps"] = round(pm["seq_tok_s"] / out["value"], 2)
            if g is not None:
                pg["speedup_vs_decode_steps"] = round(pg["seq_tok_s"] / g["seq_tok_s"], 2)
            sec["mamba2_prefill_b256_512tok"] = pm
            sec["gdn_prefill_b256_512tok"] = pg
        out["secondary"] = sec
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(syn)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
