"""The dual-precision Gated DeltaNet stack at full length and at the serving
shape: 12 independent layers x 4096 steps, batch 256 x 32 heads (dk = dv =
128), S_0 = 0, alpha = exp(-softplus(N(0,1))), beta = sigmoid(N(0,1)), q and k
unit-norm, v ~ N(0,1), fresh inputs every step; commit every 8 steps
(explainer, "Separate precisions for serving vs updating state": a
low-precision copy serves the output reads, only the fp32 checkpoint takes the
folds).  The batch holds 16 seeded sequences, each 16 times (sequence
c * 16 + b is a copy of sequence b): the kernels run the full batch-256 launch
shape, the fp64 oracle follows the 16 distinct sequences, and every copy's
outputs must equal its original's bit for bit (the sequences are independent
and each (sequence, head) is computed alone).

Every output vector of every scheme is compared with the fp64 oracle's eager
recurrence on the same inputs, e = ||o - o_exact||_inf / ||o_exact||_inf.

Gates:
* dual bf16 and dual E4M3, every step and every vector: the one-quantisation
  bound |o - o_exact| <= sum_j delta(S_c[r, j]) |q~_j| + 1e-4 ||o_exact||_inf,
  with S_c the exact checkpoint of the last commit, q~ the query carried back
  through the buffered entries (oracle.drivers.gdn_carry_batched) and delta the
  codec's half step (bf16: 2^-8 |s|; E4M3: max(2^-4 |s|, 2^-10 scale)): the
  rounding of one quantisation, never compounded by later folds.  The 1e-4
  term is the fp32 tolerance of the unquantised part; for the few vectors that
  exceed it, it is taken relative to the row-sum scale below (reading 31, as
  for the fp32 control: right after a commit of a zero state, for instance,
  the bound's quantisation term is 0 and the output is a cancelled fp32 dot
  product), and the report counts them;
* no upward drift of the dual schemes' mean error over the 512-step windows;
* the fp32 replay (control) within 1e-4 of every vector's scale, where the
  scale is ||o_exact||_inf or, for the rare vector whose output is far smaller
  than the terms it is summed from, the largest row sum sum_j |S_rj q_j| of
  the exact state (reading 31: an fp32 result is accurate relative to its
  terms, not to a cancelled sum).
The shared schemes are comparison schemes: reported, not gated.

One test per layer keeps each under half a minute; the last test pools the
layers, checks the drift and prints the report."""
import time

import numpy as np
import pytest

import oracle
from oracle import drivers
from linear_attention_decode_replayssm_amd import rssm as R
from linear_attention_decode_replayssm_amd import synthetic as syn
import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "alpha", "beta")
LAYERS, STEPS, B, H, D, INTERVAL, CHUNK, WINDOW = 12, 4096, 16, 32, 128, 8, 64, 512
REP = 16          # copies of the B distinct sequences: the launches run batch B * REP = 256
SCHEMES = [("dual-bf16", R.RSSM_DUAL, R.RSSM_BF16), ("shared-bf16", R.RSSM_SHARED, R.RSSM_BF16),
           ("dual-e4m3", R.RSSM_DUAL, R.RSSM_E4M3), ("shared-e4m3", R.RSSM_SHARED, R.RSSM_E4M3),
           ("fp32", R.RSSM_F32, R.RSSM_LP_NONE)]
NWIN = STEPS // WINDOW
_RESULTS = {}   # layer -> {scheme: (window error sums, max e)}, fp32 ill-conditioned list


class _Bounds:
    """One-quantisation bounds of one interval's steps: sum_j delta(Sc[u, r, j])
    |q~[u, j, t]| with the codec's half step delta at the exact checkpoint Sc
    [b,H,r,c] (bf16: 2^-8 |s|; E4M3: max(2^-4 |s|, 2^-10 scale), scale =
    amax / 448) and q~ [U, c, t] (float32 arithmetic: the bound is a
    tolerance).  The bf16 bound is 2^-8 |Sc| |q~|; for E4M3 the same product
    gives the lower bound max(2^-4 |Sc| |q~|, 2^-10 scale sum_j |q~_j|) of the
    exact bound, which is formed only for the units where an error exceeds
    that lower bound."""

    def __init__(self, Sc, qt):
        import torch
        self.a = torch.from_numpy(Sc.reshape(-1, D, D)).float().abs_()
        self.q = torch.from_numpy(np.abs(qt)).float()
        prod = torch.bmm(self.a, self.q)                                   # [U, r, t]
        amax = self.a.amax(dim=(1, 2))
        self.sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        low = torch.maximum(prod * 2.0 ** -4, (self.sc * 2.0 ** -10)[:, None, None] *
                            self.q.sum(1, keepdim=True))
        self.bf16 = self._tbhr(prod * 2.0 ** -8)
        self.e4m3_low = self._tbhr(low)

    @staticmethod
    def _tbhr(x):
        return x.numpy().astype(np.float64).reshape(B, H, D, -1).transpose(3, 0, 1, 2)

    def e4m3_exact(self, u):
        """The exact E4M3 bound of unit u (b * H + h): [t, r]."""
        import torch
        delta = torch.maximum(self.a[u] * 2.0 ** -4, self.sc[u] * 2.0 ** -10)
        return (delta @ self.q[u]).numpy().astype(np.float64).T


@pytest.mark.parametrize("layer", range(LAYERS))
def test_stack_layer_full_length(layer):
    t_ = gu.torch()
    t0 = time.time()
    S0 = syn.gdn_state0(0, B, H, D, D, layer=layer)
    S = S0.astype(np.float64)
    L = {}
    for n, scheme, lp in SCHEMES:
        L[n] = gu.gdn_layer(np.tile(S0, (REP, 1, 1, 1)), INTERVAL, scheme=scheme, lp=lp)
        if scheme == R.RSSM_DUAL:
            R.rssm_commit(L[n], None, 0)          # the copy starts as Q(S_0)
    esum = {n: np.zeros(NWIN) for n, _, _ in SCHEMES}
    emax = {n: 0.0 for n, _, _ in SCHEMES}
    margin = {"dual-bf16": -np.inf, "dual-e4m3": -np.inf}
    cancelled = {n: [] for n in margin}
    ill = []
    o = t_.empty((CHUNK, REP * B, H, D), dtype=t_.float32, device="cuda")
    o_rep = o.view(CHUNK, REP, B, H, D)
    U = B * H
    for c0 in range(0, STEPS, CHUNK):
        st = syn.gdn_steps(0, c0, CHUNK, B, H, D, D, layer=layer)
        # every input tiled over the batch: copy c of sequence b at c * B + b
        dv = {k: gu.dev(v).repeat(1, REP, *([1] * (v.ndim - 2))).contiguous()
              for k, v in st.items()}
        # exact outputs, the checkpoint at the start of every interval, and the
        # one-quantisation bound of each step
        o_exact = np.empty((CHUNK, B, H, D))
        bounds = []
        S_start = S.copy()
        for i0 in range(0, CHUNK, INTERVAL):
            sl = slice(i0, i0 + INTERVAL)
            Sc = S.copy()
            o_exact[sl] = oracle.gdn_eager(*(st[k][sl] for k in NAMES), S)
            qt = np.empty((U, D, INTERVAL))
            for j in range(INTERVAL):
                qt[:, :, j], _ = drivers.gdn_carry_batched(
                    st["q"][i0 + j].reshape(U, D),
                    st["k"][i0:i0 + j + 1].transpose(1, 2, 0, 3).reshape(U, -1, D),
                    st["alpha"][i0:i0 + j + 1].transpose(1, 2, 0).reshape(U, -1),
                    st["beta"][i0:i0 + j + 1].transpose(1, 2, 0).reshape(U, -1))
            bounds.append(_Bounds(Sc, qt))
        den = np.abs(o_exact).max(-1)
        slack = 1e-4 * den[..., None]
        for n, scheme, lp in SCHEMES:
            fused = scheme == R.RSSM_F32
            for i in range(CHUNK):
                commit = (c0 + i + 1) % INTERVAL == 0
                R.rssm_gdn_step(L[n], *(dv[k][i] for k in NAMES), o[i],
                                commit_after=fused and commit)
                if commit and not fused:
                    R.rssm_commit(L[n], None, 0)
            same = bool((o_rep == o_rep[:, :1]).all())
            assert same, (n, layer, c0, "a copy of a sequence differs from its original")
            err = np.abs(gu.host(o_rep[:, 0].contiguous()).astype(np.float64) - o_exact)
            e = err.max(-1) / den
            esum[n][c0 // WINDOW] += e.sum()
            emax[n] = max(emax[n], float(e.max()))
            if n in margin:
                over = _excess(n, err, slack, bounds)
                vec = over.max(-1) > 0
                if vec.any():      # reading 31: the fp32 slack of a cancelled sum
                    idx = np.argwhere(vec)
                    for (t, bb, hh), c in zip(idx, _row_sum_scales(st, S_start, idx, den)):
                        over[t, bb, hh] -= gu.TOL_F32 * (max(1.0, c) - 1.0) * den[t, bb, hh]
                        cancelled[n].append(c)
                margin[n] = max(margin[n], float((over / den[..., None]).max()))
                assert np.all(over <= 0), (n, layer, c0, np.unravel_index(np.argmax(over), over.shape))
            if fused and e.max() > gu.TOL_F32:
                idx = np.argwhere(e > gu.TOL_F32)
                ill.extend(zip(e[e > gu.TOL_F32].tolist(), _row_sum_scales(st, S_start, idx, den)))
    for n, _, _ in SCHEMES:
        assert R.rssm_status(L[n]) == 0
    for x, c in ill:                                  # reading 31, fp32 control only
        assert x <= gu.TOL_F32 * max(1.0, c), (layer, x, c)
    _RESULTS[layer] = ({n: (esum[n], emax[n]) for n in esum}, ill, margin, cancelled)
    del L
    t_.cuda.empty_cache()
    print(f"layer {layer}: {time.time() - t0:.0f} s; worst excess over the dual bound "
          f"(relative to ||o_exact||): bf16 {margin['dual-bf16']:.2e}, "
          f"e4m3 {margin['dual-e4m3']:.2e}", flush=True)


def _excess(n, err, slack, bounds):
    """err - bound - slack for every vector of a chunk ([t, b, H, r]); <= 0
    everywhere when the one-quantisation bound holds."""
    over = np.empty_like(err)
    for k, bd in enumerate(bounds):
        sl = slice(k * INTERVAL, (k + 1) * INTERVAL)
        if n == "dual-bf16":
            over[sl] = err[sl] - bd.bf16 - slack[sl]
            continue
        ov = err[sl] - bd.e4m3_low - slack[sl]
        for bb, hh in {(int(x[1]), int(x[2])) for x in np.argwhere(ov > 0)}:
            ov[:, bb, hh] = err[sl][:, bb, hh] - bd.e4m3_exact(bb * H + hh) - slack[sl][:, bb, hh]
        over[sl] = ov
    return over


def test_stack_pooled_drift_and_report():
    """Pooled over the layers: the dual schemes' mean error does not drift up
    across the 512-step windows (no compounding); the report gives every
    scheme's mean and max error, per-layer spread and window means."""
    if len(_RESULTS) != LAYERS:
        pytest.skip("needs every layer of test_stack_layer_full_length in this session")
    per = B * H * WINDOW
    lines, ill_all = [], []
    for n, _, _ in SCHEMES:
        es = np.array([_RESULTS[l][0][n][0] for l in range(LAYERS)])        # [layer, window]
        mx = max(_RESULTS[l][0][n][1] for l in range(LAYERS))
        wmean = es.sum(0) / (LAYERS * per)
        lmean = es.sum(1) / (NWIN * per)
        lines.append(f"{n:12s} mean e {es.sum() / (LAYERS * NWIN * per):.3e}  max e {mx:.3e}  "
                     f"per-layer mean {lmean.min():.3e}..{lmean.max():.3e}  per-512-step window "
                     + " ".join(f"{x:.2e}" for x in wmean))
        if n.startswith("dual"):
            assert wmean[-1] <= 1.2 * wmean[0], (n, wmean)
    for l in range(LAYERS):
        ill_all.extend(_RESULTS[l][1])
    worst = {n: max(_RESULTS[l][2][n] for l in range(LAYERS)) for n in ("dual-bf16", "dual-e4m3")}
    canc = {n: sum((_RESULTS[l][3][n] for l in range(LAYERS)), []) for n in worst}
    lines.append(f"dual one-quantisation bound held for all {LAYERS * STEPS * B * H} vectors; "
                 f"largest (error - bound - fp32 slack) / ||o||: bf16 {worst['dual-bf16']:.2e}, "
                 f"e4m3 {worst['dual-e4m3']:.2e}; vectors that needed the row-sum slack "
                 f"(reading 31): bf16 {len(canc['dual-bf16'])}, e4m3 {len(canc['dual-e4m3'])}, "
                 f"largest row-sum / ||o||: "
                 + " ".join(f"{max(canc[n], default=0):.1f}" for n in worst))
    lines.append(f"fp32 vectors above 1e-4 of ||o_exact||_inf: {len(ill_all)} of "
                 f"{LAYERS * STEPS * B * H}; (e, sum_j |S_rj q_j| / ||o_exact||_inf): "
                 + " ".join(f"({x:.2e}, {c:.1f})" for x, c in sorted(ill_all)[-8:]))
    print("\nGDN stack, 12 layers x 4096 steps, batch 256 (16 sequences x 16 copies) x 32 "
          "heads:\n" + "\n".join(lines), flush=True)


def _row_sum_scales(st, S_start, idx, den):
    """For the vectors idx ([k, 3] rows of (step, b, h) within a chunk): step
    the oracle from the chunk's start state to each step and return max_r
    sum_j |S_rj q_j| / ||o_exact||_inf, S being the exact state the output
    reads: the size of the terms an fp32 output is summed from, relative to
    the output."""
    out = {}
    S = S_start.copy()
    last = int(idx[:, 0].max())
    for i in range(last + 1):
        oracle.gdn_eager(*(st[k][i:i + 1] for k in NAMES), S)
        for t, bb, hh in idx[idx[:, 0] == i]:
            scale = (np.abs(S[bb, hh]) @ np.abs(st["q"][i, bb, hh].astype(np.float64))).max()
            out[(int(t), int(bb), int(hh))] = float(scale / den[t, bb, hh])
    return [out[(int(t), int(bb), int(hh))] for t, bb, hh in idx]
