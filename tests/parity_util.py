"""Helpers for GPU-vs-oracle parity checks (test infrastructure).

Selection rule: chunk ids must match the oracle exactly wherever the gap
between the K-th and (K+1)-th group scores exceeds TIE_BAND; inside the band a
different choice is accepted only if every chosen chunk scores within
TIE_BAND of the oracle's K-th score (several selections are then correct),
and such rows are counted and reported.  Outputs are compared on every row
whose selection matches the oracle's (bf16: max-abs 2e-2; fp32: max-abs error
relative to the largest reference magnitude, 1e-5).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import hils_oracle as O

TIE_BAND = 1e-4
TOL_BF16_ABS = 2e-2
TOL_F32_REL = 1e-5


def np32(t):
    """Exact float32 copy of a torch tensor (bf16 values are exact in float32)."""
    return t.detach().cpu().float().numpy()


def check_selection(gpu_sel, ref, K):
    """gpu_sel: int array [K] (-1 padded); ref: oracle row result for one group
    (needs 'sel', 'gap', 's_hat').  Returns 'exact', 'tie' or raises."""
    n = ref["s_hat"].shape[1]
    kk = min(K, n)
    got = np.asarray(gpu_sel)
    assert np.all(got[kk:] == -1), f"padding wrong: {got}"
    got = got[:kk]
    assert np.all(np.diff(got) > 0), f"selection not strictly ascending: {got}"
    want = ref["sel"]
    if np.array_equal(got, want):
        return "exact"
    gap = ref["gap"]
    assert not (gap > TIE_BAND), f"selection differs outside the tie band (gap={gap}): {got} vs {want}"
    gs = O.ref_group_scores(ref["s_hat"])
    kth = np.sort(gs)[::-1][kk - 1]
    assert np.all(gs[got] >= kth - TIE_BAND), "tie-band alternative is not a valid top-K"
    return "tie"


def out_error(got, want, dtype):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max()
    if dtype == "f32":
        return err / max(np.abs(want).max(), 1e-30), TOL_F32_REL
    return err, TOL_BF16_ABS


class Tally:
    def __init__(self):
        self.exact = 0
        self.tie = 0
        self.rows = 0
        self.max_err = 0.0
        self.tol = None

    def __repr__(self):
        return (f"rows={self.rows} sel_exact={self.exact} tie_band={self.tie} "
                f"max_err={self.max_err:.3g} tol={self.tol}")


def compare_prefill_rows(res, gpu_out, gpu_sel, rows, w, tally=None):
    """res: oracle results {(b,i): ...}; gpu_out [B,Hq,N,d] np; gpu_sel [B,Hkv,N,K] np."""
    t = tally or Tally()
    G = w.Hq // w.Hkv
    for (b, i) in rows:
        r = res[(b, i)]
        t.rows += 1
        for g in range(w.Hkv):
            sub = dict(sel=r["sel"][g], gap=r["gap"][g], s_hat=r["s_hat"][g])
            kind = check_selection(gpu_sel[b, g, i], sub, w.K)
            if kind == "exact":
                t.exact += 1
                hs = slice(g * G, (g + 1) * G)
                err, tol = out_error(gpu_out[b, hs, i], r["out"][hs], w.dtype)
                t.tol = tol
                t.max_err = max(t.max_err, err)
                assert err <= tol, f"output error {err} > {tol} at b={b} i={i} g={g}"
            else:
                t.tie += 1
    return t


def sample_rows(w, count, seed=0, include=()):
    """Query rows spanning the sequence: the first rows with candidates, the
    last row, chunk boundaries and random rows."""
    rng = np.random.default_rng(seed)
    first = w.W + w.S - 1
    base = {0, 1, min(first - 1, w.N - 1), min(first, w.N - 1), w.N - 1,
            min(first + w.S, w.N - 1), min(w.N - 1, (w.N // 2) // w.S * w.S),
            min(w.N - 1, (w.N // 2) // w.S * w.S - 1)}
    base |= set(int(x) for x in include)
    extra = rng.integers(0, w.N, size=max(0, count - len(base)))
    rows = sorted(base | set(int(x) for x in extra))
    return [(b, i) for b in range(w.B) for i in rows if 0 <= i < w.N]
