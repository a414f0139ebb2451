"""Helpers for GPU-vs-oracle parity checks (test infrastructure).

Selection rule (routing equation of section 3: I_i = the chunks of rank < K):
chunk ids must lie in [0, |C_i|), be strictly ascending and -1 padded, and
match the oracle exactly wherever the gap between the K-th and (K+1)-th group
scores exceeds TIE_BAND.  Inside the band a different choice is a valid top-K
only if it holds every chunk scoring above the oracle's K-th score + TIE_BAND
and nothing scoring below the K-th score - TIE_BAND; such rows are counted,
and their outputs are compared with the oracle re-run on the GPU's selection.

Outputs: bf16 max-abs 2e-2 against the fp64 oracle, plus, per head, the
largest error over the compared rows relative to that head's largest
reference magnitude (REL_BF16), so that a head whose outputs are small (1/sqrt(d)
scaled inputs) is still held to its own scale; fp32: max-abs error relative
to the largest reference magnitude, 1e-5.
"""
from __future__ import annotations

import numpy as np

from oracle import hils_oracle as O

TIE_BAND = 1e-4
TOL_BF16_ABS = 2e-2
TOL_F32_REL = 1e-5
# bf16 path: bf16 inputs are exact for the oracle; the kernels round the
# softmax weights fed to the matrix cores, the per-chunk outputs and the final
# output to bf16 (2^-9 relative each), so the error is a few 2^-9 of the
# output's own scale
REL_BF16 = 2e-2


def np32(t):
    """Exact float32 copy of a torch tensor (bf16 values are exact in float32)."""
    return t.detach().cpu().float().numpy()


def check_selection(gpu_sel, ref, K):
    """gpu_sel: int array [K] (-1 padded); ref: oracle row result for one group
    (needs 'sel', 'gap', 's_hat').  Returns 'exact', 'tie' or raises."""
    n = ref["s_hat"].shape[1]
    kk = min(K, n)
    got = np.asarray(gpu_sel).astype(np.int64)
    assert got.shape[0] == K, f"selection has {got.shape[0]} slots, expected {K}"
    assert np.all(got[kk:] == -1), f"padding wrong: {got}"
    got = got[:kk]
    assert np.all((got >= 0) & (got < n)), f"chunk id outside [0, {n}): {got}"
    assert np.all(np.diff(got) > 0), f"selection not strictly ascending: {got}"
    want = ref["sel"]
    if np.array_equal(got, want):
        return "exact"
    gap = ref["gap"]
    assert not (gap > TIE_BAND), f"selection differs outside the tie band (gap={gap}): {got} vs {want}"
    gs = O.ref_group_scores(ref["s_hat"])
    kth = np.sort(gs)[::-1][kk - 1]
    must = np.nonzero(gs > kth + TIE_BAND)[0]
    missing = np.setdiff1d(must, got)
    assert missing.size == 0, f"tie-band selection drops chunks clearly in the top-K: {missing}"
    assert np.all(gs[got] >= kth - TIE_BAND), "tie-band alternative holds a chunk below the K-th score"
    return "tie"


def out_error(got, want, dtype):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max()
    if dtype == "f32":
        return err / max(np.abs(want).max(), 1e-30), TOL_F32_REL
    return err, TOL_BF16_ABS


class Tally:
    """Counts of exact and tie-band rows, the largest output error, and per
    head the largest error and reference magnitude (for the relative view)."""

    def __init__(self):
        self.exact = 0
        self.tie = 0
        self.tie_checked = 0
        self.rows = 0
        self.max_err = 0.0
        self.tol = None
        self.head_err = {}
        self.head_ref = {}

    def add(self, key, got, want, dtype, what):
        err, tol = out_error(got, want, dtype)
        self.tol = tol
        self.max_err = max(self.max_err, err)
        assert err <= tol, f"output error {err} > {tol} at {what}"
        got = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
        want = np.asarray(want, np.float64).reshape(got.shape)
        for r in range(got.shape[0]):
            h = (key, r)
            self.head_err[h] = max(self.head_err.get(h, 0.0), float(np.abs(got[r] - want[r]).max()))
            self.head_ref[h] = max(self.head_ref.get(h, 0.0), float(np.abs(want[r]).max()))

    def max_rel(self):
        """Largest per-head error relative to that head's largest reference magnitude."""
        rel = [self.head_err[h] / self.head_ref[h] for h in self.head_err if self.head_ref[h] > 0]
        return max(rel) if rel else 0.0

    def check_rel(self, dtype):
        if dtype == "bf16":
            assert self.max_rel() <= REL_BF16, f"per-head relative error {self.max_rel()} > {REL_BF16}"

    def __repr__(self):
        return (f"rows={self.rows} sel_exact={self.exact} tie_band={self.tie} "
                f"(outputs re-checked on the GPU's selection: {self.tie_checked}) "
                f"max_err={self.max_err:.3g} tol={self.tol} max_rel_per_head={self.max_rel():.3g}")


def compare_prefill_rows(res, gpu_out, gpu_sel, rows, w, tally=None, rerun=None, head_key=0):
    """res: oracle results {(b,i): ...}; gpu_out [B,Hq,N,d] np; gpu_sel [B,Hkv,N,K] np.

    rerun(b, i, forced) -> oracle result of row (b, i) with the selections in
    `forced` ({(b, g, i): ids}) held fixed; used for every tie-band row."""
    t = tally or Tally()
    G = w.Hq // w.Hkv
    for (b, i) in rows:
        r = res[(b, i)]
        t.rows += 1
        ties = {}
        for g in range(w.Hkv):
            sub = dict(sel=r["sel"][g], gap=r["gap"][g], s_hat=r["s_hat"][g])
            kind = check_selection(gpu_sel[b, g, i], sub, w.K)
            hs = slice(g * G, (g + 1) * G)
            if kind == "exact":
                t.exact += 1
                t.add((head_key, b, g), gpu_out[b, hs, i], r["out"][hs], w.dtype, f"b={b} i={i} g={g}")
            else:
                t.tie += 1
                ties[g] = [int(c) for c in gpu_sel[b, g, i] if c >= 0]
        if ties:
            assert rerun is not None, "tie-band rows need the oracle re-run on the GPU's selection"
            rr = rerun(b, i, {(b, g, i): s for g, s in ties.items()})
            for g in ties:
                hs = slice(g * G, (g + 1) * G)
                assert list(rr["sel"][g]) == ties[g]
                t.add((head_key, b, g), gpu_out[b, hs, i], rr["out"][hs], w.dtype,
                      f"tie row b={b} i={i} g={g} (GPU selection)")
                t.tie_checked += 1
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
