"""Test oracle for the HiLS attention forward pass (prefill rows and single-step decode).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
shares no code with it.

This is a plain, slow, obviously-correct NumPy float64 restatement of the
definitions in "Hierarchical Sparse Attention Done Right: Toward Infinite
Context Modeling" (Hu et al., arXiv 2607.02980; cited below as "HiLS paper").
Citations name the section / equation of that paper.  Every array is float64;
inputs are the exact values of the (bf16- or fp32-) tensors handed to the GPU.

Notation (0-based tokens and chunks):
  S chunk size, W window size, K top-K, tau = 1/sqrt(d) unless given,
  c(j) = floor(j/S), l(i) = floor((i-W+1)/S)*S, C_i = {0..l(i)/S-1},
  window = [max(0,l(i)), i].
GQA: q heads h = g*G + r share KV head g (G = Hq/Hkv).

Readings of points the paper leaves open:
  * chunks/tokens are 0-based; l(i) uses floor division (negative numerators
    round toward -inf); C_i is empty when l(i) <= 0 and the window starts at 0;
  * |C_i| < K selects all of C_i; equal scores rank the lower chunk id first;
  * GQA "normalised chunk weights" = per-head softmax over C_i of the scores
    (the window mass excluded), max over the heads of a group, then top-K;
    with G = 1 the raw score is ranked directly (same order);
  * the landmark tensor holds one landmark *query* q'_c per chunk per query
    head; the summary is Attn(q'_c, K_c, K_c) over the S chunk tokens only;
  * the routing query q_hat (low-rank query calibration) enters only the
    chunk scores; token logits use q;
  * the summary key k'_c is stored in the input dtype (bf16 rounding by
    round-to-nearest-even from the exact value) and b'_c in fp32; scores use
    the stored values.  This is the summary cache's boundary format.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

__all__ = [
    "bf16_round", "f32_round", "store_round", "window_left", "n_candidates",
    "ref_summarize", "ref_chunk_scores", "ref_exact_logz", "ref_group_scores", "ref_decode_multi", "ref_backward",
    "ref_select", "ref_row", "ref_prefill_rows", "ref_decode",
    "ref_full_causal", "ref_naive_bsa", "ref_overlap", "ref_brute_force_mass_topk",
]

# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's 8-bit
    exponent.  Rounding is done directly from the float64 value (a single
    rounding), so it never double-rounds through fp32.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    mant, expo = np.frexp(xf)            # xf = mant * 2**expo, 0.5 <= |mant| < 1
    # normal bf16 range: |x| >= 2**-126  <=>  expo >= -125
    normal = expo >= -125
    r = np.empty_like(xf)
    # 8 significant bits: scale mantissa to [128, 256), round half to even
    r[normal] = np.ldexp(np.round(np.ldexp(mant[normal], 8)), expo[normal] - 8)
    # subnormal bf16: fixed spacing 2**-133
    sub = ~normal
    r[sub] = np.ldexp(np.round(np.ldexp(xf[sub], 133)), -133)
    # overflow: beyond the largest finite bf16 rounds to inf
    big = np.abs(r) >= 2.0 ** 128
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    return out


def f32_round(x) -> np.ndarray:
    """Round float64 to the nearest fp32 (IEEE default rounding), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def store_round(x, fmt: str) -> np.ndarray:
    """Round to a storage format: 'bf16', 'f32' or 'f64' (no rounding)."""
    if fmt == "bf16":
        return bf16_round(x)
    if fmt == "f32":
        return f32_round(x)
    if fmt == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# index sets (HiLS paper, section 2.1)
# ---------------------------------------------------------------------------

def window_left(i: int, W: int, S: int) -> int:
    """Aligned window boundary l(i) = floor((i - W + 1)/S) * S  (section 2.1)."""
    return ((i - W + 1) // S) * S          # Python // is floor division


def n_candidates(i: int, W: int, S: int) -> int:
    """|C_i| with C_i = {0, ..., l(i)/S - 1}; empty when l(i) <= 0 (section 2.1)."""
    return max(0, window_left(i, W, S) // S)


def _window_start(i: int, W: int, S: int) -> int:
    return max(0, window_left(i, W, S))


def _lse(x, axis=-1):
    m = np.max(x, axis=axis, keepdims=True)
    return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))


# ---------------------------------------------------------------------------
# chunk summaries (HiLS paper, section 3, Proposition 3.1 and the landmark text)
# ---------------------------------------------------------------------------

def ref_summarize(k, lm, S, scale=None, mode="surrogate", store="bf16"):
    """Landmark chunk summaries (k'_c, b'_c) for every complete chunk.

    k  : [B, Hkv, N, d]  keys
    lm : [B, Hq, nC, d]  landmark queries q'_c (nC = floor(N/S))
    For mode 'surrogate' (Proposition 3.1, section 3):
        p_j   = softmax_{j in T_c}(q'_c . k_j * scale)
        k'_c  = sum_j p_j k_j              (= Attn(q'_c, K_c, K_c))
        b'_c  = -sum_j p_j log p_j         (entropy of p, natural log)
    For mode 'landmark_key' (ablation "w/o Prop. 3.1", Table 5): the landmark
        row itself is the routing key and b'_c = 0.
    For mode 'mean_pool' (section 2.2 mean-pooled key; ablation "w/ mean
        pooling", Table 5): k'_c = (1/S) sum_j k_j and b'_c = ln S, i.e. the
        Proposition 3.1 summary of a landmark query equal to zero (uniform p),
        so s_hat is the mean logit plus the log-mass of a uniform chunk.
    Returns (ks [B,Hq,nC,d] rounded to `store`, bs [B,Hq,nC] rounded to fp32;
    with store='f64' neither is rounded).
    """
    k = np.asarray(k)
    lm = np.asarray(lm)
    B, Hkv, N, d = k.shape
    Hq, nC = lm.shape[1], lm.shape[2]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    ks = np.zeros((B, Hq, nC, d))
    bs = np.zeros((B, Hq, nC))
    if mode == "landmark_key":
        return store_round(lm.astype(np.float64), store), bs
    if mode == "mean_pool":
        for b in range(B):
            for h in range(Hq):
                kc = k[b, h // G, : nC * S].reshape(nC, S, d).astype(np.float64)
                ks[b, h] = kc.sum(axis=1) / S
        bs[:] = math.log(S)
        return store_round(ks, store), (bs if store == "f64" else f32_round(bs))
    if mode != "surrogate":
        raise ValueError(mode)
    for b in range(B):
        for h in range(Hq):
            kc = k[b, h // G, : nC * S].reshape(nC, S, d).astype(np.float64)
            t = tau * np.einsum("cd,csd->cs", lm[b, h].astype(np.float64), kc)
            t = t - t.max(axis=1, keepdims=True)
            e = np.exp(t)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            logp = t - np.log(z)               # finite even where p underflows
            ks[b, h] = np.einsum("cs,csd->cd", p, kc)
            bs[b, h] = -(p * logp).sum(axis=1)
    return store_round(ks, store), (bs if store == "f64" else f32_round(bs))


# ---------------------------------------------------------------------------
# routing (section 3 routing equation; section 4.1 query calibration and GQA)
# ---------------------------------------------------------------------------

def ref_chunk_scores(qr_rows, ks, bs, n, scale):
    """Surrogate scores s_hat[h, c] = scale * q_hat_h . k'_{h,c} + b'_{h,c} for c < n.

    qr_rows : [G, d] routing queries of the G heads of one group at one position
    ks, bs  : [G, nC, d], [G, nC] summaries of those heads
    """
    return scale * np.einsum("hd,hcd->hc", qr_rows, ks[:, :n]) + bs[:, :n]


def ref_exact_logz(q_rows, kg, n, S, scale):
    """Exact chunk log-masses log Z_{i,c} = log sum_{j in T_c} exp(s_ij), c < n (section 2.1)."""
    if n == 0:
        return np.zeros((q_rows.shape[0], 0))
    s = scale * np.einsum("hd,jd->hj", q_rows, kg[: n * S].astype(np.float64))
    return _lse(s.reshape(q_rows.shape[0], n, S), axis=2)


def ref_group_scores(s_hat):
    """Group-level chunk score for GQA shared selection (section 4.1).

    G == 1: the raw score.  G > 1: per head, the log of the softmax over the
    candidate chunks (s_hat - LSE_c s_hat), then the maximum over the heads.
    """
    if s_hat.shape[0] == 1 or s_hat.shape[1] == 0:
        return s_hat[0].copy()
    L = _lse(s_hat, axis=1)
    return np.max(s_hat - L[:, None], axis=0)


def ref_select(gscore, K):
    """Top-K by (score descending, chunk id ascending)  (section 3, rank_down(s) < K).

    Returns (sel ascending int array of min(K, n) ids, gap) where gap is the
    difference between the K-th and (K+1)-th ranked scores (inf if n <= K).
    """
    n = gscore.shape[0]
    order = np.lexsort((np.arange(n), -gscore))
    kk = min(K, n)
    sel = np.sort(order[:kk])
    gap = float(gscore[order[K - 1]] - gscore[order[K]]) if n > K else math.inf
    return sel, gap


# ---------------------------------------------------------------------------
# one query position, all heads of one KV group
# ---------------------------------------------------------------------------

def ref_row(q, k, v, i, S, W, K, scale, s_hat_fn, forced_sel=None, want_weights=False):
    """HiLS output for one position i and the G heads of one KV group.

    q      : [G, d] token queries at position i
    k, v   : [N', d] keys/values of the group (at least i+1 rows)
    s_hat_fn(n) -> [G, n] fusion/routing logits of the candidate chunks
    Steps (HiLS paper section 3, hierarchical-softmax equation):
      window softmax over [max(0,l(i)), i] -> o_swa, log Z_swa;
      top-K of the group scores over C_i;
      per selected chunk an independent softmax over its S tokens -> o_c;
      chunk-level softmax over {s_hat_c : c selected} U {log Z_swa}, whose
      weights mix o_c and o_swa (Z_hat_{c(j)} = Z_swa on window tokens).
    Returns dict(out [G,d], sel, gap, s_hat [G,n], logz_swa [G], weights [G,i+1]?).
    """
    G, d = q.shape
    n = n_candidates(i, W, S)
    w0 = _window_start(i, W, S)
    s_hat = s_hat_fn(n)
    if forced_sel is None:
        sel, gap = ref_select(ref_group_scores(s_hat), K)
    else:
        sel, gap = np.asarray(forced_sel, dtype=np.int64), math.nan
    out = np.zeros((G, d))
    logz_swa = np.zeros(G)
    weights = np.zeros((G, i + 1)) if want_weights else None
    kw, vw = k[w0: i + 1].astype(np.float64), v[w0: i + 1].astype(np.float64)
    for r in range(G):
        sw = scale * (kw @ q[r])
        m = sw.max()
        ew = np.exp(sw - m)
        zw = ew.sum()
        o_sw = (ew @ vw) / zw
        logz_swa[r] = m + math.log(zw)
        lam = np.concatenate([s_hat[r, sel], [logz_swa[r]]])
        lam_max = lam.max()
        a = np.exp(lam - lam_max)
        a = a / a.sum()
        acc = a[-1] * o_sw
        if want_weights:
            weights[r, w0: i + 1] = a[-1] * ew / zw
        for t, c in enumerate(sel):
            kc = k[c * S:(c + 1) * S].astype(np.float64)
            vc = v[c * S:(c + 1) * S].astype(np.float64)
            sc = scale * (kc @ q[r])
            ec = np.exp(sc - sc.max())
            zc = ec.sum()
            acc = acc + a[t] * ((ec @ vc) / zc)
            if want_weights:
                weights[r, c * S:(c + 1) * S] = a[t] * ec / zc
        out[r] = acc
    res = dict(out=out, sel=sel, gap=gap, s_hat=s_hat, logz_swa=logz_swa, n=n)
    if want_weights:
        res["weights"] = weights
    return res


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _arr(x):
    """Keep float32/float64 input arrays as they are (bf16 and fp32 values are exact
    in float32); every slice is upcast to float64 before any arithmetic."""
    return None if x is None else np.asarray(x)


def ref_prefill_rows(q, k, v, lm, rows, S, W, K, q_route=None, scale=None,
                     mode="surrogate", store="bf16", summaries=None,
                     forced_sel=None, want_weights=False):
    """HiLS prefill outputs for a subset of query rows.

    q [B,Hq,N,d], k/v [B,Hkv,N,d], lm [B,Hq,nC,d] (unused in 'exact' mode),
    rows: iterable of (b, i).  mode: 'surrogate' | 'landmark_key' | 'mean_pool' | 'exact'.
    summaries: optional precomputed (ks, bs) from ref_summarize.
    forced_sel: optional dict {(b, g, i): sel} to evaluate a given selection.
    Returns dict keyed by (b, i) -> dict(out [Hq,d], sel {g: ids}, gap {g: gap}, ...).
    """
    q, k, v, lm, q_route = map(_arr, (q, k, v, lm, q_route))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    qr = q if q_route is None else q_route
    if mode != "exact" and summaries is None:
        summaries = ref_summarize(k, lm, S, tau, mode=mode, store=store)
    results = {}
    for (b, i) in rows:
        out = np.zeros((Hq, d))
        sels, gaps, shats, lzs, wts = {}, {}, {}, {}, {}
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            kg, vg = k[b, g], v[b, g]
            qrow = q[b, hs, i].astype(np.float64)
            if mode == "exact":
                fn = (lambda n, qq=qrow, kk=kg: ref_exact_logz(qq, kk, n, S, tau))
            else:
                ks, bs = summaries
                fn = (lambda n, qq=qr[b, hs, i].astype(np.float64), kk=ks[b, hs], bb=bs[b, hs]:
                      ref_chunk_scores(qq, kk, bb, n, tau))
            fs = None if forced_sel is None else forced_sel.get((b, g, i))
            r = ref_row(qrow, kg, vg, i, S, W, K, tau, fn, forced_sel=fs,
                        want_weights=want_weights)
            out[hs] = r["out"]
            sels[g], gaps[g], shats[g], lzs[g] = r["sel"], r["gap"], r["s_hat"], r["logz_swa"]
            if want_weights:
                wts[g] = r["weights"]
        res = dict(out=out, sel=sels, gap=gaps, s_hat=shats, logz_swa=lzs,
                   n=n_candidates(i, W, S))
        if want_weights:
            res["weights"] = wts
        results[(b, i)] = res
    return results


def ref_decode(q, k_cache, v_cache, seqlen, lm, S, W, K, q_route=None, scale=None,
               mode="surrogate", store="bf16", forced_sel=None):
    """Single-step decode: the new token is already in the cache, i = T_b - 1.

    q [B,Hq,d] (or [B,Hq,1,d]); k_cache/v_cache [B,Hkv,T,d]; seqlen [B];
    lm [B,Hq,>=floor(max T/S),d].  Summaries are computed here from the cache
    (same definition as prefill); only chunks c < |C_i| are scored.
    Returns dict b -> dict(out [Hq,d], sel {g: ids}, gap {g: gap}, ...).
    """
    q = np.asarray(q, np.float64)
    if q.ndim == 4:
        q = q[:, :, 0]
    qr = q if q_route is None else np.asarray(q_route, np.float64).reshape(q.shape)
    k_cache, v_cache = _arr(k_cache), _arr(v_cache)
    lm = _arr(lm)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    results = {}
    for b in range(B):
        T = int(seqlen[b])
        i = T - 1
        n = n_candidates(i, W, S)
        out = np.zeros((Hq, d))
        sels, gaps = {}, {}
        summ = None
        if mode != "exact" and n > 0:
            summ = ref_summarize(k_cache[b:b + 1, :, : n * S], lm[b:b + 1, :, :n], S, tau,
                                 mode=mode, store=store)
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            kg, vg = k_cache[b, g, :T], v_cache[b, g, :T]
            if mode == "exact":
                fn = (lambda nn, qq=q[b, hs], kk=kg: ref_exact_logz(qq, kk, nn, S, tau))
            elif n == 0:
                fn = (lambda nn: np.zeros((G, 0)))
            else:
                ks, bs = summ
                fn = (lambda nn, qq=qr[b, hs], kk=ks[0, hs], bb=bs[0, hs]:
                      ref_chunk_scores(qq, kk, bb, nn, tau))
            fs = None if forced_sel is None else forced_sel.get((b, g))
            r = ref_row(q[b, hs], kg, vg, i, S, W, K, tau, fn, forced_sel=fs)
            out[hs] = r["out"]
            sels[g], gaps[g] = r["sel"], r["gap"]
        results[b] = dict(out=out, sel=sels, gap=gaps, n=n)
    return results


def ref_decode_multi(q, k_cache, v_cache, seqlen, lm, S, W, K, q_route=None, scale=None,
                     mode="surrogate", store="bf16"):
    """Decode of a block of M new tokens per sequence, all already in the cache.

    Token m of sequence b sits at position i = T_b - M + m (evaluated at 0 if
    that is negative) and is computed exactly as the prefill row i (section 3:
    its own window [max(0, l(i)), i], its own candidates C_i, so the block is
    causal among its tokens).  q [B,Hq,M,d]; k_cache/v_cache [B,Hkv,T,d];
    seqlen [B]; lm [B,Hq,>=floor(max T/S),d].  Summaries come from the cache as
    in ref_decode.  Returns dict (b, m) -> dict(out [Hq,d], sel {g: ids},
    gap {g: gap}, s_hat {g: [G,n]}, n).
    """
    q = np.asarray(q, np.float64)
    B, Hq, M, d = q.shape
    qr = q if q_route is None else np.asarray(q_route, np.float64).reshape(q.shape)
    k_cache, v_cache, lm = _arr(k_cache), _arr(v_cache), _arr(lm)
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    results = {}
    for b in range(B):
        T = int(seqlen[b])
        pos = [max(T - M + m, 0) for m in range(M)]
        n_top = max(n_candidates(i, W, S) for i in pos)
        summ = None
        if mode != "exact" and n_top > 0:
            summ = ref_summarize(k_cache[b:b + 1, :, : n_top * S], lm[b:b + 1, :, :n_top], S, tau,
                                 mode=mode, store=store)
        for m, i in enumerate(pos):
            n = n_candidates(i, W, S)
            out = np.zeros((Hq, d))
            sels, gaps, shats = {}, {}, {}
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                kg, vg = k_cache[b, g, : i + 1], v_cache[b, g, : i + 1]
                if mode == "exact":
                    fn = (lambda nn, qq=q[b, hs, m], kk=kg: ref_exact_logz(qq, kk, nn, S, tau))
                elif n == 0:
                    fn = (lambda nn: np.zeros((G, 0)))
                else:
                    ks, bs = summ
                    fn = (lambda nn, qq=qr[b, hs, m], kk=ks[0, hs], bb=bs[0, hs]:
                          ref_chunk_scores(qq, kk, bb, nn, tau))
                r = ref_row(q[b, hs, m], kg, vg, i, S, W, K, tau, fn)
                out[hs] = r["out"]
                sels[g], gaps[g], shats[g] = r["sel"], r["gap"], r["s_hat"]
            results[(b, m)] = dict(out=out, sel=sels, gap=gaps, s_hat=shats, n=n)
    return results


def ref_backward(q, k, v, lm, dout, S, W, K, q_route=None, scale=None, sel=None,
                 mode="surrogate", store="bf16", rows=None):
    """Gradients of L = sum(dout * out) for the HiLS prefill of every position.

    The top-K selection is a discrete choice and is held fixed (given as `sel`
    [B,Hkv,N,K], -1 padded, or computed by the forward); every other step of
    section 3 is differentiated exactly:
      out = sum_c alpha_c o_c + alpha_w o_w, alpha = softmax({s_hat_c} U {log Z_swa});
      o_c = softmax_j(tau q.k_j) V over chunk c;  o_w, log Z_swa over the window;
      s_hat_c = tau q_hat.k'_c + b'_c  (section 3 routing equation);
      k'_c = sum_j pi_j k_j, b'_c = -sum_j pi_j log pi_j, pi = softmax_j(tau q'_c.k_j)
      (Proposition 3.1);  'landmark_key': k'_c = q'_c, b'_c = 0;
      'mean_pool': k'_c = mean_j k_j, b'_c = ln S.
    The stored (rounded per `store`) summaries enter s_hat as in the forward;
    their rounding is not differentiated.  Returns dict(dq, dk, dv, dlm,
    dq_route (None without q_route), sel).

    `rows` (a set of (b, g, i)), when given, keeps only those query rows'
    terms: dq of a listed row is then exact, and so are dk, dv of a key (and
    dlm of a chunk) all of whose attending rows (window and selecting) are
    listed; everything else is partial.
    """
    q, k, v, lm, dout, q_route = map(_arr, (q, k, v, lm, dout, q_route))
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nC = N // S
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    qr = q if q_route is None else q_route
    q64, k64, v64, lm64, do64, qr64 = (x.astype(np.float64) for x in (q, k, v, lm, dout, qr))
    ks, bs = ref_summarize(k, lm, S, tau, mode=mode, store=store)
    if sel is None:
        res = ref_prefill_rows(q, k, v, lm, [(b, i) for b in range(B) for i in range(N)], S, W,
                               K, q_route=q_route, scale=scale, mode=mode, store=store,
                               summaries=(ks, bs))
        sel = -np.ones((B, Hkv, N, K), dtype=np.int64)
        for (b, i), r in res.items():
            for g in range(Hkv):
                sel[b, g, i, :len(r["sel"][g])] = r["sel"][g]
    sel = np.asarray(sel)
    dq, dqr = np.zeros_like(q64), np.zeros_like(q64)
    dk, dv = np.zeros_like(k64), np.zeros_like(v64)
    dks, dbs = np.zeros((B, Hq, nC, d)), np.zeros((B, Hq, nC))
    for b in range(B):
        for g in range(Hkv):
            for i in range(N):
                if rows is not None and (b, g, i) not in rows:
                    continue
                w0 = _window_start(i, W, S)
                chunks = [int(c) for c in sel[b, g, i] if c >= 0]
                kw, vw = k64[b, g, w0:i + 1], v64[b, g, w0:i + 1]
                for r in range(G):
                    h = g * G + r
                    qi, qh, go = q64[b, h, i], qr64[b, h, i], do64[b, h, i]
                    sw = tau * (kw @ qi)
                    lzw = _lse(sw)
                    pw = np.exp(sw - lzw)
                    ow = pw @ vw
                    pcs, ocs, lam = [], [], []
                    for c in chunks:
                        kc, vc = k64[b, g, c * S:(c + 1) * S], v64[b, g, c * S:(c + 1) * S]
                        sc = tau * (kc @ qi)
                        pc = np.exp(sc - _lse(sc))
                        pcs.append(pc)
                        ocs.append(pc @ vc)
                        lam.append(tau * (qh @ ks[b, h, c]) + bs[b, h, c])
                    logits = np.array(lam + [lzw])
                    alpha = np.exp(logits - _lse(logits))
                    out = sum(alpha[t] * ocs[t] for t in range(len(chunks))) + alpha[-1] * ow
                    gbar = go @ out
                    gw = go @ ow
                    dlzw = alpha[-1] * (gw - gbar)
                    # window: through o_w and log Z_swa
                    dsw = alpha[-1] * pw * (vw @ go - gw) + dlzw * pw
                    dq[b, h, i] += tau * (dsw @ kw)
                    dk[b, g, w0:i + 1] += tau * np.outer(dsw, qi)
                    dv[b, g, w0:i + 1] += alpha[-1] * np.outer(pw, go)
                    dqh = np.zeros(d)
                    for t, c in enumerate(chunks):
                        kc, vc = k64[b, g, c * S:(c + 1) * S], v64[b, g, c * S:(c + 1) * S]
                        gc = go @ ocs[t]
                        dlam = alpha[t] * (gc - gbar)
                        ds = alpha[t] * pcs[t] * (vc @ go - gc)
                        dq[b, h, i] += tau * (ds @ kc)
                        dk[b, g, c * S:(c + 1) * S] += tau * np.outer(ds, qi)
                        dv[b, g, c * S:(c + 1) * S] += alpha[t] * np.outer(pcs[t], go)
                        dqh += tau * dlam * ks[b, h, c]
                        dks[b, h, c] += tau * dlam * qh
                        dbs[b, h, c] += dlam
                    if q_route is None:
                        dq[b, h, i] += dqh
                    else:
                        dqr[b, h, i] += dqh
    # summaries (Proposition 3.1 and the mode variants)
    dlm = np.zeros_like(lm64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for c in range(nC):
                kc = k64[b, g, c * S:(c + 1) * S]
                if mode == "landmark_key":
                    dlm[b, h, c] = dks[b, h, c]
                    continue
                if mode == "mean_pool":
                    dk[b, g, c * S:(c + 1) * S] += dks[b, h, c] / S
                    continue
                t = tau * (kc @ lm64[b, h, c])
                logpi = t - _lse(t)
                pi = np.exp(logpi)
                dpi = kc @ dks[b, h, c] + dbs[b, h, c] * (-logpi - 1.0)
                dt = pi * (dpi - pi @ dpi)
                dlm[b, h, c] = tau * (dt @ kc)
                dk[b, g, c * S:(c + 1) * S] += tau * np.outer(dt, lm64[b, h, c]) + np.outer(pi, dks[b, h, c])
    return dict(dq=dq, dk=dk, dv=dv, dlm=dlm, dq_route=(dqr if q_route is not None else None),
                sel=sel)


def ref_attending_rows(sel, b, g, j, S, W):
    """The query rows (b, g, i) whose attention reads key j of KV group g of
    sequence b (section 2.1 window, section 3 selection): those whose window
    [window_start(i), i] holds j and those whose selection holds j's chunk."""
    sel = np.asarray(sel)
    N = sel.shape[2]
    c = j // S
    rows = {(b, g, i) for i in range(j, N) if _window_start(i, W, S) <= j}
    rows |= {(b, g, int(i)) for i in np.nonzero((sel[b, g] == c).any(axis=-1))[0]}
    return rows


# ---------------------------------------------------------------------------
# independent routes used as pins
# ---------------------------------------------------------------------------

def ref_full_causal(q, k, v, scale=None):
    """Textbook causal softmax attention, all positions: out[b,h,i] = softmax_{j<=i}(q.k*scale) V."""
    q, k, v = map(_as64, (q, k, v))
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    tau = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    out = np.zeros_like(q)
    mask = np.tril(np.ones((N, N), dtype=bool))
    for b in range(B):
        for h in range(Hq):
            s = tau * q[b, h] @ k[b, h // G].T
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, h // G]
    return out


def ref_naive_bsa(q, k, v, i, sel, S, W, scale):
    """Naive block-sparse attention for one position and the heads of one group.

    One softmax over the selected tokens only (window plus the tokens of the
    selected chunks); every other token gets weight 0 (section 2.1 prose).
    q [G,d], k/v [N',d].  Returns (out [G,d], weights [G,i+1]).
    """
    q, k, v = map(_as64, (q, k, v))
    w0 = _window_start(i, W, S)
    idx = [np.arange(w0, i + 1)] + [np.arange(c * S, (c + 1) * S) for c in sel]
    idx = np.concatenate(idx)
    s = scale * (q @ k[idx].T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    w = np.zeros((q.shape[0], i + 1))
    w[:, idx] = p
    return p @ v[idx], w


def ref_brute_force_mass_topk(logz, K):
    """All K-subsets of the candidates; the one with the largest retained mass sum exp(log Z_c)."""
    n = logz.shape[0]
    kk = min(K, n)
    best, best_set = -math.inf, None
    z = np.exp(logz - logz.max())
    for comb in itertools.combinations(range(n), kk):
        m = z[list(comb)].sum()
        if m > best:
            best, best_set = m, comb
    return np.array(best_set, dtype=np.int64)


def ref_overlap(sel_sets, K):
    """Normalised chunk overlap of M adjacent queries (section 7.2):
    (M*K - |union of I_m|) / ((M-1)*K)."""
    M = len(sel_sets)
    u = set()
    for s in sel_sets:
        u |= set(int(c) for c in s)
    return (M * K - len(u)) / ((M - 1) * K)
