"""Pins for the fp64 oracle: facts fixed by the HiLS paper and by mathematics.

Each test checks the oracle against something other than itself: a value
derived by hand from the definitions (tests/golden), a closed form, an
invariant, a special case that reduces to textbook attention, or brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import hils_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _tiny(**kw):
    w = synth.get_workload("tiny_fp32", **kw)
    x = synth.make_prefill_inputs(w)
    return w, {k: _np(v) for k, v in x.items()}


# --- number format ---------------------------------------------------------

def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact bf16 midpoints (ties) in both parities, and subnormals
        (np.arange(1, 2000) * 2 + 1).astype(np.float64) * 2.0 ** -8,
        np.array([1e-40, -3e-39, 2.0 ** -133, 3 * 2.0 ** -134, 5e-45]),
    ]).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.bf16_round(x), want)


def test_bf16_round_is_single_rounding_from_f64():
    # 1 + 2^-8 is the exact midpoint between bf16 1 and 1+2^-7: ties to even -> 1.
    # Just above it (by 2^-40) must round up; via fp32 it would become the tie.
    assert O.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    assert O.bf16_round(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    # largest finite bf16 is (2 - 2^-7) * 2^127; the midpoint to 2^128 rounds to inf
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert O.bf16_round(np.array([big * (1 + 2.0 ** -10)]))[0] == big
    assert O.bf16_round(np.array([(2 - 2.0 ** -8) * 2.0 ** 127]))[0] == math.inf


# --- window geometry (section 2.1) ------------------------------------------

def test_window_geometry_golden():
    fx = json.load(open(os.path.join(GOLD, "window_geometry.json")))
    for case in fx["cases"]:
        S, W, first = case["S"], case["W"], case["first"]
        assert O.n_candidates(first - 1, W, S) == 0
        assert O.n_candidates(first, W, S) == 1
        for i, l in case["l"].items():
            assert O.window_left(int(i), W, S) == l


# --- hand-derived worked example -------------------------------------------

def test_hand_example_d1():
    fx = json.load(open(os.path.join(GOLD, "hand_example_d1.json")))
    st = fx["setup"]
    val = {"0": 0.0, "ln2": math.log(2), "ln3": math.log(3)}
    k = np.array([val[s] for s in st["k"]]).reshape(1, 1, 8, 1)
    v = np.array(st["v"], dtype=np.float64).reshape(1, 1, 8, 1)
    q = np.ones((1, 1, 8, 1))
    lm = np.zeros((1, 1, 4, 1))
    res = O.ref_prefill_rows(q, k, v, lm, [(0, i) for i in range(8)], S=2, W=2, K=1,
                             scale=1.0, store="f64")
    for i in range(8):
        r = res[(0, i)]
        num, den = fx["expected_out"][str(i)]
        assert abs(r["out"][0, 0] - num / den) < 1e-12, i
        assert r["sel"][0].tolist() == fx["expected_sel"][str(i)]
        assert r["n"] == fx["expected_n_candidates"][str(i)]


# --- hand-derived example at the default scale 1/sqrt(d) (d = 4) -----------

_LOGS = {"0": 0.0, "ln2": math.log(2), "ln3": math.log(3), "ln6": math.log(6)}


def _d4_example():
    """tests/golden/hand_example_d4_default_scale.json: q = (2,0,0,0) at every
    position, keys (x_j,0,0,0), values (j,1,-j,0), landmark queries (2,0,0,0)."""
    fx = json.load(open(os.path.join(GOLD, "hand_example_d4_default_scale.json")))
    x = np.array([_LOGS[s] for s in fx["setup"]["k_first_component"]])
    N, d = x.shape[0], 4
    j = np.arange(N, dtype=np.float64)
    q = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 2.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, :, 0] = x
    v = np.zeros((1, 1, N, d))
    v[0, 0, :, 0], v[0, 0, :, 1], v[0, 0, :, 2] = j, 1.0, -j
    lm = np.zeros((1, 1, N // 2, d))
    lm[0, 0, :, 0] = 2.0
    return fx, q, k, v, lm


def test_hand_example_default_scale_summaries_and_scores():
    # Proposition 3.1 summaries and the routing scores at scale 1/sqrt(d) = 1/2,
    # through ref_summarize's default scale and ref_chunk_scores itself
    fx, q, k, v, lm = _d4_example()
    ln2, ln3, ln6 = math.log(2), math.log(3), math.log(6)
    ks, bs = O.ref_summarize(k, lm, 2, store="f64")
    np.testing.assert_allclose(ks[0, 0, :, 0], [0.0, ln2, ln3, ln3 / 3 + 2 * ln6 / 3, 0.0],
                               rtol=0, atol=1e-14)
    assert np.all(ks[0, 0, :, 1:] == 0.0)
    np.testing.assert_allclose(bs[0, 0], [ln2, ln2, ln2, ln3 - 2 * ln2 / 3, ln2], rtol=0,
                               atol=1e-14)
    s = O.ref_chunk_scores(q[0, :, 9], ks[0], bs[0], 4, 1 / math.sqrt(4))
    np.testing.assert_allclose(s[0], [ln2, math.log(4), ln6, math.log(9)], rtol=0, atol=1e-14)


def test_hand_example_default_scale_outputs():
    fx, q, k, v, lm = _d4_example()
    res = O.ref_prefill_rows(q, k, v, lm, [(0, i) for i in range(10)], S=2, W=2, K=1,
                             store="f64")
    for i in range(10):
        num, den = fx["expected_out_surrogate"][str(i)]
        o = res[(0, i)]["out"][0]
        np.testing.assert_allclose(o, [num / den, 1.0, -num / den, 0.0], rtol=0, atol=1e-12,
                                   err_msg=f"row {i}")
        assert res[(0, i)]["sel"][0].tolist() == fx["expected_sel_surrogate"][str(i)], i


def test_hand_example_landmark_key_mode():
    # ablation 'w/o Prop. 3.1' (section 5.3, Table 5): the landmark row is the
    # routing key as it is and the entropy bias is absent (b' = 0), which the
    # fusion weight against the window fixes (b' = ln S would give other outputs)
    fx, q, k, v, _ = _d4_example()
    lm = np.zeros((1, 1, 5, 4))
    lm[0, 0, 0, 0] = math.log(5)
    ks, bs = O.ref_summarize(k, lm, 2, mode="landmark_key", store="f64")
    np.testing.assert_array_equal(ks, lm)
    assert np.all(bs == 0.0)
    rows = [(0, int(i)) for i in fx["expected_out_landmark_key"]]
    res = O.ref_prefill_rows(q, k, v, lm, rows, S=2, W=2, K=1, mode="landmark_key", store="f64")
    for (_, i) in rows:
        num, den = fx["expected_out_landmark_key"][str(i)]
        np.testing.assert_allclose(res[(0, i)]["out"][0], [num / den, 1.0, -num / den, 0.0],
                                   rtol=0, atol=1e-12, err_msg=f"row {i}")
        assert res[(0, i)]["sel"][0].tolist() == fx["expected_sel_landmark_key"][str(i)], i


def test_surrogate_tangent_point_through_chunk_scores():
    # Proposition 3.1: the routing score equals the exact chunk log-mass when the
    # routing query is the chunk's landmark query, at the default scale 1/sqrt(d);
    # everywhere else it stays below it (convexity of log-sum-exp)
    rng = np.random.default_rng(11)
    S, d, n = 64, 128, 6
    tau = 1 / math.sqrt(d)
    k = rng.standard_normal((1, 1, n * S, d))
    lm = rng.standard_normal((1, 2, n, d)) * 3.0
    ks, bs = O.ref_summarize(k, lm, S, store="f64")
    for c in range(n):
        s = O.ref_chunk_scores(lm[0, :, c], ks[0], bs[0], n, tau)
        logz = O.ref_exact_logz(lm[0, :, c], k[0, 0], n, S, tau)
        np.testing.assert_allclose(s[:, c], logz[:, c], rtol=0, atol=1e-11)
        assert np.all(s <= logz + 1e-11)


# --- P1: exact masses with K >= |C_i| reproduce full causal attention ------

def test_exact_mode_full_k_equals_full_causal():
    w, x = _tiny()
    Kmax = O.n_candidates(w.N - 1, w.W, w.S)          # 14 for N=512, S=32, W=64
    assert Kmax == 14
    rows = [(0, i) for i in range(w.N)]
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], None, rows, w.S, w.W, Kmax, mode="exact")
    full = O.ref_full_causal(x["q"], x["k"], x["v"])
    got = np.stack([res[(0, i)]["out"] for i in range(w.N)], axis=1)
    np.testing.assert_allclose(got, full[0], rtol=0, atol=1e-12)


# --- P2: naive-BSA exact-mass top-K is the max-mass subset; fusion = naive BSA

def test_exact_topk_is_brute_force_max_mass():
    w, x = _tiny()
    tau = 1 / math.sqrt(w.d)
    checked = 0
    for i in range(w.W + w.S, w.N, 7):
        n = O.n_candidates(i, w.W, w.S)
        for h in range(2):
            logz = O.ref_exact_logz(x["q"][0, h:h + 1, i], x["k"][0, h], n, w.S, tau)[0]
            sel, _ = O.ref_select(logz, w.K)
            bf = O.ref_brute_force_mass_topk(logz, w.K)
            assert sorted(bf.tolist()) == sel.tolist(), i
            checked += 1
    assert checked > 100


def test_exact_fusion_equals_naive_bsa():
    w, x = _tiny()
    tau = 1 / math.sqrt(w.d)
    rows = [(0, i) for i in range(0, w.N, 5)]
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], None, rows, w.S, w.W, w.K,
                             mode="exact", want_weights=True)
    for (b, i) in rows:
        r = res[(b, i)]
        for g in range(2):
            o, wts = O.ref_naive_bsa(x["q"][0, g:g + 1, i], x["k"][0, g], x["v"][0, g], i,
                                     r["sel"][g], w.S, w.W, tau)
            np.testing.assert_allclose(r["out"][g], o[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(r["weights"][g][0], wts[0], rtol=0, atol=1e-13)


# --- P3: weights sum to 1 over selected tokens and are exactly 0 elsewhere --

@pytest.mark.parametrize("mode", ["surrogate", "exact", "landmark_key"])
def test_weights_normalised_and_zero_elsewhere(mode):
    w, x = _tiny()
    rows = [(0, i) for i in range(0, w.N, 3)]
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], x["lm"], rows, w.S, w.W, w.K,
                             mode=mode, store="f32", want_weights=True)
    for (b, i) in rows:
        r = res[(b, i)]
        w0 = max(0, O.window_left(i, w.W, w.S))
        for g in range(2):
            wt = r["weights"][g][0]
            allowed = np.zeros(i + 1, dtype=bool)
            allowed[w0:] = True
            for c in r["sel"][g]:
                allowed[c * w.S:(c + 1) * w.S] = True
            assert abs(wt.sum() - 1.0) < 1e-12
            assert np.all(wt[~allowed] == 0.0)
            assert np.all(wt[allowed] > 0.0)
            # the weighted sum of values is the output
            np.testing.assert_allclose(wt @ x["v"][0, g, : i + 1], r["out"][g], atol=1e-12)


# --- P4: Proposition 3.1 properties ----------------------------------------

def _one_chunk(seed, S=64, d=128, scale_q=1.0):
    rng = np.random.default_rng(seed)
    kc = rng.standard_normal((S, d))
    lmq = rng.standard_normal(d) * scale_q
    k = kc.reshape(1, 1, S, d)
    lm = lmq.reshape(1, 1, 1, d)
    ks, bs = O.ref_summarize(k, lm, S, store="f64")
    return kc, lmq, ks[0, 0, 0], bs[0, 0, 0]


def test_surrogate_exact_at_tangent_point():
    tau = 1 / math.sqrt(128)
    for seed in range(20):
        kc, lmq, ks, bs = _one_chunk(seed)
        logz = O._lse(tau * kc @ lmq)
        assert abs((tau * lmq @ ks + bs) - logz) < 1e-12


def test_surrogate_is_lower_bound_of_logz():
    tau = 1 / math.sqrt(128)
    rng = np.random.default_rng(7)
    for seed in range(10):
        kc, lmq, ks, bs = _one_chunk(seed)
        for _ in range(50):
            q = rng.standard_normal(128) * rng.uniform(0.1, 3)
            assert tau * q @ ks + bs <= O._lse(tau * kc @ q) + 1e-12


def test_entropy_bias_limits():
    S = 64
    for seed in range(10):
        kc, lmq, ks, bs = _one_chunk(seed)
        assert 0.0 <= bs <= math.log(S) + 1e-12
    # q' = 0: uniform p, mean key, b' = log S (section 2.2 mean pooling)
    kc, lmq, ks, bs = _one_chunk(0, scale_q=0.0)
    np.testing.assert_allclose(ks, kc.mean(axis=0), atol=1e-14)
    assert abs(bs - math.log(S)) < 1e-14
    # q' scaled up: one logit dominates, b' -> 0 and k' -> the arg-max key
    kc, lmq, ks, bs = _one_chunk(3, scale_q=1e4)
    j = np.argmax(kc @ lmq)
    assert bs < 1e-6
    np.testing.assert_allclose(ks, kc[j], atol=1e-8)


# --- P5: no candidates or a window covering everything = causal attention ---

def test_no_candidate_rows_equal_causal():
    w, x = _tiny()
    full = O.ref_full_causal(x["q"], x["k"], x["v"])
    first = w.W + w.S - 1
    rows = [(0, i) for i in range(first)]
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], x["lm"], rows, w.S, w.W, w.K)
    for (b, i) in rows:
        assert res[(b, i)]["n"] == 0
        np.testing.assert_allclose(res[(b, i)]["out"], full[0, :, i], atol=1e-12)


def test_window_covering_sequence_equals_causal():
    w, x = _tiny()
    full = O.ref_full_causal(x["q"], x["k"], x["v"])
    rows = [(0, i) for i in range(0, w.N, 17)]
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], x["lm"], rows, w.S, w.N, w.K)
    for (b, i) in rows:
        np.testing.assert_allclose(res[(b, i)]["out"], full[0, :, i], atol=1e-12)


# --- P6: GQA reductions (section 4.1) ---------------------------------------

def test_gqa_single_head_ranking_unchanged_by_normalisation():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((1, 200))
    g = O.ref_group_scores(s)
    L = O._lse(s, axis=1)
    np.testing.assert_array_equal(np.argsort(-g, kind="stable"),
                                  np.argsort(-(s[0] - L[0]), kind="stable"))


def test_gqa_identical_heads_equal_mha():
    rng = np.random.default_rng(4)
    N, d, S, W, K = 1024, 64, 32, 64, 4
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    q1 = rng.standard_normal((1, 1, N, d))
    lm1 = rng.standard_normal((1, 1, N // S, d))
    q2, lm2 = np.repeat(q1, 3, axis=1), np.repeat(lm1, 3, axis=1)
    rows = [(0, i) for i in range(100, N, 37)]
    r1 = O.ref_prefill_rows(q1, k, v, lm1, rows, S, W, K)
    r3 = O.ref_prefill_rows(q2, k, v, lm2, rows, S, W, K)
    for key in rows:
        assert r1[key]["sel"][0].tolist() == r3[key]["sel"][0].tolist()
        for h in range(3):
            np.testing.assert_allclose(r3[key]["out"][h], r1[key]["out"][0], atol=1e-12)


def test_gqa_max_over_heads_hand_case():
    # head 0 strongly prefers chunk 3; head 1 is spread and dislikes it; a chunk that
    # matters to any one head is selected (section 4.1).
    s = np.array([[0.0, 0.0, 0.0, 5.0, 0.0],
                  [1.0, 1.2, 1.1, -20.0, 0.9]])
    g = O.ref_group_scores(s)
    L0 = math.log(4 + math.exp(5))
    L1 = math.log(sum(math.exp(t) for t in s[1]))
    want = np.maximum(s[0] - L0, s[1] - L1)
    np.testing.assert_allclose(g, want, atol=1e-14)
    sel, gap = O.ref_select(g, 2)
    assert sel.tolist() == [1, 3]
    # the mean over heads would have picked chunk 1 and 2 instead of 3
    mean_sel = np.argsort(-(s - np.array([[L0], [L1]])).mean(axis=0), kind="stable")[:2]
    assert sorted(mean_sel.tolist()) != sel.tolist()


def test_gqa_rows_without_candidates_are_window_attention():
    w, x = _tiny()
    q2 = np.concatenate([x["q"], x["q"][:, ::-1]], axis=1)       # 4 q heads, 2 KV heads
    lm2 = np.concatenate([x["lm"], x["lm"][:, ::-1]], axis=1)
    res = O.ref_prefill_rows(q2, x["k"], x["v"], lm2, [(0, 10), (0, 94)], w.S, w.W, w.K)
    full = O.ref_full_causal(q2, x["k"], x["v"])
    for i in (10, 94):
        assert res[(0, i)]["n"] == 0 and all(len(s) == 0 for s in res[(0, i)]["sel"].values())
        np.testing.assert_allclose(res[(0, i)]["out"], full[0, :, i], atol=1e-12)


def test_select_ties_and_short_candidate_lists():
    sel, gap = O.ref_select(np.array([1.0, 2.0, 2.0, 0.5, 2.0]), 2)
    assert sel.tolist() == [1, 2] and gap == 0.0
    sel, gap = O.ref_select(np.array([0.3, 0.1]), 4)
    assert sel.tolist() == [0, 1] and gap == math.inf
    sel, gap = O.ref_select(np.zeros(0), 4)
    assert sel.tolist() == []


# --- P7: LSE regimes ----------------------------------------------------------

def test_equal_logits_logz_is_s_plus_log_s():
    S, d = 64, 16
    kg = np.tile(np.linspace(-1, 1, d), (3 * S, 1))
    q = np.linspace(0.3, -0.2, d)[None, :]
    logz = O.ref_exact_logz(q, kg, 3, S, 1.0)
    s = float(q[0] @ kg[0])
    np.testing.assert_allclose(logz[0], s + math.log(S), atol=1e-13)


def test_one_dominant_logit_logz_is_max():
    S = 64
    kg = np.zeros((S, 1))
    kg[5, 0] = 200.0
    logz = O.ref_exact_logz(np.ones((1, 1)), kg, 1, S, 1.0)
    assert abs(logz[0, 0] - 200.0) < 1e-12


# --- P8: overlap formula (section 7.2) --------------------------------------

def test_overlap_formula():
    assert O.ref_overlap([[1, 2, 3], [1, 2, 3], [1, 2, 3]], 3) == 1.0
    assert O.ref_overlap([[1, 2], [3, 4]], 2) == 0.0
    assert O.ref_overlap([[1, 2], [2, 3]], 2) == 0.5


# --- decode is the prefill row at i = T-1 -----------------------------------

def test_decode_equals_last_prefill_row():
    w = synth.get_workload("decode_512k", N=2048, B=2, Hq=4, Hkv=2, W=256, K=4)
    x = synth.make_decode_inputs(w, seqlen=[2048, 1500])
    q, k, v, lm = (_np(x[n]) for n in ("q", "k", "v", "lm"))
    dec = O.ref_decode(q, k, v, [2048, 1500], lm, w.S, w.W, w.K)
    for b, T in enumerate([2048, 1500]):
        qq = np.zeros((1, w.Hq, T, w.d))
        qq[0, :, T - 1] = q[b, :, 0]
        pre = O.ref_prefill_rows(qq, k[b:b + 1, :, :T], v[b:b + 1, :, :T], lm[b:b + 1, :, : T // w.S],
                                 [(0, T - 1)], w.S, w.W, w.K)[(0, T - 1)]
        np.testing.assert_allclose(dec[b]["out"], pre["out"], atol=1e-12)
        for g in range(w.Hkv):
            assert dec[b]["sel"][g].tolist() == pre["sel"][g].tolist()


def test_decode_multi_rows_are_causal_prefill_rows():
    """Each token of a multi-token decode block is the prefill row at its own
    position (section 3), M = 1 is the single-step decode, and a token's output
    does not change when later tokens of the block change (causality)."""
    w = synth.get_workload("decode_512k", N=2048, B=3, Hq=4, Hkv=2, W=256, K=4)
    M = 3
    T = [2048, 1500, 2]                                  # the last one is shorter than M
    x = synth.make_decode_inputs(w, seqlen=T)
    k, v, lm = (_np(x[n]) for n in ("k", "v", "lm"))
    rng = np.random.default_rng(5)
    q = rng.standard_normal((w.B, w.Hq, M, w.d))
    dec = O.ref_decode_multi(q, k, v, T, lm, w.S, w.W, w.K)
    for b in range(w.B):
        for m in range(M):
            i = max(T[b] - M + m, 0)
            qq = np.zeros((1, w.Hq, i + 1, w.d))
            qq[0, :, i] = q[b, :, m]
            nck = (i + 1) // w.S
            pre = O.ref_prefill_rows(qq, k[b:b + 1, :, : i + 1], v[b:b + 1, :, : i + 1],
                                     lm[b:b + 1, :, :nck], [(0, i)], w.S, w.W, w.K)[(0, i)]
            np.testing.assert_allclose(dec[(b, m)]["out"], pre["out"], atol=1e-12)
            for g in range(w.Hkv):
                assert dec[(b, m)]["sel"][g].tolist() == pre["sel"][g].tolist()
    one = O.ref_decode_multi(q[:, :, -1:], k, v, T, lm, w.S, w.W, w.K)
    ref1 = O.ref_decode(q[:, :, -1], k, v, T, lm, w.S, w.W, w.K)
    for b in range(w.B):
        np.testing.assert_allclose(one[(b, 0)]["out"], ref1[b]["out"], atol=1e-12)
    # changing the last token of the block leaves the earlier tokens' outputs alone
    k2, v2 = k.copy(), v.copy()
    k2[0, :, T[0] - 1] += 3.0
    v2[0, :, T[0] - 1] -= 2.0
    dec2 = O.ref_decode_multi(q, k2, v2, T, lm, w.S, w.W, w.K)
    for m in range(M - 1):
        np.testing.assert_allclose(dec2[(0, m)]["out"], dec[(0, m)]["out"], atol=1e-12)
    assert np.abs(dec2[(0, M - 1)]["out"] - dec[(0, M - 1)]["out"]).max() > 1e-3


def _hils_loss(x, dout, S, W, K, sel, mode, q_route=None):
    """sum(dout * out) of every prefill row with the selection held at `sel`."""
    B, Hq, N, d = x["q"].shape
    Hkv = x["k"].shape[1]
    rows = [(0, i) for i in range(N)]
    forced = {(0, g, i): [int(c) for c in sel[0, g, i] if c >= 0] for g in range(Hkv) for i in range(N)}
    res = O.ref_prefill_rows(x["q"], x["k"], x["v"], x["lm"], rows, S, W, K, q_route=q_route,
                             mode=mode, store="f64", forced_sel=forced)
    return sum(float(np.sum(dout[0, :, i] * res[(0, i)]["out"])) for i in range(N))


@pytest.mark.parametrize("mode,route", [("surrogate", False), ("surrogate", True),
                                        ("landmark_key", False), ("mean_pool", False)])
def test_backward_matches_finite_differences(mode, route):
    """The oracle's gradients (selection held fixed) equal central finite
    differences of sum(dout * out) along random directions, for q, the routing
    query, k, v and the landmark queries."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, N, d, S, W, K = 1, 4, 2, 160, 8, 16, 32, 3
    x = {"q": rng.standard_normal((B, Hq, N, d)), "k": rng.standard_normal((B, Hkv, N, d)),
         "v": rng.standard_normal((B, Hkv, N, d)),
         "lm": rng.standard_normal((B, Hq, N // S, d))}
    qr = rng.standard_normal((B, Hq, N, d)) if route else None
    dout = rng.standard_normal((B, Hq, N, d))
    gr = O.ref_backward(x["q"], x["k"], x["v"], x["lm"], dout, S, W, K, q_route=qr, mode=mode,
                        store="f64")
    sel = gr["sel"]
    assert (sel[..., 0] >= 0).sum() > 0 and (sel[..., K - 1] >= 0).sum() > 0
    names = [("q", "dq"), ("k", "dk"), ("v", "dv")]
    if mode != "mean_pool":
        names.append(("lm", "dlm"))
    eps = 1e-5
    for name, gname in names + ([("q_route", "dq_route")] if route else []):
        u = rng.standard_normal(x[name].shape if name != "q_route" else qr.shape)
        def loss(sgn):
            y = dict(x)
            r2 = qr
            if name == "q_route":
                r2 = qr + sgn * eps * u
            else:
                y[name] = x[name] + sgn * eps * u
            return _hils_loss(y, dout, S, W, K, sel, mode, q_route=r2)
        fd = (loss(1) - loss(-1)) / (2 * eps)
        an = float(np.sum(gr[gname] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (mode, name, fd, an)


def test_backward_row_restriction_is_exact_where_complete():
    """With `rows` restricted to the rows attending a key (plus some query
    rows), the key's dk, dv, its chunk's dlm and the listed rows' dq are those
    of the unrestricted backward, term for term; a key whose attending rows
    are left out gets a different dk."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, N, d, S, W, K = 1, 4, 2, 200, 8, 16, 40, 3
    q, qr, dout = (rng.standard_normal((B, Hq, N, d)) for _ in range(3))
    k, v = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    lm = rng.standard_normal((B, Hq, N // S, d))
    full = O.ref_backward(q, k, v, lm, dout, S, W, K, q_route=qr, store="f64")
    sel = full["sel"]
    g, j = 1, 37                                     # a key of chunk 2, selected by later rows
    assert (sel[0, g] == j // S).any()
    rows = O.ref_attending_rows(sel, 0, g, j, S, W) | {(0, 0, 150), (0, 1, 199)}
    part = O.ref_backward(q, k, v, lm, dout, S, W, K, q_route=qr, sel=sel, store="f64", rows=rows)
    np.testing.assert_array_equal(part["dk"][0, g, j], full["dk"][0, g, j])
    np.testing.assert_array_equal(part["dv"][0, g, j], full["dv"][0, g, j])
    for h in range(g * (Hq // Hkv), (g + 1) * (Hq // Hkv)):
        np.testing.assert_array_equal(part["dlm"][0, h, j // S], full["dlm"][0, h, j // S])
    for (b, gg, i) in [(0, 0, 150), (0, 1, 199)]:
        for h in range(gg * (Hq // Hkv), (gg + 1) * (Hq // Hkv)):
            np.testing.assert_array_equal(part["dq"][b, h, i], full["dq"][b, h, i])
            np.testing.assert_array_equal(part["dq_route"][b, h, i], full["dq_route"][b, h, i])
    # a key of the other group, whose rows are not all listed, differs
    assert np.abs(part["dk"][0, 0, 37] - full["dk"][0, 0, 37]).max() > 1e-6


def test_backward_window_only_is_causal_attention_gradient():
    """With the window covering every position (no candidate chunks) HiLS is
    causal softmax attention; its gradients equal torch autograd of the
    textbook formula (float64, CPU)."""
    import torch
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, d, S = 1, 4, 2, 48, 8, 8
    q, k, v = (rng.standard_normal(sh) for sh in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    lm = rng.standard_normal((B, Hq, N // S, d))
    dout = rng.standard_normal((B, Hq, N, d))
    gr = O.ref_backward(q, k, v, lm, dout, S, N + S, 2, store="f64")
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    s = (tq @ kk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    out = torch.softmax(s, dim=-1) @ vv
    (out * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(gr["dq"], tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(gr["dk"], tk.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(gr["dv"], tv.grad.numpy(), atol=1e-10)
    assert np.abs(gr["dlm"]).max() == 0.0


def test_mean_pool_is_surrogate_at_zero_landmark_query():
    """Mean pooling (section 2.2 equation) equals the Proposition 3.1 summary of
    a zero landmark query: uniform weights give the mean key and entropy ln S."""
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, 2, 96, 8))
    lm0 = np.zeros((1, 4, 6, 8))
    ks_m, bs_m = O.ref_summarize(k, lm0, 16, mode="mean_pool", store="f64")
    ks_s, bs_s = O.ref_summarize(k, lm0, 16, mode="surrogate", store="f64")
    np.testing.assert_allclose(ks_m, ks_s, rtol=0, atol=1e-14)
    np.testing.assert_allclose(bs_m, bs_s, rtol=0, atol=1e-14)
    # the mean key, chunk by chunk, written out directly
    assert abs(ks_m[0, 3, 2, 5] - k[0, 1, 32:48, 5].mean()) < 1e-15
    assert np.all(bs_m == math.log(16))
