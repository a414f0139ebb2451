"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Inputs come from the seeded generators in synth/; expected values come only
from oracle/.  Every test prints what it covered (selection exact / tie-band
counts and the largest output error).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import hils_oracle as O
from tests.parity_util import (Tally, check_selection, compare_prefill_rows, np32, out_error,
                               sample_rows)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import chunk_wise_hierarchical_amd as hils


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu_inputs(w, device="cuda", **kw):
    gen_dev = "cpu" if w.B * w.Hq * w.N * w.d <= (1 << 26) else device
    x = synth.make_prefill_inputs(w, device=gen_dev, **kw)
    return {k: v.to(device) for k, v in x.items()}


def _run_prefill(w, x, mode="surrogate", generic=False, union=False):
    B, Hq, N, d = x["q"].shape
    nC = N // w.S
    ks = torch.empty((B, Hq, nC, d), dtype=x["q"].dtype, device="cuda")
    bs = torch.empty((B, Hq, nC), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, w.Hkv, N, w.K), dtype=torch.int32, device="cuda")
    out = hils.prefill(x["q"], x["k"], x["v"], x["lm"], w.S, w.W, w.K, q_route=x.get("q_route"),
                       mode=mode, sel=sel, summaries=(ks, bs), generic=generic, union=union)
    torch.cuda.synchronize()
    return out, sel, ks, bs


def _oracle_summaries(w, xn, mode="surrogate"):
    return O.ref_summarize(xn["k"], xn["lm"], w.S, mode=mode, store=w.dtype)


def _check_summaries(w, ks, bs, ref):
    rks, rbs = ref
    gks = np32(ks).astype(np.float64)
    gbs = np32(bs).astype(np.float64)
    nbad = int((gks != rks).sum())
    # k' is the correctly rounded exact summary on both sides: expect identity
    assert nbad <= max(1, gks.size // 10**6), f"{nbad} summary-key elements differ"
    rel = np.abs(gbs - rbs) / np.maximum(np.abs(rbs), 1e-30)
    assert rel.size == 0 or rel.max() <= 1e-6, f"b' rel err {rel.max()}"   # N < S: no chunks
    return nbad


def _prefill_case(w, rows=None, mode="surrogate", generic=False, q_route=False, label="",
                  union=False):
    _say(f"[prefill] {label} {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} "
         f"W={w.W} K={w.K} dtype={w.dtype} mode={mode} generic={generic} union={union}")
    x = _gpu_inputs(w, with_q_route=q_route)
    out, sel, ks, bs = _run_prefill(w, x, mode=mode, generic=generic, union=union)
    xn = {k: np32(v) for k, v in x.items()}
    summ, nbad = None, 0
    if mode != "exact":               # exact scoring has no summaries
        summ = _oracle_summaries(w, xn, mode)
        nbad = _check_summaries(w, ks, bs, summ)
    if rows is None:
        rows = [(b, i) for b in range(w.B) for i in range(w.N)]
    res = O.ref_prefill_rows(xn["q"], xn["k"], xn["v"], xn["lm"], rows, w.S, w.W, w.K,
                             q_route=xn.get("q_route"), mode=mode, store=w.dtype, summaries=summ)

    def rerun(b, i, forced):
        return O.ref_prefill_rows(xn["q"], xn["k"], xn["v"], xn["lm"], [(b, i)], w.S, w.W, w.K,
                                  q_route=xn.get("q_route"), mode=mode, store=w.dtype,
                                  summaries=summ, forced_sel=forced)[(b, i)]

    t = compare_prefill_rows(res, np32(out), sel.cpu().numpy(), rows, w, rerun=rerun)
    _say(f"   summaries: {nbad} k' elements differ; {t}")
    assert t.exact >= 0.9 * (t.exact + t.tie)
    t.check_rel(w.dtype)
    return t


# ---------------------------------------------------------------------------
# prefill, generic kernels
# ---------------------------------------------------------------------------

def test_prefill_8k_full_size_sampled():
    # the 8K training-length workload at its stated size: B=2, N=8192, 16/16
    # heads, d=128, S=64, W=512, K=16, inputs N(0,1)/sqrt(d), heads 8-15 peaked;
    # 2048 positions per sequence (every head of each), all boundary rows included
    w = synth.get_workload("prefill_8k")
    assert (w.B, w.N, w.Hq, w.Hkv, w.d, w.S, w.W, w.K) == (2, 8192, 16, 16, 128, 64, 512, 16)
    _prefill_case(w, rows=sample_rows(w, 2048, include=[w.N - 2, 8191 - 64]),
                  label="8K full size, 4096 rows")


def test_prefill_tiny_fp32_all_rows():
    w = synth.get_workload("tiny_fp32")
    _prefill_case(w, label="tiny fp32 all rows")


def test_prefill_bf16_mha_peaked_all_rows():
    w = synth.get_workload("prefill_8k", N=2048, B=2)
    _prefill_case(w, label="8K-geometry MHA, N=2048")


def test_prefill_bf16_gqa_sampled():
    w = synth.get_workload("prefill_64k", N=8192, W=1024, K=32)
    _prefill_case(w, rows=sample_rows(w, 160), label="64K-geometry GQA 4:1, N=8192")


def test_prefill_ragged_and_degenerate():
    # N not a multiple of S, K larger than some candidate sets, GQA 2:1
    w = synth.get_workload("prefill_64k", N=1000, Hq=4, Hkv=2, d=64, S=32, W=100, K=8,
                           regime="iid")
    _prefill_case(w, label="ragged N=1000 S=32")
    # window covering the whole sequence: no candidates anywhere
    w2 = w.with_(N=300, W=400)
    _prefill_case(w2, label="W > N")
    # one token, one chunk
    w3 = w.with_(N=1, W=1, S=1, K=1)
    _prefill_case(w3, label="N=1")


def test_prefill_q_route_and_landmark_key():
    w = synth.get_workload("prefill_64k", N=2048, Hq=8, Hkv=2, W=256, K=8)
    _prefill_case(w, rows=sample_rows(w, 120), q_route=True, label="q_route")
    _prefill_case(w, rows=sample_rows(w, 120), mode="landmark_key", label="landmark_key")


def test_prefill_mean_pool_fast_and_generic():
    # mean-pooled chunk keys with b' = ln S (Table 5 ablation), both kernel families
    w = synth.get_workload("prefill_64k", N=4096, W=512, K=16)
    _prefill_case(w, rows=sample_rows(w, 120), mode="mean_pool", label="mean_pool fast")
    _prefill_case(w, rows=sample_rows(w, 120), mode="mean_pool", generic=True,
                  label="mean_pool generic")
    # the landmark queries are not read in this mode
    x = _gpu_inputs(w)
    o1 = hils.prefill(x["q"], x["k"], x["v"], x["lm"], w.S, w.W, w.K, mode="mean_pool")
    o2 = hils.prefill(x["q"], x["k"], x["v"], None, w.S, w.W, w.K, mode="mean_pool")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_prefill_exact_scoring():
    # exact chunk log-masses from the token query (section 2.1), generic kernels
    w = synth.get_workload("tiny_fp32")
    _prefill_case(w, mode="exact", label="exact tiny fp32")
    w2 = synth.get_workload("prefill_8k", N=1024, B=1, Hq=4, Hkv=2, W=128, K=4)
    _prefill_case(w2, rows=sample_rows(w2, 80), mode="exact", label="exact bf16 GQA")


def test_prefill_exact_all_chunks_is_full_attention():
    # with every candidate chunk selected, exact fusion weights reproduce dense
    # causal softmax attention (section 3: the hierarchical softmax is exact then)
    w = synth.get_workload("tiny_fp32", K=16)           # N/S = 16 chunks
    x = _gpu_inputs(w)
    out = hils.prefill(x["q"], x["k"], x["v"], None, w.S, w.W, w.K, mode="exact")
    torch.cuda.synchronize()
    ref = O.ref_full_causal(np32(x["q"]), np32(x["k"]), np32(x["v"]))
    err, tol = out_error(np32(out), ref, "f32")
    _say(f"   exact K=|C| vs dense causal: rel err {err:.3g} (tol {tol})")
    assert err <= tol


def test_prefill_generic_kernels_bf16():
    # the same geometries through the vector-ALU kernels (HILS_FLAG_GENERIC)
    w = synth.get_workload("prefill_8k", N=1024, B=1)
    _prefill_case(w, generic=True, label="generic MHA")
    w = synth.get_workload("prefill_64k", N=4096, W=512, K=16)
    _prefill_case(w, rows=sample_rows(w, 100), generic=True, label="generic GQA")


def test_prefill_fast_ragged():
    # fast path (bf16, d=128, S=64) with N not a multiple of 64 and of the query block,
    # both attention organisations (per-chunk buckets, query-block unions)
    for union in (False, True):
        for G, N in ((2, 3001), (4, 2049), (1, 1500)):
            w = synth.get_workload("prefill_64k", N=N, Hq=2 * G, Hkv=2, W=200, K=8, regime="mod3")
            _prefill_case(w, label=f"fast ragged G={G}", union=union)


def test_prefill_fast_without_candidates():
    # fast path (bf16, d=128, S=64): no complete chunk at all (N < S), and chunks
    # but a window covering the whole sequence (W > N), in both attention
    # organisations
    for union in (False, True):
        w = synth.get_workload("prefill_64k", N=50, Hq=8, Hkv=2, W=256, K=8, regime="iid")
        _prefill_case(w, label="fast N < S", union=union)
        w = synth.get_workload("prefill_64k", N=300, Hq=8, Hkv=2, W=400, K=8, regime="iid")
        _prefill_case(w, label="fast W > N", union=union)


def test_prefill_pairs_across_slices():
    # more queries than one bucket slice (131072), ragged last slice, q_route
    w = synth.get_workload("prefill_64k", N=140000, Hq=4, Hkv=1, W=1024, K=32)
    _prefill_case(w, rows=sample_rows(w, 300, include=[131071, 131072, 139999]), q_route=True,
                  label="two slices")


def test_prefill_pairs_many_buckets():
    # 2 x 8 x 312 = 4992 (KV group, chunk) buckets: the bucket prefix sums span
    # two scan workgroups (4096 buckets each), the second one partial
    w = synth.get_workload("prefill_64k", N=20000, B=2, W=1024, K=32)
    assert w.B * w.Hkv * (w.N // w.S) == 4992
    _prefill_case(w, rows=sample_rows(w, 120, include=[19999]), label="4992 buckets")


def test_union_and_pairs_agree():
    w = synth.get_workload("prefill_64k", N=4096, W=512, K=16)
    x = _gpu_inputs(w)
    o1, s1, _, _ = _run_prefill(w, x)
    o2, s2, _, _ = _run_prefill(w, x, union=True)
    assert torch.equal(s1, s2)
    err = (o1.float() - o2.float()).abs().max().item()
    _say(f"   union/pairs max |out diff| {err:.3g}")
    assert err < 2e-2


def test_fast_and_generic_agree():
    w = synth.get_workload("prefill_64k", N=4096, W=512, K=16)
    x = _gpu_inputs(w)
    o1, s1, _, _ = _run_prefill(w, x, generic=False)
    o2, s2, _, _ = _run_prefill(w, x, generic=True)
    same = (s1 == s2).all(dim=-1).cpu().numpy()           # [B, Hkv, N]
    frac = float(same.mean())
    err = np.abs(np32(o1) - np32(o2))[same.repeat(w.G, axis=1)]
    _say(f"   fast/generic identical selections: {frac:.5f}; max |out diff| {err.max():.3g}")
    assert frac > 0.999
    assert err.max() < 2e-2


def _group_slice(x, w, g):
    G = w.G
    return dict(q=x["q"][:, g * G:(g + 1) * G], k=x["k"][:, g:g + 1], v=x["v"][:, g:g + 1],
                lm=x["lm"][:, g * G:(g + 1) * G])


def _large_sampled(w, groups, nrows, label):
    _say(f"[prefill] {label} {w.name} N={w.N} Hq={w.Hq} Hkv={w.Hkv} K={w.K} W={w.W} groups={groups}")
    x = {k2: v2 for k2, v2 in synth.make_prefill_inputs(w, device="cuda").items()}
    _run_prefill(w, x)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    out, sel, ks, bs = _run_prefill(w, x)
    t1.record()
    torch.cuda.synchronize()
    _say(f"   prefill time {t0.elapsed_time(t1):.2f} ms")
    rows = sample_rows(w, nrows, include=[w.N - 2, w.N - 65])
    t = Tally()
    wg = w.with_(Hq=w.G, Hkv=1)
    for g in groups:
        _say(f"   group {g}: oracle summaries")
        xg = {k2: np32(v2) for k2, v2 in _group_slice(x, w, g).items()}
        summ = O.ref_summarize(xg["k"], xg["lm"], w.S, store=w.dtype)
        gk = np32(ks[:, g * w.G:(g + 1) * w.G]).astype(np.float64)
        assert int((gk != summ[0]).sum()) <= max(1, gk.size // 10**6)
        _say(f"   group {g}: oracle rows")
        res = O.ref_prefill_rows(xg["q"], xg["k"], xg["v"], xg["lm"], rows, w.S, w.W, w.K,
                                 store=w.dtype, summaries=summ)

        def rerun(b, i, forced, xg=xg, summ=summ):
            return O.ref_prefill_rows(xg["q"], xg["k"], xg["v"], xg["lm"], [(b, i)], w.S, w.W,
                                      w.K, store=w.dtype, summaries=summ,
                                      forced_sel=forced)[(b, i)]

        compare_prefill_rows(res, np32(out[:, g * w.G:(g + 1) * w.G]),
                             sel[:, g:g + 1].cpu().numpy(), rows, wg, tally=t, rerun=rerun,
                             head_key=g)
    _say(f"   {t}")
    assert t.exact >= 0.9 * (t.exact + t.tie)
    t.check_rel(w.dtype)


def test_prefill_full_64k_sampled():
    w = synth.get_workload("prefill_64k")
    _large_sampled(w, groups=[0, 5], nrows=96, label="full 64K")


def test_prefill_full_512k_sampled():
    w = synth.get_workload("prefill_512k")
    _large_sampled(w, groups=[0, 7], nrows=48, label="full 512K")


def test_prefill_deterministic():
    w = synth.get_workload("prefill_64k", N=4096, W=512, K=16)
    x = _gpu_inputs(w)
    o1, s1, _, _ = _run_prefill(w, x)
    o2, s2, _, _ = _run_prefill(w, x)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _decode_case(w, seqlen, label="", q_route=False, seqs=None, mode="surrogate"):
    _say(f"[decode] {label} {w.name} B={w.B} T={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} "
         f"W={w.W} K={w.K} seqlen={seqlen[:4]}...")
    gen_dev = "cpu" if w.B * w.Hkv * w.N * w.d <= (1 << 26) else "cuda"
    x = synth.make_decode_inputs(w, device=gen_dev, seqlen=seqlen, with_q_route=q_route)
    x = {k: v.cuda() for k, v in x.items()}
    ks, bs = hils.summarize(x["k"], x["lm"], w.S, mode=mode)
    sel = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    out = hils.decode(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K,
                      q_route=x.get("q_route"), sel=sel, mode=mode)
    torch.cuda.synchronize()
    seqs = range(w.B) if seqs is None else seqs
    t = Tally()
    gsel = sel.cpu().numpy()
    gout = np32(out)
    for b in seqs:
        _say(f"   checking sequence {b}")
        T = int(seqlen[b])
        n = O.n_candidates(T - 1, w.W, w.S)
        kb = np32(x["k"][b:b + 1, :, :T])
        vb = np32(x["v"][b:b + 1, :, :T])
        lb = np32(x["lm"][b:b + 1, :, :max(n, 1)])
        qb = np32(x["q"][b:b + 1])
        qrb = np32(x["q_route"][b:b + 1]) if q_route else None
        summ = (O.ref_summarize(kb[:, :, :n * w.S], lb[:, :, :n], w.S, mode=mode, store=w.dtype)
                if n else None)
        # the decode query stands at position T-1 (a zero-copy broadcast view over positions)
        qq = np.broadcast_to(qb, (1, w.Hq, T, w.d))
        qr = np.broadcast_to(qrb, (1, w.Hq, T, w.d)) if q_route else None
        # decode is the prefill row i = T-1 (same definition)
        sm = summ if n else (np.zeros((1, w.Hq, 0, w.d)), np.zeros((1, w.Hq, 0)))

        def oracle(forced=None):
            return O.ref_prefill_rows(qq, kb, vb, lb, [(0, T - 1)], w.S, w.W, w.K, q_route=qr,
                                      mode=mode, store=w.dtype, summaries=sm,
                                      forced_sel=forced)[(0, T - 1)]

        r = oracle()
        t.rows += 1
        G = w.G
        for g in range(w.Hkv):
            kind = check_selection(gsel[b, g], dict(sel=r["sel"][g], gap=r["gap"][g],
                                                    s_hat=r["s_hat"][g]), w.K)
            hs = slice(g * G, (g + 1) * G)
            if kind == "exact":
                t.exact += 1
                t.add((b, g), gout[b, hs, 0], r["out"][hs], w.dtype, f"decode b={b} g={g}")
            else:
                t.tie += 1
                ids = [int(c) for c in gsel[b, g] if c >= 0]
                rr = oracle({(0, g, T - 1): ids})
                t.add((b, g), gout[b, hs, 0], rr["out"][hs], w.dtype,
                      f"decode tie b={b} g={g} (GPU selection)")
                t.tie_checked += 1
    _say(f"   {t}")
    assert t.exact >= 0.9 * (t.exact + t.tie)
    t.check_rel(w.dtype)
    return t


def test_decode_small_ragged():
    w = synth.get_workload("decode_512k", N=8192, B=4)
    _decode_case(w, [8192, 5000, 700, 1], label="ragged seqlen")


def test_decode_fp32_and_q_route():
    w = synth.get_workload("decode_512k", N=4096, B=2, dtype="f32", Hq=4, Hkv=2, d=64, K=8,
                           W=256)
    _decode_case(w, [4096, 3001], label="fp32", q_route=True)


def test_decode_full_512k_sampled_sequences():
    w = synth.get_workload("decode_512k")
    _decode_case(w, [w.N] * w.B, label="full size, 2 sequences checked", seqs=[0, 15])


def test_decode_mha_and_wide_groups():
    # G = 1 ranks raw scores; G = 8 is the widest group the kernels take
    w = synth.get_workload("decode_512k", N=8192, B=2, Hq=8, Hkv=8, K=16, W=512)
    _decode_case(w, [8192, 4097], label="G=1")
    w = synth.get_workload("decode_512k", N=8192, B=2, Hq=4, Hkv=2, K=16, W=512)
    _decode_case(w, [8192, 5000], label="G=2")
    w = synth.get_workload("decode_512k", N=8192, B=2, Hq=16, Hkv=2, K=16, W=512)
    _decode_case(w, [8192, 6001], label="G=8")
    # group sizes the selection does not specialise on (heads taken in a loop)
    w = synth.get_workload("decode_512k", N=8192, B=2, Hq=6, Hkv=2, K=16, W=512)
    _decode_case(w, [8192, 6001], label="G=3")
    w = synth.get_workload("decode_512k", N=6000, B=1, Hq=6, Hkv=1, K=100, W=300)
    _decode_case(w, [5999], label="G=6, K=100")
    # chunk size that is not a multiple of 4, window not a multiple of the chunk
    w = synth.get_workload("decode_512k", N=4400, B=2, Hq=4, Hkv=2, S=22, W=100, K=6)
    _decode_case(w, [4400, 3333], label="S=22")


def test_decode_mean_pool_and_landmark_key():
    w = synth.get_workload("decode_512k", N=8192, B=3)
    _decode_case(w, [8192, 6000, 129], label="mean_pool", mode="mean_pool")
    _decode_case(w, [8192, 6000, 129], label="landmark_key", mode="landmark_key")


def test_decode_4m_context_sampled_groups():
    # 4M-token cache, batch 1, W=2048, K=64: 65504 candidate chunks per query;
    # the oracle checks two KV groups (their own summaries, selection, output)
    w = synth.get_workload("decode_4m")
    T = w.N
    _say(f"[decode] 4M {w.name} B={w.B} T={T} Hq={w.Hq} Hkv={w.Hkv} W={w.W} K={w.K}")
    x = synth.make_decode_inputs(w, device="cuda")
    ks, bs = hils.summarize(x["k"], x["lm"], w.S)
    sel = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    out = hils.decode(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, sel=sel)
    torch.cuda.synchronize()
    n = O.n_candidates(T - 1, w.W, w.S)
    G = w.G
    t = Tally()
    t.rows = 1
    gsel, gout = sel.cpu().numpy(), np32(out)
    for g in (0, w.Hkv - 1):
        _say(f"   group {g}: oracle summaries over {n} chunks")
        hs = slice(g * G, (g + 1) * G)
        kg = np32(x["k"][:, g:g + 1])
        vg = np32(x["v"][:, g:g + 1])
        lg = np32(x["lm"][:, hs, :n])
        summ = O.ref_summarize(kg[:, :, :n * w.S], lg, w.S, store=w.dtype)
        gk = np32(ks[:, hs, :n]).astype(np.float64)
        assert int((gk != summ[0]).sum()) <= max(1, gk.size // 10**6)
        _say(f"   group {g}: oracle row {T - 1}")
        qq = np.broadcast_to(np32(x["q"][:, hs]), (1, G, T, w.d))
        r = O.ref_prefill_rows(qq, kg, vg, lg, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                               summaries=summ)[(0, T - 1)]
        kind = check_selection(gsel[0, g], dict(sel=r["sel"][0], gap=r["gap"][0],
                                                s_hat=r["s_hat"][0]), w.K)
        if kind == "exact":
            t.exact += 1
        else:
            t.tie += 1
            ids = [int(c) for c in gsel[0, g] if c >= 0]
            r = O.ref_prefill_rows(qq, kg, vg, lg, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                                   summaries=summ, forced_sel={(0, 0, T - 1): ids})[(0, T - 1)]
            t.tie_checked += 1
        t.add((0, g), gout[0, hs, 0], r["out"], w.dtype, f"4M decode group {g}")
    _say(f"   {t}")
    assert t.exact >= 1
    t.check_rel(w.dtype)


def test_decode_candidates_beyond_lds():
    # more candidate chunks than the selection kernel keeps in LDS (24576)
    w = synth.get_workload("decode_512k", N=409600, B=1, Hq=2, Hkv=1, d=64, S=16, W=256, K=8)
    _decode_case(w, [409600], label="n > 24576")


def test_decode_equal_scores_take_lowest_ids():
    # Partitioned selection (two rows, 8191 candidates: two partitions of 4096,
    # then a merge).  Sequence 0: every summary row of a head identical and
    # b' = 0, so all candidates score alike, the bound admits every key of a
    # partition (more than the 1024 ranked directly) and the radix passes pick
    # each partition's lowest ids; the merge then ranks its 32 equal keys
    # directly.  The top-K must be the K lowest chunk ids (section 3 ranking,
    # ties to the lower id).  Sequence 1 (distinct rows) takes the ranked
    # short path in both phases.
    w = synth.get_workload("decode_512k", N=524288, B=2, Hq=4, Hkv=1, K=16, W=512)
    T = w.N
    _say(f"[decode] equal scores {w.name} B={w.B} T={T} Hq={w.Hq} Hkv={w.Hkv} K={w.K}")
    x = synth.make_decode_inputs(w, device="cuda", seqlen=[T, T])
    ks, bs = hils.summarize(x["k"], x["lm"], w.S)
    ks[0] = ks[0, :, :1].expand(-1, ks.shape[2], -1).clone()
    bs[0] = 0.0
    sel = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    out = hils.decode(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, sel=sel)
    torch.cuda.synchronize()
    n = O.n_candidates(T - 1, w.W, w.S)
    assert n > 4096
    gsel, gout = sel.cpu().numpy(), np32(out)
    assert (gsel[0] == np.arange(w.K)[None, :]).all(), gsel[0]
    t = Tally()
    for b in range(w.B):
        _say(f"   checking sequence {b}")
        kb, vb = np32(x["k"][b:b + 1]), np32(x["v"][b:b + 1])
        lb = np32(x["lm"][b:b + 1, :, :n])
        summ = (np32(ks[b:b + 1, :, :n]).astype(np.float64), np32(bs[b:b + 1, :, :n]).astype(np.float64))
        qq = np.broadcast_to(np32(x["q"][b:b + 1]), (1, w.Hq, T, w.d))
        r = O.ref_prefill_rows(qq, kb, vb, lb, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                               summaries=summ)[(0, T - 1)]
        t.rows += 1
        for g in range(w.Hkv):
            hs = slice(g * w.G, (g + 1) * w.G)
            if b == 0:
                assert list(r["sel"][g]) == list(range(w.K))
            kind = check_selection(gsel[b, g], dict(sel=r["sel"][g], gap=r["gap"][g],
                                                    s_hat=r["s_hat"][g]), w.K)
            rr = r
            if kind == "exact":
                t.exact += 1
            else:
                t.tie += 1
                ids = [int(c) for c in gsel[b, g] if c >= 0]
                rr = O.ref_prefill_rows(qq, kb, vb, lb, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                                        summaries=summ, forced_sel={(0, g, T - 1): ids})[(0, T - 1)]
                t.tie_checked += 1
            t.add((b, g), gout[b, hs, 0], rr["out"][hs], w.dtype, f"equal-score decode b={b} g={g}")
    _say(f"   {t}")
    t.check_rel(w.dtype)


def test_decode_partitioned_selection():
    # 299999 candidate chunks, K = 128: the selection runs as partitions of
    # 5120 chunks (the 128-key lists of at most 64 partitions fit one merge),
    # then one merge; a shorter sequence takes fewer partitions
    w = synth.get_workload("decode_512k", N=300000, B=2, Hq=2, Hkv=1, d=32, S=1, W=1, K=128,
                           regime="iid")
    _decode_case(w, [300000, 7000], label="partitioned selection")
