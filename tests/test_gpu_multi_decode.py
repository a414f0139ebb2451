"""GPU parity of the multi-token decode (hils_decode_multi) against the oracle.

A block of M new tokens per sequence; token m is the prefill row at position
T_b - M + m.  Inputs come from the seeded generators in synth/, expected values
only from oracle/.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import hils_oracle as O
from tests.parity_util import Tally, check_selection, np32

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import chunk_wise_hierarchical_amd as hils


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(w, M, seqlen, q_route=False, seed=11, corr=0.0):
    gen_dev = "cpu" if w.B * w.Hkv * w.N * w.d <= (1 << 26) else "cuda"
    x = synth.make_decode_inputs(w, device=gen_dev, seqlen=seqlen, with_q_route=q_route)
    x = {k: v.cuda() for k, v in x.items()}
    # M query rows per sequence: the generator's decode query (with its planted
    # structure) for the last token, seeded normals of the same scale before it
    g = torch.Generator(device="cpu").manual_seed(seed)
    f = (1.0 / w.d ** 0.5) if w.scaled else 1.0
    qm = (torch.randn((w.B, w.Hq, M, w.d), generator=g) * f).cuda()
    if corr > 0.0:                 # the block's queries share most of their direction
        qm = qm * (1.0 - corr) ** 0.5 + x["q"][:, :, 0:1].float() * corr ** 0.5
    qm = qm.to(x["q"].dtype)
    qm[:, :, M - 1] = x["q"][:, :, 0]
    x["qm"] = qm.contiguous()
    if q_route:
        qrm = (torch.randn((w.B, w.Hq, M, w.d), generator=g) * 0.25 * f).cuda()
        x["qrm"] = (qm.float() + qrm).to(x["q"].dtype).contiguous()
    return x


def _multi_case(w, M, seqlen, label="", q_route=False, mode="surrogate", seqs=None, corr=0.0):
    _say(f"[decode_multi] {label} {w.name} B={w.B} T={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
         f"S={w.S} W={w.W} K={w.K} M={M} seqlen={seqlen[:4]} dtype={w.dtype} mode={mode}")
    x = _inputs(w, M, seqlen, q_route, corr=corr)
    ks, bs = hils.summarize(x["k"], x["lm"], w.S, mode=mode)
    sel = torch.empty((w.B, w.Hkv, M, w.K), dtype=torch.int32, device="cuda")
    out = hils.decode_multi(x["qm"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K,
                            q_route=x.get("qrm"), sel=sel, mode=mode)
    torch.cuda.synchronize()
    gsel, gout = sel.cpu().numpy(), np32(out)
    t = Tally()
    G = w.G
    for b in (range(w.B) if seqs is None else seqs):
        T = int(seqlen[b])
        nmx = max(O.n_candidates(max(T - M + m, 0), w.W, w.S) for m in range(M))
        qb = np32(x["qm"][b:b + 1])
        qrb = np32(x["qrm"][b:b + 1]) if q_route else None
        res = O.ref_decode_multi(qb, np32(x["k"][b:b + 1, :, :T]), np32(x["v"][b:b + 1, :, :T]),
                                 [T], np32(x["lm"][b:b + 1, :, :max(nmx, 1)]), w.S, w.W, w.K,
                                 q_route=qrb, mode=mode, store=w.dtype)
        for m in range(M):
            r = res[(0, m)]
            t.rows += 1
            for g in range(w.Hkv):
                kind = check_selection(gsel[b, g, m], dict(sel=r["sel"][g], gap=r["gap"][g],
                                                           s_hat=r["s_hat"][g]), w.K)
                hs = slice(g * G, (g + 1) * G)
                if kind == "exact":
                    t.exact += 1
                    t.add((b, m, g), gout[b, hs, m], r["out"][hs], w.dtype, f"b={b} m={m} g={g}")
                else:
                    t.tie += 1
                    rr = _forced_token(x, w, b, T, M, m, mode, q_route,
                                       {g: [int(c) for c in gsel[b, g, m] if c >= 0]})
                    t.add((b, m, g), gout[b, hs, m], rr["out"][hs], w.dtype,
                          f"tie b={b} m={m} g={g} (GPU selection)")
                    t.tie_checked += 1
    _say(f"   {t}")
    assert t.exact >= 0.9 * (t.exact + t.tie)
    t.check_rel(w.dtype)
    return out, sel


def _forced_token(x, w, b, T, M, m, mode, q_route, forced):
    """Oracle output of token m of sequence b (the prefill row at its position,
    section 3) with the selections of the groups in `forced` held fixed."""
    i = max(T - M + m, 0)
    n = O.n_candidates(i, w.W, w.S)
    qq = np.broadcast_to(np32(x["qm"][b:b + 1, :, m:m + 1]), (1, w.Hq, i + 1, w.d))
    qr = (np.broadcast_to(np32(x["qrm"][b:b + 1, :, m:m + 1]), (1, w.Hq, i + 1, w.d))
          if q_route else None)
    kb, vb = np32(x["k"][b:b + 1, :, :i + 1]), np32(x["v"][b:b + 1, :, :i + 1])
    lb = np32(x["lm"][b:b + 1, :, :max(n, 1)])
    summ = (O.ref_summarize(kb[:, :, :n * w.S], lb[:, :, :n], w.S, mode=mode, store=w.dtype)
            if n else (np.zeros((1, w.Hq, 0, w.d)), np.zeros((1, w.Hq, 0))))
    return O.ref_prefill_rows(qq, kb, vb, lb, [(0, i)], w.S, w.W, w.K, q_route=qr, mode=mode,
                              store=w.dtype, summaries=summ,
                              forced_sel={(0, g, i): s for g, s in forced.items()})[(0, i)]


def test_multi_decode_gqa_ragged():
    # 4 tokens per sequence, GQA 4:1, ragged lengths (one without candidates)
    w = synth.get_workload("decode_512k", N=8192, B=3)
    _multi_case(w, 4, [8192, 6001, 700], label="M=4")


def test_multi_decode_seven_tokens_groups_and_fp32():
    # M = 7: two query groups in the scoring pass, the second partial
    w = synth.get_workload("decode_512k", N=4096, B=2, Hq=8, Hkv=8, K=16, W=512)
    _multi_case(w, 7, [4096, 3000], label="G=1 M=7")
    w = synth.get_workload("decode_512k", N=4096, B=2, Hq=16, Hkv=2, K=16, W=512)
    _multi_case(w, 7, [4096, 2222], label="G=8 M=7")
    w = synth.get_workload("decode_512k", N=4096, B=2, dtype="f32", Hq=4, Hkv=2, d=64, K=8, W=256)
    _multi_case(w, 5, [4096, 3001], label="fp32 q_route M=5", q_route=True)


def test_multi_decode_max_block_short_sequence_and_mean_pool():
    w = synth.get_workload("decode_512k", N=2048, B=2, Hq=4, Hkv=2, d=64, S=32, W=128, K=8)
    _multi_case(w, 16, [2048, 1333], label="M=16")
    # a sequence shorter than the block: positions below 0 are evaluated at 0
    _multi_case(w, 4, [2048, 2], label="seqlen < M")
    _multi_case(w, 3, [2048, 999], label="mean_pool", mode="mean_pool")


def test_multi_decode_union_at_its_limits():
    # bf16, d=128, S=64 blocks take the union attention (one load per distinct
    # chunk or window tile of the block): M*K at its limit of 1024 ids, G = 2,
    # a sequence shorter than the block (positions clamp at 0) and one whose
    # tokens straddle a chunk boundary; then G = 1 with correlated queries, so
    # that many chunks are shared by several tokens
    w = synth.get_workload("decode_512k", N=8192, B=3, Hq=8, Hkv=4, K=64, W=512)
    _multi_case(w, 16, [8192, 5000 + 70, 9], label="M=16 K=64 G=2")
    w = synth.get_workload("decode_512k", N=8192, B=2, Hq=4, Hkv=4, K=32, W=1024)
    _multi_case(w, 8, [8192, 6400 + 3], label="M=8 G=1", corr=0.9)


def test_multi_decode_one_token_is_decode():
    # M = 1 runs the single-step decode: identical outputs and selections
    w = synth.get_workload("decode_512k", N=8192, B=4)
    x = _inputs(w, 1, [8192, 5000, 700, 1])
    ks, bs = hils.summarize(x["k"], x["lm"], w.S)
    s1 = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    s2 = torch.empty((w.B, w.Hkv, 1, w.K), dtype=torch.int32, device="cuda")
    o1 = hils.decode(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, sel=s1)
    o2 = hils.decode_multi(x["qm"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, sel=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2[:, :, 0])


def test_multi_decode_full_512k_two_sequences():
    # the 512K decode workload with a 4-token block; two sequences checked
    w = synth.get_workload("decode_512k")
    _multi_case(w, 4, [w.N] * w.B, label="512K M=4", seqs=[0, 15])
