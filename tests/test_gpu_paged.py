"""Paged-KV decode (one chunk per page) against the contiguous decode and the
oracle, and a decode step captured into a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import synth
import chunk_wise_hierarchical_amd as hils
from oracle import hils_oracle as O
from parity_util import check_selection, out_error

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _paged_copy(w, x, seqlen, seed=3):
    """Scatter a contiguous cache into randomly permuted pages; table entries of
    chunks past a sequence's tokens and the spare pages hold junk."""
    B, Hkv, N, d = x["k"].shape
    S = w.S
    maxp = N // S
    g = torch.Generator().manual_seed(seed)
    P = B * maxp + 5
    perm = torch.randperm(P, generator=g)
    table = torch.full((B, maxp), -7, dtype=torch.int32)
    k_pages = torch.randn((P, Hkv, S, d), generator=g).to(x["k"].dtype).cuda()
    v_pages = torch.randn((P, Hkv, S, d), generator=g).to(x["k"].dtype).cuda()
    lm_pages = torch.randn((P, w.Hq, d), generator=g).to(x["k"].dtype).cuda()
    used = []
    for b in range(B):
        nchunk = (int(seqlen[b]) + S - 1) // S
        for c in range(nchunk):
            p = int(perm[b * maxp + c])
            table[b, c] = p
            k_pages[p] = x["k"][b, :, c * S:(c + 1) * S]
            v_pages[p] = x["v"][b, :, c * S:(c + 1) * S]
            if c < x["lm"].shape[2]:
                lm_pages[p] = x["lm"][b, :, c]
                if (c + 1) * S <= int(seqlen[b]):
                    used.append(p)
        if nchunk < maxp:
            table[b, nchunk:] = 10 ** 9          # never read
    return table.cuda(), k_pages, v_pages, lm_pages, torch.tensor(used, dtype=torch.int32).cuda()


def _case(w, lens):
    x = {k: v.cuda() for k, v in synth.make_decode_inputs(w, device="cpu", seqlen=lens).items()}
    seqlen = x["seqlen"]
    ks, bs = hils.summarize(x["k"], x["lm"], w.S)
    sel_c = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    out_c = hils.decode(x["q"], x["k"], x["v"], seqlen, ks, bs, w.S, w.W, w.K, sel=sel_c)
    table, kp, vp, lmp, used = _paged_copy(w, x, lens)
    ksp, bsp = hils.summarize_paged(kp, lmp, used, w.S, w.N)
    return x, seqlen, (ks, bs, out_c, sel_c), (table, kp, vp, ksp, bsp)


def test_paged_decode_equals_contiguous_and_oracle():
    w = synth.get_workload("decode_512k", N=8192, B=3)
    lens = [8192, 5000, 1500]
    _say(f"[paged] B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} W={w.W} K={w.K} seqlen={lens}")
    x, seqlen, (ks, bs, out_c, sel_c), (table, kp, vp, ksp, bsp) = _case(w, lens)
    # page summaries equal the contiguous ones, chunk by chunk
    tab = table.cpu().numpy()
    for b, T in enumerate(lens):
        for c in range(T // w.S):
            assert torch.equal(ksp[tab[b, c]], ks[b, :, c]), (b, c)
            assert torch.equal(bsp[tab[b, c]], bs[b, :, c]), (b, c)
    sel_p = torch.empty_like(sel_c)
    out_p = hils.decode_paged(x["q"], kp, vp, table, seqlen, ksp, bsp, w.S, w.W, w.K, sel=sel_p)
    torch.cuda.synchronize()
    assert torch.equal(sel_p, sel_c)
    assert torch.equal(out_p, out_c)
    # and the oracle, sequence 1 (ragged length)
    b, T = 1, lens[1]
    n = O.n_candidates(T - 1, w.W, w.S)
    f = lambda t: t.float().cpu().numpy()
    kb, vb = f(x["k"][b:b + 1, :, :T]), f(x["v"][b:b + 1, :, :T])
    lb = f(x["lm"][b:b + 1, :, :n])
    summ = O.ref_summarize(kb[:, :, :n * w.S], lb, w.S, store=w.dtype)
    qq = np.broadcast_to(f(x["q"][b:b + 1]), (1, w.Hq, T, w.d))
    r = O.ref_prefill_rows(qq, kb, vb, lb, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                           summaries=summ)[(0, T - 1)]
    gsel = sel_p.cpu().numpy()
    for g in range(w.Hkv):
        kind = check_selection(gsel[b, g], dict(sel=r["sel"][g], gap=r["gap"][g],
                                               s_hat=r["s_hat"][g]), w.K)
        rg = r
        if kind != "exact":      # a valid alternative in the tie band: the oracle on it
            ids = [int(c) for c in gsel[b, g] if c >= 0]
            rg = O.ref_prefill_rows(qq, kb, vb, lb, [(0, T - 1)], w.S, w.W, w.K, store=w.dtype,
                                    summaries=summ, forced_sel={(0, g, T - 1): ids})[(0, T - 1)]
        hs = slice(g * w.G, (g + 1) * w.G)
        err, tol = out_error(f(out_p[b, hs, 0]), rg["out"][hs], w.dtype)
        assert err <= tol, (g, err, tol)
    _say("   paged decode identical to contiguous decode; oracle agrees")


def test_paged_decode_graph_replay():
    w = synth.get_workload("decode_512k", N=4096, B=2)
    lens = [4096, 3001]
    x, seqlen, _, (table, kp, vp, ksp, bsp) = _case(w, lens)
    q = x["q"].clone()
    out = torch.empty_like(q)
    sel = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    cfg = hils.make_cfg(w.B, table.shape[1] * w.S, w.Hq, w.Hkv, w.d, w.S, w.W, w.K, q.dtype)
    ws = torch.empty(hils.workspace_bytes(cfg, True), dtype=torch.uint8, device="cuda")

    def step():
        hils.decode_paged(q, kp, vp, table, seqlen, ksp, bsp, w.S, w.W, w.K, out=out, sel=sel, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(11)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_out, got_sel = out.clone(), sel.clone()
        step()                                 # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_sel, sel), rep
        assert torch.equal(got_out, out), rep
    _say("   4 graph replays identical to eager decode")
