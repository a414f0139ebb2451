#!/usr/bin/env python3
"""HiLS attention forward on one MI355X: prefill tokens/s and decode steps/s at 512K context.

A step is one HiLS prefill of the prefill workload (summaries, scoring and
top-K, window + selected-chunk attention, fusion); the decode workload's
single-step decode is timed in the same run and reported under "decode".
Inputs are seeded synthetic tensors (synth/) already resident in HBM when the
timed region starts.  Headline times are taken with the library's kernel
timing off; a second timed pass with it on (HIP events the library records
around each kernel on the kernel's own stream, hils_profile_enable) gives the
per-kernel table and the rooflines.  After the headline prefill and decode
workloads, further workloads are timed the same way ("more_workloads": the
64K GQA and 8K MHA prefills and the 4M-token decode by default).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_512k]
                    [--decode-workload decode_512k] [--decode-steps 50] [--no-cpu]
                    [--calibrate-copy]

`roofline.traffic` is the dominant kernel's HBM bytes per launch measured with
rocprofv3 FETCH_SIZE and WRITE_SIZE counters (profiles/*_pmc.md), scaled by
what the same counters read for a plain 1 GiB copy kernel (--calibrate-copy
runs that copy first so one profiled command holds both).  It is reported
only while the kernel's sources still hash to the value recorded with the
counters, and is null otherwise.
"""
import hashlib
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# fp32 vector peak without packed-fp32 instructions (which this build turns off):
# 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP (FMA) x 2.4 GHz = 78.6 TFLOP/s
PEAK_FP32_VALU_TFLOPS = 78.6


def _geometry(N, W, S):
    i = np.arange(N, dtype=np.int64)
    left = np.floor_divide(i - W + 1, S) * S
    n = np.maximum(0, left // S)
    win = i - np.maximum(0, left) + 1
    return n, win


def prefill_work(w):
    """Algorithmic FLOPs: (scoring, summaries, attention) for one prefill."""
    n, win = _geometry(w.N, w.W, w.S)
    score = 2.0 * w.d * float(n.sum()) * w.Hq * w.B
    summ = 4.0 * w.B * w.Hq * (w.N // w.S) * w.S * w.d
    attn = 4.0 * w.d * float((np.minimum(w.K, n) * w.S + win).sum()) * w.Hq * w.B
    return score, summ, attn


def window_work(w):
    """Algorithmic FLOPs of the attention split into (window part, selected-chunk part)."""
    n, win = _geometry(w.N, w.W, w.S)
    win_f = 4.0 * w.d * float(win.sum()) * w.Hq * w.B
    sel_f = 4.0 * w.d * float((np.minimum(w.K, n) * w.S).sum()) * w.Hq * w.B
    return win_f, sel_f


def decode_work(w, T):
    """Algorithmic HBM bytes of one decode step (all sequences at length T), and the
    bytes of the scoring launch (k', b' read, scores written; for bf16 d=128 S=64
    single-token steps it also carries the window tiles' K and V)."""
    n, win = _geometry(T, w.W, w.S)
    n, win = int(n[-1]), int(win[-1])
    e = 2 if w.dtype == "bf16" else 4
    win_bytes = w.Hkv * win * w.d * e * 2
    per_seq = (w.Hq * n * (w.d * e + 4) + w.Hkv * min(w.K, n) * w.S * w.d * e * 2
               + win_bytes + 2 * w.Hq * w.d * e)
    score_bytes = w.B * w.Hq * n * (w.d * e + 4 + 4)
    if w.dtype == "bf16" and w.d == 128 and w.S == 64 and w.G in (1, 2, 4):
        score_bytes += w.B * win_bytes
    return per_seq * w.B, score_bytes


# sources whose text decides each kernel's code (for the counter staleness check)
KERNEL_SOURCES = {
    "k_attn_fast": ["fast_attn.hip", "fast_common.h", "hils_device.h"],
    "k_score_fast": ["fast_score.hip", "fast_common.h", "hils_device.h"],
    "k_pair_attn": ["fast_pairs.hip", "fast_common.h", "hils_device.h", "hils_internal.h"],
    "k_win_fuse": ["fast_pairs.hip", "fast_common.h", "hils_device.h", "hils_internal.h"],
    "k_dec_score": ["decode.hip", "fast_common.h", "hils_device.h", "hils_internal.h"],
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "chunk_wise_hierarchical_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>_<workload>_pmc.md, or None
    when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("- ") and ":" in ln:
                k, v = ln[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(torch, dev, log):
    """A plain device copy of 1 GiB (fp32 elementwise kernel), three times, so a
    rocprofv3 counter run can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x {n * 4} bytes read and written")
    del a, b


def timed(torch, _lib, fn, steps, profile, group=16, median=False):
    """ms per call of fn over `steps` calls, timed between HIP events on the
    current stream in groups of at most `group` calls with the host
    synchronised between groups (the time between a group's two events is
    device time: the host enqueues far faster than the device runs).  The
    result is the mean over all calls, or with median=True the median of the
    groups' per-call times: sub-millisecond steps are exposed to rare stalls of
    the host's enqueueing (tens of ms, seen in kernel traces as gaps inside an
    otherwise back-to-back group), which the median of short groups ignores.
    With profile=True the library also brackets every kernel with HIP events
    (hils_profile_enable) and the per-kernel table is returned; the headline
    numbers come from runs with profile=False."""
    torch.cuda.synchronize()
    if profile:
        _lib.profile_enable(True)
        _lib.profile_read()
    total = 0.0
    per_group = []
    done = 0
    while done < steps:
        n = min(group, steps - done)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        total += t
        per_group.append(t / n)
        done += n
    ms = float(np.median(per_group)) if median else total / steps
    kt = None
    if profile:
        kt = _kernel_table(_lib.profile_read(), steps)
        _lib.profile_enable(False)
    return ms, kt


def _kernel_table(records, steps):
    agg = {}
    for name, ms in records:
        a = agg.setdefault(name, [0.0, 0])
        a[0] += ms
        a[1] += 1
    return {k: {"ms_per_step": v[0] / steps, "calls": v[1], "avg_ms": v[0] / v[1]} for k, v in agg.items()}


def pair_path_bytes(sel, w, launches):
    """Design-traffic bytes per prefill of the chunk-bucket path's pair
    attention and fused window + fusion kernel, from the selection sel
    [B,Hkv,N,K] (-1 padded).  Pair attention, per (query, KV group, selected
    chunk) pair: the G gathered query rows and the G bf16 per-chunk output rows
    (G*d*2 B each), G fp32 fusion logits and the 4-byte list entry; per
    (slice, KV group, chunk) bucket: the chunk's K and V^T (S*d*2 B each), k'
    (G*d*2 B) and b' (G*4 B).  Window + fusion, per pair: the G output rows and
    logits read back; per (query, head): its query row read and the bf16
    output written (the window's K/V tiles are shared through L2)."""
    import torch
    B, Hkv, N, K = sel.shape
    G, d, S = w.G, w.d, w.S
    nC = max(N // S, 1)
    qs = -(-N // int(round(launches)))
    pairs, buckets = 0, 0
    bgi = torch.arange(B * Hkv, device=sel.device, dtype=torch.int64).view(B, Hkv, 1, 1)
    for i0 in range(0, N, qs):
        s = sel[:, :, i0:i0 + qs]
        v = s >= 0
        pairs += int(v.sum())
        buckets += int(torch.unique((bgi * nC + s.long())[v]).numel())
    attn = pairs * (2 * G * d * 2 + G * 4 + 4) + buckets * (2 * S * d * 2 + G * d * 2 + G * 4)
    red = pairs * G * (d * 2 + 4) + B * Hkv * N * G * (d * 2 + d * 2)
    return float(attn), float(red)


def _overlap(sel, K, M=16, blocks=64):
    """Normalised chunk overlap of M adjacent queries (section 7.2) over the
    last `blocks` full blocks of KV group 0 (rows with at least K candidates)."""
    s = sel[0, 0].cpu().numpy()
    N = s.shape[0]
    vals = []
    for bidx in range(blocks):
        hi = N - bidx * M
        blk = s[hi - M:hi]
        if (blk < 0).any():
            break
        u = len(set(blk.ravel().tolist()))
        vals.append((M * K - u) / ((M - 1) * K))
    return float(np.mean(vals)) if vals else None


def cpu_baseline_prefill(x, w, rows=4096):
    """Oracle on one KV group: summaries of every chunk + `rows` query rows;
    full-prefill time extrapolated to all groups and positions."""
    from threadpoolctl import threadpool_limits
    from oracle import hils_oracle as O
    G = w.G
    with threadpool_limits(1):
        qg = x["q"][:, :G].float().cpu().numpy()
        kg = x["k"][:, :1].float().cpu().numpy()
        vg = x["v"][:, :1].float().cpu().numpy()
        lg = x["lm"][:, :G].float().cpu().numpy()
        t0 = time.perf_counter()
        summ = O.ref_summarize(kg, lg, w.S, store=w.dtype)
        t1 = time.perf_counter()
        idx = np.linspace(w.W + w.S, w.N - 1, rows).astype(int)
        O.ref_prefill_rows(qg, kg, vg, lg, [(0, int(i)) for i in idx], w.S, w.W, w.K,
                           store=w.dtype, summaries=summ)
        t2 = time.perf_counter()
    t_full = w.Hkv * w.B * ((t1 - t0) + (t2 - t1) * w.N / rows)
    return {"value": w.B * w.N / t_full, "unit": "tokens/s", "cores": 1,
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": (f"KV group 0 of {w.Hkv}: summaries of all {w.N // w.S} chunks "
                       f"({t1 - t0:.1f} s) + {rows} query rows spread over the sequence "
                       f"({t2 - t1:.1f} s); full prefill extrapolated = {w.Hkv * w.B} groups x "
                       f"(summaries + rows x {w.N}/{rows}) = {t_full:.0f} s; NumPy float64, 1 BLAS thread "
                       f"(host has {os.cpu_count()} cores)")}


def cpu_baseline_decode(xd, wd, nseq=8):
    """Oracle decode step (scoring over the summary cache, top-K, window and
    chunk attention, fusion) of every KV group of `nseq` sequences; each summary
    cache is computed first by the oracle and, as on the GPU, not timed.  The
    step is the prefill row i = T - 1 (same definition)."""
    from threadpoolctl import threadpool_limits
    from oracle import hils_oracle as O
    G = wd.G
    T = wd.N
    n = O.n_candidates(T - 1, wd.W, wd.S)
    ts = tsum = 0.0
    nseq = min(nseq, wd.B)
    with threadpool_limits(1):
        for b in range(nseq):
            for g in range(wd.Hkv):
                hs = slice(g * G, (g + 1) * G)
                q = xd["q"][b:b + 1, hs].float().cpu().numpy()
                k = xd["k"][b:b + 1, g:g + 1].float().cpu().numpy()
                v = xd["v"][b:b + 1, g:g + 1].float().cpu().numpy()
                lm = xd["lm"][b:b + 1, hs, :n].float().cpu().numpy()
                t0 = time.perf_counter()
                summ = O.ref_summarize(k[:, :, :n * wd.S], lm, wd.S, store=wd.dtype)
                tsum += time.perf_counter() - t0
                qq = np.broadcast_to(q, (1, G, T, wd.d))
                t0 = time.perf_counter()
                O.ref_prefill_rows(qq, k, v, lm, [(0, T - 1)], wd.S, wd.W, wd.K, store=wd.dtype,
                                   summaries=summ)
                ts += time.perf_counter() - t0
    t_step = ts * wd.B / nseq
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": 1,
            "host_cores": os.cpu_count(), "kind": "oracle",
            "sample": (f"all {wd.Hkv} KV groups of sequences 0..{nseq - 1}: {ts:.2f} s for their "
                       f"single-token steps over {n}-chunk summary caches (the caches, "
                       f"{tsum:.1f} s, built by the oracle beforehand and not timed, as on the "
                       f"GPU); step time extrapolated x {wd.B}/{nseq} sequences = {t_step:.2f} s; "
                       f"NumPy float64, 1 BLAS thread "
                       f"(host has {os.cpu_count()} cores)")}


def paged_decode_bench(torch, hils, _lib, xd, wd, ks, bs, steps, log):
    """Decode over a paged copy of the cache: pages hold one chunk each and are
    placed by a random permutation; the page summaries are built with
    hils_summarize_paged.  Times the step eagerly and as a replayed graph."""
    B, Hkv, T, d = xd["k"].shape
    S = wd.S
    maxp = T // S
    P = B * maxp
    dev = xd["k"].device
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).to(dev)
    table = perm.view(B, maxp).to(torch.int32).contiguous()

    def paged(t, heads):                       # [B,H,T,d] -> [P,H,S,d] at the permuted slots
        lg = t.view(B, heads, maxp, S, d).permute(0, 2, 1, 3, 4).reshape(P, heads, S, d)
        out = torch.empty_like(lg)
        out[perm] = lg
        return out

    kp, vp = paged(xd["k"], Hkv), paged(xd["v"], Hkv)
    lmp = torch.empty((P, wd.Hq, d), dtype=xd["lm"].dtype, device=dev)
    lmp[perm] = xd["lm"].permute(0, 2, 1, 3).reshape(P, wd.Hq, d)
    ksp, bsp = hils.summarize_paged(kp, lmp, perm.to(torch.int32), S, T)
    torch.cuda.synchronize()
    same = bool(torch.equal(ksp[perm].view(B, maxp, wd.Hq, d).permute(0, 2, 1, 3), ks))
    out = torch.empty_like(xd["q"])
    sel = torch.empty((B, Hkv, wd.K), dtype=torch.int32, device=dev)
    cfg = hils.make_cfg(B, T, wd.Hq, Hkv, d, S, wd.W, wd.K, xd["q"].dtype)
    ws = torch.empty(max(1, hils.workspace_bytes(cfg, True)), dtype=torch.uint8, device=dev)

    def step():
        hils.decode_paged(xd["q"], kp, vp, table, xd["seqlen"], ksp, bsp, S, wd.W, wd.K,
                          out=out, sel=sel, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager_ms, _ = timed(torch, _lib, step, steps, profile=False, group=8, median=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    graph_ms, _ = timed(torch, _lib, graph.replay, steps, profile=False, group=8, median=True)
    log(f"paged decode {eager_ms:.3f} ms/step eager, {graph_ms:.3f} ms/step graph replay "
        f"({P} pages; page summaries identical to contiguous: {same})")
    del kp, vp, lmp, ksp, bsp, ws, graph
    return {"pages": P, "page_tokens": S, "ms_per_step": eager_ms, "steps_per_s": 1000.0 / eager_ms,
            "graph_ms_per_step": graph_ms, "graph_steps_per_s": 1000.0 / graph_ms,
            "page_summaries_identical": same}


def multi_decode_bench(torch, hils, _lib, xd, wd, ks, bs, M, steps, log, corr=0.0):
    """Decode of a block of M new tokens per sequence (the cache already holds
    them; token m at position T - M + m).  The per-step summary read is shared
    by the block's tokens, so tokens/s should grow with M at nearly the
    single-step cost.  The block's earlier queries are seeded normals; with
    corr > 0 they share that fraction of their variance with the last token's
    query (adjacent positions route to overlapping chunks, section 7.2)."""
    B, Hq, _, d = xd["q"].shape
    g = torch.Generator(device="cpu").manual_seed(17)
    noise = torch.randn((B, Hq, M, d), generator=g).to(xd["q"].device)
    last = xd["q"][:, :, 0:1].float()
    qm = (noise * math.sqrt(1.0 - corr) + last * math.sqrt(corr)).to(xd["q"].dtype)
    qm[:, :, M - 1] = xd["q"][:, :, 0]
    qm = qm.contiguous()
    out = torch.empty_like(qm)
    sel = torch.empty((B, wd.Hkv, M, wd.K), dtype=torch.int32, device=qm.device)
    cfg = hils.make_cfg(B, wd.N, wd.Hq, wd.Hkv, d, wd.S, wd.W, wd.K, qm.dtype)
    ws = torch.empty(max(1, _lib.lib().hils_decode_multi_workspace_bytes(ctypes.byref(cfg), M)),
                     dtype=torch.uint8, device=qm.device)

    def step():
        hils.decode_multi(qm, xd["k"], xd["v"], xd["seqlen"], ks, bs, wd.S, wd.W, wd.K, out=out,
                          sel=sel, ws=ws)

    for _ in range(3):
        step()
    ms, _ = timed(torch, _lib, step, steps, profile=False, group=8, median=True)
    _, kt = timed(torch, _lib, step, steps, profile=True)
    s_np = sel.cpu().numpy()
    union = float(np.mean([len(set(s_np[b, gg].ravel().tolist()) - {-1})
                           for b in range(B) for gg in range(wd.Hkv)]))
    log(f"decode block of {M} tokens (query correlation {corr}) {ms:.3f} ms/step; distinct chunks "
        f"per (sequence, KV group) {union:.1f}; kernels {json.dumps(kt)}")
    del ws, out, sel, qm
    return {"M": M, "query_correlation": corr, "ms_per_step": ms, "steps_per_s": 1000.0 / ms,
            "tokens_per_s": B * M * 1000.0 / ms, "distinct_chunks_per_group": union,
            "kernels": kt}


def backward_bench(torch, hils, _lib, wb, steps, log):
    """Prefill backward (selection held fixed) on a training-length workload:
    forward once for the selection, then time the backward."""
    import synth
    xb = synth.make_prefill_inputs(wb, device="cuda")
    sel = torch.empty((wb.B, wb.Hkv, wb.N, wb.K), dtype=torch.int32, device="cuda")
    ks = torch.empty((wb.B, wb.Hq, wb.N // wb.S, wb.d), dtype=xb["q"].dtype, device="cuda")
    bs = torch.empty((wb.B, wb.Hq, wb.N // wb.S), dtype=torch.float32, device="cuda")
    hils.prefill(xb["q"], xb["k"], xb["v"], xb["lm"], wb.S, wb.W, wb.K, sel=sel, summaries=(ks, bs))
    g = torch.Generator(device="cuda").manual_seed(9)
    dout = torch.randn(xb["q"].shape, generator=g, device="cuda").to(xb["q"].dtype)
    cfg = hils.make_cfg(wb.B, wb.N, wb.Hq, wb.Hkv, wb.d, wb.S, wb.W, wb.K, xb["q"].dtype)
    ws = torch.empty(_lib.lib().hils_prefill_backward_workspace_bytes(ctypes.byref(cfg)),
                     dtype=torch.uint8, device="cuda")

    def step():
        return hils.prefill_backward(xb["q"], xb["k"], xb["v"], xb["lm"], dout, sel, wb.S, wb.W,
                                     wb.K, summaries=(ks, bs), ws=ws)

    for _ in range(2):
        step()
    ms, _ = timed(torch, _lib, step, steps, profile=False)
    _, kt = timed(torch, _lib, step, steps, profile=True)
    # algorithmic FLOPs: per attended (query, head, token) the five products of an
    # attention backward (logit and dout.v recompute, dq, dk, dv): 10 d.  For bf16
    # with d in {64, 128} and S a multiple of 16 all five run on the matrix cores
    # (priced against the bf16 MFMA peak), else on the fp32 vector ALU.
    n, win = _geometry(wb.N, wb.W, wb.S)
    att = float((np.minimum(wb.K, n) * wb.S + win).sum()) * wb.Hq * wb.B
    flops = 10.0 * wb.d * att
    achieved = flops / (ms * 1e-3) / 1e12
    on_mfma = wb.dtype == "bf16" and wb.d in (64, 128) and wb.S % 16 == 0
    bound, peak = ("mfma", PEAK_BF16_TFLOPS) if on_mfma else ("alu", PEAK_FP32_VALU_TFLOPS)
    log(f"backward {wb.name}: {ms:.2f} ms/step; kernels {json.dumps(kt)}")
    del xb, sel, ks, bs, dout, ws
    return {"workload": wb.name, "ms_per_step": ms, "tokens_per_s": wb.B * wb.N / (ms * 1e-3),
            "config": {"B": wb.B, "N": wb.N, "Hq": wb.Hq, "Hkv": wb.Hkv, "d": wb.d, "S": wb.S,
                       "W": wb.W, "K": wb.K},
            "roofline": {"bound": bound, "achieved": achieved, "peak": peak,
                         "unit": "TFLOP/s", "frac": achieved / peak,
                         "algorithmic_flops_per_step": flops},
            "kernels": kt}


def prefill_bench(torch, hils, _lib, w, steps, warmup, union, log, want_sel=False):
    """One workload's prefill: the headline time with the library's kernel
    timing off, then a second timed pass with it on for the per-kernel table
    and the rooflines.  Rooflines are useful (algorithmic) FLOPs against the
    bf16 MFMA peak: per kernel (FLOPs per launch over the kernel's average
    launch time) and for the whole step."""
    dev = torch.device("cuda:0")
    log(f"prefill inputs {w.name}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} "
        f"W={w.W} K={w.K}")
    x = synth_inputs(w, dev)
    out = torch.empty_like(x["q"])
    sel = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.int32, device=dev)
    cfg = hils.make_cfg(w.B, w.N, w.Hq, w.Hkv, w.d, w.S, w.W, w.K, x["q"].dtype, union=union)
    ws = torch.empty(max(1, hils.workspace_bytes(cfg, False)), dtype=torch.uint8, device=dev)

    def step():
        hils.prefill(x["q"], x["k"], x["v"], x["lm"], w.S, w.W, w.K, out=out, sel=sel, ws=ws,
                     union=union)

    for _ in range(warmup):
        step()
    ms, _ = timed(torch, _lib, step, steps, profile=False)
    ms_prof, kern = timed(torch, _lib, step, steps, profile=True)
    log(f"prefill {w.name} {ms:.3f} ms/step ({ms_prof:.3f} with kernel timing); "
        f"kernels {json.dumps(kern)}")
    score_f, summ_f, attn_f = prefill_work(w)
    win_f, sel_f = window_work(w)
    # algorithmic FLOPs per step of the contraction kernels; per launch is that
    # over the launches per step (the bucket-path kernels run once per slice)
    step_flops = {"k_attn_fast": attn_f, "k_attn_generic": attn_f, "k_score_fast": score_f,
                  "k_select_generic": score_f, "k_summarize": summ_f, "k_win_fuse": win_f,
                  "k_pair_attn": sel_f}

    def roofline(kname):
        launches = kern[kname]["calls"] / steps
        per_launch = step_flops[kname] / launches
        achieved = per_launch / (kern[kname]["avg_ms"] * 1e-3) / 1e12
        return {"kernel": kname, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": counter_traffic(kname, w.name),
                "algorithmic_flops_per_launch": per_launch, "launches_per_step": launches}

    rooflines = {k2: roofline(k2) for k2 in kern if k2 in step_flops}
    # design-traffic diagnostic: the bucket path's pair attention and reduction
    # move per-pair gathers and partial rows, counted from the selection
    hbm_rooflines = {}
    if "k_pair_attn" in kern:
        attn_b, red_b = pair_path_bytes(sel, w, kern["k_pair_attn"]["calls"] / steps)
        for kname, step_bytes in (("k_pair_attn", attn_b), ("k_win_fuse", red_b)):
            if kname not in kern:
                continue
            launches = kern[kname]["calls"] / steps
            per_launch = step_bytes / launches
            achieved = per_launch / (kern[kname]["avg_ms"] * 1e-3) / 1e9
            hbm_rooflines[kname] = {"kernel": kname, "bound": "hbm", "achieved": achieved,
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": achieved / PEAK_HBM_GBS,
                                    "traffic": counter_traffic(kname, w.name),
                                    "design_bytes_per_launch": per_launch,
                                    "launches_per_step": launches}
    # the dominant kernel among those doing the method's contractions
    dom = max(rooflines, key=lambda k2: kern[k2]["ms_per_step"])
    total_flops = score_f + summ_f + attn_f
    step_tflops = total_flops / (ms * 1e-3) / 1e12
    rec = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.N / (ms * 1e-3),
           "ms_per_step_with_kernel_timing": ms_prof,
           "config": {"workload": w.name, "B": w.B, "N": w.N, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                      "S": w.S, "W": w.W, "K": w.K, "regime": w.regime,
                      "attention": "query-block unions" if union else "chunk buckets"},
           "algorithmic_tflop": {"scoring": score_f / 1e12, "summaries": summ_f / 1e12,
                                 "attention": attn_f / 1e12},
           "roofline": rooflines[dom],
           "step_roofline": {"bound": "mfma", "achieved": step_tflops, "peak": PEAK_BF16_TFLOPS,
                             "unit": "TFLOP/s", "frac": step_tflops / PEAK_BF16_TFLOPS,
                             "algorithmic_flops_per_step": total_flops},
           "kernel_rooflines": rooflines, "design_traffic_hbm": hbm_rooflines, "kernels": kern}
    if w.N >= 16 * 64:
        rec["config"]["chunk_overlap_M16"] = _overlap(sel, w.K)
    del out, ws
    if not want_sel:
        del sel, x
        torch.cuda.empty_cache()
        return rec, None, None
    return rec, x, sel


def synth_inputs(w, dev):
    import synth
    return synth.make_prefill_inputs(w, device=dev)


def decode_bench(torch, hils, _lib, wd, steps, warmup, log, keep=False):
    """Single-step decode of every sequence of the workload (the cache is full,
    T = capacity), headline time with kernel timing off, then the kernel table."""
    import synth
    dev = torch.device("cuda:0")
    log(f"decode inputs {wd.name}: B={wd.B} T={wd.N} Hq={wd.Hq} Hkv={wd.Hkv} W={wd.W} K={wd.K}")
    xd = synth.make_decode_inputs(wd, device=dev)
    ks, bs = hils.summarize(xd["k"], xd["lm"], wd.S)
    outd = torch.empty_like(xd["q"])
    cfgd = hils.make_cfg(wd.B, wd.N, wd.Hq, wd.Hkv, wd.d, wd.S, wd.W, wd.K, xd["q"].dtype)
    wsd = torch.empty(max(1, hils.workspace_bytes(cfgd, True)), dtype=torch.uint8, device=dev)

    def dstep():
        hils.decode(xd["q"], xd["k"], xd["v"], xd["seqlen"], ks, bs, wd.S, wd.W, wd.K,
                    out=outd, ws=wsd)

    for _ in range(max(3, warmup)):
        dstep()
    dec_ms, _ = timed(torch, _lib, dstep, steps, profile=False, group=8, median=True)
    ms_prof, dk = timed(torch, _lib, dstep, steps, profile=True)
    log(f"decode {wd.name} {dec_ms:.4f} ms/step ({ms_prof:.4f} with kernel timing); "
        f"kernels {json.dumps(dk)}")
    step_bytes, score_bytes = decode_work(wd, wd.N)
    sc = dk.get("k_dec_score")
    dach = score_bytes / (sc["avg_ms"] * 1e-3) / 1e9 if sc else None
    step_gbs = step_bytes / (dec_ms * 1e-3) / 1e9
    rec = {"workload": wd.name, "metric": "decode steps/s", "value": 1000.0 / dec_ms,
           "unit": "steps/s", "ms_per_step": dec_ms, "tokens_per_s": wd.B * 1000.0 / dec_ms,
           "ms_per_step_with_kernel_timing": ms_prof,
           "config": {"workload": wd.name, "B": wd.B, "T": wd.N, "Hq": wd.Hq, "Hkv": wd.Hkv,
                      "d": wd.d, "S": wd.S, "W": wd.W, "K": wd.K},
           "step_roofline": {"bound": "hbm", "achieved": step_gbs, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": step_gbs / PEAK_HBM_GBS,
                             "algorithmic_bytes_per_step": step_bytes},
           "roofline": {"kernel": "k_dec_score", "bound": "hbm", "achieved": dach,
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": (dach / PEAK_HBM_GBS) if dach else None,
                        "traffic": counter_traffic("k_dec_score", wd.name),
                        "algorithmic_bytes_per_launch": score_bytes},
           "kernels": dk}
    if keep:
        return rec, (xd, ks, bs)
    del xd, ks, bs, outd, wsd
    torch.cuda.empty_cache()
    return rec, None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_512k")
    ap.add_argument("--decode-workload", default="decode_512k")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--more-prefill", default="prefill_64k,prefill_8k",
                    help="further prefill workloads timed after the headline one ('' skips)")
    ap.add_argument("--more-decode", default="decode_4m",
                    help="further decode workloads timed after the headline one ('' skips)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--union", action="store_true",
                    help="prefill attention by query block over the union of its chunks "
                         "instead of the default per-chunk buckets")
    ap.add_argument("--backward-workload", default="prefill_8k,prefill_64k",
                    help="workloads of the backward measurement, comma-separated: the first "
                         "is `backward`, the others `backward_more` ('' skips it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB copy first (counter scale for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import chunk_wise_hierarchical_amd as hils
    from chunk_wise_hierarchical_amd import _lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        calibrate_copy(torch, dev, log)

    # ---------------- prefill (headline workload) ----------------
    w = synth.get_workload(args.workload)
    pre, x, sel = prefill_bench(torch, hils, _lib, w, args.steps, args.warmup, args.union, log,
                                want_sel=not args.no_cpu)
    cpu_pre = None
    if not args.no_cpu:
        log("oracle baseline (prefill sample)")
        cpu_pre = cpu_baseline_prefill(x, w)
    del x, sel
    torch.cuda.empty_cache()

    more = {}
    for name in [n for n in args.more_prefill.split(",") if n]:
        wm = synth.get_workload(name)
        more[name], _, _ = prefill_bench(torch, hils, _lib, wm, max(args.steps, 10),
                                         args.warmup, args.union, log)

    # ---------------- decode ----------------
    dec = None
    if not args.no_decode:
        wd = synth.get_workload(args.decode_workload)
        dec, kept = decode_bench(torch, hils, _lib, wd, args.decode_steps, args.warmup, log,
                                 keep=True)
        xd, ks, bs = kept
        # the same step over a paged cache (one chunk per page, pages randomly
        # placed), eagerly and replayed from a captured HIP graph
        dec["paged"] = paged_decode_bench(torch, hils, _lib, xd, wd, ks, bs, args.decode_steps, log)
        # a block of 4 new tokens per sequence (draft / verification tokens)
        dec["multi_token"] = multi_decode_bench(torch, hils, _lib, xd, wd, ks, bs, 4,
                                                args.decode_steps, log)
        dec["multi_token_correlated"] = multi_decode_bench(torch, hils, _lib, xd, wd, ks, bs, 4,
                                                           args.decode_steps, log, corr=0.9)
        if not args.no_cpu:
            log("oracle baseline (decode sample)")
            dec["cpu_baseline"] = cpu_baseline_decode(xd, wd)
        del xd, ks, bs, kept
        torch.cuda.empty_cache()
        for name in [n for n in args.more_decode.split(",") if n]:
            more[name], _ = decode_bench(torch, hils, _lib, synth.get_workload(name),
                                         args.decode_steps, args.warmup, log)

    bwd, bwd_more = None, {}
    for n, name in enumerate([n for n in args.backward_workload.split(",") if n]):
        torch.cuda.empty_cache()
        rec = backward_bench(torch, hils, _lib, synth.get_workload(name), args.steps, log)
        if n == 0:
            bwd = rec
        else:
            bwd_more[name] = rec

    line = {
        "metric": "prefill tokens/s and decode steps/s at 512K ctx; % of MFMA/HBM roofline",
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": pre["config"],
        "roofline": pre["roofline"],
        "step_roofline": pre["step_roofline"],
        "algorithmic_tflop": pre["algorithmic_tflop"],
        "kernel_rooflines": pre["kernel_rooflines"],
        "design_traffic_hbm": pre["design_traffic_hbm"],
        "cpu_baseline": cpu_pre,
        "kernels": pre["kernels"],
        "ms_per_step_with_kernel_timing": pre["ms_per_step_with_kernel_timing"],
        "decode": dec,
        "more_workloads": more,
        "backward": bwd,
        "backward_more": bwd_more,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
