"""GPU parity of the prefill backward (hils_prefill_backward) against the oracle.

The selection is a hard choice held fixed in the backward; the oracle computes
it (with its own summaries) and both sides differentiate at that selection.
Gradients are fp32 on the GPU and fp64 in the oracle; tolerance: max |g - g_ref|
over max |g_ref| per tensor <= 1e-5, the fp32 forward bar (fp32 accumulation
over at most a few thousand terms per element with the hardware exp/log; about
1.5e-6 is observed).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import hils_oracle as O
from tests.parity_util import np32

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import chunk_wise_hierarchical_amd as hils

TOL = 1e-5


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(w, mode="surrogate", q_route=False, label="", seed=21, reverse_slots=False):
    _say(f"[backward] {label} {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} "
         f"W={w.W} K={w.K} dtype={w.dtype} mode={mode} q_route={q_route}")
    x = {k: v.cuda() for k, v in synth.make_prefill_inputs(w, with_q_route=q_route).items()}
    g = torch.Generator(device="cpu").manual_seed(seed)
    dout = torch.randn(x["q"].shape, generator=g).to(x["q"].dtype).cuda()
    xn = {k: np32(v) for k, v in x.items()}
    ref = O.ref_backward(xn["q"], xn["k"], xn["v"], xn["lm"], np32(dout), w.S, w.W, w.K,
                         q_route=xn.get("q_route"), mode=mode, store=w.dtype)
    sel = torch.tensor(ref["sel"], dtype=torch.int32).cuda().contiguous()
    if reverse_slots:      # empty slots (-1) first: the gradients depend on the set only
        sel = sel.flip(-1).contiguous()
    lm = None if mode == "mean_pool" else x["lm"]
    gr = hils.prefill_backward(x["q"], x["k"], x["v"], lm, dout, sel, w.S, w.W, w.K,
                               q_route=x.get("q_route"), mode=mode)
    torch.cuda.synchronize()
    names = ["dq", "dk", "dv"] + (["dlm"] if mode != "mean_pool" and w.N >= w.S else []) \
        + (["dq_route"] if q_route else [])
    errs = {}
    for n in names:
        got = gr[n].cpu().numpy().astype(np.float64)
        want = ref[n]
        errs[n] = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
    _say("   relative gradient errors " + ", ".join(f"{n} {e:.3g}" for n, e in errs.items()))
    for n, err in errs.items():
        assert err <= TOL, f"{n}: relative error {err:.3g} > {TOL}"
    return gr, (x, dout, sel)


def test_backward_tiny_fp32_with_routing_query():
    w = synth.get_workload("tiny_fp32")
    _case(w, label="tiny fp32")
    _case(w, q_route=True, label="tiny fp32 q_route")


def test_backward_bf16_gqa_ragged():
    # GQA 4:1, d = 128, S = 64, N not a multiple of S, K below the candidate count
    w = synth.get_workload("prefill_64k", N=1000, Hq=8, Hkv=2, W=128, K=4)
    _case(w, label="bf16 GQA ragged")


def test_backward_many_selected_keys():
    # G = 4 and K = 32 chunks of 64: the keys a row attends do not fit the
    # all-keys row kernel's LDS budget, so the chunk-at-a-time row kernel runs
    w = synth.get_workload("prefill_64k", N=2500, Hq=8, Hkv=2, W=128, K=32, regime="iid")
    _case(w, label="bf16 GQA K=32")


def test_backward_summary_modes():
    w = synth.get_workload("prefill_64k", N=520, Hq=4, Hkv=2, d=64, S=32, W=96, K=3, regime="iid",
                           dtype="f32")
    _case(w, mode="landmark_key", label="landmark_key")
    _case(w, mode="mean_pool", label="mean_pool")


def test_backward_matrix_core_columns_all_modes():
    # bf16 with d = 128 and S = 64 (and d = 64, S = 32): dk and dv come from the
    # matrix-core column pass, the summaries' share of dk and dlm from the
    # summary pass; routing query, landmark key and mean pool; a sequence
    # shorter than one chunk (window only, no summaries)
    w = synth.get_workload("prefill_64k", N=700, Hq=4, Hkv=2, W=100, K=4, regime="iid")
    _case(w, q_route=True, label="mf q_route")
    _case(w, mode="landmark_key", label="mf landmark_key")
    _case(w, mode="mean_pool", label="mf mean_pool")
    w = synth.get_workload("prefill_64k", N=333, Hq=8, Hkv=1, d=64, S=32, W=40, K=6, regime="depth10")
    _case(w, label="mf d64 S32 G8")
    w = synth.get_workload("prefill_64k", N=50, Hq=2, Hkv=1, W=30, K=2)
    _case(w, label="mf N < S")
    w = synth.get_workload("prefill_64k", N=1, Hq=2, Hkv=1, W=30, K=2)
    _case(w, label="mf N = 1")
    w = synth.get_workload("prefill_64k", N=65, Hq=4, Hkv=1, W=1, K=3, regime="iid")
    _case(w, label="mf N = S + 1, W = 1")
    # a group size that is not a power of two (the summary pass's generic form)
    w = synth.get_workload("prefill_64k", N=400, Hq=6, Hkv=2, W=80, K=5, regime="half_peaked4")
    _case(w, label="mf G3")


def test_backward_selection_slot_order():
    # early queries have fewer candidates than K; with the slots reversed their
    # -1 entries come first, in both the matrix-core (bf16) and VALU (fp32) paths
    w = synth.get_workload("prefill_64k", N=600, Hq=4, Hkv=2, W=64, K=6, regime="iid")
    _case(w, label="bf16 reversed slots", reverse_slots=True)
    w = synth.get_workload("prefill_64k", N=300, Hq=2, Hkv=1, d=64, S=32, W=40, K=5, regime="iid",
                           dtype="f32")
    _case(w, label="fp32 reversed slots", reverse_slots=True)


def test_backward_query_slices(monkeypatch):
    # the matrix-core backward in several query slices (at these sizes it
    # normally takes one): slice bounds inside chunks and windows, dk and dv
    # added up over the slices, the lists cut per slice
    monkeypatch.setenv("HILS_BWD_SLICE_QUERIES", "300")
    w = synth.get_workload("prefill_64k", N=1000, Hq=8, Hkv=2, W=128, K=4)
    _case(w, q_route=True, label="4 slices of 300")
    monkeypatch.setenv("HILS_BWD_SLICE_QUERIES", "64")
    w = synth.get_workload("prefill_64k", N=333, Hq=4, Hkv=1, d=64, S=32, W=100, K=5,
                           regime="depth10")
    _case(w, label="6 slices of 64")


def test_backward_lists_over_several_workgroups():
    # N > 4096: the selection lists are built by two workgroups per (sequence,
    # KV group), each wavefront scattering its own sub-range of the queries
    w = synth.get_workload("prefill_64k", N=5000, Hq=4, Hkv=2, W=128, K=4, regime="iid")
    _case(w, label="lists over 2 workgroups")


def test_backward_full_size_sampled():
    """prefill_8k at its full size (B=2, N=8192, 16/16 heads, W=512, K=16), the
    launch bench.py times.  The selection is an input of the backward (held
    fixed): a seeded random choice of min(K, |C_i|) candidate chunks per row,
    the same for both sides.  The oracle runs only the rows attending three
    sampled keys plus 24 sampled query rows, which makes those keys' dk, dv,
    their chunks' dlm and those rows' dq exact (ref_backward, `rows`)."""
    w = synth.get_workload("prefill_8k")
    x = {k2: v2.cuda() for k2, v2 in synth.make_prefill_inputs(w).items()}
    g0 = torch.Generator(device="cpu").manual_seed(31)
    dout = torch.randn(x["q"].shape, generator=g0).to(x["q"].dtype).cuda()
    B, Hkv, N, S, W, K = w.B, w.Hkv, w.N, w.S, w.W, w.K
    nC = N // S
    rng = np.random.default_rng(8192)
    ncand = np.array([O.n_candidates(i, W, S) for i in range(N)])
    keys = rng.random((B, Hkv, N, nC), dtype=np.float32)
    keys[:, :, np.arange(nC)[None, :] >= ncand[:, None]] = np.inf
    order = np.argsort(keys, axis=-1)[..., :K]
    sel = np.where(np.arange(K)[None, :] < np.minimum(K, ncand)[:, None], order, -1).astype(np.int32)
    _say(f"[backward] full-size prefill_8k, random selection ({(sel >= 0).sum()} pairs)")
    gr = hils.prefill_backward(x["q"], x["k"], x["v"], x["lm"], dout,
                               torch.from_numpy(sel).cuda().contiguous(), S, W, K)
    torch.cuda.synchronize()
    samp_keys = [(0, 0, 1000), (1, 5, 4100), (0, 15, N - 70)]
    samp_rows = {(int(rng.integers(B)), int(rng.integers(Hkv)), int(rng.integers(N))) for _ in range(24)}
    rows = set(samp_rows)
    for (b, g, j) in samp_keys:
        rows |= O.ref_attending_rows(sel, b, g, j, S, W)
    _say(f"   oracle over {len(rows)} rows")
    xn = {k2: np32(v2) for k2, v2 in x.items()}
    ref = O.ref_backward(xn["q"], xn["k"], xn["v"], xn["lm"], np32(dout), S, W, K, sel=sel,
                         store=w.dtype, rows=rows)
    G = w.Hq // Hkv
    pairs = {"dk": [(b, g, j) for (b, g, j) in samp_keys], "dv": [(b, g, j) for (b, g, j) in samp_keys],
             "dlm": [(b, g * G + r, j // S) for (b, g, j) in samp_keys for r in range(G)],
             "dq": [(b, g * G + r, i) for (b, g, i) in samp_rows for r in range(G)]}
    errs = {}
    for n, idx in pairs.items():
        got = np.stack([gr[n][t].cpu().numpy().astype(np.float64) for t in idx])
        want = np.stack([ref[n][t] for t in idx])
        errs[n] = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
    _say("   relative gradient errors " + ", ".join(f"{n} {e:.3g}" for n, e in errs.items()))
    for n, err in errs.items():
        assert err <= TOL, f"{n}: relative error {err:.3g} > {TOL}"


def test_backward_more_than_64_slots():
    # K = 100 selected chunks of 16: slots 64.. live in a second register of
    # the row pass and a second ballot word of the dq reduction (bf16, matrix
    # cores); the fp32 case takes the vector-ALU kernels
    w = synth.get_workload("prefill_64k", N=2200, Hq=2, Hkv=1, S=16, W=64, K=100, regime="iid")
    _case(w, q_route=True, label="K = 100 bf16")
    w = synth.get_workload("prefill_64k", N=1900, Hq=2, Hkv=2, d=64, S=16, W=48, K=100,
                           regime="iid", dtype="f32")
    _case(w, label="K = 100 fp32")
    # the row pass keeps the slots' k' pieces in registers up to 16 rows per
    # lane: K = 64 at d = 128 (4 rows per load instruction, the most it
    # keeps) and K = 100 at d = 64 (8 rows per instruction, slots past 64)
    w = synth.get_workload("prefill_64k", N=1500, Hq=4, Hkv=2, S=16, W=32, K=64, regime="iid")
    _case(w, q_route=True, label="K = 64 bf16, row pieces in registers")
    w = synth.get_workload("prefill_64k", N=2000, Hq=2, Hkv=1, d=64, S=16, W=40, K=100,
                           regime="half_peaked4")
    _case(w, label="K = 100 bf16 d = 64, row pieces in registers")


def test_backward_deterministic():
    w = synth.get_workload("prefill_64k", N=700, Hq=4, Hkv=1, d=64, S=32, W=64, K=4, regime="iid")
    gr, (x, dout, sel) = _case(w, label="determinism")
    gr2 = hils.prefill_backward(x["q"], x["k"], x["v"], x["lm"], dout, sel, w.S, w.W, w.K)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dlm"):
        assert torch.equal(gr[n], gr2[n]), n
