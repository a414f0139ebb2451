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


def _case(w, mode="surrogate", q_route=False, label="", seed=21):
    _say(f"[backward] {label} {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} "
         f"W={w.W} K={w.K} dtype={w.dtype} mode={mode} q_route={q_route}")
    x = {k: v.cuda() for k, v in synth.make_prefill_inputs(w, with_q_route=q_route).items()}
    g = torch.Generator(device="cpu").manual_seed(seed)
    dout = torch.randn(x["q"].shape, generator=g).to(x["q"].dtype).cuda()
    xn = {k: np32(v) for k, v in x.items()}
    ref = O.ref_backward(xn["q"], xn["k"], xn["v"], xn["lm"], np32(dout), w.S, w.W, w.K,
                         q_route=xn.get("q_route"), mode=mode, store=w.dtype)
    sel = torch.tensor(ref["sel"], dtype=torch.int32).cuda().contiguous()
    lm = None if mode == "mean_pool" else x["lm"]
    gr = hils.prefill_backward(x["q"], x["k"], x["v"], lm, dout, sel, w.S, w.W, w.K,
                               q_route=x.get("q_route"), mode=mode)
    torch.cuda.synchronize()
    names = ["dq", "dk", "dv"] + (["dlm"] if mode != "mean_pool" and w.N >= w.S else []) \
        + (["dq_route"] if q_route else [])
    worst = 0.0
    for n in names:
        got = gr[n].cpu().numpy().astype(np.float64)
        want = ref[n]
        err = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
        worst = max(worst, err)
        assert err <= TOL, f"{n}: relative error {err:.3g} > {TOL}"
    _say(f"   max relative gradient error {worst:.3g} over {names}")
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


def test_backward_deterministic():
    w = synth.get_workload("prefill_64k", N=700, Hq=4, Hkv=1, d=64, S=32, W=64, K=4, regime="iid")
    gr, (x, dout, sel) = _case(w, label="determinism")
    gr2 = hils.prefill_backward(x["q"], x["k"], x["v"], x["lm"], dout, sel, w.S, w.W, w.K)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dlm"):
        assert torch.equal(gr[n], gr2[n]), n
