"""GPU parity over a seeded sweep of shapes: the HIP library against the fp64
oracle on configurations drawn at random from the supported space (fast MFMA
path and generic kernels, bf16 and fp32, every head-structure regime, ragged
lengths, windows shorter and longer than the sequence, K from 1 to 64).

The draws are fixed by the seed, so every run checks the same cases; each case
prints its shape before it runs.
"""
import numpy as np
import pytest

import synth
from tests.parity_util import sample_rows
from tests.test_gpu_parity import _decode_case, _prefill_case

pytestmark = pytest.mark.gpu

REGIMES = ["iid", "mod3", "half_peaked4", "depth10", "needle_chunk"]


def _prefill_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        fast = c % 2 == 0
        if fast:                          # shapes the MFMA path takes
            d, S, dtype = 128, 64, "bf16"
            G = int(rng.choice([1, 2, 4]))
        else:                             # generic kernels
            d = int(rng.choice([32, 64, 96]))
            S = int(rng.choice([16, 32, 48]))
            dtype = str(rng.choice(["bf16", "f32"]))
            G = int(rng.choice([1, 2, 3, 8]))
        Hkv = int(rng.choice([1, 2]))
        N = int(rng.integers(S, 40 * S))
        W = int(rng.integers(1, 12 * S))
        K = int(rng.integers(1, 65 if fast else 33))
        regime = REGIMES[int(rng.integers(0, 4))]
        out.append(dict(B=int(rng.integers(1, 3)), N=N, Hq=G * Hkv, Hkv=Hkv, d=d, S=S, W=W,
                        K=K, dtype=dtype, regime=regime, seed=int(rng.integers(0, 1 << 30)),
                        scaled=bool(rng.integers(0, 2)), q_route=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _prefill_draws(24, seed=20261203),
                         ids=lambda c: f"N{c['N']}_G{c['Hq'] // c['Hkv']}_d{c['d']}_S{c['S']}_"
                                       f"W{c['W']}_K{c['K']}_{c['dtype']}")
def test_prefill_sweep(case):
    c = dict(case)
    q_route = c.pop("q_route")
    w = synth.get_workload("prefill_64k", **c)
    _prefill_case(w, rows=sample_rows(w, 120, seed=c["seed"] % 1000), q_route=q_route,
                  label="sweep")


def _decode_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 5))
        N = int(rng.integers(512, 6000))
        out.append(dict(B=B, N=N, Hq=G * Hkv, Hkv=Hkv, W=int(rng.integers(1, 1200)),
                        K=int(rng.integers(1, 65)), regime=REGIMES[int(rng.integers(0, 5))],
                        seed=int(rng.integers(0, 1 << 30)),
                        seqlen=[int(x) for x in rng.integers(1, N + 1, size=B)]))
    return out


@pytest.mark.parametrize("case", _decode_draws(12, seed=20261204),
                         ids=lambda c: f"B{c['B']}_T{c['N']}_G{c['Hq'] // c['Hkv']}_W{c['W']}_K{c['K']}")
def test_decode_sweep(case):
    c = dict(case)
    seqlen = c.pop("seqlen")
    w = synth.get_workload("decode_512k", **c)
    _decode_case(w, seqlen, label="sweep")


def _backward_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        dtype = "bf16" if c % 2 == 0 else "f32"
        d = int(rng.choice([64, 128])) if dtype == "bf16" else int(rng.choice([32, 64, 96, 128]))
        S = int(rng.choice([16, 32, 64]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        out.append(dict(B=int(rng.integers(1, 3)), N=int(rng.integers(S, 24 * S)), Hq=G * Hkv,
                        Hkv=Hkv, d=d, S=S, W=int(rng.integers(1, 8 * S)),
                        K=int(rng.integers(1, 17)), dtype=dtype, regime=REGIMES[int(rng.integers(0, 4))],
                        seed=int(rng.integers(0, 1 << 30)), scaled=bool(rng.integers(0, 2)),
                        q_route=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _backward_draws(10, seed=20261205),
                         ids=lambda c: f"N{c['N']}_G{c['Hq'] // c['Hkv']}_d{c['d']}_S{c['S']}_"
                                       f"W{c['W']}_K{c['K']}_{c['dtype']}")
def test_backward_sweep(case):
    from tests.test_gpu_backward import _case as backward_case
    c = dict(case)
    q_route = c.pop("q_route")
    w = synth.get_workload("prefill_64k", **c)
    backward_case(w, q_route=q_route, label="sweep", seed=c["seed"] % 1000)


def _multi_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        B = int(rng.integers(1, 4))
        N = int(rng.integers(256, 5000))
        M = int(rng.integers(1, 17))
        out.append(dict(B=B, N=N, Hq=G * Hkv, Hkv=Hkv, W=int(rng.integers(1, 1200)),
                        K=int(rng.integers(1, 65)), regime=REGIMES[int(rng.integers(0, 5))],
                        seed=int(rng.integers(0, 1 << 30)), M=M,
                        seqlen=[int(x) for x in rng.integers(M, N + 1, size=B)]))
    return out


@pytest.mark.parametrize("case", _multi_draws(8, seed=20261206),
                         ids=lambda c: f"B{c['B']}_T{c['N']}_G{c['Hq'] // c['Hkv']}_M{c['M']}_"
                                       f"W{c['W']}_K{c['K']}")
def test_multi_decode_sweep(case):
    from tests.test_gpu_multi_decode import _multi_case
    c = dict(case)
    seqlen, M = c.pop("seqlen"), c.pop("M")
    w = synth.get_workload("decode_512k", **c)
    _multi_case(w, M, seqlen, label="sweep")


def _long_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.choice([1, 2, 4]))
        out.append(dict(N=int(rng.integers(3000, 20000)), Hq=G * Hkv, Hkv=Hkv,
                        W=int(rng.integers(64, 3000)), K=int(rng.integers(1, 65)),
                        regime=REGIMES[int(rng.integers(0, 4))], seed=int(rng.integers(0, 1 << 30)),
                        scaled=bool(rng.integers(0, 2)), union=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _long_draws(6, seed=20261207),
                         ids=lambda c: f"N{c['N']}_G{c['Hq'] // c['Hkv']}_W{c['W']}_K{c['K']}_"
                                       f"{'union' if c['union'] else 'buckets'}")
def test_prefill_long_sweep(case):
    # several score tiles, window tiles and (for the buckets) pair tiles per
    # query block, on both attention organisations
    c = dict(case)
    union = c.pop("union")
    w = synth.get_workload("prefill_64k", **c)
    _prefill_case(w, rows=sample_rows(w, 40, seed=c["seed"] % 1000), union=union, label="sweep")


def _paged_draws(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        B = int(rng.integers(1, 4))
        N = int(rng.integers(2, 80)) * 64
        out.append(dict(B=B, N=N, Hq=G * Hkv, Hkv=Hkv, W=int(rng.integers(1, 2000)),
                        K=int(rng.integers(1, 65)), regime=REGIMES[int(rng.integers(0, 5))],
                        seed=int(rng.integers(0, 1 << 30)),
                        lens=[int(x) for x in rng.integers(1, N + 1, size=B)]))
    return out


@pytest.mark.parametrize("case", _paged_draws(8, seed=20261208),
                         ids=lambda c: f"B{c['B']}_T{c['N']}_G{c['Hq'] // c['Hkv']}_W{c['W']}_K{c['K']}")
def test_paged_decode_sweep(case):
    # decode over randomly placed pages equals decode over the contiguous
    # cache (selection and output, bit for bit)
    import torch
    import chunk_wise_hierarchical_amd as hils
    from tests.test_gpu_paged import _case as paged_case
    c = dict(case)
    lens = c.pop("lens")
    w = synth.get_workload("decode_512k", **c)
    x, seqlen, (ks, bs, out_c, sel_c), (table, kp, vp, ksp, bsp) = paged_case(w, lens)
    sel_p = torch.empty_like(sel_c)
    out_p = hils.decode_paged(x["q"], kp, vp, table, seqlen, ksp, bsp, w.S, w.W, w.K, sel=sel_p)
    torch.cuda.synchronize()
    assert torch.equal(sel_p, sel_c)
    assert torch.equal(out_p, out_c)
