"""Seeded synthetic input tensors for HiLS prefill and decode.

Recipe (all draws seeded; values then rounded to the workload dtype with
torch's round-to-nearest-even):
  * q, k, v and the landmark queries are N(0, f^2) with f = 1/sqrt(d) for
    "scaled" workloads and f = 1 otherwise, drawn in that order from one
    torch generator on the target device, one (batch, head) slice at a time;
  * a "peaked" query head h gets a unit direction u_h; its queries and landmark
    queries get + a*u_h (a = 1 when scaled, a = sqrt(d) otherwise), and needle
    keys k* = k0 + (lam*sqrt(d)/a)*u_h are planted in its KV head, which gives
    the needle a token logit about lam above the background (lam = 4 for
    prefill, 8 for decode);
  * optionally (q_share > 0) queries carry a component shared by runs of
    q_seg adjacent tokens, q_i = sqrt(1-q_share)*e_i + sqrt(q_share)*z_seg(i),
    which keeps each element N(0, f^2) while making adjacent queries route to
    overlapping chunks.
Structure (directions, needle positions) comes from a CPU generator seeded
with seed+1, so it is identical whatever device draws the bulk tensors.
"""
from __future__ import annotations

import math

import torch

from .workloads import Workload

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fill_normal(out, gen, std, share=0.0, seg=1):
    """Fill out[..., N, d] (one 2-D slice per leading index) with N(0, std^2)."""
    lead = out.shape[:-2]
    N, d = out.shape[-2], out.shape[-1]
    for idx in _ndindex(lead):
        x = torch.randn((N, d), generator=gen, device=out.device, dtype=torch.float32)
        if share > 0.0:
            nseg = (N + seg - 1) // seg
            z = torch.randn((nseg, d), generator=gen, device=out.device, dtype=torch.float32)
            z = z.repeat_interleave(seg, dim=0)[:N]
            x = math.sqrt(1.0 - share) * x + math.sqrt(share) * z
        out[idx] = (x * std).to(out.dtype)


def _ndindex(shape):
    if len(shape) == 0:
        yield ()
        return
    import itertools
    yield from itertools.product(*[range(s) for s in shape])


def _window_left(i, W, S):
    return ((i - W + 1) // S) * S


def _plan_structure(w: Workload, seed: int, ncand: int):
    """Needle plan: list of (b, q_head, [(chunk, token_offset), ...])."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1)
    plan = []
    nC = max(ncand, 1)

    def rint(hi):
        return int(torch.randint(0, max(hi, 1), (1,), generator=g).item())

    for b in range(w.B):
        if w.regime == "iid":
            break
        if w.regime == "half_peaked4":
            for h in range(w.Hq // 2, w.Hq):
                chunks = torch.randperm(nC, generator=g)[:4].tolist()
                plan.append((b, h, [(c, rint(w.S)) for c in chunks]))
        elif w.regime == "mod3":
            for h in range(w.Hq):
                if h % 3 == 1:
                    plan.append((b, h, [(rint(nC), rint(w.S))]))
                elif h % 3 == 2:
                    m = 2 + rint(7)                       # 2..8 chunks (fewer if nC < m)
                    chunks = torch.randperm(nC, generator=g)[:m].tolist()
                    plan.append((b, h, [(chunks[rint(len(chunks))], rint(w.S)) for _ in range(8)]))
        elif w.regime == "needle_chunk":
            c = rint(nC)
            for h in range(w.Hq):
                plan.append((b, h, [(c, rint(w.S))]))
        elif w.regime == "depth10":
            chunks = [min(nC - 1, int((k + 0.5) / 10 * nC)) for k in range(10)]
            for h in range(0, w.Hq, 2):
                plan.append((b, h, [(c, rint(w.S)) for c in chunks]))
        else:
            raise ValueError(w.regime)
    dirs = torch.randn((w.B, w.Hq, w.d), generator=g, dtype=torch.float64)
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    return plan, dirs


def _apply_structure(w, plan, dirs, q, k, lm, lam):
    """Plant needles: peaked heads share a direction between queries, landmark
    queries and the planted keys (see module docstring)."""
    a = 1.0 if w.scaled else math.sqrt(w.d)
    coef = lam * math.sqrt(w.d) / a
    G = w.G
    dev = q.device
    for (b, h, needles) in plan:
        u = dirs[b, h].to(device=dev, dtype=torch.float32)
        q[b, h] = (q[b, h].float() + a * u).to(q.dtype)
        lm[b, h] = (lm[b, h].float() + a * u).to(lm.dtype)
        for (c, off) in needles:
            t = c * w.S + off
            if t >= k.shape[2]:      # a sequence shorter than one chunk: nothing to plant
                continue
            k[b, h // G, t] = (k[b, h // G, t].float() + coef * u).to(k.dtype)


def make_prefill_inputs(w: Workload, device="cpu", seed=None, with_q_route=False):
    """q [B,Hq,N,d], k/v [B,Hkv,N,d], lm [B,Hq,floor(N/S),d] (+ q_route)."""
    seed = w.seed if seed is None else seed
    dt = _TORCH_DTYPE[w.dtype]
    f = (1.0 / math.sqrt(w.d)) if w.scaled else 1.0
    nC = w.N // w.S
    gen = _gen(device, seed)
    q = torch.empty((w.B, w.Hq, w.N, w.d), dtype=dt, device=device)
    k = torch.empty((w.B, w.Hkv, w.N, w.d), dtype=dt, device=device)
    v = torch.empty((w.B, w.Hkv, w.N, w.d), dtype=dt, device=device)
    lm = torch.empty((w.B, w.Hq, nC, w.d), dtype=dt, device=device)
    _fill_normal(q, gen, f, w.q_share, w.q_seg)
    _fill_normal(k, gen, f)
    _fill_normal(v, gen, f)
    _fill_normal(lm, gen, f)
    ncand = max(0, _window_left(w.N - 1, w.W, w.S) // w.S)
    plan, dirs = _plan_structure(w, seed, ncand)
    _apply_structure(w, plan, dirs, q, k, lm, lam=4.0)
    out = dict(q=q, k=k, v=v, lm=lm)
    if with_q_route:
        qr = torch.empty_like(q)
        _fill_normal(qr, gen, 0.25 * f)
        out["q_route"] = (q.float() + qr.float()).to(dt)
    return out


def make_decode_inputs(w: Workload, device="cpu", seed=None, seqlen=None, with_q_route=False):
    """q [B,Hq,1,d], k_cache/v_cache [B,Hkv,T,d], lm [B,Hq,floor(T/S),d], seqlen [B] int32."""
    seed = w.seed if seed is None else seed
    dt = _TORCH_DTYPE[w.dtype]
    f = (1.0 / math.sqrt(w.d)) if w.scaled else 1.0
    T = w.N
    nC = T // w.S
    gen = _gen(device, seed)
    q = torch.empty((w.B, w.Hq, 1, w.d), dtype=dt, device=device)
    k = torch.empty((w.B, w.Hkv, T, w.d), dtype=dt, device=device)
    v = torch.empty((w.B, w.Hkv, T, w.d), dtype=dt, device=device)
    lm = torch.empty((w.B, w.Hq, nC, w.d), dtype=dt, device=device)
    _fill_normal(q, gen, f)
    _fill_normal(k, gen, f)
    _fill_normal(v, gen, f)
    _fill_normal(lm, gen, f)
    if seqlen is None:
        seqlen = [T] * w.B
    seqlen = torch.tensor(seqlen, dtype=torch.int32)
    ncand = max(0, _window_left(int(seqlen.min()) - 1, w.W, w.S) // w.S)
    plan, dirs = _plan_structure(w, seed, ncand)
    _apply_structure(w, plan, dirs, q[:, :, 0], k, lm, lam=8.0)
    out = dict(q=q, k=k, v=v, lm=lm, seqlen=seqlen.to(device))
    if with_q_route:
        qr = torch.empty_like(q)
        _fill_normal(qr, gen, 0.25 * f)
        out["q_route"] = (q.float() + qr.float()).to(dt)
    return out
