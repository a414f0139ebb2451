"""Torch-facing wrappers of the HiLS C ABI: prefill, decode, summarize.

Torch provides device memory and the current stream; every step of the
computation runs in the HIP kernels of libhils.so.  Tensors must be contiguous
CUDA (HIP) tensors of dtype bfloat16 or float32 with the layouts documented in
include/hils.h.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import HilsCfg, check

_DT = {torch.bfloat16: _lib.HILS_BF16, torch.float32: _lib.HILS_F32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name, shape):
    """Exact shape check (the C ABI takes bare pointers, so a mis-shaped tensor
    would be read or written out of bounds on the device)."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _check_tensor(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_cfg(B, N, Hq, Hkv, d, S, W, K, dtype, mode="surrogate", scale=0.0, generic=False,
             union=False):
    flags = (_lib.HILS_FLAG_GENERIC if generic else 0) | (_lib.HILS_FLAG_UNION if union else 0)
    return HilsCfg(B=B, N=N, Hq=Hq, Hkv=Hkv, d=d, S=S, W=W, K=K, dtype=_DT[dtype],
                   mode=_lib.MODES[mode], scale=float(scale), flags=flags)


def workspace_bytes(cfg: HilsCfg, decode: bool) -> int:
    return int(_lib.lib().hils_workspace_bytes(ctypes.byref(cfg), 1 if decode else 0))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(cfg, decode, device, ws):
    need = workspace_bytes(cfg, decode)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, need


def prefill(q, k, v, lm, S, W, K, q_route=None, mode="surrogate", scale=0.0, out=None,
            sel=None, summaries=None, ws=None, generic=False, union=False):
    """HiLS prefill. q [B,Hq,N,d]; k,v [B,Hkv,N,d]; lm [B,Hq,N//S,d].

    mode: "surrogate" (the method), "landmark_key", "mean_pool" (lm may be None) or
    "exact" (token-query chunk log-mass; generic kernels, lm may be None).
    generic forces the vector-ALU kernels; union selects the MFMA attention by
    query block over the union of the block's chunks instead of the default
    per-chunk buckets.
    sel (optional) [B,Hkv,N,K] int32 receives the selected chunk ids;
    summaries (optional) (k_sum [B,Hq,N//S,d], b_sum [B,Hq,N//S] fp32) receive the
    chunk summaries.  Returns out [B,Hq,N,d].
    """
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    nC = N // S if S > 0 else 0
    ks = bs = None
    if summaries is not None:
        ks, bs = summaries
    for name, t, shape in (("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d)),
                           ("lm", lm, (B, Hq, nC, d)), ("q_route", q_route, (B, Hq, N, d)),
                           ("out", out, (B, Hq, N, d)), ("sel", sel, (B, Hkv, N, K)),
                           ("k_sum", ks, (B, Hq, nC, d)), ("b_sum", bs, (B, Hq, nC))):
        _expect(t, name, shape)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("lm", lm), ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    if summaries is not None:
        _check_tensor(ks, "k_sum", q.dtype, dev)
        _check_tensor(bs, "b_sum", torch.float32, dev)
    cfg = make_cfg(B, N, Hq, Hkv, d, S, W, K, q.dtype, mode, scale, generic, union)
    ws, need = _workspace(cfg, False, dev, ws)
    st = _lib.lib().hils_prefill(ctypes.byref(cfg), _ptr(q), _ptr(q_route), _ptr(k), _ptr(v),
                                 _ptr(lm), _ptr(out), _ptr(sel), _ptr(ks), _ptr(bs), _ptr(ws),
                                 ctypes.c_size_t(ws.numel()), _stream(dev))
    check(st, "hils_prefill")
    return out


def summarize(k, lm, S, c0=0, c1=None, out=None, mode="surrogate", scale=0.0, Hq=None):
    """Chunk summaries for chunks [c0, c1): returns (k_sum [B,Hq,N//S,d], b_sum [B,Hq,N//S]).
    In "mean_pool" mode lm may be None (then pass Hq)."""
    B, Hkv, N, d = _dims(k, "k", 4)
    if Hq is None:
        if lm is None:
            raise ValueError("summarize: Hq is required when lm is None")
        Hq = _dims(lm, "lm", 4)[1]
    nC = N // S if S > 0 else 0
    c1 = nC if c1 is None else c1
    _expect(lm, "lm", (B, Hq, nC, d))
    if out is not None:
        _expect(out[0], "k_sum", (B, Hq, nC, d))
        _expect(out[1], "b_sum", (B, Hq, nC))
    dev = k.device
    _check_tensor(k, "k", None, dev)
    _check_tensor(lm, "lm", k.dtype, dev)
    if out is None:
        out = (torch.empty((B, Hq, nC, d), dtype=k.dtype, device=dev),
               torch.empty((B, Hq, nC), dtype=torch.float32, device=dev))
    ks, bs = out
    _check_tensor(ks, "k_sum", k.dtype, dev)
    _check_tensor(bs, "b_sum", torch.float32, dev)
    cfg = make_cfg(B, N, Hq, Hkv, d, S, 1, 1, k.dtype, mode, scale)
    st = _lib.lib().hils_summarize(ctypes.byref(cfg), _ptr(k), _ptr(lm), int(c0), int(c1),
                                   _ptr(ks), _ptr(bs), _stream(dev))
    check(st, "hils_summarize")
    return ks, bs


def decode(q, k_cache, v_cache, seqlen, k_sum, b_sum, S, W, K, q_route=None, mode="surrogate",
           scale=0.0, out=None, sel=None, ws=None):
    """HiLS single-step decode. q [B,Hq,1,d]; caches [B,Hkv,T,d]; seqlen [B] int32 (device);
    k_sum [B,Hq,T//S,d], b_sum [B,Hq,T//S].  Returns out [B,Hq,1,d]."""
    B, Hq, one, d = _dims(q, "q", 4)
    if one != 1:
        raise ValueError(f"decode takes one query per sequence: q has shape {tuple(q.shape)}")
    Hkv, T = _dims(k_cache, "k_cache", 4)[1:3]
    nC = T // S if S > 0 else 0
    for name, t, shape in (("k_cache", k_cache, (B, Hkv, T, d)), ("v_cache", v_cache, (B, Hkv, T, d)),
                           ("seqlen", seqlen, (B,)), ("k_sum", k_sum, (B, Hq, nC, d)),
                           ("b_sum", b_sum, (B, Hq, nC)), ("q_route", q_route, (B, Hq, 1, d)),
                           ("out", out, (B, Hq, 1, d)), ("sel", sel, (B, Hkv, K))):
        _expect(t, name, shape)
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_sum", k_sum),
                    ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    _check_tensor(seqlen, "seqlen", torch.int32, dev)
    _check_tensor(b_sum, "b_sum", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    cfg = make_cfg(B, T, Hq, Hkv, d, S, W, K, q.dtype, mode, scale)
    ws, need = _workspace(cfg, True, dev, ws)
    st = _lib.lib().hils_decode(ctypes.byref(cfg), _ptr(q), _ptr(q_route), _ptr(k_cache),
                                _ptr(v_cache), _ptr(seqlen), _ptr(k_sum), _ptr(b_sum), _ptr(out),
                                _ptr(sel), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    check(st, "hils_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, seqlen, k_sum, b_sum, S, W, K, q_route=None,
                   mode="surrogate", scale=0.0, out=None, sel=None):
    """hils_decode_noalloc: the single-step decode with the library's own
    per-GPU scratch instead of a workspace (no device allocation in the call
    when `out` is given).  Same arguments and result as decode() without ws."""
    B, Hq, one, d = _dims(q, "q", 4)
    if one != 1:
        raise ValueError(f"decode takes one query per sequence: q has shape {tuple(q.shape)}")
    Hkv, T = _dims(k_cache, "k_cache", 4)[1:3]
    nC = T // S if S > 0 else 0
    for name, t, shape in (("k_cache", k_cache, (B, Hkv, T, d)), ("v_cache", v_cache, (B, Hkv, T, d)),
                           ("seqlen", seqlen, (B,)), ("k_sum", k_sum, (B, Hq, nC, d)),
                           ("b_sum", b_sum, (B, Hq, nC)), ("q_route", q_route, (B, Hq, 1, d)),
                           ("out", out, (B, Hq, 1, d)), ("sel", sel, (B, Hkv, K))):
        _expect(t, name, shape)
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_sum", k_sum),
                    ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    _check_tensor(seqlen, "seqlen", torch.int32, dev)
    _check_tensor(b_sum, "b_sum", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    cfg = make_cfg(B, T, Hq, Hkv, d, S, W, K, q.dtype, mode, scale)
    st = _lib.lib().hils_decode_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(q_route), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(seqlen), _ptr(k_sum), _ptr(b_sum),
                                        _ptr(out), _ptr(sel), _stream(dev))
    check(st, "hils_decode_noalloc")
    return out


def decode_multi(q, k_cache, v_cache, seqlen, k_sum, b_sum, S, W, K, q_route=None,
                 mode="surrogate", scale=0.0, out=None, sel=None, ws=None):
    """HiLS decode of M new tokens per sequence. q [B,Hq,M,d] (token m at position
    seqlen[b] - M + m); caches [B,Hkv,T,d]; seqlen [B] int32 (device);
    k_sum [B,Hq,T//S,d], b_sum [B,Hq,T//S].  Returns out [B,Hq,M,d]; sel, if
    given, [B,Hkv,M,K] int32 receives the selected chunk ids."""
    B, Hq, M, d = _dims(q, "q", 4)
    Hkv, T = _dims(k_cache, "k_cache", 4)[1:3]
    nC = T // S if S > 0 else 0
    for name, t, shape in (("k_cache", k_cache, (B, Hkv, T, d)), ("v_cache", v_cache, (B, Hkv, T, d)),
                           ("seqlen", seqlen, (B,)), ("k_sum", k_sum, (B, Hq, nC, d)),
                           ("b_sum", b_sum, (B, Hq, nC)), ("q_route", q_route, (B, Hq, M, d)),
                           ("out", out, (B, Hq, M, d)), ("sel", sel, (B, Hkv, M, K))):
        _expect(t, name, shape)
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_sum", k_sum),
                    ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    _check_tensor(seqlen, "seqlen", torch.int32, dev)
    _check_tensor(b_sum, "b_sum", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    cfg = make_cfg(B, T, Hq, Hkv, d, S, W, K, q.dtype, mode, scale)
    need = _lib.lib().hils_decode_multi_workspace_bytes(ctypes.byref(cfg), int(M))
    if need == 0:
        raise ValueError(f"decode_multi: unsupported configuration (M={M})")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.lib().hils_decode_multi(ctypes.byref(cfg), int(M), _ptr(q), _ptr(q_route),
                                      _ptr(k_cache), _ptr(v_cache), _ptr(seqlen), _ptr(k_sum),
                                      _ptr(b_sum), _ptr(out), _ptr(sel), _ptr(ws),
                                      ctypes.c_size_t(ws.numel()), _stream(dev))
    check(st, "hils_decode_multi")
    return out


def prefill_backward(q, k, v, lm, dout, sel, S, W, K, q_route=None, mode="surrogate", scale=0.0,
                     summaries=None, ws=None):
    """Gradients of sum(dout * prefill(...)) with the forward's selection `sel`
    [B,Hkv,N,K] held fixed.  Returns a dict of fp32 tensors dq, dk, dv, dlm
    (None in mean_pool mode) and dq_route (None without q_route)."""
    B, Hq, N, d = _dims(q, "q", 4)
    Hkv = _dims(k, "k", 4)[1]
    nC = N // S if S > 0 else 0
    for name, t, shape in (("k", k, (B, Hkv, N, d)), ("v", v, (B, Hkv, N, d)),
                           ("lm", lm, (B, Hq, nC, d)), ("dout", dout, (B, Hq, N, d)),
                           ("q_route", q_route, (B, Hq, N, d)), ("sel", sel, (B, Hkv, N, K))):
        _expect(t, name, shape)
    if summaries is not None:
        _expect(summaries[0], "k_sum", (B, Hq, nC, d))
        _expect(summaries[1], "b_sum", (B, Hq, nC))
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("lm", lm), ("dout", dout), ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    ks = bs = None
    if summaries is not None:
        ks, bs = summaries
        _check_tensor(ks, "k_sum", q.dtype, dev)
        _check_tensor(bs, "b_sum", torch.float32, dev)
    cfg = make_cfg(B, N, Hq, Hkv, d, S, W, K, q.dtype, mode, scale)
    need = _lib.lib().hils_prefill_backward_workspace_bytes(ctypes.byref(cfg))
    if need == 0:
        raise ValueError("prefill_backward: unsupported configuration")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dqr = torch.empty(q.shape, **f32) if q_route is not None else None
    dlm = torch.empty((B, Hq, N // S, d), **f32) if (mode != "mean_pool" and N // S > 0) else None
    st = _lib.lib().hils_prefill_backward(ctypes.byref(cfg), _ptr(q), _ptr(q_route), _ptr(k), _ptr(v),
                                          _ptr(lm), _ptr(dout), _ptr(sel), _ptr(ks), _ptr(bs),
                                          _ptr(dq), _ptr(dqr), _ptr(dk), _ptr(dv), _ptr(dlm),
                                          _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    check(st, "hils_prefill_backward")
    return dict(dq=dq, dk=dk, dv=dv, dlm=dlm, dq_route=dqr)


def summarize_paged(k_pages, lm_pages, pages, S, N, out=None, mode="surrogate", scale=0.0):
    """Summaries of the pages listed in `pages` (int32 device tensor) of a paged
    cache: k_pages [P,Hkv,S,d], lm_pages [P,Hq,d].  Returns (k_sum_pages [P,Hq,d],
    b_sum_pages [P,Hq]); `out` reuses existing page-summary tensors."""
    P, Hkv, S_, d = _dims(k_pages, "k_pages", 4)
    if lm_pages is None:
        raise ValueError("summarize_paged: lm_pages is required (it sets Hq)")
    Hq = _dims(lm_pages, "lm_pages", 3)[1]
    if S_ != S:
        raise ValueError(f"k_pages page size {S_} != S={S}")
    _expect(lm_pages, "lm_pages", (P, Hq, d))
    _dims(pages, "pages", 1)
    if out is not None:
        _expect(out[0], "k_sum_pages", (P, Hq, d))
        _expect(out[1], "b_sum_pages", (P, Hq))
    dev = k_pages.device
    _check_tensor(k_pages, "k_pages", None, dev)
    _check_tensor(lm_pages, "lm_pages", k_pages.dtype, dev)
    _check_tensor(pages, "pages", torch.int32, dev)
    if out is None:
        out = (torch.empty((P, Hq, d), dtype=k_pages.dtype, device=dev),
               torch.empty((P, Hq), dtype=torch.float32, device=dev))
    ks, bs = out
    _check_tensor(ks, "k_sum_pages", k_pages.dtype, dev)
    _check_tensor(bs, "b_sum_pages", torch.float32, dev)
    cfg = make_cfg(1, N, Hq, Hkv, d, S, 1, 1, k_pages.dtype, mode, scale)
    st = _lib.lib().hils_summarize_paged(ctypes.byref(cfg), _ptr(k_pages), _ptr(lm_pages),
                                         _ptr(pages), int(pages.numel()), P, _ptr(ks), _ptr(bs),
                                         _stream(dev))
    check(st, "hils_summarize_paged")
    return out


def decode_paged(q, k_pages, v_pages, page_table, seqlen, k_sum_pages, b_sum_pages, S, W, K,
                 q_route=None, mode="surrogate", scale=0.0, out=None, sel=None, ws=None):
    """HiLS single-step decode over a paged cache (one chunk per page).
    q [B,Hq,1,d]; k_pages/v_pages [P,Hkv,S,d]; page_table [B,max_pages] int32;
    seqlen [B] int32; k_sum_pages [P,Hq,d]; b_sum_pages [P,Hq].  Returns out."""
    B, Hq, one, d = _dims(q, "q", 4)
    if one != 1:
        raise ValueError(f"decode takes one query per sequence: q has shape {tuple(q.shape)}")
    P, Hkv = _dims(k_pages, "k_pages", 4)[:2]
    maxp = _dims(page_table, "page_table", 2)[1]
    for name, t, shape in (("k_pages", k_pages, (P, Hkv, S, d)), ("v_pages", v_pages, (P, Hkv, S, d)),
                           ("page_table", page_table, (B, maxp)), ("seqlen", seqlen, (B,)),
                           ("k_sum_pages", k_sum_pages, (P, Hq, d)),
                           ("b_sum_pages", b_sum_pages, (P, Hq)), ("q_route", q_route, (B, Hq, 1, d)),
                           ("out", out, (B, Hq, 1, d)), ("sel", sel, (B, Hkv, K))):
        _expect(t, name, shape)
    dev = q.device
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("k_sum_pages", k_sum_pages), ("q_route", q_route)):
        _check_tensor(t, name, q.dtype, dev)
    _check_tensor(page_table, "page_table", torch.int32, dev)
    _check_tensor(seqlen, "seqlen", torch.int32, dev)
    _check_tensor(b_sum_pages, "b_sum_pages", torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", q.dtype, dev)
    _check_tensor(sel, "sel", torch.int32, dev)
    cfg = make_cfg(B, maxp * S, Hq, Hkv, d, S, W, K, q.dtype, mode, scale)
    ws, need = _workspace(cfg, True, dev, ws)
    st = _lib.lib().hils_decode_paged(ctypes.byref(cfg), _ptr(q), _ptr(q_route), _ptr(k_pages),
                                      _ptr(v_pages), P, _ptr(page_table), maxp, _ptr(seqlen),
                                      _ptr(k_sum_pages), _ptr(b_sum_pages), _ptr(out), _ptr(sel),
                                      _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    check(st, "hils_decode_paged")
    return out
