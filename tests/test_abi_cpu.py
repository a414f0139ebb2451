"""CPU-only checks of the C-ABI library: it loads, exports every symbol
include/hils.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from chunk_wise_hierarchical_amd import _lib
from chunk_wise_hierarchical_amd._lib import HilsCfg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")
PKG = os.path.join(ROOT, "chunk_wise_hierarchical_amd")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hils_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libhils.so is not built (run python -m chunk_wise_hierarchical_amd.build)")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) >= set(_lib.EXPORTED)
    for n in names:
        assert hasattr(L, n), f"{n} declared in hils.h but not exported"


def test_version_and_strerror(L):
    assert L.hils_abi_version() == 1
    assert L.hils_strerror(0) == b"ok"
    assert b"workspace" in L.hils_strerror(3)


def _cfg(**kw):
    base = dict(B=1, N=1024, Hq=8, Hkv=2, d=128, S=64, W=256, K=8, dtype=0, mode=0, scale=0.0,
                flags=0)
    base.update(kw)
    return HilsCfg(**base)


def test_workspace_bytes(L):
    # generic kernels: summaries + selection ids + fusion logits (each 256-byte aligned)
    n = L.hils_workspace_bytes(ctypes.byref(_cfg(flags=_lib.HILS_FLAG_GENERIC)), 0)
    want = (1 * 8 * 16 * 128 * 2) + (1 * 8 * 16 * 4) + (1 * 2 * 1024 * 8 * 4) + (1 * 8 * 1024 * 8 * 4)
    assert want <= n <= want + 4 * 256
    # MFMA fast path (bf16, d=128, S=64), query-block unions: summaries + selection
    # ids + per-chunk V^T + k' in MFMA fragment order (per query head and 32-chunk
    # tile, nine 1 KB fragments)
    n = L.hils_workspace_bytes(ctypes.byref(_cfg(flags=_lib.HILS_FLAG_UNION)), 0)
    base = (1 * 8 * 16 * 128 * 2) + (1 * 8 * 16 * 4) + (1 * 2 * 1024 * 8 * 4) + (1 * 2 * 16 * 128 * 64 * 2) \
        + (1 * 8 * 1 * 9 * 1024)
    assert base <= n <= base + 5 * 256
    # default per-chunk buckets add, for one slice of 1024 queries (G=4, 16 pairs a tile):
    # 4 bucket arrays, totals, scan-block totals, tile table, pair list, pair fusion
    # logits, bf16 per-chunk outputs
    n = L.hils_workspace_bytes(ctypes.byref(_cfg()), 0)
    F, P = 2 * 16, 2 * 1024 * 8
    want = base + 4 * F * 4 + 16 + 8 + (P // 16 + F) * 8 + P * 4 + P * 4 * 4 + P * 4 * 128 * 2
    assert want <= n <= want + 16 * 256
    assert L.hils_workspace_bytes(ctypes.byref(_cfg()), 1) > 0
    for bad in (dict(Hq=7), dict(d=0), dict(K=0), dict(dtype=5), dict(mode=9), dict(N=0)):
        assert L.hils_workspace_bytes(ctypes.byref(_cfg(**bad)), 0) == 0, bad


def _prefill(L, c, ws_bytes=1 << 30, null_q=False, misalign=False, null_lm=False):
    p = ctypes.c_void_p(0x10000)
    q = None if null_q else ctypes.c_void_p(0x10000 + (8 if misalign else 0))
    lm = None if null_lm else p
    return L.hils_prefill(ctypes.byref(c), q, None, p, p, lm, p, None, None, None, p,
                          ctypes.c_size_t(ws_bytes), None)


def test_argument_errors_return_before_launch(L):
    assert _prefill(L, _cfg(Hq=6, Hkv=4)) == _lib.HILS_E_ARG
    assert _prefill(L, _cfg(), null_q=True) == _lib.HILS_E_ARG
    assert _prefill(L, _cfg(), misalign=True) == _lib.HILS_E_ARG
    assert _prefill(L, _cfg(d=512)) == _lib.HILS_E_UNSUPPORTED
    assert _prefill(L, _cfg(S=128)) == _lib.HILS_E_UNSUPPORTED
    # the landmark queries are needed by the Proposition 3.1 and landmark-key modes only
    assert _prefill(L, _cfg(mode=0), null_lm=True) == _lib.HILS_E_ARG
    assert _prefill(L, _cfg(mode=1), null_lm=True) == _lib.HILS_E_ARG
    for m in (2, 3):
        assert _prefill(L, _cfg(mode=m), ws_bytes=16, null_lm=True) == _lib.HILS_E_WORKSPACE
    assert _prefill(L, _cfg(), ws_bytes=16) == _lib.HILS_E_WORKSPACE
    p = ctypes.c_void_p(0x10000)
    # k_sum without b_sum
    assert L.hils_prefill(ctypes.byref(_cfg()), p, None, p, p, p, p, None, p, None, p,
                          ctypes.c_size_t(1 << 30), None) == _lib.HILS_E_ARG
    # summarize: chunk range outside [0, N/S]
    assert L.hils_summarize(ctypes.byref(_cfg()), p, p, 0, 17, p, p, None) == _lib.HILS_E_ARG
    assert L.hils_summarize(ctypes.byref(_cfg()), p, p, 3, 2, p, p, None) == _lib.HILS_E_ARG
    assert L.hils_summarize(ctypes.byref(_cfg()), p, p, 2, 2, p, p, None) == _lib.HILS_OK
    # decode: missing seqlen, head dim not a multiple of the vector width
    assert L.hils_decode(ctypes.byref(_cfg()), p, None, p, p, None, p, p, p, None, p,
                         ctypes.c_size_t(1 << 30), None) == _lib.HILS_E_ARG
    assert L.hils_decode(ctypes.byref(_cfg(d=12)), p, None, p, p, p, p, p, p, None, p,
                         ctypes.c_size_t(1 << 30), None) == _lib.HILS_E_UNSUPPORTED
    # exact scoring is a prefill test mode; decode and summaries reject it
    assert L.hils_decode(ctypes.byref(_cfg(mode=2)), p, None, p, p, p, p, p, p, None, p,
                         ctypes.c_size_t(1 << 30), None) == _lib.HILS_E_UNSUPPORTED
    assert L.hils_summarize(ctypes.byref(_cfg(mode=2)), p, p, 0, 2, p, p, None) == _lib.HILS_E_ARG
    assert L.hils_summarize(ctypes.byref(_cfg(mode=4)), p, p, 0, 2, p, p, None) == _lib.HILS_E_ARG


def test_paged_entry_points_reject_bad_arguments(L):
    p = ctypes.c_void_p(0x10000)
    c = _cfg(N=1024)                      # 16 chunks of 64
    ws = ctypes.c_size_t(1 << 30)
    # decode: table narrower than the capacity, no pages, missing table
    assert L.hils_decode_paged(ctypes.byref(c), p, None, p, p, 40, p, 15, p, p, p, p, None, p, ws,
                               None) == _lib.HILS_E_ARG
    assert L.hils_decode_paged(ctypes.byref(c), p, None, p, p, 0, p, 16, p, p, p, p, None, p, ws,
                               None) == _lib.HILS_E_ARG
    assert L.hils_decode_paged(ctypes.byref(c), p, None, p, p, 40, None, 16, p, p, p, p, None, p,
                               ws, None) == _lib.HILS_E_ARG
    assert L.hils_decode_paged(ctypes.byref(c), p, None, p, p, 40, p, 16, p, p, p, p, None, p,
                               ctypes.c_size_t(16), None) == _lib.HILS_E_WORKSPACE
    # summaries: negative count, no pages; zero listed pages is a no-op
    assert L.hils_summarize_paged(ctypes.byref(c), p, p, p, -1, 40, p, p, None) == _lib.HILS_E_ARG
    assert L.hils_summarize_paged(ctypes.byref(c), p, p, p, 3, 0, p, p, None) == _lib.HILS_E_ARG
    assert L.hils_summarize_paged(ctypes.byref(c), p, p, p, 0, 40, p, p, None) == _lib.HILS_OK


def test_multi_decode_arguments_and_workspace(L):
    p = ctypes.c_void_p(0x10000)
    c = _cfg(N=1024)
    ws = ctypes.c_size_t(1 << 30)

    def call(M, cfg=c, wsb=ws, seqlen=p):
        return L.hils_decode_multi(ctypes.byref(cfg), M, p, None, p, p, seqlen, p, p, p, None, p,
                                   wsb, None)
    assert call(0) == _lib.HILS_E_ARG
    assert call(17) == _lib.HILS_E_UNSUPPORTED
    assert call(4, seqlen=None) == _lib.HILS_E_ARG
    assert call(4, cfg=_cfg(N=1024, mode=2)) == _lib.HILS_E_UNSUPPORTED
    assert call(4, wsb=ctypes.c_size_t(16)) == _lib.HILS_E_WORKSPACE
    # the per-row buffers of an M-token block are those of B*M single decodes,
    # plus (bf16, d=128, S=64) the block's chunk union per (sequence, KV group):
    # its size and M*K ids, and a slot byte per (union element, token)
    one = L.hils_decode_multi_workspace_bytes(ctypes.byref(c), 1)
    assert one == L.hils_workspace_bytes(ctypes.byref(c), 1)
    four = L.hils_decode_multi_workspace_bytes(ctypes.byref(c), 4)
    bg, mk = c.B * c.Hkv, 4 * c.K
    align = lambda x: (x + 255) // 256 * 256
    union = align(bg * (mk + 1) * 4 + bg * mk * 4) - align(8)
    assert four == L.hils_workspace_bytes(ctypes.byref(_cfg(N=1024, B=4 * c.B)), 1) + union
    c32 = _cfg(N=1024, dtype=1)                    # fp32 blocks attend token by token
    assert (L.hils_decode_multi_workspace_bytes(ctypes.byref(c32), 4)
            == L.hils_workspace_bytes(ctypes.byref(_cfg(N=1024, B=4, dtype=1)), 1))
    assert L.hils_decode_multi_workspace_bytes(ctypes.byref(c), 0) == 0
    assert L.hils_decode_multi_workspace_bytes(ctypes.byref(c), 17) == 0


def test_backward_head_dim_granularity(L):
    # the column pass reads each thread's d / 8 elements as whole 16-byte vectors
    ok = L.hils_prefill_backward_workspace_bytes
    assert ok(ctypes.byref(_cfg(d=128))) > 0 and ok(ctypes.byref(_cfg(d=64))) > 0
    assert ok(ctypes.byref(_cfg(d=32))) == 0                       # bf16: d % 64
    assert ok(ctypes.byref(_cfg(d=32, dtype=1))) > 0               # fp32: d % 32
    assert ok(ctypes.byref(_cfg(d=16, dtype=1))) == 0


def test_backward_workspace_holds_the_dq_partials(L):
    # the matrix-core backward (bf16, d in {64, 128}, S % 16 == 0) keeps one fp32
    # dq partial row per (query, head, selected slot or window chunk) and the
    # window partials; fp32 inputs take the vector-ALU kernels without them
    ok = L.hils_prefill_backward_workspace_bytes
    c = _cfg(N=1024, W=256, K=8)
    nwin = -(-(256 + 64 - 1) // 64)
    parts = 1 * 8 * 1024 * (8 + nwin) * 128 * 4 + 1 * 8 * 1024 * nwin * 16
    bf16, f32 = ok(ctypes.byref(c)), ok(ctypes.byref(_cfg(N=1024, W=256, K=8, dtype=1)))
    assert bf16 >= parts
    # fp32 summaries are twice the size; everything else is shared
    assert 0 < f32 < bf16 - parts + 1 * 8 * 16 * 128 * 2 + 4096
    # long sequences run in query slices whose partials fit 4 GiB
    big = _cfg(N=1 << 20, Hq=32, Hkv=8, W=2048, K=64)
    big_parts = (1 << 20) * 32 * (64 + 33) * 128 * 4
    assert 0 < ok(ctypes.byref(big)) < big_parts


def test_decode_rejects_batches_beyond_the_scoring_grid(L):
    # the decode scoring grid holds (sequence, query head) in its y dimension:
    # B * Hq = 8192 * 8 is one past its limit of 65535
    p = ctypes.c_void_p(0x10000)
    c = _cfg(N=1024, B=8192, Hq=8, Hkv=2)
    ws = ctypes.c_size_t(L.hils_workspace_bytes(ctypes.byref(c), 1))
    assert ws.value > 0
    args = (p, None, p, p, p, p, p, p, None, p, ws, None)
    assert L.hils_decode(ctypes.byref(c), *args) == _lib.HILS_E_UNSUPPORTED
    assert L.hils_decode_multi(ctypes.byref(c), 1, *args) == _lib.HILS_E_UNSUPPORTED
    assert L.hils_decode_paged(ctypes.byref(c), p, None, p, p, 16, p, 16, p, p, p, p, None, p, ws,
                               None) == _lib.HILS_E_UNSUPPORTED


def test_product_path_does_not_touch_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f), errors="ignore").read()
                assert "oracle" not in txt.lower(), f"{f} mentions the oracle"


def test_wrappers_reject_mis_shaped_tensors():
    """The torch wrappers check every tensor's exact shape against (B, Hq, Hkv,
    N, d, S, K) before anything reaches the C ABI, which takes bare pointers."""
    import torch
    import chunk_wise_hierarchical_amd as hils

    B, Hq, Hkv, N, d, S, W, K = 1, 4, 2, 256, 16, 32, 64, 4
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros(B, Hq, N, d, **bf)
    k = torch.zeros(B, Hkv, N, d, **bf)
    v = torch.zeros(B, Hkv, N, d, **bf)
    lm = torch.zeros(B, Hq, N // S, d, **bf)

    def bad(fn, *a, **kw):
        with pytest.raises(ValueError, match="shape|dimensions"):
            fn(*a, **kw)

    bad(hils.prefill, q, k, v, lm, S, W, K, sel=torch.zeros(B, Hkv, N, K - 1, dtype=torch.int32))
    bad(hils.prefill, q, k[:, :, :N - 1].contiguous(), v, lm, S, W, K)
    bad(hils.prefill, q, k, v, lm[:, :, :N // S - 1].contiguous(), S, W, K)
    bad(hils.prefill, q, k, v, lm, S, W, K, out=torch.zeros(B, Hq, N, d + 8, **bf))
    bad(hils.prefill, q, k, v, lm, S, W, K,
        summaries=(torch.zeros(B, Hq, N // S + 1, d, **bf), torch.zeros(B, Hq, N // S + 1)))
    bad(hils.summarize, k, lm[:, :, :3].contiguous(), S)
    qd = torch.zeros(B, Hq, 1, d, **bf)
    ks = torch.zeros(B, Hq, N // S, d, **bf)
    bs = torch.zeros(B, Hq, N // S)
    sl = torch.full((B,), N, dtype=torch.int32)
    bad(hils.decode, qd, k, v, sl, ks[:, :, :2].contiguous(), bs, S, W, K)
    bad(hils.decode, qd, k, v, torch.full((B + 1,), N, dtype=torch.int32), ks, bs, S, W, K)
    bad(hils.decode, qd, k, v, sl, ks, bs, S, W, K, sel=torch.zeros(B, Hkv, K - 1, dtype=torch.int32))
    bad(hils.decode, torch.zeros(B, Hq, 2, d, **bf), k, v, sl, ks, bs, S, W, K)
    bad(hils.decode_multi, torch.zeros(B, Hq, 3, d, **bf), k, v, sl, ks, bs, S, W, K,
        sel=torch.zeros(B, Hkv, 2, K, dtype=torch.int32))
    bad(hils.prefill_backward, q, k, v, lm, torch.zeros(B, Hq, N - 1, d, **bf),
        torch.zeros(B, Hkv, N, K, dtype=torch.int32), S, W, K)
    P = 8
    kp = torch.zeros(P, Hkv, S, d, **bf)
    bad(hils.summarize_paged, kp, torch.zeros(P + 1, Hq, d, **bf),
        torch.zeros(P, dtype=torch.int32), S, N)
    bad(hils.decode_paged, qd, kp, kp, torch.zeros(B + 1, N // S, dtype=torch.int32), sl,
        torch.zeros(P, Hq, d, **bf), torch.zeros(P, Hq), S, W, K)
    # well-shaped host tensors get past the shape checks and stop at the device check
    with pytest.raises(ValueError, match="GPU tensor"):
        hils.prefill(q, k, v, lm, S, W, K)


def test_decode_noalloc_refuses_oversized_workspace_before_any_launch(L):
    """The allocation-free decode checks its scratch size before it looks up
    the device buffer or enqueues anything (so this runs without a GPU)."""
    c = _cfg(B=16, N=1 << 22, Hq=32, Hkv=8, W=2048, K=64)
    assert L.hils_workspace_bytes(ctypes.byref(c), 1) > _lib.HILS_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(4096)          # never dereferenced: the call returns first
    st = L.hils_decode_noalloc(ctypes.byref(c), p, None, p, p, p, p, p, p, None, None)
    assert st == _lib.HILS_E_WORKSPACE
    bad = _cfg(Hq=7, Hkv=2)
    assert L.hils_decode_noalloc(ctypes.byref(bad), p, None, p, p, p, p, p, p, None, None) == _lib.HILS_E_ARG
