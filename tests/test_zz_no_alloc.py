"""The allocation-free decode entry point (hils_decode_noalloc, through the C
ABI) against the workspace entry point (hils_decode): identical outputs and
selections on two calls in a row, the second with a smaller input, so the
shared per-GPU scratch keeps the first call's contents when the second runs."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import chunk_wise_hierarchical_amd as hils


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pair(w, seqlen):
    _say(f"[decode_noalloc] B={w.B} T={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d} S={w.S} W={w.W} "
         f"K={w.K} seqlen={seqlen}")
    x = synth.make_decode_inputs(w, device="cpu", seqlen=seqlen)
    x = {k: v.cuda() for k, v in x.items()}
    ks, bs = hils.summarize(x["k"], x["lm"], w.S)
    s1 = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
    s2 = torch.full_like(s1, -7)
    o1 = hils.decode(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, sel=s1)
    o2 = torch.full_like(o1, 3.0)
    hils.decode_noalloc(x["q"], x["k"], x["v"], x["seqlen"], ks, bs, w.S, w.W, w.K, out=o2, sel=s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(o1, o2)
    _say("   identical to hils_decode")


def test_decode_noalloc_equals_decode_twice_second_smaller():
    big = synth.get_workload("decode_512k", N=16384, B=4)
    _pair(big, [16384, 9000, 700, 1])
    small = synth.get_workload("decode_512k", N=4096, B=2, Hq=8, Hkv=2, K=16, W=512)
    _pair(small, [4096, 3001])


def test_decode_noalloc_rejects_oversized_configuration():
    # a decode workspace beyond the scratch size is refused before any launch
    cfg = hils.make_cfg(16, 1 << 22, 32, 8, 128, 64, 2048, 64, torch.bfloat16)
    need = hils.workspace_bytes(cfg, True)
    from chunk_wise_hierarchical_amd import _lib
    assert need > _lib.HILS_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((16, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((16, 8, 64, 128), dtype=torch.bfloat16, device="cuda")
    import ctypes
    st = _lib.lib().hils_decode_noalloc(ctypes.byref(cfg), ctypes.c_void_p(q.data_ptr()), None,
                                        ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
                                        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(q.data_ptr()),
                                        None, None)
    assert st == _lib.HILS_E_WORKSPACE
