"""The synthetic workloads, shaped like the HiLS paper's settings.

Shapes follow the paper's sparsity settings (chunk size 64, windows 512-2048,
top-K 16-64, 345M/7B-style head counts; "Hierarchical Sparse Attention Done
Right", sections 5.1 and 7.1) at 8K, 64K, 512K and 4M tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    N: int               # prefill length, or KV-cache length for decode
    Hq: int
    Hkv: int
    d: int
    S: int
    W: int
    K: int
    dtype: str           # "bf16" or "f32"
    scaled: bool         # q/k/v/landmarks drawn N(0,1)/sqrt(d) instead of N(0,1)
    regime: str          # head-structure recipe, see synth.generate
    seed: int = 0
    q_share: float = 0.0  # fraction of query variance shared within a segment (0 = i.i.d.)
    q_seg: int = 1        # segment length (tokens) of the shared query component
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    # tiny fp32 prefill: N=512, 2 heads, d=64, S=32, W=64, K=4, i.i.d. N(0,1)
    "tiny_fp32": Workload("tiny_fp32", "prefill", 1, 512, 2, 2, 64, 32, 64, 4,
                          "f32", False, "iid"),
    # bf16 prefill at the 8K training length: B=2, 16/16 heads, d=128, S=64,
    # W=512, K=16; N(0,1)/sqrt(d); heads 8-15 peaked (4 needles in random chunks)
    "prefill_8k": Workload("prefill_8k", "prefill", 2, 8192, 16, 16, 128, 64, 512, 16,
                           "bf16", True, "half_peaked4"),
    # bf16 long prefill: N=65536, 32/8 heads, d=128, S=64, W=1024, K=32; N(0,1);
    # q head h mod 3: uniform / single needle / 8-token cluster over 2-8 chunks
    "prefill_64k": Workload("prefill_64k", "prefill", 1, 65536, 32, 8, 128, 64, 1024, 32,
                            "bf16", False, "mod3"),
    # bf16 decode: B=16, 512K-token KV cache, 32/8 heads, d=128, S=64, W=1024,
    # K=32; N(0,1) KV; one needle chunk per sequence at a random depth
    "decode_512k": Workload("decode_512k", "decode", 16, 524288, 32, 8, 128, 64, 1024, 32,
                            "bf16", False, "needle_chunk"),
    # bf16 extreme context prefill: N=524288, 32/8 heads, d=128, S=64, W=2048,
    # K=64; needles at 10 evenly spaced depths; half the heads peaked
    "prefill_512k": Workload("prefill_512k", "prefill", 1, 524288, 32, 8, 128, 64, 2048, 64,
                             "bf16", False, "depth10"),
    # the same prefill with adjacent queries sharing most of their direction
    # (90% of the variance shared within 512-token segments), so that the
    # M=16 chunk overlap of adjacent queries is in the range trained models show
    "prefill_512k_corr": Workload("prefill_512k_corr", "prefill", 1, 524288, 32, 8, 128, 64,
                                  2048, 64, "bf16", False, "depth10", q_share=0.9, q_seg=512),
    # bf16 extreme context decode: B=1, 4M-token KV cache, same heads/S/W/K
    "decode_4m": Workload("decode_4m", "decode", 1, 4194304, 32, 8, 128, 64, 2048, 64,
                          "bf16", False, "depth10"),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
