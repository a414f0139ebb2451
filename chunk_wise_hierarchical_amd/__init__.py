"""HiLS (Hierarchical Landmark Sparse) attention forward pass for AMD MI355X (gfx950).

The computation lives in libhils.so (hand-written HIP kernels behind the C ABI
of include/hils.h); this package only marshals torch tensors into that ABI.
"""
from .api import (decode, decode_multi, decode_noalloc, decode_paged, make_cfg, prefill,  # noqa: F401
                  prefill_backward, summarize, summarize_paged, workspace_bytes)
from ._lib import HilsError, LIB_PATH  # noqa: F401

__all__ = ["prefill", "prefill_backward", "decode", "decode_multi", "decode_noalloc", "decode_paged", "summarize", "summarize_paged", "workspace_bytes",
           "make_cfg", "HilsError", "LIB_PATH"]
