"""Seeded synthetic inputs for HiLS attention (shared by tests, bench and smoke).

Holds no part of the attention method's arithmetic: it only draws random
tensors and plants structure (needles) into them.
"""
from .workloads import WORKLOADS, Workload, get_workload
from .generate import make_prefill_inputs, make_decode_inputs

__all__ = ["WORKLOADS", "Workload", "get_workload", "make_prefill_inputs", "make_decode_inputs"]
