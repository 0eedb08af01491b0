"""Seeded synthetic workloads for the attention forward pass.

This package only draws random inputs and stores them in the storage type
(fp32, fp16 or bf16 bit patterns).  It holds none of the attention
arithmetic, so both the fp64 oracle and the GPU library can consume its
output without sharing any computation.
"""

from .configs import CONFIGS, HEADLINE, ORDER, PAGE_TABLE, Workload, flops, get, min_bytes, naive_bytes, score_matrix_bytes  # noqa: F401
from .inputs import make_inputs, round_to_storage, storage_itemsize  # noqa: F401
