"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the GPU library.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_backward_dq_rows,
    attention_forward,
    attention_forward_block_sparse,
    attention_forward_block_sparse_rows,
    attention_forward_kv,
    block_visibility,
    attention_forward_rows,
    scores,
    softmax_rows,
)
from . import fp8  # noqa: F401  (FP8 forward with incoherent processing)
