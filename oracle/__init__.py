"""Test infrastructure: a plain CPU float64 oracle for fused linear + cross-entropy.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package imports nothing from
the product path.
"""
from .flce_oracle import (  # noqa: F401
    logits,
    apply_softcap,
    row_logsumexp,
    valid_mask,
    flce_forward_backward,
    flce_forward,
    flce_rows,
    flce_vocab_rows,
    flce_blocked,
    flce_sequences,
)
