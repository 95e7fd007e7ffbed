"""CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The GPU library never calls it, links it or falls back
to it; the two share no code.

Contents
  attention.py     plain fp64 exact attention: materialised P, explicit
                   softmax-Jacobian backward (and the same map in factored
                   form for long rows), row / key-column subset modes.
  memory_model.py  the training-memory accounting of the FlashAttention
                   recomputation page, pinned to the page's printed table.

Parity status: every function here is pinned by tests/test_oracle.py
(closed forms, invariants, finite differences, mpmath, an independent
library routine -- the batched wrappers head by head against torch's float64
scaled-dot-product attention with per-sequence lengths) or
tests/test_memory_model.py (values printed on the page).  Nothing here is
"parity unpinned".
"""
from .attention import (allowed_mask, head_forward, head_backward, attention_forward, attention_backward,
                        rows_forward_backward, key_columns_backward, to_f64)
from .memory_model import training_memory, MemoryRow

__all__ = ["allowed_mask", "head_forward", "head_backward", "attention_forward", "attention_backward",
           "rows_forward_backward", "key_columns_backward", "to_f64", "training_memory", "MemoryRow"]
