"""Training-memory accounting of stored attention activations (TEST INFRASTRUCTURE ONLY).

Follows the analytic model of Brenndoerfer, "FlashAttention Algorithm >
Recomputation Strategy", code cell In[17] and its printed table Out[18]
(GPT-2 config, 16-bit values), restated here from its description:

  * standard attention keeps, per layer, two [heads, N, N] matrices (the
    scores and the softmax weights) plus the four [N, d_model] activations
    Q, K, V and O;
  * the recomputing method keeps the same four [N, d_model] activations
    plus two per-row statistics (running max m and normaliser L) for every
    (position, head);
  * every stored value takes `elem_bytes` bytes; totals are per model
    (times the number of layers) and reported in units of 1e9 bytes.

This is the page's own accounting and is pinned to its printed table by
tests/test_memory_model.py.  Note the page's prose below the table ("over
24 GB", "97%") disagrees with the table; the table is what the model gives.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class MemoryRow:
    seq_len: int
    standard_gb: float
    recompute_gb: float
    savings_pct: float
    attn_matrix_gb: float


def training_memory(seq_len: int, d_model: int = 768, heads: int = 12, layers: int = 12,
                    elem_bytes: int = 2) -> MemoryRow:
    activations = 4 * seq_len * d_model            # Q, K, V, O values per layer
    square = 2 * heads * seq_len * seq_len         # scores + weights values per layer
    row_stats = 2 * heads * seq_len                # (m, L) per position and head
    std_bytes = layers * elem_bytes * (activations + square)
    rec_bytes = layers * elem_bytes * (activations + row_stats)
    return MemoryRow(
        seq_len=seq_len,
        standard_gb=std_bytes / 1e9,
        recompute_gb=rec_bytes / 1e9,
        savings_pct=100.0 * (std_bytes - rec_bytes) / std_bytes,
        attn_matrix_gb=layers * elem_bytes * square / 1e9,
    )
