"""The training-memory model against the values the recomputation page prints.

Fixtures: tests/golden/memory_table_gpt2_fp16.txt (Brenndoerfer, "FlashAttention
Algorithm > Recomputation Strategy", console Out[18]) and
tests/golden/attention_matrix_8192.txt (same page, "Why Recomputation Makes Sense").
"""
import os

import pytest

from oracle import training_memory

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [float(x) for x in line.split()]


def _printed(x, ref, decimals):
    return round(x, decimals) == pytest.approx(ref, abs=10 ** -(decimals + 3))


def test_table_matches_printed_values():
    rows = list(_rows("memory_table_gpt2_fp16.txt"))
    assert len(rows) == 4
    for n, std, rec, sav, attn in rows:
        r = training_memory(int(n), d_model=768, heads=12, layers=12, elem_bytes=2)
        assert _printed(r.standard_gb, std, 2), (n, r.standard_gb, std)
        assert _printed(r.recompute_gb, rec, 3), (n, r.recompute_gb, rec)
        assert _printed(r.savings_pct, sav, 1), (n, r.savings_pct, sav)
        assert _printed(r.attn_matrix_gb, attn, 2), (n, r.attn_matrix_gb, attn)


def test_single_attention_matrix_size():
    (n, eb, mb), = list(_rows("attention_matrix_8192.txt"))
    assert int(n) ** 2 * int(eb) == 134_217_728
    assert round(int(n) ** 2 * int(eb) / 1e6) == int(mb)


def test_recompute_memory_is_linear_in_sequence_length():
    a = training_memory(4096).recompute_gb
    b = training_memory(8192).recompute_gb
    c = training_memory(16384).recompute_gb
    assert b == pytest.approx(2 * a) and c == pytest.approx(2 * b)
    s1, s2 = training_memory(4096).attn_matrix_gb, training_memory(8192).attn_matrix_gb
    assert s2 == pytest.approx(4 * s1)
