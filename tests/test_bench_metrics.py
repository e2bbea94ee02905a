"""The arithmetic behind bench.py's reported figures (CPU only): prefill work counted pair by pair
against its closed form, and the decode step's algorithmic bytes counted by hand."""
import numpy as np
import pytest

import bench
from workloads import make_decode_workload, make_workload


def _pairs_brute(q_lens, ctx):
    """Visible (query, key) pairs, one query at a time: a query at position p sees keys 0..p."""
    n = 0
    for ql, c in zip(q_lens, ctx):
        if ql <= 1:  # decode rows are not prefill work
            continue
        for t in range(ql):
            pos = c - ql + t
            for k in range(c):
                if k <= pos:
                    n += 1
    return n


@pytest.mark.parametrize("q_lens,ctx", [([5], [5]), ([3, 1, 7], [3, 40, 12]), ([2, 64, 1], [2, 200, 9])])
def test_prefill_flops_counts_visible_pairs(q_lens, ctx):
    hq, d = 4, 64
    assert bench.prefill_flops(q_lens, ctx, hq, d) == 4 * d * hq * _pairs_brute(q_lens, ctx)


def test_prefill_flops_closed_form_without_cached_prefix():
    # a prompt of L tokens with no cached prefix: L(L+1)/2 visible pairs, 2·Hq·d·L(L+1) flops
    for L in (2, 17, 200, 2048):
        assert bench.prefill_flops([L], [L], 40, 128) == 2 * 40 * 128 * L * (L + 1)


def test_decode_bytes_by_hand():
    ctx = [1, 16, 17, 100]
    w = make_decode_workload(9, ctx, 8, 2, 64, "bf16", 16, name="bytes")
    kv, total = bench.decode_algorithmic_bytes(ctx, w, 4)
    per_token = 2 * 2 * 64 * 2  # K and V, 2 kv heads, 64 dims, 2 bytes
    assert w.kv_bytes_per_token() == per_token
    assert kv == sum(ctx) * per_token
    q = 4 * 8 * 64 * 2          # 4 sequences x 8 query heads x 64 dims, bf16
    out = 4 * 8 * 64 * 4        # fp32 output
    tables = (1 + 1 + 2 + 7) * 4 + 4 * 4  # ceil(ctx / 16) entries and one length per sequence
    assert total == kv + q + out + tables


def test_headline_kv_bytes_per_token():
    # the GQA configuration: 8 kv heads x 128 dims x bf16, K and V: 4096 bytes per attended token
    w = make_workload("gqa", "full")
    assert (w.num_kv_heads, w.head_dim, w.dtype) == (8, 128, "bf16")
    assert w.kv_bytes_per_token() == 4096
