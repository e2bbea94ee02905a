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


class _Pool:
    def __init__(self, free):
        self.free = free

    def num_free(self):
        return self.free


class _W:
    def __init__(self, lens, block_size, num_blocks):
        self.context_lens, self.block_size, self.num_blocks = lens, block_size, num_blocks


@pytest.mark.parametrize("B", [8, 16, 32])
def test_last_block_waste_over_a_full_period(B):
    # lengths 1..kB cover every residue of B k times: the mean of the empty slots is (B - 1) / 2
    lens = list(range(1, 3 * B + 1))
    used = sum(-(-L // B) for L in lens)
    u = bench.kv_utilisation(_W(lens, B, used + 5), _Pool(5), 3 * B)
    assert u["last_block_empty_slots_mean"] == (B - 1) / 2 == u["last_block_empty_slots_even_residues"]
    assert u["blocks_in_use"] == used
    assert u["paged"] == round(sum(lens) / (used * B), 4)


def test_last_block_waste_by_hand():
    u = bench.kv_utilisation(_W([1, 16, 17, 100], 16, 20), _Pool(9), 128)
    assert u["last_block_empty_slots_mean"] == (15 + 0 + 15 + 12) / 4
    assert u["blocks_in_use"] == 11 and u["max_len_prealloc"] == round(134 / 512, 4)


def test_split_seqs_counts_contexts_beyond_one_partition():
    hist = [np.array([100, 2048, 2049, 9000]), np.array([2049, 1, 5000, 2048])]
    assert bench.split_seqs(hist, 2048) == 2.0
    assert bench.split_seqs(hist, 1024) == 3.0
