"""Helpers shared by the tests: contiguous histories, pool-layout decoding, bitwise pool
comparison, and the oracle's attention run over groups of sequences on several threads.

Nothing here computes attention or allocates blocks itself.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


def contiguous_history(w, seqs=None) -> Dict[int, tuple]:
    """Each sequence's K and V rows in token order, straight from the script.

    A fork copies the parent's rows; appends extend. No block table, slot or
    pool is involved, so this is an independent view of what attention sees.
    """
    hist: Dict[int, List] = {}
    for op in w.ops:
        kind = type(op).__name__
        if kind == "AddOp":
            hist[op.seq] = ([], [])
        elif kind == "ForkOp":
            hist[op.child] = (list(hist[op.parent][0]), list(hist[op.parent][1]))
        elif kind == "FreeOp":
            hist.pop(op.seq)
        elif kind == "AppendOp":
            k, v = w.append_values(op)
            pos = 0
            for s, n in zip(op.seqs, op.n_tokens):
                hist[s][0].append(k[pos:pos + n])
                hist[s][1].append(v[pos:pos + n])
                pos += n
    out = {}
    for s, (ks, vs) in hist.items():
        if seqs is not None and s not in seqs:
            continue
        shape = (0, w.num_kv_heads, w.head_dim)
        out[s] = (np.concatenate(ks) if ks else np.zeros(shape), np.concatenate(vs) if vs else np.zeros(shape))
    return out


def device_pool_to_oracle_layout(dev: np.ndarray, num_blocks: int, block_size: int, hkv: int, d: int):
    """Decode the device pool layout into the oracle's ``[N, B, Hkv, d]``.

    The device layout contract (include/pagedkv.h): element (block b, kv head h,
    slot o, dim i) sits at linear index ((b*Hkv + h)*B + o)*d + i.
    """
    return dev.reshape(num_blocks, hkv, block_size, d).transpose(0, 2, 1, 3)


def _storage_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def _nan_mask(a: np.ndarray, dtype: str) -> np.ndarray:
    """NaN positions of storage values (bf16 held as uint16 bits: exponent all ones, mantissa != 0)."""
    if dtype == "bf16":
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    return np.isnan(a)


def compare_pool_bits(dev_storage: np.ndarray, ref: np.ndarray, w) -> int:
    """The device pool (its own layout, as storage values) against the oracle's pool: every slot
    the oracle wrote holds the same bits, every slot it did not write is still NaN. Returns the
    number of written elements compared."""
    got = device_pool_to_oracle_layout(dev_storage, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    written = ~_nan_mask(ref, w.dtype)
    assert np.array_equal(_nan_mask(got, w.dtype), ~written), "written-slot sets differ"
    assert np.array_equal(_storage_bits(np.ascontiguousarray(got))[written], _storage_bits(ref)[written]), \
        "pool bits differ"
    return int(written.sum())


def oracle_attention_threaded(w, st, threads: int = 16, groups: int = 64) -> np.ndarray:
    """``oracle.paged_ragged`` over the oracle state ``st`` for every sequence of ``w``'s query,
    evaluated on groups of sequences in parallel threads (one BLAS thread each). Each group's rows
    come from its own call; no arithmetic is done here."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits

    tables, lens = st.bm.padded_tables(w.query_seqs, w.max_blocks_per_seq())
    q, cu = w.queries(), w.cu_seqlens()
    n = len(w.query_seqs)
    # interleaved groups balance long and short sequences
    parts = [list(range(i, n, groups)) for i in range(min(groups, n))]
    out = np.zeros((q.shape[0], w.num_q_heads, w.head_dim), dtype=np.float64)

    def one(idx):
        res = oracle.paged_ragged(q, cu, lens, tables, st.pool_k, st.pool_v, w.scale, w.block_size, w.dtype,
                                  only_seqs=idx)
        for i in idx:
            out[cu[i]:cu[i + 1]] = res[cu[i]:cu[i + 1]]

    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, parts))
    return out
