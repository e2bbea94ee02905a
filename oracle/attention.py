"""Attention over a paged KV cache, by the plain definition, in float64.

Test infrastructure only (see the package docstring).

Definition followed: 「PagedAttention原理」 §为什么会有 KV cache gives the decode
output of the newest token as o_t = softmax(q_t Kᵀ / √d) V over every cached key
and value of the sequence; §实现一个虚拟内存 splits the keys into blocks of B
tokens and states that attention over the blocks up to ⌈i/B⌉ gives the same
o_i. Paging is a storage change, not an approximation, so the oracle
*gathers* each sequence's keys and values into a contiguous array through the
block table and applies the plain softmax there. Readings taken where the pages
are silent or loose:
  * positions and blocks are 0-based (the page writes them 1-based);
  * the scale is an explicit argument (1/√d in the page's formula);
  * the block-wise denominator sums every scalar score of the attended
    blocks, i.e. ordinary softmax over tokens, and a query at position i only
    sees keys 0..i (the ⌈i/B⌉ limit makes the last block partial);
  * grouped query heads: query head h reads KV head ⌊h / g⌋, g = Hq / Hkv;
  * a sequence with no context yields a zero output.
"""
from __future__ import annotations

import numpy as np


def upcast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of storage values to float64 (bf16 is held as uint16 bits)."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def gather_kv(pool: np.ndarray, table, ctx: int, block_size: int) -> np.ndarray:
    """Rows 0..ctx-1 of one sequence, in logical order: ``[ctx, Hkv, d]`` storage values.

    Position p lives in logical block ⌊p/B⌋ at offset p mod B; the block table
    maps the logical block to a physical one (「PagedAttention原理」
    §实现一个虚拟内存, block table figure).
    """
    rows = []
    for p in range(ctx):
        phys = int(table[p // block_size])
        rows.append(pool[phys, p % block_size])
    if not rows:
        return pool[:0, 0]
    return np.stack(rows)


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      key_limit=None) -> np.ndarray:
    """o = softmax(scale · q kᵀ) v for float64 ``q [n, d]``, ``k, v [m, d]``.

    ``key_limit[i]`` (optional) is the number of leading keys query row i may
    see; the others are excluded from the softmax. Rows that see no key give 0.
    """
    n, m = q.shape[0], k.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    if m == 0 or n == 0:
        return out
    logits = scale * (q @ k.T)
    if key_limit is None:
        lim = np.full(n, m, dtype=np.int64)
    else:
        lim = np.minimum(np.asarray(key_limit, dtype=np.int64), m)
    seen = np.arange(m)[None, :] < lim[:, None]
    live = lim > 0
    logits = np.where(seen, logits, -np.inf)[live]
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    out[live] = (w / w.sum(axis=1, keepdims=True)) @ v
    return out


def paged_decode(q: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray, block_tables,
                 context_lens, scale: float, block_size: int, dtype: str) -> np.ndarray:
    """One query row per sequence at position ctx-1 attending keys 0..ctx-1.

    ``q``: ``[S, Hq, d]`` storage values; pools: oracle layout ``[N, B, Hkv, d]``.
    Returns float64 ``[S, Hq, d]``.
    """
    S, hq, d = q.shape
    hkv = pool_k.shape[2]
    g = hq // hkv
    out = np.zeros((S, hq, d), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        K = upcast(gather_kv(pool_k, block_tables[s], ctx, block_size), dtype)
        V = upcast(gather_kv(pool_v, block_tables[s], ctx, block_size), dtype)
        qs = upcast(q[s], dtype)
        for h in range(hq):
            kh = h // g
            out[s, h] = softmax_attention(qs[h:h + 1], K[:, kh], V[:, kh], scale)[0]
    return out


def paged_ragged(q: np.ndarray, cu_seqlens, context_lens, block_tables, pool_k: np.ndarray,
                 pool_v: np.ndarray, scale: float, block_size: int, dtype: str,
                 only_seqs=None) -> np.ndarray:
    """Selective-batching attention over a flattened ragged batch.

    Sequence s owns query rows cu[s]..cu[s+1]-1; its q_len = cu[s+1]-cu[s] rows
    are the last q_len positions of its context, so row t sits at position
    ctx - q_len + t and sees keys 0..that position (causal). A decode is the
    case q_len = 1. The attention is split per request only here; everything
    else in the batch is row-wise (「Paged Attention&Orca Paper笔记与解读」
    §Orca的Solution, selective batching).

    ``only_seqs`` limits the work to some sequences (other rows stay zero).
    Returns float64 ``[T, Hq, d]``.
    """
    T, hq, d = q.shape
    hkv = pool_k.shape[2]
    g = hq // hkv
    out = np.zeros((T, hq, d), dtype=np.float64)
    S = len(context_lens)
    want = None if only_seqs is None else set(int(s) for s in only_seqs)
    for s in range(S):
        if want is not None and s not in want:
            continue
        q0, q1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        ql, ctx = q1 - q0, int(context_lens[s])
        if ql == 0 or ctx == 0:
            continue
        K = upcast(gather_kv(pool_k, block_tables[s], ctx, block_size), dtype)
        V = upcast(gather_kv(pool_v, block_tables[s], ctx, block_size), dtype)
        qs = upcast(q[q0:q1], dtype)
        limits = [ctx - ql + t + 1 for t in range(ql)]
        for h in range(hq):
            kh = h // g
            out[q0:q1, h] = softmax_attention(qs[:, h], K[:, kh], V[:, kh], scale, limits)
    return out
