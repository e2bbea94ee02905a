"""The oracle's KV pool: storage values, token-major ``[N, B, Hkv, d]``.

Test infrastructure only (see the package docstring).

The KV cache is cut into fixed-size blocks of B slots, each slot holding one
token's K (or V) rows for every KV head (「PagedAttention原理」 §从虚拟内存的启发
and §实现一个虚拟内存). Slot s of the pool is block ⌊s/B⌋, offset s mod B.
Unwritten slots hold NaN so any read of one that reaches a result shows up.
The layout here is token-major on purpose; the device library uses its own.
"""
from __future__ import annotations

import numpy as np

_NAN_BITS = {"bf16": np.uint16(0x7FC0)}


def new_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: str):
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    if dtype == "bf16":
        return np.full(shape, _NAN_BITS["bf16"], dtype=np.uint16)
    st = {"f32": np.float32, "f16": np.float16}[dtype]
    return np.full(shape, np.nan, dtype=st)


def write_slots(pool_k: np.ndarray, pool_v: np.ndarray, k: np.ndarray, v: np.ndarray, slots) -> None:
    """pool[slot[t]] <- (k[t], v[t]) bit for bit; a negative slot means "skip".

    Each decode step stores the new token's K and V after computing them, and a
    prefill stores the whole prompt's (「vllm」 §2.1 Prefill, §2.2 Decode).
    """
    B = pool_k.shape[1]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        b, o = divmod(s, B)
        pool_k[b, o] = k[t]
        pool_v[b, o] = v[t]


def copy_blocks(pool_k: np.ndarray, pool_v: np.ndarray, pairs) -> None:
    """pool[dst] <- pool[src] for every (src, dst): all B slots, K and V, bit for bit.

    Step (2) of copy-on-write copies the shared block's contents into the new
    block (「PagedAttention原理」 §解决COW); the whole block is copied.
    """
    for src, dst in pairs:
        pool_k[int(dst)] = pool_k[int(src)]
        pool_v[int(dst)] = pool_v[int(src)]


def copy_between(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray, pairs) -> None:
    """dst[d] <- src[s] for every (s, d): whole blocks between two pools (GPU pool and host
    swap pool), bit for bit (「PagedAttention原理」 §swap)."""
    for s_, d_ in pairs:
        dst_k[int(d_)] = src_k[int(s_)]
        dst_v[int(d_)] = src_v[int(s_)]
