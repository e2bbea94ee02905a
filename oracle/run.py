"""Run a synthetic workload script through the oracle.

Test infrastructure only (see the package docstring). Plays the script's
add / append / fork / free operations on the oracle block manager, performs
the copy-on-write copies and slot writes on the oracle pool, and finally
evaluates the attention the script asks for.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .attention import paged_ragged
from .block_manager import BlockManager
from .pool import copy_between, copy_blocks, new_pool, write_slots


@dataclass
class OracleState:
    bm: BlockManager
    pool_k: np.ndarray
    pool_v: np.ndarray
    host_k: np.ndarray = None
    host_v: np.ndarray = None
    slots_per_append: List[List[int]] = field(default_factory=list)
    pairs_per_append: List[List[Tuple[int, int]]] = field(default_factory=list)


def run_workload(w, only_seqs: Optional[Sequence[int]] = None, attend: bool = True,
                 threads: int = 1):
    """Returns (state, out) where out is float64 ``[T, Hq, d]`` (None if not attending).

    ``only_seqs`` writes values (and evaluates attention) only for those
    sequences and for the sequences they were forked from; the block manager
    still plays every operation so tables and slots match the full run.
    """
    # Writes that land in blocks a kept sequence can read come from the kept
    # sequence itself or from an ancestor it was forked from.
    keep = None
    if only_seqs is not None:
        parent = {}
        for op in w.ops:
            if type(op).__name__ == "ForkOp":
                parent[op.child] = op.parent
        keep = set()
        for s in only_seqs:
            s = int(s)
            while s is not None and s not in keep:
                keep.add(s)
                s = parent.get(s)
    bm = BlockManager(w.num_blocks, w.block_size, w.free_order)
    pk = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    pv = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    st = OracleState(bm, pk, pv)
    if getattr(w, "num_host_blocks", 0):
        bm.attach_host_pool(w.num_host_blocks, w.host_free_order)
        st.host_k = new_pool(w.num_host_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
        st.host_v = new_pool(w.num_host_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    for op in w.ops:
        kind = type(op).__name__
        if kind == "SwapOutOp":
            pairs = bm.swap_out(op.seqs)
            st.pairs_per_append.append(pairs)
            copy_between(st.host_k, st.host_v, pk, pv, pairs)
        elif kind == "SwapInOp":
            pairs = bm.swap_in(op.seqs)
            st.pairs_per_append.append(pairs)
            copy_between(pk, pv, st.host_k, st.host_v, pairs)
        elif kind == "AddOp":
            bm.add_seq(op.seq)
        elif kind == "ForkOp":
            bm.fork(op.parent, op.child)
        elif kind == "FreeOp":
            bm.free_seq(op.seq)
        elif kind == "AppendOp":
            slots, pairs = bm.append(op.seqs, op.n_tokens)
            st.slots_per_append.append(slots)
            st.pairs_per_append.append(pairs)
            copy_blocks(pk, pv, pairs)
            k, v = w.append_values(op, None if keep is None else keep, threads=threads)
            if keep is None:
                write_slots(pk, pv, k, v, slots)
            else:
                sel, pos = [], 0
                for s, n in zip(op.seqs, op.n_tokens):
                    if s in keep:
                        sel.extend(slots[pos:pos + n])
                    pos += n
                write_slots(pk, pv, k, v, sel)
        else:
            raise TypeError(kind)
    if not attend:
        return st, None
    tables, lens = bm.padded_tables(w.query_seqs, w.max_blocks_per_seq())
    assert [int(x) for x in lens] == list(w.context_lens), "script and context lengths disagree"
    q = w.queries()
    out = paged_ragged(q, w.cu_seqlens(), lens, tables, pk, pv, w.scale, w.block_size, w.dtype,
                       only_seqs=None if only_seqs is None else
                       [i for i, s in enumerate(w.query_seqs) if s in set(only_seqs)])
    return st, out
