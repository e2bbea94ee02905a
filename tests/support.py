"""Helpers shared by the tests: contiguous histories and pool-layout decoding.

Nothing here computes attention or allocates blocks.
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
