"""Play a workload script through the library: host block manager + HIP kernels.

This is the engine-side loop in miniature: for every append it asks the C++ block manager for
slots and copy-on-write pairs, runs copy_blocks before kv_cache_write on one stream, and at the
end runs the attention the script asks for (decode or the ragged mixed step). PyTorch provides
device memory and the stream only.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import native as pk

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage values (bf16 as uint16 bits) -> device tensor of the matching dtype, bit for bit."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device, non_blocking=False)


def to_host_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> storage values on the host (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def nan_fill_(pool: torch.Tensor) -> torch.Tensor:
    """Fill a pool with NaN so that any read of an unwritten slot reaching a result shows up."""
    return pool.fill_(float("nan"))


@dataclass
class DeviceState:
    bm: pk.BlockManager
    desc: pk.CacheDesc
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    slots_per_append: List[np.ndarray] = field(default_factory=list)
    pairs_per_append: List[np.ndarray] = field(default_factory=list)
    host_k: Optional[torch.Tensor] = None  # pinned host swap pool
    host_v: Optional[torch.Tensor] = None


def make_pools(w, device="cuda", fill_nan=True):
    shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
    kc = torch.empty(shape, dtype=TORCH_DTYPE[w.dtype], device=device)
    vc = torch.empty(shape, dtype=TORCH_DTYPE[w.dtype], device=device)
    if fill_nan:
        nan_fill_(kc)
        nan_fill_(vc)
    return kc, vc


def play_script(w, device="cuda", threads: int = 8, fill_nan: bool = True, chunk_tokens: int = 1 << 16) -> DeviceState:
    """Run every op of the script; values come from the shared generator."""
    kc, vc = make_pools(w, device, fill_nan)
    desc = pk.CacheDesc.make(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    bm = pk.BlockManager(w.num_blocks, w.block_size, w.free_order)
    st = DeviceState(bm, desc, kc, vc)
    if getattr(w, "num_host_blocks", 0):
        bm.attach_host_pool(w.num_host_blocks, w.host_free_order)
        hshape = (w.num_host_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        st.host_k = torch.empty(hshape, dtype=TORCH_DTYPE[w.dtype], pin_memory=True)
        st.host_v = torch.empty(hshape, dtype=TORCH_DTYPE[w.dtype], pin_memory=True)
        if fill_nan:
            st.host_k.fill_(float("nan"))
            st.host_v.fill_(float("nan"))
    for op in w.ops:
        kind = type(op).__name__
        if kind in ("SwapOutOp", "SwapInOp"):
            out = kind == "SwapOutOp"
            pairs = bm.swap_out(op.seqs) if out else bm.swap_in(op.seqs)
            st.pairs_per_append.append(pairs)
            if len(pairs):
                pd = torch.from_numpy(np.ascontiguousarray(pairs)).to(device)
                if out:
                    pk.swap_blocks(st.host_k, st.host_v, kc, vc, pd, desc)
                else:
                    pk.swap_blocks(kc, vc, st.host_k, st.host_v, pd, desc)
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
            if len(pairs):
                pk.copy_blocks(kc, vc, torch.from_numpy(np.ascontiguousarray(pairs)).to(device), desc)
            # values in bounded chunks of sequences so host memory stays modest
            seqs, ns = list(op.seqs), list(op.n_tokens)
            pos, i = 0, 0
            while i < len(seqs):
                j, tok = i, 0
                while j < len(seqs) and (tok == 0 or tok + ns[j] <= chunk_tokens):
                    tok += ns[j]
                    j += 1
                sub = type(op)(seqs[i:j], ns[i:j], op.tag)
                k, v = w.append_values(sub, threads=threads)
                if tok:
                    kd = to_device(k, w.dtype, device)
                    vd = to_device(v, w.dtype, device)
                    sd = torch.from_numpy(np.ascontiguousarray(slots[pos:pos + tok])).to(device)
                    pk.kv_cache_write(kd, vd, kc, vc, sd, desc)
                pos += tok
                i = j
        else:
            raise TypeError(kind)
    return st


def attention(w, st: DeviceState, out_dtype: Optional[str] = "f32", device="cuda", partition_size: int = 0,
              q: Optional[torch.Tensor] = None):
    """Run the script's final attention; returns (out [T, Hq, D] tensor, inputs dict)."""
    max_blocks = w.max_blocks_per_seq()
    tables, lens = st.bm.block_tables(w.query_seqs, max_blocks)
    bt = torch.from_numpy(tables).to(device)
    cl = torch.from_numpy(lens).to(device)
    if q is None:
        q = to_device(w.queries(), w.dtype, device)
    odt = TORCH_DTYPE[out_dtype or w.dtype]
    # NaN-filled, so a row the kernels leave unwritten fails the callers' finiteness checks
    out = torch.full(q.shape, float("nan"), dtype=odt, device=device)
    max_ctx = int(lens.max()) if len(lens) else 0
    if w.is_decode:
        nbytes = pk.decode_workspace_bytes(len(lens), w.num_q_heads, max_ctx, st.desc, partition_size)
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        pk.paged_attention_decode(out, q, st.k_cache, st.v_cache, bt, cl, w.scale, max_ctx, st.desc, ws,
                                  partition_size)
    else:
        cu = torch.from_numpy(w.cu_seqlens()).to(device)
        max_q = int(max(w.q_lens))
        nbytes = pk.ragged_workspace_bytes(len(lens), q.shape[0], w.num_q_heads, max_q, max_ctx, st.desc)
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        pk.paged_attention_ragged(out, q, cu, cl, st.k_cache, st.v_cache, bt, w.scale, max_q, max_ctx, st.desc, ws)
    return out, dict(block_tables=bt, context_lens=cl, q=q, workspace=ws, tables_host=tables, lens_host=lens)
