"""The fused cache write + decode entry point (pkv_paged_attention_decode_append) against the
separate calls: the same outputs and the same pools, bit for bit, for dense and work-list launches,
every head grouping and dtype, empty contexts (nothing stored) and newest tokens that open a block."""
import sys

import numpy as np
import pytest

from workloads import make_decode_workload, make_workload

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _bits(t):
    import torch
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


CASES = [
    ("gqa", 16, "items", 128), ("gqa", 32, "dense", 0), ("llama7b", None, "dense", 256), ("tiny", None, "items", 64),
    ("shared_prefix", None, "items", 256),
]
DECODE_CASES = [
    # (seed, ctx, hq, hkv, d, dtype, B, launch, partition)
    (601, [0, 1, 16, 17, 700, 2049, 33, 5000], 64, 8, 128, "bf16", 8, "items", 256),   # 8 heads per kv head: MFMA scores
    (602, [3000, 1, 64, 65, 0, 1500], 64, 8, 64, "f16", 32, "dense", 0),
    (603, [100, 2000, 1, 0, 4097], 8, 4, 128, "f32", 16, "items", 512),
    (604, [9000, 8, 24, 250], 8, 8, 64, "bf16", 16, "dense", 0),
]


def _run(w, launch, partition):
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    st = R.play_script(w)  # the pools hold every token, each sequence's newest included
    ref, inp = R.attention(w, st, "f32", partition_size=partition)
    lens, tables = inp["lens_host"], inp["tables_host"]
    B = w.block_size
    live = np.nonzero(lens > 0)[0]
    pos = lens[live].astype(np.int64) - 1
    blocks = torch.from_numpy(tables[live, pos // B].astype(np.int64)).cuda()
    offs = torch.from_numpy(pos % B).cuda()
    slots_h = np.full(len(lens), -1, dtype=np.int32)
    slots_h[live] = (tables[live, pos // B].astype(np.int64) * B + pos % B).astype(np.int32)
    slots = torch.from_numpy(slots_h).cuda()
    shape = (len(lens), w.num_kv_heads, w.head_dim)
    k_new = torch.zeros(shape, dtype=st.k_cache.dtype, device="cuda")
    v_new = torch.zeros_like(k_new)
    live_d = torch.from_numpy(live).cuda()
    k_new[live_d] = st.k_cache[blocks, :, offs, :]
    v_new[live_d] = st.v_cache[blocks, :, offs, :]
    k_ref, v_ref = st.k_cache.clone(), st.v_cache.clone()
    st.k_cache[blocks, :, offs, :] = float("nan")  # the newest rows are not in the pool yet
    st.v_cache[blocks, :, offs, :] = float("nan")
    out = torch.full_like(ref, float("nan"))
    mx = int(lens.max())
    items = None
    part = partition
    if launch == "items":
        items = torch.from_numpy(np.ascontiguousarray(pk.decode_items(lens, partition))).cuda()
    pk.paged_attention_decode_append(out, inp["q"], k_new, v_new, slots, st.k_cache, st.v_cache, inp["block_tables"],
                                     inp["context_lens"], w.scale, mx, st.desc, inp["workspace"], part, items)
    torch.cuda.synchronize()
    assert torch.equal(_bits(st.k_cache), _bits(k_ref)), "K pool differs from the separate cache write"
    assert torch.equal(_bits(st.v_cache), _bits(v_ref)), "V pool differs from the separate cache write"
    assert torch.equal(out, ref), "output differs from the separate calls"


@pytest.mark.parametrize("name,B,launch,partition", CASES)
def test_append_equals_write_then_decode(name, B, launch, partition):
    w = make_workload(name, "small" if name != "tiny" else "full", block_size=B)
    _announce(f"append {w.name} {launch} partition={partition}")
    _run(w, launch, partition)


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[5]}-{c[2]}/{c[3]}-d{c[4]}-B{c[6]}-{c[7]}")
def test_append_shapes(case):
    seed, ctx, hq, hkv, d, dt, B, launch, partition = case
    w = make_decode_workload(seed, ctx, hq, hkv, d, dt, B, name=f"append-{dt}-{hq}-{hkv}-d{d}")
    _announce(f"{w.name} ctx={ctx} {launch}")
    _run(w, launch, partition)
