"""GPU parity of the ragged mixed prefill + decode step vs the oracle.

Outputs in fp32, max-abs tolerance 2e-3 for f16/bf16 inputs; pools and bookkeeping bit-exact.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from workloads import make_ragged_workload, make_workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def _announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _run(w, out_dtype="f32", rows=None):
    from paged_kv_cache_323_amd import runner as R
    st = R.play_script(w, threads=16)
    out, _ = R.attention(w, st, out_dtype)
    return st, out


def _check(w, out, ref, rows=None, tol=None):
    got = out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    tol = tol if tol is not None else TOL[w.dtype]
    assert err <= tol, f"{w.name}: max abs err {err:.3g} > {tol}"
    return err


def test_mixed_small():
    w = make_workload("mixed", "small")
    _announce(w.name)
    st_or, ref = oracle.run_workload(w)
    st, out = _run(w)
    for a, b in zip(st.slots_per_append, st_or.slots_per_append):
        assert [int(x) for x in a] == list(b)
    err = _check(w, out, ref)
    print(f"  max abs err {err:.3g}")


RAGGED_CASES = [
    # (dtype, B, d, hq, hkv, q_lens, ctx)
    ("bf16", 16, 128, 4, 4, [1, 130, 1, 2, 257, 1], [90, 130, 1, 40, 300, 700]),     # prefill + cached prefix
    ("f16", 16, 128, 4, 4, [128, 1, 129, 3], [128, 2000, 129, 3]),
    ("bf16", 8, 128, 8, 2, [65, 1, 200], [65, 33, 450]),                               # GQA, chunked prefill
    ("bf16", 32, 64, 4, 2, [17, 1, 1, 300], [17, 64, 1025, 300]),                       # head_dim 64
    ("f16", 32, 64, 2, 2, [2, 0, 40], [2, 5, 100]),                                     # a sequence with no rows
    ("bf16", 16, 128, 16, 2, [1, 1, 1], [5, 1100, 2500]),                               # decode-only ragged
    # f32 pools: every row through the decode kernels, one item per query row
    ("f32", 16, 128, 4, 4, [1, 130, 1, 2, 257, 1], [90, 130, 1, 40, 300, 700]),
    ("f32", 8, 64, 8, 2, [65, 1, 200, 0], [65, 33, 450, 5]),                            # GQA, empty sequence
    ("f32", 16, 128, 4, 2, [300, 1], [5000, 3000]),                                     # split partitions
    ("f32", 16, 64, 4, 2, [3, 1], [20000, 500]),      # few rows, many partitions each: 8-thread merge
    # 16-bit chunks of at most g rows: every row through the decode kernels as well
    ("bf16", 16, 128, 32, 8, [2, 4, 1, 3], [1500, 40, 700, 3]),
    ("f16", 16, 64, 8, 1, [8, 1, 5], [100, 2000, 8]),
    # a prefill chunk behind 19800 cached tokens at B=8: 2500 blocks, more than the prefill
    # kernel's 1024-entry LDS table window, so the window moves during the key loop
    ("bf16", 8, 64, 4, 2, [200, 1], [20000, 9000]),
]


@pytest.mark.parametrize("case", RAGGED_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-d{c[2]}-{c[3]}/{c[4]}-{len(c[5])}seqs")
def test_ragged_shapes(case):
    dt, B, d, hq, hkv, ql, ctx = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    w = make_ragged_workload(seed, ql, ctx, hq, hkv, d, dt, B, name=f"ragged-{dt}-B{B}-d{d}")
    _announce(f"{w.name} q_lens={ql} ctx={ctx}")
    _, ref = oracle.run_workload(w)
    _, out = _run(w)
    _check(w, out, ref)


HINT_CASES = [
    # (dtype, B, d, hq, hkv, q_lens, ctx, min_q_len)
    ("bf16", 16, 128, 4, 4, [130, 2, 257], [130, 40, 300], 2),            # prefill only: no decode launches
    ("f16", 32, 64, 8, 2, [65, 200, 17], [65, 450, 17], 17),              # GQA; the bound is the shortest chunk
    # a bound that is wrong: the single rows run on the prefill kernel (one-row tiles)
    ("bf16", 16, 128, 4, 4, [1, 130, 1, 2, 257, 1], [90, 130, 1, 40, 300, 700], 2),
    ("f16", 8, 128, 8, 2, [1, 65, 0, 1], [33, 65, 5, 4000], 2),            # and an empty sequence
    ("bf16", 16, 64, 4, 4, [40, 40, 40], [40, 900, 3000], 40),            # the bound equals max_q_len
    # causal-rows mode (an f32 pool; 16-bit chunks of at most g rows): the bound has no effect
    ("f32", 16, 128, 4, 4, [1, 130, 2, 257], [90, 130, 40, 300], 2),
    ("bf16", 16, 128, 32, 8, [2, 4, 3], [1500, 40, 3], 2),
]


@pytest.mark.parametrize("case", HINT_CASES, ids=lambda c: f"{c[0]}-{len(c[5])}seqs-min{c[7]}")
def test_ragged_min_q_len_hint(case):
    """pkv_paged_attention_ragged_ex with a lower bound on q_len: the oracle's outputs within the
    tolerance, and every row of a multi-row sequence bit-identical to the call without the bound
    (the same prefill kernel computes it)."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    dt, B, d, hq, hkv, ql, ctx, min_q = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    w = make_ragged_workload(seed, ql, ctx, hq, hkv, d, dt, B, name=f"ragged-hint-{dt}-B{B}-d{d}")
    _announce(f"{w.name} q_lens={ql} ctx={ctx} min_q_len={min_q}")
    _, ref = oracle.run_workload(w)
    st = R.play_script(w, threads=16)
    out, inp = R.attention(w, st, "f32")
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    hinted = torch.full_like(out, float("nan"))
    pk.paged_attention_ragged(hinted, inp["q"], cu, inp["context_lens"], st.k_cache, st.v_cache, inp["block_tables"],
                              w.scale, int(max(ql)), int(inp["lens_host"].max()), st.desc, inp["workspace"],
                              min_q_len=min_q)
    torch.cuda.synchronize()
    err = _check(w, hinted, ref)
    cuh = w.cu_seqlens()
    multi = np.concatenate([np.arange(cuh[i], cuh[i + 1]) for i in range(len(ql)) if ql[i] >= 2])
    assert torch.equal(hinted[multi].view(torch.int32), out[multi].view(torch.int32)), "prefill rows differ"
    if dt == "f32" or max(ql) <= hq // hkv:  # causal-rows mode: every row, bit for bit
        assert torch.equal(hinted.view(torch.int32), out.view(torch.int32)), "rows mode must ignore the bound"
    print(f"  max abs err {err:.3g}")


ITEM_CASES = [
    # (dtype, B, d, hq, hkv, q_lens, ctx)
    ("bf16", 16, 128, 4, 4, [1, 130, 1, 1, 257, 1], [900, 130, 5000, 1, 300, 2100]),  # long decodes split
    ("f16", 16, 128, 32, 8, [1, 1, 65, 1], [3000, 40, 65, 9000]),        # four query heads per kv head
    ("bf16", 32, 64, 64, 8, [1, 200, 1], [4500, 200, 77]),               # eight: the one-pass kernel
    ("bf16", 16, 128, 40, 40, [1] * 6, [300, 1200, 17, 640, 1280, 5]),   # decode rows only
    ("bf16", 16, 128, 32, 8, [2, 4, 3], [1500, 40, 3]),                  # causal-rows mode: list unused
]


@pytest.mark.parametrize("case", ITEM_CASES, ids=lambda c: f"{c[0]}-{c[3]}q{c[4]}kv-d{c[2]}-{len(c[5])}seqs")
def test_ragged_work_list(case):
    """pkv_paged_attention_ragged_items: at the automatic partition size every output row equals
    the dense-grid call bit for bit, whatever the order of the work list; at a smaller partition
    size the oracle's outputs within the tolerance."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    dt, B, d, hq, hkv, ql, ctx = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    w = make_ragged_workload(seed, ql, ctx, hq, hkv, d, dt, B, name=f"ragged-items-{dt}-B{B}-d{d}")
    _announce(f"{w.name} q_lens={ql} ctx={ctx}")
    _, ref = oracle.run_workload(w)
    st = R.play_script(w, threads=16)
    out, inp = R.attention(w, st, "f32")
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    lens = inp["lens_host"]
    S, mx, mq = len(ql), int(lens.max()), int(max(ql))
    p_auto = pk.decode_partition_size(S, hq, mx, st.desc)
    for p in (p_auto, 256):
        host_items = pk.decode_items(lens, p)
        ws = torch.zeros(max(pk.ragged_workspace_bytes(S, int(inp["q"].shape[0]), hq, mq, mx, st.desc),
                             pk.decode_workspace_bytes(S, hq, mx, st.desc, p), 1), dtype=torch.uint8, device="cuda")
        for order in ("longest first", "reversed"):
            it = host_items if order == "longest first" else host_items[::-1].copy()
            items = torch.from_numpy(np.ascontiguousarray(it)).cuda()
            got = torch.full_like(out, float("nan"))
            pk.paged_attention_ragged(got, inp["q"], cu, inp["context_lens"], st.k_cache, st.v_cache,
                                      inp["block_tables"], w.scale, mq, mx, st.desc, ws, min_q_len=int(min(ql)),
                                      partition_size=p, items=items)
            torch.cuda.synchronize()
            err = _check(w, got, ref)
            if p == p_auto:
                assert torch.equal(got.view(torch.int32), out.view(torch.int32)), f"partition {p}, {order}"
            print(f"  partition {p} ({len(it)} items, {order}): max abs err {err:.3g}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_ragged_sharp_scores(dt):
    """Scores scaled by 4.0 instead of 1/sqrt(d): along a prefill row the maximum keeps rising by
    more than the kernel's 2^8 lazy-rescale threshold, and attention is close to one-hot."""
    import dataclasses
    w = make_ragged_workload(51, [300, 1, 257, 2], [300, 2000, 600, 40], 8, 4, 128, dt, 16, name=f"ragged-sharp-{dt}")
    w = dataclasses.replace(w, scale=4.0)
    _announce(w.name)
    _, ref = oracle.run_workload(w)
    _, out = _run(w)
    err = _check(w, out, ref)
    print(f"  max abs err {err:.3g}")


def test_ragged_native_out_dtype():
    w = make_workload("mixed", "small")
    _announce("mixed native out")
    _, ref = oracle.run_workload(w)
    _, out = _run(w, out_dtype=w.dtype)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= TOL[w.dtype] + 2.0 ** -8 * np.abs(ref))


def test_ragged_short_rows_precision():
    """Prefill rows that see only 1-4 keys are where a P rounded once to bf16 (8 bits) would break
    the tolerance; the kernel's P operand rounded once to f16 (11 bits) keeps them within 2e-3
    (here: 1e-3). The split bf16 P is only taken for values beyond the f16 range (tested below)."""
    w = make_ragged_workload(42, [300], [300], 8, 8, 128, "bf16", 16, name="short-rows")
    _announce(w.name)
    _, ref = oracle.run_workload(w)
    _, out = _run(w)
    _check(w, out, ref, rows=list(range(8)), tol=1e-3)
    _check(w, out, ref)


def test_mixed_full_every_row():
    """The full 13B-shaped mixed step (8 prefills + 248 decodes, 40 heads, bf16): every row of every
    prompt and every decode row against the oracle, every append's slots, and both full pools bit
    for bit after the setup writes and the step's own cache write (about 548 k tokens, the cache
    write's grid-stride path); the benchmark's work-list call bit for bit equal to the dense one."""
    from paged_kv_cache_323_amd import runner as R
    from support import compare_pool_bits, oracle_attention_threaded
    w = make_workload("mixed", "full")
    _announce(f"{w.name}: {len(w.query_seqs)} seqs, {sum(w.q_lens)} rows, sum ctx {sum(w.context_lens)}")
    st = R.play_script(w, threads=16)
    out, inp = R.attention(w, st, "f32")
    # the benchmark's call: decode rows from the longest-first work list, bit for bit the same
    import torch
    from paged_kv_cache_323_amd import native as pk
    lens = inp["lens_host"]
    p = pk.decode_partition_size(len(lens), w.num_q_heads, int(lens.max()), st.desc)
    items = torch.from_numpy(pk.decode_items(lens, p)).cuda()
    got_items = torch.full_like(out, float("nan"))
    pk.paged_attention_ragged(got_items, inp["q"], torch.from_numpy(w.cu_seqlens()).cuda(), inp["context_lens"],
                              st.k_cache, st.v_cache, inp["block_tables"], w.scale, int(max(w.q_lens)),
                              int(lens.max()), st.desc, inp["workspace"], min_q_len=1, partition_size=p, items=items)
    torch.cuda.synchronize()
    assert torch.equal(got_items.view(torch.int32), out.view(torch.int32)), "work-list call differs"
    del got_items, items
    got = out.cpu().numpy()
    st_or, _ = oracle.run_workload(w, attend=False, threads=16)
    for a, b in zip(st.slots_per_append, st_or.slots_per_append):
        assert np.array_equal(np.asarray(a, dtype=np.int64), np.asarray(b, dtype=np.int64))
    n_k = compare_pool_bits(R.to_host_storage(st.k_cache, w.dtype), st_or.pool_k, w)
    n_v = compare_pool_bits(R.to_host_storage(st.v_cache, w.dtype), st_or.pool_v, w)
    del st
    ref = oracle_attention_threaded(w, st_or)
    assert np.isfinite(got).all(), "non-finite output"
    n_pre = sum(1 for x in w.q_lens if x > 1)
    cu = w.cu_seqlens()
    err_pre = float(np.max(np.abs(got[: cu[n_pre]] - ref[: cu[n_pre]])))
    err_dec = float(np.max(np.abs(got[cu[n_pre]:] - ref[cu[n_pre]:])))
    assert max(err_pre, err_dec) <= TOL[w.dtype], (err_pre, err_dec)
    print(f"  all {cu[-1]} rows: prefill max abs err {err_pre:.3g}, decode {err_dec:.3g}; pools bit-exact "
          f"({n_k + n_v} written elements)", flush=True)


def test_ragged_prefill_row_tiles_beyond_one_grid_dimension():
    """65535 two-row prefill chunks (131070 rows, one head, d 64): the prefill launch sizes its
    row-tile slots as T/128 + min(S, T/2) = 66559, more than one grid dimension holds, so the
    slots continue in the grid's third dimension. Every row against the oracle."""
    S = 65535
    rng = np.random.default_rng(23)
    ctx = (2 + rng.integers(0, 31, S)).tolist()
    w = make_ragged_workload(23, [2] * S, ctx, 1, 1, 64, "bf16", 16, name="ragged-65535-prefills")
    _announce(f"{w.name}: {S} sequences of 2 rows")
    st, out = _run(w)
    ref = oracle_attention_rows(w)
    err = _check(w, out, ref)
    print(f"  max abs err {err:.3g}", flush=True)


def oracle_attention_rows(w):
    from support import oracle_attention_threaded
    st_or, _ = oracle.run_workload(w, attend=False, threads=16)
    return oracle_attention_threaded(w, st_or, groups=256)


def test_ragged_on_caller_stream():
    """The ragged step on a non-default stream: a copy enqueued on that stream right after the
    call sees every row, prefill and decode (outputs start as NaN), for two calls on two streams."""
    import torch
    from paged_kv_cache_323_amd import runner as R
    cases = [make_ragged_workload(31, [300, 1, 1, 257], [300, 900, 40, 400], 8, 4, 128, "bf16", 16, name="join-a"),
             make_ragged_workload(32, [1, 129, 1], [2000, 129, 3], 4, 4, 64, "f16", 16, name="join-b")]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    copies = []
    for w, s in zip(cases, streams):
        _announce(f"ragged on a side stream {w.name}")
        st = R.play_script(w, threads=16)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            out, _ = R.attention(w, st, "f32")
            copies.append(out.clone())  # same stream: ordered after both launches
    for s in streams:
        s.synchronize()
    for w, got in zip(cases, copies):
        _, ref = oracle.run_workload(w)
        _check(w, got, ref)


@pytest.mark.parametrize("shift", [10, 17])
def test_ragged_bf16_values_beyond_f16(shift):
    """A bf16 V pool scaled by 2^shift (exact). Prefill stages bf16 values as f16: at 2^10 every
    value still fits; at 2^17 values pass 65504, so every prefill tile is recomputed with bf16 Vᵀ
    and a split P. Attention is linear in V, so the oracle's output times 2^shift is the
    reference, with the tolerance scaled alike."""
    from paged_kv_cache_323_amd import runner as R
    w = make_ragged_workload(41, [130, 1, 257, 1, 64], [130, 700, 300, 50, 1000], 8, 4, 128, "bf16", 16,
                             name=f"bf16-v-x2^{shift}")
    _announce(f"{w.name}")
    _, ref = oracle.run_workload(w)
    st = R.play_script(w, threads=16)
    st.v_cache.mul_(2.0 ** shift)
    out, _ = R.attention(w, st, "f32")
    err = _check(w, out, ref * 2.0 ** shift, tol=TOL[w.dtype] * 2.0 ** shift)
    print(f"  max abs err {err:.3g} (scale 2^{shift})")


def test_ragged_f32_many_sequences():
    """An f32 pool's ragged step over 300 sequences (290 decode rows, 10 prefill chunks): each
    query row finds its sequence by counting row offsets, which takes two passes over 256 threads."""
    rng = np.random.default_rng(17)
    q_lens = [1] * 290 + [5] * 10
    rng.shuffle(q_lens)
    ctx = [int(q) + int(rng.integers(0, 300)) for q in q_lens]
    w = make_ragged_workload(17, q_lens, ctx, 4, 2, 64, "f32", 16, name="ragged-f32-300seqs")
    _announce(f"{w.name}")
    _, ref = oracle.run_workload(w)
    _, out = _run(w)
    _check(w, out, ref)


def test_ragged_bf16_many_sequences():
    """A bf16 ragged step over 600 sequences, mostly decode rows, with MFMA prefill chunks in the
    first, middle and last of the prefill kernel's 256-sequence passes over the row offsets (each
    workgroup finds its row tile by counting tiles back from the last sequence)."""
    rng = np.random.default_rng(23)
    q_lens = [1] * 600
    for i, q in ((0, 130), (1, 2), (255, 70), (256, 129), (300, 257), (511, 9), (599, 65)):
        q_lens[i] = q
    ctx = [int(q) + int(rng.integers(0, 200)) for q in q_lens]
    w = make_ragged_workload(23, q_lens, ctx, 4, 2, 64, "bf16", 16, name="ragged-bf16-600seqs")
    _announce(f"{w.name}")
    _, ref = oracle.run_workload(w)
    _, out = _run(w)
    _check(w, out, ref)


def test_ragged_step_graph_replay_matches_eager():
    """The ragged mixed step (decode rows, then MFMA prefill rows) captured in a HIP graph: every
    replay, with eager GPU work between replays, gives the eager output bit for bit."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    w = make_workload("mixed", "small")
    _announce(f"ragged step in a HIP graph {w.name}")
    st = R.play_script(w, threads=16)
    eager, inp = R.attention(w, st, "f32")
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    mx, mq = int(inp["lens_host"].max()), int(max(w.q_lens))
    out = torch.full_like(eager, float("nan"))

    def step():
        pk.paged_attention_ragged(out, inp["q"], cu, inp["context_lens"], st.k_cache, st.v_cache,
                                  inp["block_tables"], w.scale, mq, mx, st.desc, inp["workspace"])

    step()
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        out.fill_(float("nan"))
        scratch = scratch @ scratch.T / 512.0
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
