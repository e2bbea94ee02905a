"""Pins for the oracle: checks against facts fixed by the pages or by mathematics.

Each ``pin_*`` raises AssertionError when the oracle disagrees. They are
called by ``test_oracle_pins.py`` on the real oracle and by
``test_oracle_mutants.py`` on deliberately broken copies of it, to show that a
plausible slip anywhere in the oracle trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import random

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from support import contiguous_history

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _to_f64_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact float64 view of storage values, through torch's own dtype conversions."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)


# ---------------------------------------------------------------------------------------------
# Attention pins
# ---------------------------------------------------------------------------------------------
def pin_sdpa(w, tol=1e-12):
    """Library routine: torch's scaled_dot_product_attention in float64 over the script's
    contiguous per-sequence K/V (no pool, no block table) equals the oracle's paged result.

    GQA is torch's own ``enable_gqa`` mapping; causal rows of a prefill chunk get an
    explicit mask (row t of q_len sees keys 0..ctx-q_len+t).
    """
    _, out = oracle.run_workload(w)
    hist = contiguous_history(w)
    q = w.queries()
    cu = w.cu_seqlens()
    worst = 0.0
    for i, s in enumerate(w.query_seqs):
        K, V = hist[s]
        ctx, ql = K.shape[0], int(w.q_lens[i])
        assert ctx == w.context_lens[i]
        qs = _to_f64_torch(q[cu[i]:cu[i + 1]], w.dtype).permute(1, 0, 2)[None]   # [1,Hq,ql,d]
        Kt = _to_f64_torch(K, w.dtype).permute(1, 0, 2)[None]                     # [1,Hkv,ctx,d]
        Vt = _to_f64_torch(V, w.dtype).permute(1, 0, 2)[None]
        mask = torch.arange(ctx)[None, :] <= (ctx - ql + torch.arange(ql))[:, None]
        ref = F.scaled_dot_product_attention(qs, Kt, Vt, attn_mask=mask, scale=w.scale,
                                             enable_gqa=True)[0].permute(1, 0, 2).numpy()
        got = out[cu[i]:cu[i + 1]]
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert np.isfinite(got).all(), f"seq {s}: non-finite oracle output"
        worst = max(worst, err)
    assert worst <= tol, f"oracle vs SDPA max abs err {worst:g} > {tol:g}"
    return worst


def pin_blockwise_equation(w, tol=1e-12, partitions=(1, 2, 3)):
    """「PagedAttention原理」 §实现一个虚拟内存: A_ij = exp(q_i·K_j/√d) / Σ_t Σ exp(q_i·K_t/√d),
    o_i = Σ_j V_j A_ijᵀ, evaluated literally block by block from the pool through the
    block table, equals the oracle. Also checks the identity the split-context path
    relies on: merging per-partition (max, sum, partial output) triples with
    log-sum-exp weights reproduces the same o_i for any grouping of blocks.
    """
    st, out = oracle.run_workload(w)
    B = w.block_size
    g = w.group
    q = w.queries()
    cu = w.cu_seqlens()
    tables, lens = st.bm.padded_tables(w.query_seqs, w.max_blocks_per_seq())
    K64 = oracle.upcast(st.pool_k, w.dtype)
    V64 = oracle.upcast(st.pool_v, w.dtype)
    q64 = oracle.upcast(q, w.dtype)
    worst = 0.0
    for i, s in enumerate(w.query_seqs):
        ctx, ql = int(lens[i]), int(w.q_lens[i])
        for t in range(ql):
            pos = ctx - ql + t               # 0-based position of this query row
            nblk = pos // B + 1              # the page's ⌈i/B⌉ with 1-based i = pos+1
            for h in range(w.num_q_heads):
                kh = h // g
                qv = q64[cu[i] + t, h]
                e_blocks, v_blocks = [], []
                for j in range(nblk):
                    phys = int(tables[i, j])
                    valid = min(B, pos + 1 - j * B)
                    Kj = K64[phys, :valid, kh]
                    Vj = V64[phys, :valid, kh]
                    e_blocks.append(np.exp((Kj @ qv) * w.scale))
                    v_blocks.append(Vj)
                denom = sum(float(e.sum()) for e in e_blocks)
                o = sum(Vj.T @ (e / denom) for e, Vj in zip(e_blocks, v_blocks))
                worst = max(worst, float(np.max(np.abs(o - out[cu[i] + t, h]))))
                # split-context merge over contiguous groups of blocks
                for nparts in partitions:
                    bounds = np.linspace(0, nblk, min(nparts, nblk) + 1).astype(int)
                    trip = []
                    for a, b in zip(bounds[:-1], bounds[1:]):
                        if a == b:
                            continue
                        sc = np.concatenate([(K64[int(tables[i, j]), :min(B, pos + 1 - j * B), kh] @ qv)
                                             * w.scale for j in range(a, b)])
                        vv = np.concatenate([V64[int(tables[i, j]), :min(B, pos + 1 - j * B), kh]
                                             for j in range(a, b)])
                        m = sc.max()
                        p = np.exp(sc - m)
                        trip.append((m, p.sum(), vv.T @ p))
                    M = max(m for m, _, _ in trip)
                    L = sum(math.exp(m - M) * l for m, l, _ in trip)
                    om = sum(math.exp(m - M) * acc for m, _, acc in trip) / L
                    worst = max(worst, float(np.max(np.abs(om - out[cu[i] + t, h]))))
    assert worst <= tol, f"block-wise equation vs oracle max abs err {worst:g}"
    return worst


def pin_permutation_invariance(w, seed=0):
    """Relabelling physical blocks (pool and tables together) leaves the oracle's
    output bit-identical: which physical block holds a logical block is storage only."""
    st, out = oracle.run_workload(w)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_blocks)       # new id of old block b is perm[b]
    pk = np.empty_like(st.pool_k)
    pv = np.empty_like(st.pool_v)
    pk[perm] = st.pool_k
    pv[perm] = st.pool_v
    tables, lens = st.bm.padded_tables(w.query_seqs, w.max_blocks_per_seq())
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out2 = oracle.paged_ragged(w.queries(), w.cu_seqlens(), lens, t2, pk, pv, w.scale,
                               w.block_size, w.dtype)
    assert np.array_equal(out, out2), "output changed under a physical relabelling"


def pin_brute_force(w, tol=1e-12, max_rows=None):
    """Scalar loops with math.exp over the script's contiguous history (tiny inputs)."""
    _, out = oracle.run_workload(w)
    hist = contiguous_history(w)
    q = w.queries()
    cu = w.cu_seqlens()
    g = w.group
    rows = 0
    for i, s in enumerate(w.query_seqs):
        K, V = hist[s]
        ctx, ql = K.shape[0], int(w.q_lens[i])
        Kf = _to_f64_torch(K, w.dtype).tolist()
        Vf = _to_f64_torch(V, w.dtype).tolist()
        for t in range(ql):
            qrow = _to_f64_torch(q[cu[i] + t], w.dtype).tolist()
            n_keys = ctx - ql + t + 1
            for h in range(w.num_q_heads):
                kh = h // g
                scores = []
                for p in range(n_keys):
                    acc = 0.0
                    for x in range(w.head_dim):
                        acc += qrow[h][x] * Kf[p][kh][x]
                    scores.append(acc * w.scale)
                mx = max(scores)
                ex = [math.exp(a - mx) for a in scores]
                tot = sum(ex)
                for x in range(w.head_dim):
                    o = 0.0
                    for p in range(n_keys):
                        o += ex[p] / tot * Vf[p][kh][x]
                    assert abs(o - out[cu[i] + t, h, x]) <= tol, (s, t, h, x, o, out[cu[i] + t, h, x])
            rows += 1
            if max_rows and rows >= max_rows:
                return


def pin_closed_forms():
    """Hand-worked softmax-attention cases (golden/attention_closed_forms.json) and
    special cases with exact answers, through the oracle's paged entry point."""
    for c in golden("attention_closed_forms.json")["cases"]:
        q = np.array([c["q"]], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        o = oracle.softmax_attention(q, k, v, c["scale"])[0]
        assert np.all(np.abs(o - np.array(c["o"])) <= c["tol"]), (c["name"], o)

    # Through the paged decode path: ctx = 1 returns v_0 exactly; q = 0 returns the mean
    # of the attended values; constant value rows return that constant; ctx = 0 gives 0.
    rng = np.random.default_rng(7)
    B, N, H, d = 4, 6, 2, 8
    pk = oracle.new_pool(N, B, H, d, "f32")
    pv = oracle.new_pool(N, B, H, d, "f32")
    table = np.array([[3, 5, 0, -1], [4, -1, -1, -1], [1, 2, -1, -1], [2, -1, -1, -1]], dtype=np.int32)
    for b in (3, 5, 0, 4, 1, 2):
        pk[b] = rng.standard_normal((B, H, d)).astype(np.float32)
        pv[b] = rng.standard_normal((B, H, d)).astype(np.float32)
    pv[1] = 0.625                                      # constant values for sequence 2
    pv[2, :2] = 0.625
    q = rng.standard_normal((4, H, d)).astype(np.float32)
    q[0] = 0.0
    lens = [10, 1, 6, 0]
    out = oracle.paged_decode(q, pk, pv, table, lens, 0.35, B, "f32")
    # seq 0: q = 0 -> plain mean of its 10 value rows (blocks 3, 5 and half of 0)
    rows = np.concatenate([pv[3], pv[5], pv[0, :2]]).astype(np.float64)
    assert np.max(np.abs(out[0] - rows.mean(axis=0))) <= 1e-14
    # seq 1: one token -> its value row, exactly
    assert np.array_equal(out[1], pv[4, 0].astype(np.float64))
    # seq 2: constant value rows
    assert np.max(np.abs(out[2] - 0.625)) <= 1e-15
    # seq 3: empty context
    assert np.array_equal(out[3], np.zeros((H, d)))


def pin_paged_decode_gqa(groups=(1, 2, 4, 8), tol=1e-12):
    """The oracle's single-query entry point (``paged_decode``) with g = Hq / Hkv query heads per
    kv head, against torch's scaled_dot_product_attention with ``enable_gqa`` (its own
    contiguous-group mapping: query head h reads kv head ⌊h/g⌋) over each sequence's contiguous
    history from the script (no pool, no block table), and against the oracle's ragged entry
    point with one query row per sequence. Eight query heads over 8, 4, 2 and 1 kv heads, so that
    h mod Hkv and ⌊h/g⌋ differ for g = 2 and 4; contexts cover an empty one, one token, a full
    block, a ragged tail and several blocks."""
    from workloads import make_decode_workload
    worst = 0.0
    for g in groups:
        for dtype, B in (("f32", 8), ("bf16", 16)):
            hq = 8
            w = make_decode_workload(900 + g, [0, 1, B, 3 * B + 5, 2 * B - 1, 70], hq, hq // g, 16, dtype, B,
                                     name=f"pin-decode-g{g}-{dtype}")
            st, _ = oracle.run_workload(w, attend=False)
            tables, lens = st.bm.padded_tables(w.query_seqs, w.max_blocks_per_seq())
            q = w.queries()
            got = oracle.paged_decode(q, st.pool_k, st.pool_v, tables, lens, w.scale, B, dtype)
            rag = oracle.paged_ragged(q, w.cu_seqlens(), lens, tables, st.pool_k, st.pool_v, w.scale, B, dtype)
            assert np.array_equal(got, rag), f"g={g} {dtype}: decode and ragged entry points differ"
            hist = contiguous_history(w)
            for i, s in enumerate(w.query_seqs):
                K, V = hist[s]
                if K.shape[0] == 0:
                    assert np.array_equal(got[i], np.zeros_like(got[i])), "empty context must give zeros"
                    continue
                qs = _to_f64_torch(q[i], dtype)[:, None, :]                       # [Hq, 1, d]
                Kt = _to_f64_torch(K, dtype).permute(1, 0, 2)                      # [Hkv, ctx, d]
                Vt = _to_f64_torch(V, dtype).permute(1, 0, 2)
                ref = F.scaled_dot_product_attention(qs, Kt, Vt, scale=w.scale, enable_gqa=True)[:, 0].numpy()
                worst = max(worst, float(np.max(np.abs(got[i] - ref))))
    assert worst <= tol, f"paged_decode vs SDPA (GQA) max abs err {worst:g}"
    return worst


# ---------------------------------------------------------------------------------------------
# Block-manager pins
# ---------------------------------------------------------------------------------------------
def play_trace(make_bm, trace):
    """Run a golden block-manager trace against an object with the oracle's API."""
    bm = make_bm(trace["num_blocks"], trace["block_size"], trace["free_order"])
    if "num_host_blocks" in trace:
        bm.attach_host_pool(trace["num_host_blocks"], trace["host_free_order"])
    for i, st in enumerate(trace["steps"]):
        op = st["op"]
        exp = st["expect"]
        if op in ("swap_out", "swap_in"):
            fn = getattr(bm, op)
            if st.get("fails"):
                try:
                    fn(st["seqs"])
                except oracle.NoFreeBlocks:
                    pass
                else:
                    raise AssertionError(f"step {i}: {op} should have failed")
            else:
                pairs = fn(st["seqs"])
                assert [list(p) for p in pairs] == exp["pairs"], (i, pairs, exp["pairs"])
        elif op == "add":
            bm.add_seq(st["seq"])
        elif op == "fork":
            bm.fork(st["parent"], st["child"])
        elif op == "free":
            bm.free_seq(st["seq"])
        elif op == "append":
            if st.get("fails"):
                try:
                    bm.append(st["seqs"], st["n"])
                except oracle.NoFreeBlocks:
                    pass
                else:
                    raise AssertionError(f"step {i}: append should have failed")
            else:
                slots, pairs = bm.append(st["seqs"], st["n"])
                assert list(slots) == exp["slots"], (i, slots, exp["slots"])
                assert [list(p) for p in pairs] == exp["pairs"], (i, pairs, exp["pairs"])
        for s, t in exp.get("tables", {}).items():
            assert bm.block_table(int(s)) == t, (i, s, bm.block_table(int(s)), t)
        for s, n in exp.get("lens", {}).items():
            assert bm.context_len(int(s)) == n, (i, s)
        for b, r in exp.get("rc", {}).items():
            assert bm.refcount(int(b)) == r, (i, b, bm.refcount(int(b)), r)
        if "free" in exp:
            assert bm.free_list() == exp["free"], (i, bm.free_list(), exp["free"])
        for b, r in exp.get("host_rc", {}).items():
            assert bm.host_refcount(int(b)) == r, (i, b, bm.host_refcount(int(b)), r)
        if "host_free" in exp:
            assert bm.host_free_list() == exp["host_free"], (i, bm.host_free_list(), exp["host_free"])


def pin_cow_trace(make_bm=None):
    play_trace(make_bm or oracle.BlockManager, golden("cow_trace.json"))


def pin_swap_trace(make_bm=None):
    play_trace(make_bm or oracle.BlockManager, golden("swap_trace.json"))


def pin_fragmentation(make_bm=None):
    """Expected internal waste over a full period of lengths is (B-1)/2, the worst is B-1,
    and the tiny configuration's per-sequence block counts are as worked out by hand."""
    make_bm = make_bm or oracle.BlockManager
    gold = golden("fragmentation.json")
    for B in (8, 16, 32):
        k = 3
        wastes = []
        nb = k * B * k + 8                     # every length uses at most k blocks
        bm = make_bm(nb, B, list(range(nb)))
        for L in range(1, k * B + 1):
            bm.add_seq(L)
            bm.append([L], [L])
            nblk = len(bm.block_table(L))
            wastes.append(nblk * B - L)
        assert float(np.mean(wastes)) == gold["expected_mean_waste"][str(B)], (B, np.mean(wastes))
        assert max(wastes) == gold["expected_max_waste"][str(B)]
    tc = gold["tiny_config"]
    bm = make_bm(64, tc["block_size"], list(range(64)))
    for i, L in enumerate(tc["context_lens"]):
        bm.add_seq(i)
        bm.append([i], [L])
    blocks = [len(bm.block_table(i)) for i in range(4)]
    assert blocks == tc["blocks_per_seq"]
    assert [b * tc["block_size"] - L for b, L in zip(blocks, tc["context_lens"])] == tc["waste_per_seq"]
    assert 64 - bm.num_free() == tc["blocks_used"]


def pin_parallel_sampling(make_bm=None, B=16, n=4, prompts=(1000, 992, 7, 16, 33)):
    """「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法 (parallel sampling):
    the ⌊L/B⌋ full prompt blocks stay shared by all n samples (count n), the partial
    prompt block is copied for the samples that write into it while it is shared
    (n-1 copies; the last writer finds count 1 and writes in place), and nothing is
    copied when L is a multiple of B."""
    make_bm = make_bm or oracle.BlockManager
    for L in prompts:
        nb = 4 * (L // B + 2) * n
        bm = make_bm(nb, B, list(range(nb)))
        bm.add_seq(0)
        bm.append([0], [L])
        for c in range(1, n):
            bm.fork(0, c)
        prompt_blocks = bm.block_table(0)
        for b in prompt_blocks:
            assert bm.refcount(b) == n
        slots, pairs = bm.append(list(range(n)), [1] * n)
        full = L // B
        if L % B == 0:
            assert pairs == [] or list(pairs) == [], (L, pairs)
        else:
            assert len(pairs) == n - 1, (L, pairs)
            assert all(int(src) == prompt_blocks[-1] for src, _ in pairs)
            assert bm.refcount(prompt_blocks[-1]) == 1
        for j in range(full):
            assert bm.refcount(prompt_blocks[j]) == n
            for c in range(n):
                assert bm.block_table(c)[j] == prompt_blocks[j]
        # every sample's newest block is private
        for c in range(n):
            assert bm.refcount(bm.block_table(c)[-1]) == 1
        assert len(set(bm.block_table(c)[-1] for c in range(n))) == n


def pin_cow_contents():
    """Copy-on-write through the oracle pool: after copy then write, the shared source
    block's bytes are untouched, each copy equals the source in every pre-existing slot,
    and the new token lands only in the writer's private block."""
    B, H, d, L, n = 4, 2, 3, 6, 3
    bm = oracle.BlockManager(16, B, list(range(16)))
    pk = oracle.new_pool(16, B, H, d, "f16")
    pv = oracle.new_pool(16, B, H, d, "f16")
    rng = np.random.default_rng(3)
    bm.add_seq(0)
    slots, pairs = bm.append([0], [L])
    k = rng.standard_normal((L, H, d)).astype(np.float16)
    v = rng.standard_normal((L, H, d)).astype(np.float16)
    oracle.write_slots(pk, pv, k, v, slots)
    for c in range(1, n):
        bm.fork(0, c)
    shared = bm.block_table(0)[-1]
    before_k, before_v = pk[shared].copy(), pv[shared].copy()
    slots, pairs = bm.append(list(range(n)), [1] * n)
    oracle.copy_blocks(pk, pv, pairs)
    for src, dst in pairs:
        assert np.array_equal(pk[dst, :L % B], before_k[:L % B], equal_nan=True)
        assert np.array_equal(pv[dst, :L % B], before_v[:L % B], equal_nan=True)
    assert np.array_equal(pk[shared], before_k, equal_nan=True)
    nk = rng.standard_normal((n, H, d)).astype(np.float16)
    nv = rng.standard_normal((n, H, d)).astype(np.float16)
    oracle.write_slots(pk, pv, nk, nv, slots)
    for c in range(n):
        b = bm.block_table(c)[-1]
        assert np.array_equal(pk[b, L % B], nk[c]) and np.array_equal(pv[b, L % B], nv[c])
        assert np.array_equal(pk[b, :L % B], before_k[:L % B])
        assert np.array_equal(pv[b, :L % B], before_v[:L % B])


def random_script(rng: random.Random, num_blocks: int, B: int, n_ops: int = 200, swap: bool = False):
    """A random add / append / fork / free script (beam-search-like sharing churn), optionally
    with swap-out / swap-in of random groups."""
    ops, live, nxt = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if swap and live and r > 0.85:
            ss = rng.sample(live, k=min(len(live), rng.randint(1, 3)))
            ops.append(("swap_out" if r > 0.925 else "swap_in", ss))
            continue
        if not live or r < 0.1:
            ops.append(("add", nxt)); live.append(nxt); nxt += 1
        elif r < 0.3:
            p = rng.choice(live)
            ops.append(("fork", p, nxt)); live.append(nxt); nxt += 1
        elif r < 0.4 and len(live) > 1:
            s = rng.choice(live)
            ops.append(("free", s)); live.remove(s)
        else:
            ss = rng.sample(live, k=min(len(live), rng.randint(1, 4)))
            ops.append(("append", ss, [rng.randint(0, 2 * B + 1) for _ in ss]))
    return ops


def pin_invariants(make_bm=None, seeds=range(6), num_blocks=48, B=4, swap=False, host_blocks=24):
    """Under random fork / append / free (and swap) churn: every count equals the number of
    table entries naming the block; free + referenced = all blocks, disjointly, in each pool;
    each table holds ⌈len/B⌉ blocks; a failed append or swap changes nothing; each COW pair's
    source is still referenced by someone else and its destination is fresh; the host swap
    space never holds more blocks than the GPU pool has."""
    make_bm = make_bm or oracle.BlockManager
    for seed in seeds:
        rng = random.Random(seed)
        order = list(range(num_blocks))
        rng.shuffle(order)
        bm = make_bm(num_blocks, B, order)
        if swap:
            horder = list(range(host_blocks))
            rng.shuffle(horder)
            bm.attach_host_pool(host_blocks, horder)
        lens = {}
        on_host = set()

        def state():
            return ({s: bm.block_table(s) for s in lens}, bm.free_list(),
                    [bm.refcount(b) for b in range(num_blocks)],
                    bm.host_free_list() if swap else None)

        for op in random_script(rng, num_blocks, B, swap=swap):
            # ops on sequences whose creation was skipped (fork of a swapped-out parent) are skipped
            named = [op[1]] if op[0] in ("free", "fork") else (list(op[1]) if op[0] != "add" else [])
            if any(x not in lens for x in named):
                continue
            if op[0] in ("swap_out", "swap_in"):
                want_host = op[0] == "swap_out"
                if any((s in on_host) == want_host for s in op[1]):
                    continue  # only valid moves are exercised here
                snap = state()
                try:
                    pairs = getattr(bm, op[0])(op[1])
                except oracle.NoFreeBlocks:
                    assert state() == snap, "failed swap changed state"
                    continue
                for s in op[1]:
                    (on_host.add if want_host else on_host.discard)(s)
                assert len(pairs) == len({b for s in op[1] for b in bm.block_table(s)})
            elif op[0] == "add":
                bm.add_seq(op[1]); lens[op[1]] = 0
            elif op[0] == "fork":
                if op[1] in on_host:
                    continue
                bm.fork(op[1], op[2]); lens[op[2]] = lens[op[1]]
            elif op[0] == "free":
                bm.free_seq(op[1]); lens.pop(op[1]); on_host.discard(op[1])
            else:
                if any(s in on_host for s in op[1]):
                    continue
                snap = state()
                try:
                    free_before = set(bm.free_list())
                    slots, pairs = bm.append(op[1], op[2])
                except oracle.NoFreeBlocks:
                    assert state() == snap, "failed append changed state"
                    continue
                for s, n in zip(op[1], op[2]):
                    lens[s] += n
                for src, dst in pairs:
                    assert dst in free_before and bm.refcount(src) >= 1
                assert len(slots) == sum(op[2])
            refs, hrefs = {}, {}
            for s in lens:
                t = bm.block_table(s)
                assert len(t) == -(-lens[s] // B), (s, len(t), lens[s])
                assert bm.context_len(s) == lens[s]
                for b in t:
                    d = hrefs if s in on_host else refs
                    d[b] = d.get(b, 0) + 1
            for b in range(num_blocks):
                assert bm.refcount(b) == refs.get(b, 0), (b, bm.refcount(b), refs.get(b, 0))
            fl = bm.free_list()
            assert len(fl) == len(set(fl)) and not (set(fl) & set(refs))
            assert len(fl) + len(refs) == num_blocks
            if swap:
                for b in range(host_blocks):
                    assert bm.host_refcount(b) == hrefs.get(b, 0)
                hfl = bm.host_free_list()
                assert len(hfl) + len(hrefs) == host_blocks and not (set(hfl) & set(hrefs))
                assert len(hrefs) <= num_blocks
