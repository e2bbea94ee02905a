"""Seeded synthetic inputs shaped like the workloads the pages discuss.

Every random value is float32 N(0,1) rounded to nearest-even into the storage
dtype; those dtype values are the ground truth for every consumer. Each draw
comes from its own counter-keyed NumPy stream ``default_rng([seed, stream,
index])`` so any subset of sequences can be regenerated without the rest.

A workload is a *script* of block-manager operations (add / append / fork /
free) plus the final query. Appends name the tokens they add but carry no
slots: slots, block tables and copy-on-write pairs are what the code under test
computes. Values for appended tokens are produced on demand by ``gen_kv``.

Streams:
  0: lengths and other integer draws (one fixed order per config)
  1: permutation of the physical pool (the allocator's free-list order)
  2: K/V rows, keyed by (append tag, sequence id)
  3: queries, keyed by sequence id
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Union

import numpy as np

DTYPES = ("f32", "f16", "bf16")
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

_S_LENGTHS, _S_PERM, _S_KV, _S_Q = 0, 1, 2, 3


def dtype_nbytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def storage_dtype(dtype: str):
    return _STORAGE[dtype]


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> storage array of ``dtype`` (bf16 is held as uint16 bits).

    Rounding is to nearest, ties to even, in every case.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        b = x.view(np.uint32)
        return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def _rng(seed: int, stream: int, *index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), *[int(i) for i in index]])


def gen_kv(seed: int, tag: int, seq: int, n: int, hkv: int, d: int, dtype: str):
    """K and V rows ``[n, hkv, d]`` for the ``n`` tokens sequence ``seq`` adds in append ``tag``."""
    r = _rng(seed, _S_KV, tag, seq)
    k = r.standard_normal((n, hkv, d), dtype=np.float32)
    v = r.standard_normal((n, hkv, d), dtype=np.float32)
    return round_to_dtype(k, dtype), round_to_dtype(v, dtype)


def gen_q(seed: int, seq: int, n: int, hq: int, d: int, dtype: str) -> np.ndarray:
    """Query rows ``[n, hq, d]`` of sequence ``seq``."""
    r = _rng(seed, _S_Q, seq)
    return round_to_dtype(r.standard_normal((n, hq, d), dtype=np.float32), dtype)


@dataclass
class AddOp:
    seq: int


@dataclass
class AppendOp:
    seqs: List[int]
    n_tokens: List[int]
    tag: int  # value stream tag for gen_kv


@dataclass
class ForkOp:
    parent: int
    child: int


@dataclass
class FreeOp:
    seq: int


@dataclass
class SwapOutOp:
    seqs: List[int]


@dataclass
class SwapInOp:
    seqs: List[int]


Op = Union[AddOp, AppendOp, ForkOp, FreeOp, SwapOutOp, SwapInOp]


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks]
    ops: List[Op]
    # final query: sequences attended, in order, and the number of query rows each
    # (1 = decode; >1 = a prefill chunk whose rows are the last q_len positions)
    query_seqs: List[int]
    q_lens: List[int]
    context_lens: List[int]  # inclusive of the rows being queried
    scale: float = field(default=0.0)
    notes: str = ""
    num_host_blocks: int = 0               # host swap pool (0: none)
    host_free_order: Optional[np.ndarray] = None

    def __post_init__(self):
        if not self.scale:
            self.scale = float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def is_decode(self) -> bool:
        return all(n == 1 for n in self.q_lens)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def max_blocks_per_seq(self, extra_tokens: int = 0) -> int:
        B = self.block_size
        return max(1, -(-(max(self.context_lens) + extra_tokens) // B))

    def kv_bytes_per_token(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * dtype_nbytes(self.dtype)

    def append_values(self, op: AppendOp, seqs: Optional[Sequence[int]] = None, threads: int = 1):
        """(k, v) for every token ``op`` adds, concatenated in the op's sequence order.

        ``seqs`` restricts generation to a subset (others yield empty arrays).
        """
        want = None if seqs is None else set(seqs)
        jobs = [(s, n) for s, n in zip(op.seqs, op.n_tokens) if want is None or s in want]

        def one(job):
            s, n = job
            return gen_kv(self.seed, op.tag, s, n, self.num_kv_heads, self.head_dim, self.dtype)

        if threads > 1 and len(jobs) > 1:
            with ThreadPoolExecutor(threads) as ex:
                parts = list(ex.map(one, jobs))
        else:
            parts = [one(j) for j in jobs]
        st = storage_dtype(self.dtype)
        shape = (0, self.num_kv_heads, self.head_dim)
        if not parts:
            return np.zeros(shape, st), np.zeros(shape, st)
        return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))

    def queries(self, seqs: Optional[Sequence[int]] = None) -> np.ndarray:
        """Query rows ``[T, Hq, d]`` in ``query_seqs`` order (or only for ``seqs``)."""
        want = None if seqs is None else set(seqs)
        parts = [gen_q(self.seed, s, n, self.num_q_heads, self.head_dim, self.dtype)
                 for s, n in zip(self.query_seqs, self.q_lens) if want is None or s in want]
        return np.concatenate(parts) if parts else np.zeros((0, self.num_q_heads, self.head_dim),
                                                            storage_dtype(self.dtype))


# --------------------------------------------------------------------------------------------
# The five configurations (full size) and small variants of the same shape for fast tests.
# --------------------------------------------------------------------------------------------
CONFIG_NAMES = ("tiny", "llama7b", "gqa", "shared_prefix", "mixed")


def _pool_size(blocks_needed: int, slack: float = 1.5) -> int:
    return int(math.ceil(slack * blocks_needed))


def _decode_script(seqs: List[int], ctx: List[int]) -> List[Op]:
    """History of ctx-1 tokens per sequence, then the current token (written, then attended)."""
    ops: List[Op] = [AddOp(s) for s in seqs]
    ops.append(AppendOp(list(seqs), [c - 1 for c in ctx], tag=0))
    ops.append(AppendOp(list(seqs), [1] * len(seqs), tag=1))
    return ops


def make_decode_workload(seed: int, ctx: List[int], hq: int, hkv: int, head_dim: int, dtype: str,
                         block_size: int, slack: float = 1.5, name: str = "decode") -> Workload:
    """A generic decode step: ctx-1 cached tokens per sequence, then the current one."""
    need = sum(-(-c // block_size) if c > 0 else 0 for c in ctx)
    nb = max(1, _pool_size(need, slack))
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    seqs = list(range(len(ctx)))
    ops: List[Op] = [AddOp(s) for s in seqs]
    ops.append(AppendOp(list(seqs), [max(c - 1, 0) for c in ctx], tag=0))
    ops.append(AppendOp(list(seqs), [1 if c > 0 else 0 for c in ctx], tag=1))
    return Workload(name, seed, dtype, block_size, hq, hkv, head_dim, nb, perm, ops, seqs, [1] * len(ctx),
                    list(ctx))


def make_ragged_workload(seed: int, q_lens: List[int], ctx: List[int], hq: int, hkv: int, head_dim: int,
                         dtype: str, block_size: int, slack: float = 1.5, name: str = "ragged") -> Workload:
    """A generic selective-batching step: sequence s has ctx[s] - q_lens[s] cached tokens, then
    appends q_lens[s] new tokens whose rows are queried (q_len 1 = decode, more = prefill chunk)."""
    assert all(0 <= q <= c for q, c in zip(q_lens, ctx))
    need = sum(-(-c // block_size) for c in ctx)
    nb = max(1, _pool_size(need, slack))
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    seqs = list(range(len(ctx)))
    ops: List[Op] = [AddOp(s) for s in seqs]
    ops.append(AppendOp(list(seqs), [c - q for c, q in zip(ctx, q_lens)], tag=0))
    ops.append(AppendOp(list(seqs), list(q_lens), tag=1))
    return Workload(name, seed, dtype, block_size, hq, hkv, head_dim, nb, perm, ops, seqs, list(q_lens),
                    list(ctx))


def make_churn_workload(seed: int, block_size: int, hq: int, hkv: int, head_dim: int, dtype: str,
                        n_ops: int = 150, max_live: int = 10, slack: float = 1.25,
                        name: str = "churn") -> Workload:
    """Beam-search-like churn: sequences are added, forked at arbitrary points, extended in
    batches and freed, so blocks are shared, copied on write and released repeatedly. The final
    query is one decode row for every live sequence with a non-empty context.

    The pool is sized from an upper bound (every live sequence's own blocks, as if nothing were
    shared), so no append can run out of blocks.
    """
    r = _rng(seed, _S_LENGTHS)
    ops: List[Op] = []
    lens = {}
    nxt = 0
    peak = 0
    for i in range(n_ops):
        x = r.random()
        live = sorted(lens)
        if not live or (x < 0.12 and len(live) < max_live):
            ops.append(AddOp(nxt)); lens[nxt] = 0; nxt += 1
        elif x < 0.35 and len(live) < max_live:
            p = int(live[r.integers(len(live))])
            ops.append(ForkOp(p, nxt)); lens[nxt] = lens[p]; nxt += 1
        elif x < 0.45 and len(live) > 2:
            sq = int(live[r.integers(len(live))])
            ops.append(FreeOp(sq)); del lens[sq]
        else:
            k = int(r.integers(1, min(len(live), 4) + 1))
            pick = [int(v) for v in r.choice(live, size=k, replace=False)]
            ns = [int(r.integers(0, 3 * block_size)) for _ in pick]
            ops.append(AppendOp(pick, ns, tag=100 + i))
            for sq, n in zip(pick, ns):
                lens[sq] += n
        peak = max(peak, sum(-(-v // block_size) for v in lens.values()))
    q = [sq for sq in sorted(lens) if lens[sq] > 0]
    nb = max(1, int(math.ceil(slack * peak)) + 4)
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    return Workload(name, seed, dtype, block_size, hq, hkv, head_dim, nb, perm, ops, q, [1] * len(q),
                    [lens[sq] for sq in q])


def make_swap_workload(seed: int, block_size: int, hq: int, hkv: int, head_dim: int, dtype: str,
                       groups: int = 4, samples: int = 3, prompt: int = 70, gen: int = 20,
                       name: str = "swap") -> Workload:
    """Preemption and restore of sequence groups: parallel-sampling groups are built, one whole
    group is swapped to the host and its GPU blocks are reused by a newcomer, two samples of
    another group are swapped out while their siblings keep running (shared blocks are copied,
    not moved), then everything is swapped back in, extended and decoded."""
    r = _rng(seed, _S_LENGTHS)
    ops: List[Op] = []
    lens = {}
    gid = lambda g, i: g * samples + i
    tag = 0
    for g in range(groups):
        p = gid(g, 0)
        ops.append(AddOp(p))
        L = prompt + int(r.integers(0, block_size))
        ops.append(AppendOp([p], [L], tag=tag)); tag += 1
        lens[p] = L
        for i in range(1, samples):
            ops.append(ForkOp(p, gid(g, i)))
            lens[gid(g, i)] = L
    seqs = sorted(lens)
    first = [int(r.integers(1, gen)) for _ in seqs]
    ops.append(AppendOp(seqs, first, tag=tag)); tag += 1
    for sq, n in zip(seqs, first):
        lens[sq] += n
    g0 = [gid(0, i) for i in range(samples)]
    ops.append(SwapOutOp(g0))                          # whole group preempted
    newcomer = groups * samples
    ops.append(AddOp(newcomer))
    ops.append(AppendOp([newcomer], [prompt * 2], tag=tag)); tag += 1   # reuses the freed GPU blocks
    lens[newcomer] = prompt * 2
    part = [gid(1, 0), gid(1, 1)]
    ops.append(SwapOutOp(part))                        # shares blocks with gid(1, 2..): copies
    rest = [sq for sq in seqs if sq not in g0 and sq not in part]
    more = [int(r.integers(1, gen)) for _ in rest]
    ops.append(AppendOp(rest, more, tag=tag)); tag += 1
    for sq, n in zip(rest, more):
        lens[sq] += n
    ops.append(FreeOp(newcomer))
    del lens[newcomer]
    ops.append(SwapInOp(part))
    ops.append(SwapInOp(g0))
    live = sorted(lens)
    last = [1] * len(live)
    ops.append(AppendOp(live, last, tag=tag)); tag += 1
    for sq in live:
        lens[sq] += 1
    total = sum(-(-v // block_size) for v in lens.values()) + 2 * prompt // block_size + 8
    nb = _pool_size(total, 1.2)
    perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
    hb = nb
    hperm = _rng(seed, _S_PERM, 1).permutation(hb).astype(np.int32)
    return Workload(name, seed, dtype, block_size, hq, hkv, head_dim, nb, perm, ops, live, [1] * len(live),
                    [lens[sq] for sq in live], num_host_blocks=hb, host_free_order=hperm)


def make_workload(name: str, size: str = "full", block_size: Optional[int] = None,
                  slack: float = 1.5) -> Workload:
    if size not in ("full", "small"):
        raise ValueError(size)
    small = size == "small"
    if name == "tiny":
        seed, B = 1, block_size or 16
        ctx = [5, 16, 33, 100]
        seqs = list(range(4))
        nb = 64
        perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
        return Workload("tiny", seed, "f32", B, 4, 4, 64, nb, perm, _decode_script(seqs, ctx),
                        seqs, [1] * 4, ctx)

    if name == "llama7b":
        seed, B = 2, block_size or 16
        S, lo, hi, H = (6, 20, 300, 4) if small else (64, 128, 2048, 32)
        ctx = _rng(seed, _S_LENGTHS).integers(lo, hi, size=S, endpoint=True).tolist()
        need = sum(-(-c // B) for c in ctx)
        nb = _pool_size(need, slack)
        perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
        seqs = list(range(S))
        return Workload(f"llama7b{'-small' if small else ''}", seed, "f16", B, H, H, 128, nb, perm,
                        _decode_script(seqs, ctx), seqs, [1] * S, ctx)

    if name == "gqa":
        seed, B = 3, block_size or 16
        S, cap, hq, hkv = (12, 1200, 8, 2) if small else (256, 8192, 32, 8)
        med = 160 if small else 1024
        z = _rng(seed, _S_LENGTHS).standard_normal(S)
        ctx = np.clip(np.rint(np.exp(np.log(med) + 1.0 * z)), 1, cap).astype(np.int64).tolist()
        need = sum(-(-c // B) for c in ctx)
        nb = _pool_size(need, slack)
        perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
        seqs = list(range(S))
        return Workload(f"gqa-B{B}{'-small' if small else ''}", seed, "bf16", B, hq, hkv, 128, nb,
                        perm, _decode_script(seqs, ctx), seqs, [1] * S, ctx)

    if name == "shared_prefix":
        seed, B = 4, block_size or 16
        R, n, prompt, gmax, H = (3, 4, 100, 40, 4) if small else (16, 4, 1000, 512, 32)
        gen = _rng(seed, _S_LENGTHS).integers(1, gmax, size=R * n, endpoint=True).tolist()
        seqs = list(range(R * n))
        ops: List[Op] = []
        for r in range(R):
            parent = r * n
            ops.append(AddOp(parent))
            ops.append(AppendOp([parent], [prompt], tag=0))
            for c in range(1, n):
                ops.append(ForkOp(parent, parent + c))
        ops.append(AppendOp(seqs, [1] * len(seqs), tag=1))       # first generated token: COW
        ops.append(AppendOp(seqs, [g - 1 for g in gen], tag=2))  # the rest of the generation
        part = prompt % B
        need = R * (prompt // B) + sum(-(-(part + g) // B) for g in gen)
        nb = _pool_size(need, slack)
        perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
        ctx = [prompt + g for g in gen]
        return Workload(f"shared_prefix{'-small' if small else ''}", seed, "f16", B, H, H, 128, nb,
                        perm, ops, seqs, [1] * len(seqs), ctx,
                        notes=f"{R} requests x {n} samples, prompt {prompt}")

    if name == "mixed":
        seed, B = 5, block_size or 16
        if small:
            n_pre, pre_lo, pre_hi, n_dec, dec_lo, dec_hi, H = 3, 20, 150, 9, 20, 300, 4
        else:
            n_pre, pre_lo, pre_hi, n_dec, dec_lo, dec_hi, H = 8, 200, 2000, 248, 256, 4096, 40
        r = _rng(seed, _S_LENGTHS)
        pre = r.integers(pre_lo, pre_hi, size=n_pre, endpoint=True).tolist()
        dec = r.integers(dec_lo, dec_hi, size=n_dec, endpoint=True).tolist()
        seqs = list(range(n_pre + n_dec))
        dseqs = seqs[n_pre:]
        ops = [AddOp(s) for s in seqs]
        ops.append(AppendOp(dseqs, [c - 1 for c in dec], tag=0))        # cached decode contexts
        ops.append(AppendOp(seqs, pre + [1] * n_dec, tag=1))             # the mixed step's tokens
        ctx = pre + dec
        need = sum(-(-c // B) for c in ctx)
        nb = _pool_size(need, slack)
        perm = _rng(seed, _S_PERM).permutation(nb).astype(np.int32)
        return Workload(f"mixed{'-small' if small else ''}", seed, "bf16", B, H, H, 128, nb, perm,
                        ops, seqs, pre + [1] * n_dec, ctx,
                        notes=f"{n_pre} prefills then {n_dec} decodes")
    raise ValueError(f"unknown config {name!r}")
