"""Block manager of the oracle: block tables, reference counts, copy-on-write.

Test infrastructure only (see the package docstring).

Rules followed, in the pages' terms:
  * 「PagedAttention原理」 §从虚拟内存的启发: a sequence takes one block of B slots at
    a time, only when the previous one is full, so its waste stays inside one
    block and there is no external fragmentation.
  * 「PagedAttention原理」 §实现一个虚拟内存: each sequence keeps a block table giving
    the physical block of each logical block and how many slots are filled.
  * 「PagedAttention原理」 §解决共享prompt / §解决COW: each physical block carries a
    reference count; a block is released when no one uses it. A write into a
    block whose count is 1 goes in place; otherwise (1) a new physical block is
    allocated, (2) the shared block's contents are copied into it, (3) the
    sequence's logical block is remapped to it, (4) the old block's count drops
    by one, (5) the new data is written into the new block.
  * 「PagedAttention原理」 §COW 区别: appending into a block that still has room is
    not a copy by itself; only a *shared* partial block is copied.
  * 「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法 (parallel
    sampling, beam search): forking shares every block of the parent and raises
    its count; freeing drops counts and releases blocks that reach zero.
  * 「PagedAttention原理」 §all-or-nothing 调度: a batch append either succeeds for
    every sequence or changes nothing (raises ``NoFreeBlocks``).
  * 「PagedAttention原理」 §抢占与恢复 / §swap and 「Paged Attention&Orca Paper笔记与解读」
    §PagedAttention的方法 (eviction to CPU memory): a group of sequences is preempted or
    restored as a whole: every block the group references moves between the GPU pool and a
    host swap pool, or nothing happens. A sequence runs only while all its blocks are on the
    GPU. A block that some sequence outside the group still references is copied instead of
    moved, so the swap space never holds more than the GPU blocks the group used.

Choices where the pages leave freedom (any choice is valid; this one is the
deterministic contract the device-side block manager must reproduce):
  * free blocks are taken from the head of a caller-given order and released
    blocks join its tail, in logical-block order;
  * sequences of one append are served in the order given, tokens in position
    order.
"""
from __future__ import annotations

import copy
from collections import deque
from typing import Dict, List, Sequence, Tuple


class NoFreeBlocks(RuntimeError):
    pass


class NotResident(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Sequence[int]):
        if sorted(int(b) for b in free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.B = int(block_size)
        self.num_blocks = int(num_blocks)
        self.free = deque(int(b) for b in free_order)
        self.rc: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.on_host: Dict[int, bool] = {}
        self.host_free = deque()
        self.host_rc: List[int] = []
        self.num_host_blocks = 0

    def attach_host_pool(self, num_host_blocks: int, free_order: Sequence[int]) -> None:
        if self.num_host_blocks:
            raise ValueError("host pool already attached")
        if sorted(int(b) for b in free_order) != list(range(num_host_blocks)):
            raise ValueError("free_order must be a permutation of the host block ids")
        self.num_host_blocks = int(num_host_blocks)
        self.host_free = deque(int(b) for b in free_order)
        self.host_rc = [0] * num_host_blocks

    # ---- sequences -------------------------------------------------------------------------
    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0
        self.on_host[seq] = False

    def _resident(self, seq: int) -> None:
        if self.on_host.get(seq):
            raise NotResident(f"sequence {seq} is swapped out")

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self._resident(parent)
        self.on_host[child] = False
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.rc[b] += 1

    def free_seq(self, seq: int) -> None:
        host = self.on_host.pop(seq)
        rc, free = (self.host_rc, self.host_free) if host else (self.rc, self.free)
        for b in self.tables.pop(seq):
            rc[b] -= 1
            if rc[b] == 0:
                free.append(b)
        del self.lens[seq]

    # ---- swap ------------------------------------------------------------------------------
    def _move(self, seqs, to_host: bool):
        """Move (or copy, when referenced outside ``seqs``) every block of ``seqs`` to the
        other pool. Returns [(src_block, dst_block)] in first-reference order."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ValueError("duplicate sequence")
        for s in seqs:
            if s not in self.tables:
                raise KeyError(f"unknown sequence {s}")
            if self.on_host[s] == to_host:
                raise NotResident(f"sequence {s} is already {'on the host' if to_host else 'resident'}")
        src_rc, src_free = (self.rc, self.free) if to_host else (self.host_rc, self.host_free)
        dst_rc, dst_free = (self.host_rc, self.host_free) if to_host else (self.rc, self.free)
        order, refs = [], {}
        for s in seqs:
            for b in self.tables[s]:
                if b not in refs:
                    order.append(b)
                    refs[b] = 0
                refs[b] += 1
        if len(order) > len(dst_free):
            raise NoFreeBlocks("swap pool exhausted" if to_host else "pool exhausted")
        mapping, pairs = {}, []
        for b in order:
            nb = dst_free.popleft()
            dst_rc[nb] = refs[b]
            mapping[b] = nb
            pairs.append((b, nb))
        for s in seqs:
            self.tables[s] = [mapping[b] for b in self.tables[s]]
            self.on_host[s] = to_host
        for b in order:
            src_rc[b] -= refs[b]
            if src_rc[b] == 0:
                src_free.append(b)
        return pairs

    def swap_out(self, seqs):
        """Preempt ``seqs`` to the host pool; returns [(gpu_block, host_block)] to copy first."""
        return self._move(seqs, True)

    def swap_in(self, seqs):
        """Restore ``seqs`` to the GPU pool; returns [(host_block, gpu_block)] to copy first."""
        return self._move(seqs, False)

    # ---- appends ---------------------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise NoFreeBlocks("pool exhausted")
        b = self.free.popleft()
        self.rc[b] = 1
        return b

    def _append_one(self, seq: int, slots: List[int], pairs: List[Tuple[int, int]]) -> None:
        table = self.tables[seq]
        p = self.lens[seq]
        j, off = divmod(p, self.B)
        if j == len(table):                 # previous block full (or none yet): a fresh block
            table.append(self._take())
        elif self.rc[table[j]] > 1:         # shared partial block: the five copy-on-write steps
            old = table[j]
            new = self._take()              # (1) allocate
            pairs.append((old, new))        # (2) copy old -> new (done by the caller's copy)
            table[j] = new                  # (3) remap
            self.rc[old] -= 1               # (4) drop the old count
        slots.append(table[j] * self.B + off)  # (5) the write goes to the (new) block
        self.lens[seq] = p + 1

    def append(self, seqs: Sequence[int], n_tokens: Sequence[int]):
        """Add ``n_tokens[i]`` positions to ``seqs[i]``; returns (slots, cow_pairs).

        All or nothing: if the pool runs out, the state is left unchanged.
        """
        saved = (copy.copy(self.free), list(self.rc), {k: list(v) for k, v in self.tables.items()},
                 dict(self.lens))
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        try:
            for s, n in zip(seqs, n_tokens):
                if s not in self.tables:
                    raise KeyError(f"unknown sequence {s}")
                self._resident(s)
                for _ in range(int(n)):
                    self._append_one(int(s), slots, pairs)
        except Exception:
            self.free, self.rc, self.tables, self.lens = saved
            raise
        return slots, pairs

    # ---- queries ---------------------------------------------------------------------------
    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def context_len(self, seq: int) -> int:
        return self.lens[seq]

    def refcount(self, block: int) -> int:
        return self.rc[block]

    def num_free(self) -> int:
        return len(self.free)

    def free_list(self) -> List[int]:
        return list(self.free)

    def host_refcount(self, block: int) -> int:
        return self.host_rc[block]

    def host_free_list(self) -> List[int]:
        return list(self.host_free)

    def is_resident(self, seq: int) -> bool:
        return not self.on_host[seq]

    def padded_tables(self, seqs: Sequence[int], max_blocks: int):
        import numpy as np
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("max_blocks too small")
            out[i, :len(t)] = t
            lens[i] = self.lens[s]
        return out, lens
