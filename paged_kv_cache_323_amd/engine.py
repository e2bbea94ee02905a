"""Iteration-level continuous batching over the paged KV cache.

A small step loop, not a serving system: requests carry a prompt length and a number of tokens to
generate, there is no model, and the new tokens' q/k/v come from a value provider (the seeded
generator for parity runs, device random numbers for throughput runs). What it exercises is the
hot path as an engine drives it, step after step with changing tables:

  * scheduling is per model step: finished requests leave and waiting ones join
    (「Paged Attention&Orca Paper笔记与解读」 §Orca的Solution, iteration-level scheduling); requests
    move through waiting -> prefilling -> decoding -> finished, admitted first come first served
    while fewer than ``max_num_seqs`` are in flight (the scheduler of the koas-w.github.io
    continuous-batching post, "Continous Batching的相关代码");
  * each step is one selective-batching call: every new prompt's tokens plus one token per
    decoding request, flattened, written to the cache, then attended in one ragged launch pair
    (「Paged Attention&Orca Paper笔记与解读」 §Orca的Solution, selective batching);
  * when the pool cannot hold the next step, the most recently admitted requests are preempted
    whole, their blocks swapped to the host pool, and they are resumed (swapped back in) before
    new requests are admitted (「PagedAttention原理」 §all-or-nothing 调度, §抢占与恢复 / §swap;
    「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法: no new admissions while
    preempted requests wait).

Every block-manager operation is recorded in an operation log (:mod:`.oplog`), so any step can
be replayed elsewhere. The new tokens' values come from a provider object: the default fills
them from a fixed random device buffer (throughput runs); a caller may pass its own provider
with ``kv(seqs, n_tokens, tag) -> (k, v)`` and ``q(seqs, n_tokens) -> q`` returning host arrays
of storage values ``[T, heads, head_dim]`` (bf16 as uint16 bits), e.g. to replay steps against
a reference.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Deque, Dict, List, Optional

import numpy as np
import torch

from . import native as pk
from .oplog import AddOp, AppendOp, FreeOp, SwapInOp, SwapOutOp
from .runner import TORCH_DTYPE, to_device

WAITING, PREFILL, DECODING, SWAPPED, FINISHED = "waiting", "prefill", "decoding", "swapped", "finished"


@dataclass
class Request:
    seq: int
    prompt_len: int
    max_new_tokens: int
    generated: int = 0
    state: str = WAITING
    admitted_step: int = -1


@dataclass
class StepRecord:
    step: int
    seqs: List[int]
    q_lens: List[int]
    context_lens: List[int]
    ops_end: int                  # number of ops in the log up to and including this step's append
    out: Optional[torch.Tensor] = None


@dataclass
class EngineStats:
    steps: int = 0
    prefill_tokens: int = 0
    decode_tokens: int = 0
    decode_kv_tokens: int = 0     # cached tokens the decode rows attended (each read in full)
    finished: int = 0
    preemptions: int = 0
    resumptions: int = 0


class Engine:
    STAGE_RING = 8    # staging sets (pinned host + device) for the per-step index upload
    MARK_EVERY = 4    # a launch-stream marker every this many steps guards their reuse

    def __init__(self, num_blocks: int, block_size: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 dtype: str, max_num_seqs: int = 64, max_step_tokens: int = 8192, num_host_blocks: int = 0,
                 seed: int = 0, values=None, keep_outputs: bool = False, device: str = "cuda",
                 copy_stream=None):
        self.B, self.hq, self.hkv, self.d, self.dtype = block_size, num_q_heads, num_kv_heads, head_dim, dtype
        self.max_num_seqs, self.max_step_tokens = max_num_seqs, max_step_tokens
        self.seed, self.values, self.keep_outputs, self.device = seed, values, keep_outputs, device
        rng = np.random.default_rng([seed, 1])
        self.free_order = rng.permutation(num_blocks).astype(np.int32)
        self.num_blocks = num_blocks
        self.bm = pk.BlockManager(num_blocks, block_size, self.free_order)
        self.desc = pk.CacheDesc.make(num_blocks, block_size, num_kv_heads, head_dim, dtype)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        tdt = TORCH_DTYPE[dtype]
        self.k_cache = torch.empty(shape, dtype=tdt, device=device).fill_(float("nan"))
        self.v_cache = torch.empty(shape, dtype=tdt, device=device).fill_(float("nan"))
        self.num_host_blocks = num_host_blocks
        self.host_free_order = None
        if num_host_blocks:
            self.host_free_order = np.random.default_rng([seed, 2]).permutation(num_host_blocks).astype(np.int32)
            self.bm.attach_host_pool(num_host_blocks, self.host_free_order)
            hshape = (num_host_blocks, num_kv_heads, block_size, head_dim)
            self.host_k = torch.empty(hshape, dtype=tdt, pin_memory=True)
            self.host_v = torch.empty(hshape, dtype=tdt, pin_memory=True)
        self.requests: Dict[int, Request] = {}
        self.waiting: Deque[int] = deque()
        self.running: List[int] = []      # admission order
        self.swapped: Deque[int] = deque()
        self.finished: List[int] = []
        self.ops: list = []
        self.records: List[StepRecord] = []
        self.stats = EngineStats()
        self.step_idx = 0
        self._next_seq = 0
        self.ws = torch.zeros(1, dtype=torch.uint8, device=device)
        self.scale = float(np.float32(1.0 / np.sqrt(head_dim)))
        # Per-step index data (slots, cu_seqlens, lengths, tables) goes up in one asynchronous copy
        # on a copy stream from a ring of staging sets (pinned host buffer + device buffer), so the
        # host prepares later steps while the GPU runs earlier ones and the copy does not sit
        # between the kernels. Step k uses set k mod STAGE_RING; before refilling it the host waits
        # on a launch-stream marker at or after step k - STAGE_RING (markers every MARK_EVERY
        # steps: an event recorded on the launch stream every step delays the next launch).
        self._stage_host: List[Optional[torch.Tensor]] = [None] * self.STAGE_RING
        self._stage_dev: List[Optional[torch.Tensor]] = [None] * self.STAGE_RING
        self._marks: Deque = deque()      # (step index, launch-stream event after that step)
        # The upload stream. HIP gives a stream a hardware queue when the stream first submits
        # work, in turn over a few queues (four by default), so a process that keeps creating
        # streams eventually puts one on the launch stream's queue, where its uploads wait behind
        # the kernels; a caller running several engines can pass one stream for all of them.
        self._copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream(device=device)
        self.max_len = 0                  # longest context any request can reach (sizes tables)

    # ---- requests -------------------------------------------------------------------------------
    def add_request(self, prompt_len: int, max_new_tokens: int) -> int:
        seq = self._next_seq
        self._next_seq += 1
        self.requests[seq] = Request(seq, int(prompt_len), int(max_new_tokens))
        self.waiting.append(seq)
        self.max_len = max(self.max_len, int(prompt_len) + int(max_new_tokens))
        return seq

    def has_work(self) -> bool:
        return bool(self.waiting or self.running or self.swapped)

    # ---- scheduling -----------------------------------------------------------------------------
    def _ops_add(self, op):
        self.ops.append(op)

    def _preempt_one(self) -> bool:
        """Make room: a request admitted this step (no cache yet) goes back to the head of the
        queue; otherwise the most recently admitted running request is swapped out whole."""
        if not self.running:
            return False
        victim = self.running[-1]
        if self.requests[victim].state == PREFILL:
            self.bm.free_seq(victim)
            self._ops_add(FreeOp(victim))
            self.running.pop()
            self.requests[victim].state = WAITING
            self.waiting.appendleft(victim)
            return True
        if not self.num_host_blocks:
            return False
        try:
            pairs = self.bm.swap_out([victim])
        except pk.NoFreeBlocksError:
            return False
        self._ops_add(SwapOutOp([victim]))
        if len(pairs):
            pk.swap_blocks(self.host_k, self.host_v, self.k_cache, self.v_cache,
                           self._pairs_to_device(pairs), self.desc)
        self.running.pop()
        self.requests[victim].state = SWAPPED
        self.swapped.appendleft(victim)
        self.stats.preemptions += 1
        return True

    def _resume(self) -> None:
        while self.swapped and len(self.running) < self.max_num_seqs:
            seq = self.swapped[0]
            try:
                pairs = self.bm.swap_in([seq])
            except pk.NoFreeBlocksError:
                return
            self._ops_add(SwapInOp([seq]))
            if len(pairs):
                pk.swap_blocks(self.k_cache, self.v_cache, self.host_k, self.host_v,
                               self._pairs_to_device(pairs), self.desc)
            self.swapped.popleft()
            self.requests[seq].state = DECODING
            self.running.append(seq)
            self.stats.resumptions += 1

    def _schedule(self):
        """Returns (seqs, n_tokens) of this step's batch (prompts first, then decodes)."""
        # retire
        for seq in [s for s in self.running if self.requests[s].state == FINISHED]:
            self.running.remove(seq)
        self._resume()
        # Admit first come first served (none while preempted requests wait), while the step's
        # token budget and the pool both hold the next prompt beside the running decodes' growth:
        # the longest prefix of the queue that fits.
        dec = [s for s in self.running if self.requests[s].state == DECODING]
        budget = self.max_step_tokens - len(dec)
        free = self.bm.num_free() - (self.bm.blocks_needed(dec, [1] * len(dec)) if dec else 0)
        while (self.waiting and not self.swapped and len(self.running) < self.max_num_seqs):
            req = self.requests[self.waiting[0]]
            need = -(-req.prompt_len // self.B)
            if req.prompt_len > budget or need > free:
                break
            free -= need
            self.waiting.popleft()
            self.bm.add_seq(req.seq)
            self._ops_add(AddOp(req.seq))
            req.state = PREFILL
            req.admitted_step = self.step_idx
            self.running.append(req.seq)
            budget -= req.prompt_len
        # make room: preempt the newest until the batch fits the pool
        while True:
            seqs, ns = self._batch()
            if not seqs:
                return seqs, ns
            if self.bm.blocks_needed(seqs, ns) <= self.bm.num_free():
                return seqs, ns
            if not self._preempt_one():
                raise RuntimeError("pool exhausted and nothing can be preempted")

    def _batch(self):
        pre = [s for s in self.running if self.requests[s].state == PREFILL]
        dec = [s for s in self.running if self.requests[s].state == DECODING]
        seqs = pre + dec
        ns = [self.requests[s].prompt_len for s in pre] + [1] * len(dec)
        return seqs, ns

    # ---- values ---------------------------------------------------------------------------------
    def _kv(self, seqs, ns, tag):
        if self.values is not None:
            k, v = self.values.kv(list(seqs), list(ns), tag)
            return to_device(k, self.dtype, self.device), to_device(v, self.dtype, self.device)
        T = int(sum(ns))
        k, v, _ = self._device_values(T)
        return k, v

    def _q(self, seqs, ns):
        if self.values is not None:
            return to_device(self.values.q(list(seqs), list(ns)), self.dtype, self.device)
        T = int(sum(ns))
        return self._device_values(T)[2]

    def _device_values(self, T):
        """Throughput runs: rows of a fixed random device buffer stand in for the model's new
        q/k/v (their values do not change the work)."""
        cap = getattr(self, "_vals_cap", 0)
        if T > cap:
            cap = max(T, 2 * cap, 1024)
            g = torch.Generator(device=self.device)
            g.manual_seed(self.seed)
            tdt = TORCH_DTYPE[self.dtype]
            self._vals = tuple(torch.randn((cap, h, self.d), device=self.device, generator=g).to(tdt)
                               for h in (self.hkv, self.hkv, self.hq))
            self._vals_cap = cap
        return tuple(x[:T] for x in self._vals)

    # ---- per-step uploads -----------------------------------------------------------------------
    def _pairs_to_device(self, pairs) -> torch.Tensor:
        """A (src, dst) pair list on the device, copied asynchronously from pinned memory (torch's
        pinned allocator keeps the host block until the copy has run), so the host does not wait
        for the GPU here."""
        host = torch.from_numpy(np.ascontiguousarray(pairs, dtype=np.int32)).pin_memory()
        return host.to(self.device, non_blocking=True)

    def _wait_step_done(self, j: int) -> None:
        """Block the host until the kernels of step j (and so its upload) have finished."""
        if j < 0:
            return
        while self._marks and self._marks[0][0] < j:
            self._marks.popleft()
        if self._marks:  # markers come every MARK_EVERY <= STAGE_RING steps, so one is there
            self._marks[0][1].synchronize()
        else:
            torch.cuda.synchronize(self.device)

    def _staging(self, n: int) -> np.ndarray:
        """An int32 view of n elements of this step's pinned staging buffer."""
        i = self.step_idx % self.STAGE_RING
        # step_idx - STAGE_RING last used this set: its upload read the host buffer and its
        # kernels read the device buffer
        self._wait_step_done(self.step_idx - self.STAGE_RING)
        buf = self._stage_host[i]
        if buf is None or buf.numel() < n:
            m = max(n, 2 * (buf.numel() if buf is not None else 0), 1 << 16)
            if buf is not None:
                torch.cuda.synchronize(self.device)  # rare: nothing in flight uses the old pair
            self._stage_host[i] = torch.empty(m, dtype=torch.int32).pin_memory()
            self._stage_dev[i] = torch.empty(m, dtype=torch.int32, device=self.device)
        return self._stage_host[i].numpy()[:n]

    def _upload(self, host: np.ndarray) -> torch.Tensor:
        """Copy this step's staging contents to the device on the copy stream and wait for it on
        the host (the copy waits on nothing on the device), so the launch stream's queue holds no
        cross-stream wait between the previous step's kernels and this step's."""
        i = self.step_idx % self.STAGE_RING
        n = len(host)
        dev = self._stage_dev[i][:n]
        with torch.cuda.stream(self._copy_stream):
            dev.copy_(self._stage_host[i][:n], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self._copy_stream)
        ev.synchronize()
        return dev

    # ---- one model step -------------------------------------------------------------------------
    def step(self) -> Optional[StepRecord]:
        seqs, ns = self._schedule()
        if not seqs:
            return None
        tag = 1000 + self.step_idx
        slots, pairs = self.bm.append(seqs, ns)
        self._ops_add(AppendOp(list(seqs), list(ns), tag))
        if len(pairs):
            pk.copy_blocks(self.k_cache, self.v_cache, self._pairs_to_device(pairs),
                           self.desc)
        k, v = self._kv(seqs, ns, tag)
        S, T = len(seqs), len(slots)
        max_blocks = -(-self.max_len // self.B)
        # work-list capacity: the automatic partition is at least 256 tokens whenever a context
        # needs more than one
        max_parts = -(-self.max_len // 256)
        tab0 = T + 2 * S + 1
        items0 = tab0 + S * max_blocks
        host = self._staging(items0 + S * max_parts)
        host[:T] = slots
        cu = host[T: T + S + 1]
        cu[0] = 0
        np.cumsum(ns, out=cu[1:])
        lens = host[T + S + 1: tab0]
        tables = host[tab0: items0].reshape(S, max_blocks)
        self.bm.block_tables(seqs, max_blocks, out=tables, ctx_out=lens)
        max_ctx, max_q, min_q = int(lens.max()), int(max(ns)), int(min(ns))
        # The decode rows run from a work list, longest partitions first (built from the host
        # lengths, uploaded with the rest); a step of prefill chunks only has none.
        n_items, part = 0, 0
        if min_q == 1:
            part = pk.decode_partition_size(S, self.hq, max_ctx, self.desc)
            n_items = pk.decode_items_into(lens, part, host[items0:])
        dev = self._upload(host[:items0 + n_items])
        sd, cu_d = dev[:T], dev[T: T + S + 1]
        lens_d = dev[T + S + 1: tab0]
        tab_d = dev[tab0: items0].view(S, max_blocks)
        items_d = dev[items0: items0 + n_items] if min_q == 1 else None
        pk.kv_cache_write(k, v, self.k_cache, self.v_cache, sd, self.desc)
        q = self._q(seqs, ns)
        out = torch.empty(q.shape, dtype=torch.float32 if self.keep_outputs else q.dtype, device=self.device)
        nbytes = pk.ragged_workspace_bytes(S, int(cu[-1]), self.hq, max_q, max_ctx, self.desc)
        if self.ws.numel() < nbytes:
            self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        # the step's shortest chunk bounds q_len from below: a step of prefill chunks only runs
        # no decode-row launches
        pk.paged_attention_ragged(out, q, cu_d, lens_d, self.k_cache, self.v_cache, tab_d, self.scale,
                                  max_q, max_ctx, self.desc, self.ws, min_q_len=min_q, partition_size=part,
                                  items=items_d)
        lens_list = lens.tolist()
        rec = StepRecord(self.step_idx, list(seqs), list(ns), lens_list, len(self.ops),
                         out if self.keep_outputs else None)
        self.records.append(rec)
        # every row group yields one generated token (the prompt's last row, or the decode row)
        for s, n, ctx in zip(seqs, ns, lens_list):
            req = self.requests[s]
            if req.state == PREFILL:
                self.stats.prefill_tokens += n
                req.state = DECODING
            else:
                self.stats.decode_tokens += 1
                self.stats.decode_kv_tokens += ctx
            req.generated += 1
            if req.generated >= req.max_new_tokens:
                req.state = FINISHED
                self.bm.free_seq(s)
                self._ops_add(FreeOp(s))
                self.finished.append(s)
                self.stats.finished += 1
        self.stats.steps += 1
        if self.step_idx % self.MARK_EVERY == self.MARK_EVERY - 1:
            ev = torch.cuda.Event()
            ev.record(torch.cuda.current_stream(self.device))
            self._marks.append((self.step_idx, ev))
        self.step_idx += 1
        return rec
