"""Benchmark of the paged-KV hot path on one MI355X.

A *step* is one decode iteration of the GQA configuration (256 sequences, 32 query heads over 8
KV heads, head_dim 128, bf16, block size 16, lognormal context lengths with median 1024 capped
at 8192, physical blocks in a seeded random order):

  1. host block manager: append one token to every sequence -> slots, copy-on-write pairs,
     block tables (C++ inside libpagedkv.so);
  2. one pinned-memory upload of slots, context lengths and block tables (on a copy stream, so
     it overlaps the previous step's kernels);
  3. copy_blocks for any copy-on-write pairs (none in this workload);
  4. kv_cache_write of the 256 new tokens and 5. paged decode attention of the 256 query rows over
     their whole contexts, in one pass: the partition launch of pkv_paged_attention_decode_append
     stores each sequence's new token before attending it, then the merge launch.

Inputs are resident in HBM before timing starts. The JSON line reports whole-step throughput
(KV bytes read by attention per second, and sequences per second), the decode kernel against
the HBM roofline (timed with HIP events on the launch stream) and against measured read, gather
and copy ceilings, the oracle timed on this host's CPU on a bounded sample, and secondary
measurements of the other workloads (block sizes 8/32, Llama-7B-shaped decode, shared prefix,
swap, the continuous-batching engine, the 13B-shaped mixed step, prefill from an f16 pool and on
long prompts), each row beside the ceiling that bounds it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--block-size 16] [--no-extra] [--no-cpu]
                    [--partition P] [--dense-grid]
    python bench.py --profile-prefill [--prefill-dtype bf16|f16]   # profiling targets
    python bench.py --profile-copy
"""
from __future__ import annotations

import argparse
import collections
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/f16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_algorithmic_bytes(ctx_lens, w, out_bytes_per_el):
    """Bytes the decode step must move: every cached K and V row once, the queries, the
    outputs, block-table entries and context lengths."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    e = 2 if w.dtype != "f32" else 4
    kv = int(ctx.sum()) * w.kv_bytes_per_token()
    q = len(ctx) * w.num_q_heads * w.head_dim * e
    out = len(ctx) * w.num_q_heads * w.head_dim * out_bytes_per_el
    tables = int((-(-ctx // w.block_size)).sum()) * 4 + len(ctx) * 4
    return kv, kv + q + out + tables


_COPY_STREAM = None


def upload_stream():
    """One upload stream for every decode loop and engine of this process. HIP gives a stream a
    hardware queue when the stream first submits work, in turn over a few queues (four by default),
    so with a new stream per loop every fourth loop's uploads shared the launch stream's queue and
    waited behind the previous step's kernels: those loops ran host-paced (the Llama-7B-shaped step
    at 221 us against 196 us, the 1024-token partition run at 327 against 300 us)."""
    global _COPY_STREAM
    import torch
    if _COPY_STREAM is None:
        _COPY_STREAM = torch.cuda.Stream()
    return _COPY_STREAM


class DecodeLoop:
    """Steady-state decode steps over a resident workload (state advances every step)."""

    RING = 8
    MARK_EVERY = 4

    def __init__(self, w, steps_total, device="cuda", work_list=True, partition=0):
        import torch
        from paged_kv_cache_323_amd import native as pk
        from paged_kv_cache_323_amd import runner as R
        self.torch, self.pk, self.R, self.w = torch, pk, R, w
        t = time.perf_counter()
        self.st = R.play_script(w, threads=16)
        torch.cuda.synchronize()
        log(f"setup {w.name}: pool {w.num_blocks} blocks, wrote {sum(w.context_lens)} tokens "
            f"in {time.perf_counter() - t:.1f}s")
        self.S = len(w.query_seqs)
        self.seqs = np.asarray(w.query_seqs, dtype=np.int64)
        self.max_ctx_final = max(w.context_lens) + steps_total
        self.max_blocks = -(-self.max_ctx_final // w.block_size)
        self.partition = partition or pk.decode_partition_size(
            self.S, w.num_q_heads, self.max_ctx_final,
            pk.CacheDesc.make(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype))
        # The partition launch takes a work list of (sequence, partition) items built on the host
        # from the lengths it uploads anyway (work_list=False: the dense grid sized for the
        # longest context in every sequence).
        self.work_list = work_list
        self.max_items = self.S * -(-self.max_ctx_final // self.partition)
        # A ring of staging sets (pinned host + device), each [slots S | ctx S | tables S*MB | items]:
        # step k fills set k % RING on the host and uploads it on a copy stream while earlier steps'
        # kernels still read their own sets. Set reuse is guarded by sparse markers on the launch
        # stream (one event every MARK_EVERY steps) that the host waits on: an event recorded on the
        # launch stream every step delays the next step's launch by several microseconds.
        self.n_items = [0] * self.RING
        self.items_off = 2 * self.S + self.S * self.max_blocks
        n = self.items_off + self.max_items
        self.host = [torch.empty(n, dtype=torch.int32).pin_memory() for _ in range(self.RING)]
        self.host_np = [h.numpy() for h in self.host]
        self.dev = [torch.empty(n, dtype=torch.int32, device=device) for _ in range(self.RING)]
        self.marks = collections.deque()  # (step index, launch-stream event recorded after that step)
        self.copy_stream = upload_stream()
        self._views(0)
        self.q = R.to_device(w.queries(), w.dtype, device)
        # new-token K/V for the steps (fixed values; only their placement changes per step)
        r = np.random.default_rng([w.seed, 77])
        from workloads import round_to_dtype
        kv = round_to_dtype(r.standard_normal((2, self.S, w.num_kv_heads, w.head_dim), dtype=np.float32), w.dtype)
        self.k_new = R.to_device(kv[0], w.dtype, device)
        self.v_new = R.to_device(kv[1], w.dtype, device)
        self.out = torch.empty_like(self.q)  # pool dtype output, as a serving engine consumes it
        nbytes = pk.decode_workspace_bytes(self.S, w.num_q_heads, self.max_ctx_final, self.st.desc, self.partition)
        self.ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.step_idx = 0
        self.ctx_history = []
        self.pairs_total = 0
        # the throughput steps use the fused cache write + decode; the event-timed steps issue the
        # cache write, the partition launch and the merge separately, to time the partition launch
        self.fused = True

    def _views(self, i):
        d = self.dev[i]
        self.slots_d = d[: self.S]
        self.ctx_d = d[self.S: 2 * self.S]
        self.tab_d = d[2 * self.S: self.items_off].view(self.S, self.max_blocks)
        self.items_d = d[self.items_off: self.items_off + self.n_items[i]]

    def attention(self):
        """The step's two attention launches (partitions, then merge)."""
        pk, w = self.pk, self.w
        args = (self.out, self.q, self.st.k_cache, self.st.v_cache, self.tab_d, self.ctx_d, w.scale,
                self.max_ctx_final, self.st.desc)
        if self.work_list:
            pk.paged_attention_decode_partitions_items(*args, self.partition, self.items_d, self.ws)
        else:
            pk.paged_attention_decode(*args, self.ws, self.partition, stage="partitions")
        yield
        pk.paged_attention_decode(*args, self.ws, self.partition, stage="merge")
        yield

    def repeat_attention(self, n):
        for _ in range(n):
            for _ in self.attention():
                pass

    def _wait_step_done(self, j):
        """Block the host until the kernels of step j (and so its upload) have finished."""
        if j < 0:
            return
        while self.marks and self.marks[0][0] < j:
            self.marks.popleft()
        if self.marks:  # markers come every MARK_EVERY <= RING steps, so one at or after step j exists
            self.marks[0][1].synchronize()
        else:
            self.torch.cuda.synchronize()

    def step(self, ev=None):
        torch, pk, w = self.torch, self.pk, self.w
        buf = self.step_idx % self.RING
        # step idx - RING last read this set (host buffer by its upload, device buffer by its kernels)
        self._wait_step_done(self.step_idx - self.RING)
        hn = self.host_np[buf]
        slots, pairs = self.st.bm.append(self.seqs, np.ones(self.S, dtype=np.int32))
        hn[: self.S] = slots
        tab = hn[2 * self.S: self.items_off].reshape(self.S, self.max_blocks)
        # only the live entries of each row: the kernels read no further, and the rest of the
        # staging row (an earlier step's shorter table, or never written) is not padding to redo
        self.st.bm.block_tables(self.seqs, self.max_blocks, out=tab, ctx_out=hn[self.S: 2 * self.S], pad=False)
        if self.work_list:
            self.n_items[buf] = pk.decode_items_into(hn[self.S: 2 * self.S], self.partition,
                                                     hn[self.items_off: self.items_off + self.max_items])
        main = torch.cuda.current_stream()
        with torch.cuda.stream(self.copy_stream):
            self.dev[buf].copy_(self.host[buf], non_blocking=True)
            e = torch.cuda.Event()
            e.record(self.copy_stream)
        # The host waits for the upload (it waits on nothing on the device, so it lands within
        # microseconds) and then launches: a cross-stream wait in the launch stream's queue left
        # about 5 us idle before every partition launch.
        e.synchronize()
        self._views(buf)
        if len(pairs):
            self.pairs_total += len(pairs)
            pk.copy_blocks(self.st.k_cache, self.st.v_cache,
                           torch.from_numpy(np.ascontiguousarray(pairs)).to("cuda", non_blocking=False), self.st.desc)
        if self.fused and ev is None and self.work_list:
            # the cache write and the partition launch in one pass (pkv_paged_attention_decode_append),
            # then the merge
            pk.paged_attention_decode_append(self.out, self.q, self.k_new, self.v_new, self.slots_d, self.st.k_cache,
                                             self.st.v_cache, self.tab_d, self.ctx_d, w.scale, self.max_ctx_final,
                                             self.st.desc, self.ws, self.partition, self.items_d)
            self._finish_step(buf, hn, main)
            return
        pk.kv_cache_write(self.k_new, self.v_new, self.st.k_cache, self.st.v_cache, self.slots_d, self.st.desc)
        if ev is not None:
            ev[0].record()
        launches = self.attention()
        next(launches)                       # partition launch
        if ev is not None:
            ev[1].record()
        next(launches, None)                 # merge launch
        if ev is not None:
            ev[2].record()
        self._finish_step(buf, hn, main)

    def _finish_step(self, buf, hn, main):
        if self.step_idx % self.MARK_EVERY == self.MARK_EVERY - 1:
            done = self.torch.cuda.Event()
            done.record(main)
            self.marks.append((self.step_idx, done))
        self.ctx_history.append(hn[self.S: 2 * self.S].copy())
        self.step_idx += 1


def _timed_windows(loop, K, min_total_s, min_windows, max_windows, ev=False):
    """Repeated K-step windows, each from the same saved block-manager state, so every window
    times the same K steps (same contexts, same slots, same values written). Each window is
    bracketed by device synchronisations on both sides. Returns per-window seconds and, with
    ``ev``, per-launch event times (partition launch, merge launch) in ms."""
    import torch
    snap = loop.snapshot
    times, kern_ms, merge_ms = [], [], []
    loop.host_s = []  # per window: host time to enqueue its K steps (before the closing synchronisation)
    while (len(times) < min_windows or sum(times) < min_total_s) and len(times) < max_windows:
        loop.st.bm = snap.clone()
        loop.ctx_history.clear()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K)] if ev else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            loop.step(evs[i] if ev else None)
        loop.host_s.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        if ev:
            kern_ms += [a.elapsed_time(b) for a, b, _ in evs]
            merge_ms += [b.elapsed_time(c) for _, b, c in evs]
    return times, kern_ms, merge_ms


def run_headline(args):
    import gc
    import torch
    from workloads import make_workload
    w = make_workload("gqa", "full", block_size=args.block_size)
    ramp_repeats = 400
    loop = DecodeLoop(w, args.warmup + args.steps + 1, work_list=not args.dense_grid, partition=args.partition)
    util = kv_utilisation(w, loop.st.bm, MAX_LEN["gqa"])
    for _ in range(args.warmup):
        loop.step()
    torch.cuda.synchronize()
    # Every timed window restarts from this state: its K steps append to the same contexts.
    loop.snapshot = loop.st.bm.clone()
    # Keep the GPU busy for a moment so clocks have ramped before the timed steps: repeat the
    # last step's attention without advancing the state (a fixed count, so every run of this
    # command times the same launches).
    loop.repeat_attention(ramp_repeats)
    torch.cuda.synchronize()
    K = args.steps
    # The interpreter's cyclic garbage collector can stop the host for milliseconds at a point
    # of its choosing; a serving loop keeps it out of its steps, and so does this one.
    gc.collect()
    gc.freeze()
    gc.disable()
    try:
        # Throughput: K-step windows with no instrumentation, repeated until they cover at least
        # 0.25 s (and at least 10 windows) -> value and ms_per_step from the median window.
        win_s, _, _ = _timed_windows(loop, K, 0.25, 10, 1000)
        host_s = list(loop.host_s)
        ctx_hist = list(loop.ctx_history)
        # the same windows with the cache write as its own launch, for reference
        loop.fused = False
        unf_s, _, _ = _timed_windows(loop, K, 0.1, 5, 1000)
        loop.fused = True
        # Roofline: more windows of the same K steps with HIP events around the partition and merge
        # launches (on the stream they run on). Event records cost about 8 us per step, which is why
        # they stay out of the throughput windows.
        _, kern_ms, merge_ms = _timed_windows(loop, K, 0.05, 5, 1000, ev=True)
        # The partition launch back to back on the last step's inputs, one event pair around the
        # whole region: the kernel's own average duration, without the dispatch overhead of an
        # event pair around every launch (about 2.5 %). The roofline uses this; the per-launch
        # event figure of the windows above is reported beside it.
        b2b_us = _partition_back_to_back(loop, B2B_LAUNCHES, B2B_WARM)
    finally:
        gc.enable()
        gc.unfreeze()
    kv_per_step = sum(decode_algorithmic_bytes(ctx, w, 2)[0] for ctx in ctx_hist) / K
    alg_per_launch = sum(decode_algorithmic_bytes(ctx, w, 2)[1] for ctx in ctx_hist) / K
    alg_b2b = decode_algorithmic_bytes(loop.ctx_history[-1], w, 2)[1]
    med_s = float(np.median(win_s))
    step_s = med_s / K
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    achieved = alg_b2b / (b2b_us * 1e-6) / 1e9
    return dict(
        w=w, loop=loop, ms_per_step=step_s * 1e3, seqs_per_s=len(w.query_seqs) / step_s,
        kv_gbs=kv_per_step / step_s / 1e9, kern_avg_us=b2b_us, kern_med_us=float(np.median(kern_ms)) * 1e3,
        kern_ev_avg_us=kern_avg_s * 1e6, achieved_ev=alg_per_launch / kern_avg_s / 1e9, alg_b2b=alg_b2b,
        achieved=achieved, alg_per_launch=alg_per_launch, kv_per_step=kv_per_step,
        kern_kv_gbs=kv_per_step / kern_avg_s / 1e9, partition=loop.partition,
        mean_ctx=float(np.mean([c.mean() for c in ctx_hist])), util=util,
        split_seqs=split_seqs(ctx_hist, loop.partition),
        merge_avg_us=float(np.mean(merge_ms)) * 1e3, kern_launches=len(kern_ms),
        windows={"count": len(win_s), "steps_each": K, "total_s": round(sum(win_s), 4),
                 "step_us_median": round(step_s * 1e6, 2),
                 "step_us_min": round(min(win_s) / K * 1e6, 2), "step_us_max": round(max(win_s) / K * 1e6, 2),
                 "step_us_p10": round(float(np.percentile(win_s, 10)) / K * 1e6, 2),
                 "step_us_p90": round(float(np.percentile(win_s, 90)) / K * 1e6, 2),
                 "step_us_median_separate_cache_write": round(float(np.median(unf_s)) / K * 1e6, 2),
                 # host time to enqueue a window's steps: near the window's own time means the
                 # host, not the GPU, paced it
                 "host_enqueue_us_per_step_median": round(float(np.median(host_s)) / K * 1e6, 2),
                 "host_enqueue_us_per_step_max": round(max(host_s) / K * 1e6, 2)})


B2B_LAUNCHES, B2B_WARM = 20, 3


def _partition_back_to_back(loop, n, warm):
    """Average duration (us) of the partition launch alone, ``n`` launches back to back on the last
    step's device inputs (its tables, lengths and work list) between one event pair, after ``warm``
    untimed launches."""
    import torch

    def launch():
        next(loop.attention())  # the partition launch (the generator's first step); no merge
    for _ in range(warm):
        launch()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        launch()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


_EVICT = None


def evict_caches():
    """Write a 512 MiB scratch buffer: flushes the 4 MB L2s and the 256 MB MALL between timed calls
    whose inputs would otherwise stay cached from the previous call."""
    global _EVICT
    import torch
    if _EVICT is None:
        _EVICT = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    _EVICT.fill_(1)


def _time_events(fn, reps=20, warm=3, evict=False):
    """Median and mean duration (us) of fn() measured with HIP events on the current stream; with
    ``evict`` the caches are flushed (untimed) before every call."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        if evict:
            evict_caches()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return float(np.median(ms)) * 1e3, float(np.mean(ms)) * 1e3


def measured_read_peak():
    """Streaming-read probe (libpkv_probe.so): 2 GiB read once with 16-byte non-temporal loads,
    best grid of 1024/2048/4096 workgroups, median of 20 each; the attainable read bandwidth
    that a read-bound kernel such as decode is measured against."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_323_amd", "libpkv_probe.so"))
    lib.pkvprobe_stream_read.restype = ctypes.c_int32
    lib.pkvprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_void_p]
    n = 2 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for grid in (1024, 2048, 4096):
        def call(g=grid):
            st = lib.pkvprobe_stream_read(ctypes.c_void_p(buf.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), g,
                                          stream)
            if st != 0:
                raise RuntimeError(f"stream-read probe failed: {st}")
        med, _ = _time_events(call, reps=20, warm=3)
        best = max(best, n / med / 1e3)
    del buf, sink
    torch.cuda.empty_cache()
    return best  # GB/s


def measured_gather_peak(loop):
    """Tile-gather probe (libpkv_probe.so) over the headline's own pools: every (block, kv head)
    tile of the current step's contexts, listed per (sequence, kv head) in table order, read from
    the K pool and then the V pool, with no arithmetic; the best of 16, 32, 64 and 128 tiles per
    workgroup, median of 20 each. The attainable rate of the decode kernel's access pattern (tiles
    of 1 or 2 KiB, or a multiple of 4 KiB; None otherwise)."""
    import ctypes
    import torch
    w = loop.w
    tile_bytes = w.block_size * w.head_dim * {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    if tile_bytes % 4096 and tile_bytes not in (1024, 2048):
        return None
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_323_amd", "libpkv_probe.so"))
    lib.pkvprobe_gather_read.restype = ctypes.c_int32
    lib.pkvprobe_gather_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    tables, lens = loop.st.bm.block_tables(loop.seqs, loop.max_blocks)
    H = w.num_kv_heads
    parts = []
    for s in range(len(lens)):
        blocks = tables[s, : -(-int(lens[s]) // w.block_size)].astype(np.int64)
        parts.append((blocks[None, :] * H + np.arange(H)[:, None]).ravel())
    tiles_h = np.concatenate(parts)
    assert tiles_h.min() >= 0 and tiles_h.max() < w.num_blocks * H  # every tile inside both pools
    tiles = torch.from_numpy(tiles_h.astype(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for per_wg in (16, 32, 64, 128):
        def call(p=per_wg):
            st = lib.pkvprobe_gather_read(ctypes.c_void_p(loop.st.k_cache.data_ptr()),
                                          ctypes.c_void_p(loop.st.v_cache.data_ptr()),
                                          ctypes.c_void_p(tiles.data_ptr()), len(tiles_h), tile_bytes, p,
                                          ctypes.c_void_p(sink.data_ptr()), stream)
            if st != 0:
                raise RuntimeError(f"gather probe failed: {st}")
        med, _ = _time_events(call, reps=20, warm=3)
        best = max(best, 2 * len(tiles_h) * tile_bytes / med / 1e3)
    return best  # GB/s


def measured_copy_peak():
    """Streaming-copy probe (libpkv_probe.so): 1 GiB copied into another 1 GiB buffer with
    16-byte non-temporal loads and stores, 4 in flight per thread, best grid of 8192/16384/32768
    workgroups, median of 20 each; counted as read + write bytes. The attainable rate of a
    contiguous copy, which copy_blocks, the cache write and swap are set against."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_323_amd", "libpkv_probe.so"))
    lib.pkvprobe_stream_copy.restype = ctypes.c_int32
    lib.pkvprobe_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for grid in (8192, 16384, 32768):
        def call(g=grid):
            st = lib.pkvprobe_stream_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n, g, 4,
                                          3, stream)
            if st != 0:
                raise RuntimeError(f"stream-copy probe failed: {st}")
        med, _ = _time_events(call, reps=20, warm=3)
        best = max(best, 2 * n / med / 1e3)
    ok = bool(torch.equal(dst[:: 1 << 20], src[:: 1 << 20]))
    del src, dst
    torch.cuda.empty_cache()
    if not ok:
        raise RuntimeError("stream-copy probe did not copy")
    return best  # GB/s


# Longest length a request of each workload may reach: what max-length preallocation reserves.
MAX_LEN = {"gqa": 8192, "llama7b": 2048, "shared_prefix": 1000 + 512, "mixed": 4096}


def kv_utilisation(w, bm, max_len, stored_tokens=None):
    """KV memory actually holding tokens, paged vs max-length preallocation (the pages quote
    20-40 % for the latter). Paged: tokens stored / slots of the blocks in use; preallocation:
    every sequence reserves max_len slots and shares nothing."""
    used = w.num_blocks - bm.num_free()
    tokens = int(sum(w.context_lens)) if stored_tokens is None else int(stored_tokens)
    # the empty slots of each sequence's last block: for lengths spread evenly over a block's
    # residues their mean is (B - 1) / 2 slots
    lens = np.asarray(w.context_lens, dtype=np.int64)
    waste = -(-lens // w.block_size) * w.block_size - lens
    return {"paged": round(tokens / (used * w.block_size), 4),
            "max_len_prealloc": round(int(sum(w.context_lens)) / (len(w.context_lens) * max_len), 4),
            "max_len": max_len, "blocks_in_use": int(used),
            "last_block_empty_slots_mean": round(float(waste.mean()), 2),
            "last_block_empty_slots_even_residues": (w.block_size - 1) / 2}


def run_decode_config(name, block_size=None, K=20, warmup=5, partition=0):
    """Decode-step loop for another configuration, timed as the headline is: K-step windows that
    restart from one saved allocation state, without instrumentation for the step time, then more
    windows with HIP events around the partition and merge launches."""
    import gc
    import torch
    from workloads import make_workload
    w = make_workload(name, "full", block_size=block_size)
    loop = DecodeLoop(w, warmup + K + 5, partition=partition)
    util = kv_utilisation(w, loop.st.bm, MAX_LEN[name])
    for _ in range(warmup):
        loop.step()
    torch.cuda.synchronize()
    loop.snapshot = loop.st.bm.clone()
    # clocks up before the timed steps, as in the headline: the last step's attention repeated
    # (the state does not advance)
    loop.repeat_attention(200)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    try:
        win_s, _, _ = _timed_windows(loop, K, 0.1, 5, 200)
        host_s = list(loop.host_s)
        ctx_hist = list(loop.ctx_history)
        _, kern_ms, merge_ms = _timed_windows(loop, K, 0.05, 3, 50, ev=True)
    finally:
        gc.enable()
    el = float(np.median(win_s)) / K
    kern = float(np.mean(kern_ms)) * 1e-3
    merge = float(np.mean(merge_ms)) * 1e-3
    kv = float(np.mean([decode_algorithmic_bytes(c, w, 2)[0] for c in ctx_hist]))
    res = {"workload": w.name, "seqs": len(w.query_seqs), "partition": loop.partition,
           "split_seqs": split_seqs(ctx_hist, loop.partition), "step_us": round(el * 1e6, 1),
           "seqs_per_s": round(len(w.query_seqs) / el, 1), "kv_gbs_step": round(kv / el / 1e9, 1),
           "partition_launch_us": round(kern * 1e6, 1), "merge_launch_us": round(merge * 1e6, 1),
           "kv_gbs_partition_launch": round(kv / kern / 1e9, 1),
           "pct_hbm_partition_launch": round(100 * kv / kern / 1e9 / HBM_PEAK_GBS, 1),
           "windows": len(win_s),
           # host time to enqueue a window's steps: near the step time means the host paced it
           "host_enqueue_us_per_step": round(float(np.median(host_s)) / K * 1e6, 1),
           "kv_memory_utilisation": util}
    # the same (block, kv head) tiles gathered with no arithmetic: this block size's pattern ceiling
    gather = measured_gather_peak(loop)
    if gather:
        res["gather_ceiling_gbs"] = round(gather, 1)
        res["partition_launch_frac_of_gather"] = round(kv / kern / 1e9 / gather, 4)
    del loop
    torch.cuda.empty_cache()
    return res


def split_seqs(ctx_history, partition):
    """Mean count per step of sequences whose context spans more than one partition (the ones the
    merge launch combines; the others take one partition's result as it stands)."""
    return round(float(np.mean([int((np.asarray(c) > partition).sum()) for c in ctx_history])), 1)


HEAD_SHAPES = ((64, 8, 128), (64, 8, 64), (32, 8, 64), (16, 8, 128), (32, 32, 128))


def run_head_shapes(shapes=HEAD_SHAPES, K=20):
    """Decode across head shapes at the GQA configuration's 256 lognormal lengths (bf16, block size
    16, automatic partition): partition launch and merge, event-timed over K-step windows restarted
    from one saved allocation state; KV bytes over the two launches' time. The headline shape
    (32 query heads over 8 kv heads, head_dim 128) is the headline row."""
    import torch
    from workloads import make_decode_workload, make_workload
    ctx = list(make_workload("gqa", "full").context_lens)
    res = {}
    for hq, hkv, d in shapes:
        w = make_decode_workload(3, ctx, hq, hkv, d, "bf16", 16, name=f"heads-{hq}-{hkv}-d{d}")
        loop = DecodeLoop(w, 5 + K + 5)
        for _ in range(5):
            loop.step()
        torch.cuda.synchronize()
        loop.snapshot = loop.st.bm.clone()
        loop.repeat_attention(100)  # clocks up
        torch.cuda.synchronize()
        _, kern_ms, merge_ms = _timed_windows(loop, K, 0.05, 3, 20, ev=True)
        kv = sum(decode_algorithmic_bytes(c, w, 2)[0] for c in loop.ctx_history) / len(loop.ctx_history)
        k_us, m_us = float(np.mean(kern_ms)) * 1e3, float(np.mean(merge_ms)) * 1e3
        row = {"partition": loop.partition, "partition_launch_us": round(k_us, 1),
               "merge_launch_us": round(m_us, 1),
               "kv_gbs": round(kv / (k_us + m_us) / 1e3, 1),
               "pct_hbm": round(100 * kv / (k_us + m_us) / 1e3 / HBM_PEAK_GBS, 1),
               "kv_gbs_partition_launch": round(kv / k_us / 1e3, 1)}
        # the same (block, kv head) tiles gathered with no arithmetic: the access pattern's ceiling
        gather = measured_gather_peak(loop)
        if gather:
            row["gather_ceiling_gbs"] = round(gather, 1)
            row["partition_launch_frac_of_gather"] = round(kv / k_us / 1e3 / gather, 4)
        res[f"{hq}/{hkv}/d{d}"] = row
        del loop
        torch.cuda.empty_cache()
    return res


def profile_heads(shape: str, K=20):
    """One decode head shape ("QH/KVH/D") at the GQA configuration's lengths (bf16, B 16, automatic
    partition): two event-timed K-step windows from a saved state after 50 repeats, for counter
    runs; prints the partition launch's mean event time."""
    import torch
    from workloads import make_decode_workload, make_workload
    hq, hkv, d = (int(x) for x in shape.split("/"))
    ctx = list(make_workload("gqa", "full").context_lens)
    w = make_decode_workload(3, ctx, hq, hkv, d, "bf16", 16, name=f"heads-{hq}-{hkv}-d{d}")
    loop = DecodeLoop(w, 5 + K + 5)
    for _ in range(5):
        loop.step()
    torch.cuda.synchronize()
    loop.snapshot = loop.st.bm.clone()
    loop.repeat_attention(50)
    torch.cuda.synchronize()
    _, kern_ms, _ = _timed_windows(loop, K, 0.0, 2, 2, ev=True)
    print(json.dumps({"shape": shape, "partition": loop.partition,
                      "partition_launch_us": round(float(np.mean(kern_ms)) * 1e3, 1)}), flush=True)


def run_shared_prefix():
    """Copy-on-write copies at the first generated token and decode over shared blocks."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    from workloads import make_workload
    w = make_workload("shared_prefix", "full")
    st = R.play_script(w, threads=16)
    pairs = st.pairs_per_append[-2]               # the first generated token's COW pairs
    pd = torch.from_numpy(np.ascontiguousarray(pairs)).cuda()
    blk_bytes = w.num_kv_heads * w.block_size * w.head_dim * 2
    # 48 pairs move 24 MiB, which would stay in the MALL between calls: flush it before each one
    med, _ = _time_events(lambda: pk.copy_blocks(st.k_cache, st.v_cache, pd, st.desc), reps=50, warm=10,
                          evict=True)
    warm_med, _ = _time_events(lambda: pk.copy_blocks(st.k_cache, st.v_cache, pd, st.desc), reps=50, warm=10)
    res = {"workload": w.name, "cow_pairs": int(len(pairs)), "copy_us": round(med, 2),
           "copy_gbs": round(2 * 2 * len(pairs) * blk_bytes / med / 1e3, 1), "copy_us_cached": round(warm_med, 2),
           "timing": "HIP events, 10 warm-ups, median of 50 (decode: 30); caches flushed before each timed call"}
    # decode at the final state
    out, inp = R.attention(w, st, w.dtype)
    bt, cl, q, ws = inp["block_tables"], inp["context_lens"], inp["q"], inp["workspace"]
    mx = int(inp["lens_host"].max())
    med, _ = _time_events(lambda: pk.paged_attention_decode(out, q, st.k_cache, st.v_cache, bt, cl, w.scale, mx,
                                                            st.desc, ws), reps=30, warm=10, evict=True)
    lens = inp["lens_host"]
    tables = inp["tables_host"]
    logical = int(lens.sum()) * w.kv_bytes_per_token()
    fill = {}
    for t, L in zip(tables, lens):
        for j in range(-(-int(L) // w.block_size)):
            fill[int(t[j])] = max(fill.get(int(t[j]), 0), min(w.block_size, int(L) - j * w.block_size))
    unique = sum(fill.values()) * w.kv_bytes_per_token()
    res["kv_memory_utilisation"] = kv_utilisation(w, st.bm, MAX_LEN["shared_prefix"], sum(fill.values()))
    res.update({"decode_us": round(med, 1), "decode_logical_gbs": round(logical / med / 1e3, 1),
                "decode_unique_gbs": round(unique / med / 1e3, 1), "seqs_per_s": round(len(lens) / med * 1e6, 1)})
    del st
    torch.cuda.empty_cache()
    # bandwidth-scale copy: 4096 pairs over a separate pool of the same block shape
    nb = 8192
    kc = torch.empty((nb, w.num_kv_heads, w.block_size, w.head_dim), dtype=torch.float16, device="cuda")
    vc = torch.empty_like(kc)
    kc.normal_()
    vc.normal_()
    desc = pk.CacheDesc.make(nb, w.block_size, w.num_kv_heads, w.head_dim, "f16")
    perm = np.random.default_rng(4).permutation(nb).astype(np.int32)
    big = torch.from_numpy(np.ascontiguousarray(perm.reshape(2, -1).T)).cuda()
    med, _ = _time_events(lambda: pk.copy_blocks(kc, vc, big, desc), reps=20)
    res["copy_4096_pairs_us"] = round(med, 1)
    res["copy_4096_pairs_gbs"] = round(2 * 2 * 4096 * blk_bytes / med / 1e3, 1)
    # the same copy between two runs of consecutive blocks: what the kernel moves when the pool's
    # placement is not scattered (the gap to the random pairs is the cost of placement)
    seq = torch.from_numpy(np.ascontiguousarray(np.stack([np.arange(4096), np.arange(4096, 8192)], 1)
                                                .astype(np.int32))).cuda()
    med, _ = _time_events(lambda: pk.copy_blocks(kc, vc, seq, desc), reps=20)
    res["copy_4096_sequential_pairs_gbs"] = round(2 * 2 * 4096 * blk_bytes / med / 1e3, 1)
    del kc, vc
    torch.cuda.empty_cache()
    return res


def run_tiny():
    """The tiny configuration (4 sequences of 5-100 tokens, 4 heads, head_dim 64, f32): a launch-
    latency case. The step's fused cache write and decode, the decode alone, and the 4-token cache
    write alone, each timed with HIP events (10 warm-ups, median of 50) with the caches flushed
    before every call: the flush keeps the stream busy, so each call's launch is queued before its
    start event fires. The fused step is timed once more without the flush, so the host paces
    every call and the event pair includes the call's host overhead."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    from workloads import make_workload
    w = make_workload("tiny", "full")
    st = R.play_script(w)
    op = w.ops[-1]  # the step: one new token per sequence, written before the decode reads it
    if list(op.seqs) != list(w.query_seqs) or any(n != 1 for n in op.n_tokens):
        raise RuntimeError("the tiny script's last append is not one token per query sequence")
    k, v = w.append_values(op)
    kd = R.to_device(k, w.dtype).contiguous()
    vd = R.to_device(v, w.dtype).contiguous()
    slots = torch.from_numpy(np.ascontiguousarray(st.slots_per_append[-1])).cuda()
    out, inp = R.attention(w, st, w.dtype)
    bt, cl, q, ws = inp["block_tables"], inp["context_lens"], inp["q"], inp["workspace"]
    mx = int(inp["lens_host"].max())

    def step():
        pk.paged_attention_decode_append(out, q, kd, vd, slots, st.k_cache, st.v_cache, bt, cl, w.scale, mx,
                                         st.desc, ws)

    res = {"workload": w.name, "seqs": len(w.query_seqs), "context_lens": [int(x) for x in inp["lens_host"]],
           "timing": "HIP events, 10 warm-ups, median of 50; caches flushed before each timed call"}
    res["step_us"], _ = _time_events(step, reps=50, warm=10, evict=True)
    res["step_us_host_paced"], _ = _time_events(step, reps=50, warm=10)
    res["decode_us"], _ = _time_events(
        lambda: pk.paged_attention_decode(out, q, st.k_cache, st.v_cache, bt, cl, w.scale, mx, st.desc, ws),
        reps=50, warm=10, evict=True)
    res["kv_cache_write_us"], _ = _time_events(
        lambda: pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, slots, st.desc), reps=50, warm=10, evict=True)
    _, empty = _time_events(lambda: None, reps=50, warm=10)
    res["event_pair_us"] = round(empty, 2)  # an event pair around no launch
    for key in ("step_us", "step_us_host_paced", "decode_us", "kv_cache_write_us"):
        res[key] = round(res[key], 2)
    res["kv_memory_utilisation"] = kv_utilisation(w, st.bm, max(w.context_lens))
    del st
    torch.cuda.empty_cache()
    return res


def run_swap():
    """Preemption traffic: whole GQA-shaped blocks (8 kv heads x 16 slots x 128 dims, bf16) moved
    between the GPU pool and a pinned host swap pool by pkv_swap_blocks, both directions."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    nb, H, B, D = 8192, 8, 16, 128
    dk = torch.empty((nb, H, B, D), dtype=torch.bfloat16, device="cuda").normal_()
    dv = torch.empty_like(dk).normal_()
    hk = torch.empty((nb, H, B, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    desc = pk.CacheDesc.make(nb, B, H, D, "bf16")
    n = 4096
    perm = np.random.default_rng(9).permutation(nb).astype(np.int32)
    out_pairs = torch.from_numpy(np.ascontiguousarray(np.stack([perm[:n], perm[n:2 * n]], 1))).cuda()
    in_pairs = torch.from_numpy(np.ascontiguousarray(np.stack([perm[n:2 * n], perm[:n]], 1))).cuda()
    out_us, _ = _time_events(lambda: pk.swap_blocks(hk, hv, dk, dv, out_pairs, desc), reps=10)
    in_us, _ = _time_events(lambda: pk.swap_blocks(dk, dv, hk, hv, in_pairs, desc), reps=10)
    moved = 2 * n * H * B * D * 2
    res = {"blocks": n, "bytes_per_direction": moved, "swap_out_us": round(out_us, 1),
           "swap_out_gbs": round(moved / out_us / 1e3, 1), "swap_in_us": round(in_us, 1),
           "swap_in_gbs": round(moved / in_us / 1e3, 1)}
    del dk, dv, hk, hv
    torch.cuda.empty_cache()
    return res


def run_engine(n_requests=512, max_steps=400):
    """Steady-state continuous batching (13B-shaped attention: 40 heads, head_dim 128, bf16,
    B=16): 512 requests with prompts U{128..1024} and 32-256 new tokens, at most 256 in flight,
    a pool too small for all of them (preemption by swap to a pinned host pool). Reports
    requests finished and tokens processed per second over the timed steps (host scheduling,
    block manager, uploads and kernels included)."""
    import torch
    from paged_kv_cache_323_amd.engine import Engine
    rng = np.random.default_rng(21)
    eng = Engine(num_blocks=9000, block_size=16, num_q_heads=40, num_kv_heads=40, head_dim=128, dtype="bf16",
                 max_num_seqs=256, max_step_tokens=8192, num_host_blocks=6000, seed=21,
                 copy_stream=upload_stream())
    for _ in range(n_requests):
        eng.add_request(int(rng.integers(128, 1025)), int(rng.integers(32, 257)))
    for _ in range(10):  # warm-up steps (first admissions)
        eng.step()
    torch.cuda.synchronize()
    s0 = dataclass_copy(eng.stats)
    t0 = time.perf_counter()
    steps = 0
    while eng.has_work() and steps < max_steps:
        eng.step()
        steps += 1
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = eng.stats
    res = {"requests": n_requests, "timed_steps": steps, "step_ms": round(el / max(steps, 1) * 1e3, 3),
           "finished_per_s": round((st.finished - s0.finished) / el, 1),
           "decode_tokens_per_s": round((st.decode_tokens - s0.decode_tokens) / el, 1),
           "prefill_tokens_per_s": round((st.prefill_tokens - s0.prefill_tokens) / el, 1),
           # KV the decode rows read (every cached token of theirs, K and V), over the whole step
           "decode_kv_gbs_step": round((st.decode_kv_tokens - s0.decode_kv_tokens) * 2 * eng.hkv * eng.d
                                       * 2 / el / 1e9, 1),
           "preemptions": st.preemptions, "resumptions": st.resumptions, "finished_total": st.finished}
    del eng
    torch.cuda.empty_cache()
    return res


def dataclass_copy(x):
    import dataclasses
    return dataclasses.replace(x)


def prefill_flops(q_lens, ctx, hq, d):
    """4·d·Hq per causal (query, key) pair: query at position p sees p+1 keys."""
    tot = 0
    for ql, c in zip(q_lens, ctx):
        if ql <= 1:
            continue
        first = c - ql  # position of the first query row
        tot += sum(int(first) + t + 1 for t in range(int(ql)))
    return 4 * int(d) * int(hq) * int(tot)


def run_mixed():
    """Selective-batching mixed step (8 prefills + 248 decodes, 40 heads, bf16): the step's
    cache write plus the ragged attention, and a prefill-only call for MFMA utilisation."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    from workloads import make_workload
    w = make_workload("mixed", "full")
    t = time.perf_counter()
    st = R.play_script(w, threads=16)
    torch.cuda.synchronize()
    log(f"setup {w.name}: wrote {sum(w.context_lens)} tokens in {time.perf_counter() - t:.1f}s")
    util = kv_utilisation(w, st.bm, MAX_LEN["mixed"])
    step_op = w.ops[-1]
    k, v = w.append_values(step_op, threads=16)
    kd, vd = R.to_device(k, w.dtype), R.to_device(v, w.dtype)
    slots = torch.from_numpy(np.ascontiguousarray(st.slots_per_append[-1])).cuda()
    q = R.to_device(w.queries(), w.dtype)
    out = torch.empty_like(q)
    tables, lens = st.bm.block_tables(w.query_seqs, w.max_blocks_per_seq())
    bt, cl = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    mx, mq = int(lens.max()), int(max(w.q_lens))
    ws = torch.zeros(max(pk.ragged_workspace_bytes(len(lens), q.shape[0], w.num_q_heads, mq, mx, st.desc), 1),
                     dtype=torch.uint8, device="cuda")

    # decode rows from the longest-first work list, built from the host lengths as a serving loop
    # would (the dense-grid call is timed beside it)
    part = pk.decode_partition_size(len(lens), w.num_q_heads, mx, st.desc)
    items = torch.from_numpy(pk.decode_items(lens, part)).cuda()

    def attention():
        pk.paged_attention_ragged(out, q, cu, cl, st.k_cache, st.v_cache, bt, w.scale, mq, mx, st.desc, ws,
                                  min_q_len=int(min(w.q_lens)), partition_size=part, items=items)

    def step():
        pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, slots, st.desc)
        attention()

    step_us, _ = _time_events(step, reps=20)
    att_us, _ = _time_events(attention, reps=20)
    att_dense_us, _ = _time_events(lambda: pk.paged_attention_ragged(out, q, cu, cl, st.k_cache, st.v_cache, bt,
                                                                     w.scale, mq, mx, st.desc, ws), reps=20)
    n_pre = sum(1 for x in w.q_lens if x > 1)
    # prefill-only call: the 8 prompt sequences alone
    cu_p = torch.from_numpy(w.cu_seqlens()[: n_pre + 1].copy()).cuda()
    T_p = int(w.cu_seqlens()[n_pre])
    ql_p, ctx_p = w.q_lens[:n_pre], list(lens[:n_pre])
    mx_p = int(max(ctx_p))
    # (its shortest prompt as the lower bound on q_len: no decode-row launches)
    pre_us, _ = _time_events(lambda: pk.paged_attention_ragged(out[:T_p], q[:T_p], cu_p, cl[:n_pre], st.k_cache,
                                                               st.v_cache, bt[:n_pre], w.scale, mq, mx_p, st.desc,
                                                               ws, min_q_len=min(ql_p)), reps=20)
    flops = prefill_flops(ql_p, ctx_p, w.num_q_heads, w.head_dim)
    dec_kv = int(sum(int(c) for c, ql in zip(lens, w.q_lens) if ql == 1)) * w.kv_bytes_per_token()
    write_bytes = 2 * 2 * int(q.shape[0]) * w.num_kv_heads * w.head_dim * 2
    res = {"workload": w.name, "tokens": int(q.shape[0]), "prefill_seqs": n_pre,
           "decode_seqs": len(lens) - n_pre, "step_us": round(step_us, 1),
           "seqs_per_s": round(len(lens) / step_us * 1e6, 1), "attention_us": round(att_us, 1),
           "attention_us_dense_grid": round(att_dense_us, 1), "decode_partition": part,
           "decode_kv_gb": round(dec_kv / 1e9, 3), "prefill_only_us": round(pre_us, 1),
           "prefill_gflop": round(flops / 1e9, 2), "prefill_tflops": round(flops / pre_us / 1e6, 1),
           "prefill_mfma_util": round(flops / pre_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
           "kv_cache_write_bytes": write_bytes, "kv_memory_utilisation": util}
    # cache write alone at the step's size
    w_us, _ = _time_events(lambda: pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, slots, st.desc), reps=20)
    res["kv_cache_write_us"] = round(w_us, 1)
    res["kv_cache_write_gbs"] = round(write_bytes / w_us / 1e3, 1)
    # from cold caches (a 512 MiB write before each call), as when the step's K/V rows come from
    # elsewhere: 186 MB moved, so part of it would otherwise stay in the 256 MB MALL
    w_us, _ = _time_events(lambda: pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, slots, st.desc), reps=20,
                           evict=True)
    res["kv_cache_write_cold_us"] = round(w_us, 1)
    res["kv_cache_write_cold_gbs"] = round(write_bytes / w_us / 1e3, 1)
    # The same rows into consecutive slots of the same pool (blocks 0, 1, 2, ... in order): the write
    # without the scatter of a paged pool's blocks. It overwrites those blocks, so it comes last.
    seq_slots = torch.arange(int(slots.numel()), dtype=torch.int32, device="cuda")
    w_us, _ = _time_events(lambda: pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, seq_slots, st.desc), reps=20)
    res["kv_cache_write_sequential_slots_gbs"] = round(write_bytes / w_us / 1e3, 1)
    del st
    torch.cuda.empty_cache()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=12.0):
    """The oracle (float64 NumPy) on the host CPU over every sequence of the benchmark's first decode
    step: once with one BLAS thread and once with all the threads the process may use (the
    thread count OMP_NUM_THREADS gives, else the CPU affinity set). Each is the median of up to 3
    runs within ``budget_s`` seconds."""
    from threadpoolctl import threadpool_limits
    import oracle
    n_all = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    seqs = list(w.query_seqs)
    st, _ = oracle.run_workload(w, only_seqs=seqs, attend=False, threads=n_all)
    tables, lens = st.bm.padded_tables(seqs, w.max_blocks_per_seq())
    q = w.queries(seqs)
    cu = np.arange(len(seqs) + 1, dtype=np.int32)
    kv = int(np.sum(lens)) * w.kv_bytes_per_token()

    def timed(threads):
        times = []
        with threadpool_limits(threads):
            for _ in range(3):
                t = time.perf_counter()
                oracle.paged_ragged(q, cu, lens, tables, st.pool_k, st.pool_v, w.scale, w.block_size, w.dtype)
                times.append(time.perf_counter() - t)
                if sum(times) > budget_s:
                    break
        return float(np.median(times)), len(times)

    t1, n1 = timed(1)
    tn, nn = timed(n_all)
    return {"value": kv / tn / 1e9, "unit": "GB/s", "cores": n_all, "kind": "oracle",
            "seqs_per_s": len(seqs) / tn,
            "single_thread": {"value": kv / t1 / 1e9, "unit": "GB/s", "cores": 1, "seqs_per_s": len(seqs) / t1},
            "cpu_model": _cpu_model(),
            "sample": f"all {len(seqs)} sequences of the first {w.name} decode step (sum ctx {int(np.sum(lens))}, "
                      f"{kv / 1e9:.2f} GB of KV), median of {nn} runs with {n_all} BLAS threads "
                      f"({n1} runs with 1 thread)"}


def source_digest(name: str = "decode.hip") -> str:
    """Digest of a kernel source's code: counter-derived figures are only valid for it. Comments
    and whitespace are left out, so editing a comment does not invalidate the counters."""
    import hashlib
    import re
    src = os.path.join(ROOT, "paged_kv_cache_323_amd", "csrc", name)
    with open(src, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
    text = re.sub(r"//[^\n]*", " ", text)                 # line comments
    code = "".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def _read_summary(path):
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    return kv


def load_copy_traffic():
    """HBM traffic over algorithmic bytes of the copy kernels (copy_blocks, the cache write, swap)
    from the committed counter summary, keyed by workload, or {} when it was taken on a different
    cache_ops.hip."""
    path = os.path.join(ROOT, "profiles", "copy_kernels_traffic.txt")
    if not os.path.exists(path):
        return {}
    kv = _read_summary(path)
    if kv.get("source_digest") != source_digest("cache_ops.hip"):
        return {}
    return {k[: -len("_traffic_over_algorithmic")]: float(v) for k, v in kv.items()
            if k.endswith("_traffic_over_algorithmic")}


def load_traffic(block_size: int):
    """The decode partition launch's HBM traffic over its algorithmic bytes, from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size), or None when
    that summary was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_gqa_B{block_size}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = _read_summary(path)
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return {"ratio": float(kv["traffic_bytes_per_launch"]) / float(kv["algorithmic_bytes_per_launch"]),
                "profile_traffic_bytes": float(kv["traffic_bytes_per_launch"]),
                "profile_algorithmic_bytes": float(kv["algorithmic_bytes_per_launch"])}
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def layout_study(layout: str):
    """The GQA decode step (B = 16) with the library PAGEDKV_LIB points to, whose pools are stored
    head-major (the product) or token-major (the tuning build of build.py --token-major): the
    partition launch's event time over 20-step windows, a row-gather probe reading exactly the
    (block, kv head) tiles of the step in that layout's pattern, and the cache write. Prints one
    JSON line; a rocprofv3 counter target as well."""
    import ctypes
    import torch
    from paged_kv_cache_323_amd import native as pk
    from workloads import make_workload
    token_major = layout == "token"
    w = make_workload("gqa", "full", block_size=16)
    loop = DecodeLoop(w, 5 + 10 * 20 + 5)
    for _ in range(5):
        loop.step()
    torch.cuda.synchronize()
    loop.snapshot = loop.st.bm.clone()
    loop.repeat_attention(200)
    torch.cuda.synchronize()
    _, kern_ms, merge_ms = _timed_windows(loop, 20, 0.05, 5, 50, ev=True)
    alg = sum(decode_algorithmic_bytes(c, w, 2)[1] for c in loop.ctx_history) / 20
    k_us = float(np.mean(kern_ms)) * 1e3
    out = loop.out.float().cpu().numpy()
    res = {"layout": "token-major" if token_major else "head-major", "library": os.path.basename(pk.LIB_PATH),
           "partition_us": round(k_us, 1), "partition_gbs": round(alg / k_us / 1e3, 1),
           "merge_us": round(float(np.mean(merge_ms)) * 1e3, 2), "algorithmic_bytes": int(alg),
           "output_checksum": int(np.frombuffer(out.tobytes(), dtype=np.uint32).astype(np.uint64).sum() % (1 << 61))}
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_323_amd", "libpkv_probe.so"))
    lib.pkvprobe_gather_rows.restype = ctypes.c_int32
    lib.pkvprobe_gather_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    tables, lens = loop.st.bm.block_tables(loop.seqs, loop.max_blocks)
    H, B, D = w.num_kv_heads, w.block_size, w.head_dim
    row_bytes = D * 2
    parts = []
    for s in range(len(lens)):
        blocks = tables[s, : -(-int(lens[s]) // B)].astype(np.int64)
        if token_major:  # tile (b, h) starts at row b*B*H + h (rows of D elements); rows H*D apart
            parts.append((blocks[None, :] * B * H + np.arange(H)[:, None]).ravel())
        else:            # tile (b, h) starts at row (b*H + h)*B; rows contiguous
            parts.append(((blocks[None, :] * H + np.arange(H)[:, None]) * B).ravel())
    t = np.concatenate(parts)
    stride = H * row_bytes if token_major else row_bytes
    assert t.min() >= 0 and t.max() * row_bytes + (B - 1) * stride + row_bytes <= w.num_blocks * H * B * row_bytes
    tiles = torch.from_numpy(t.astype(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for per_wg in (16, 32, 64):
        def call(p=per_wg):
            st = lib.pkvprobe_gather_rows(ctypes.c_void_p(loop.st.k_cache.data_ptr()),
                                          ctypes.c_void_p(loop.st.v_cache.data_ptr()), ctypes.c_void_p(tiles.data_ptr()),
                                          len(t), row_bytes, B, row_bytes, stride, p, ctypes.c_void_p(sink.data_ptr()),
                                          stream)
            if st != 0:
                raise RuntimeError(f"row-gather probe failed: {st}")
        med, _ = _time_events(call, reps=20, warm=3)
        best = max(best, 2 * len(t) * B * row_bytes / med / 1e3)
    res["row_gather_probe_gbs"] = round(best, 1)
    res["partition_frac_of_probe"] = round(alg / k_us / 1e3 / best, 4)
    T = 65536
    slots = torch.from_numpy(np.random.default_rng(1).permutation(w.num_blocks * B)[:T].astype(np.int32)).cuda()
    k = torch.randn((T, H, D), device="cuda").to(torch.bfloat16)
    v = torch.randn_like(k)
    wus, _ = _time_events(lambda: pk.kv_cache_write(k, v, loop.st.k_cache, loop.st.v_cache, slots, loop.st.desc),
                          reps=20, warm=3)
    res["write_65536_tokens_gbs"] = round(2 * 2 * T * H * D * 2 / wus / 1e3, 1)
    print(json.dumps(res), flush=True)


def profile_copy(reps: int = 10):
    """Counter target and calibration for HBM counters: copy_blocks of 4096 whole blocks (f16, 32
    heads x 16 slots x 128 dims, random pairs), 1 GiB read and 1 GiB written per launch."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    nb, H, B, D = 8192, 32, 16, 128
    kc = torch.empty((nb, H, B, D), dtype=torch.float16, device="cuda").normal_()
    vc = torch.empty_like(kc).normal_()
    desc = pk.CacheDesc.make(nb, B, H, D, "f16")
    perm = np.random.default_rng(4).permutation(nb).astype(np.int32)
    pairs = torch.from_numpy(np.ascontiguousarray(perm.reshape(2, -1).T)).cuda()
    for _ in range(reps):
        pk.copy_blocks(kc, vc, pairs, desc)
    torch.cuda.synchronize()
    print(json.dumps({"copy_blocks_pairs": 4096, "bytes_read_per_launch": 2 * 4096 * H * B * D * 2,
                      "bytes_written_per_launch": 2 * 4096 * H * B * D * 2, "launches": reps}))


def profile_write(reps: int = 10):
    """Counter target: kv_cache_write of the 13B-shaped mixed step's new tokens (9421 tokens x 40
    kv heads x 128 dims, bf16, B=16) into the slots the block manager gives them."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    from workloads import make_workload
    w = make_workload("mixed", "full")
    st = R.play_script(w, threads=16)
    step_op = w.ops[-1]
    k, v = w.append_values(step_op, threads=16)
    kd, vd = R.to_device(k, w.dtype), R.to_device(v, w.dtype)
    slots = torch.from_numpy(np.ascontiguousarray(st.slots_per_append[-1])).cuda()
    torch.cuda.synchronize()
    for _ in range(reps):
        pk.kv_cache_write(kd, vd, st.k_cache, st.v_cache, slots, st.desc)
    torch.cuda.synchronize()
    T = int(kd.shape[0])
    row = w.num_kv_heads * w.head_dim * 2
    print(json.dumps({"kv_cache_write_tokens": T, "bytes_read_per_launch": 2 * T * row,
                      "bytes_written_per_launch": 2 * T * row, "launches": reps,
                      "setup_launches_before": "the script's own cache writes (one per append)"}))


def profile_swap(reps: int = 5):
    """Counter target: pkv_swap_blocks of 4096 GQA-shaped blocks (8 kv heads x 16 slots x 128 dims,
    bf16) out to a pinned host pool, then back in; 256 MiB each way per launch."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    nb, H, B, D = 8192, 8, 16, 128
    dk = torch.empty((nb, H, B, D), dtype=torch.bfloat16, device="cuda").normal_()
    dv = torch.empty_like(dk).normal_()
    hk = torch.empty((nb, H, B, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    desc = pk.CacheDesc.make(nb, B, H, D, "bf16")
    n = 4096
    perm = np.random.default_rng(9).permutation(nb).astype(np.int32)
    out_pairs = torch.from_numpy(np.ascontiguousarray(np.stack([perm[:n], perm[n:2 * n]], 1))).cuda()
    in_pairs = torch.from_numpy(np.ascontiguousarray(np.stack([perm[n:2 * n], perm[:n]], 1))).cuda()
    for _ in range(reps):
        pk.swap_blocks(hk, hv, dk, dv, out_pairs, desc)
    torch.cuda.synchronize()
    for _ in range(reps):
        pk.swap_blocks(dk, dv, hk, hv, in_pairs, desc)
    torch.cuda.synchronize()
    print(json.dumps({"swap_blocks": n, "bytes_per_direction_per_launch": 2 * n * H * B * D * 2,
                      "launches_out_then_in": reps}))


def prefill_only(dtype: str = "bf16", reps: int = 20, warm: int = 50, prompts=None):
    """The prefill kernel alone on the 8 prompt sequences of the 13B-shaped mixed step (or the
    given prompt lengths; 40 heads, head_dim 128, B=16, no cached prefix) in the given pool dtype:
    ``warm`` untimed launches (clock ramp), then ``reps`` timed ones; median duration and MFMA
    utilisation."""
    import torch
    from paged_kv_cache_323_amd import native as pk
    from paged_kv_cache_323_amd import runner as R
    from workloads import make_ragged_workload, make_workload
    pre = list(prompts) if prompts else [q for q in make_workload("mixed", "full").q_lens if q > 1]
    w = make_ragged_workload(5, pre, pre, 40, 40, 128, dtype, 16, name=f"prefill{len(pre)}-{dtype}")
    st = R.play_script(w, threads=16)
    q = R.to_device(w.queries(), w.dtype)
    out = torch.empty_like(q)
    tables, lens = st.bm.block_tables(w.query_seqs, w.max_blocks_per_seq())
    bt, cl = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    cu = torch.from_numpy(w.cu_seqlens()).cuda()
    mx = int(lens.max())
    ws = torch.zeros(max(pk.ragged_workspace_bytes(len(lens), q.shape[0], w.num_q_heads, mx, mx, st.desc), 1),
                     dtype=torch.uint8, device="cuda")
    med, _ = _time_events(lambda: pk.paged_attention_ragged(out, q, cu, cl, st.k_cache, st.v_cache, bt, w.scale,
                                                            mx, mx, st.desc, ws, min_q_len=min(pre)),
                          reps=reps, warm=warm)
    flops = prefill_flops(pre, pre, w.num_q_heads, w.head_dim)
    res = {"dtype": dtype, "prefill_rows": int(sum(pre)), "sequences": len(pre), "launches": reps + warm,
           "gflop_per_launch": round(flops / 1e9, 2), "median_us": round(med, 1),
           "tflops": round(flops / med / 1e6, 1), "mfma_util": round(flops / med / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
    del st
    torch.cuda.empty_cache()
    return res


def profile_prefill(dtype: str = "bf16", prompts: str = ""):
    """Profiling target for the prefill kernel (see prefill_only); prints one JSON line. prompts:
    "LENxCOUNT" (e.g. 8192x4) instead of the 13B-shaped step's prompts."""
    if prompts:
        n, c = (int(x) for x in prompts.lower().split("x"))
        print(json.dumps(prefill_only(dtype, reps=8, warm=5, prompts=[n] * c)))
    else:
        print(json.dumps(prefill_only(dtype)))


HOST_LINK_GBS = 64.0  # PCIe 5.0 x16 per direction, the swap path's link


def row_rooflines(result, extra, read_peak, copy_peak, copy_traffic=None):
    """Each hot-path row beside the ceiling that bounds it: achieved, ceiling, fraction. HBM rows
    are set against the 8 TB/s specification and the measured read (decode) or copy (write and
    copy kernels, read + write) ceiling; prefill against the bf16 MFMA peak; swap against the
    host link."""
    def hbm(achieved, measured):
        return {"achieved_gbs": round(achieved, 1), "frac_of_spec": round(achieved / HBM_PEAK_GBS, 4),
                "measured_ceiling_gbs": round(measured, 1), "frac_of_measured": round(achieved / measured, 4)}
    copy_traffic = copy_traffic or {}
    rows = {"a5_a6_decode_gqa": dict(hbm(result["roofline"]["achieved"], read_peak),
                                     kernel_us=result["roofline"]["kernel_avg_us"])}
    if "measured_gather_peak" in result["roofline"]:  # the same tiles read with no arithmetic
        rows["a5_a6_decode_gqa"]["gather_ceiling_gbs"] = result["roofline"]["measured_gather_peak"]
        rows["a5_a6_decode_gqa"]["frac_of_gather"] = result["roofline"]["frac_of_measured_gather_peak"]
    for key in ("llama7b", "gqa_B32", "gqa_B8"):
        e = extra.get(key, {})
        if "kv_gbs_partition_launch" in e:
            rows[f"a5_decode_{key}"] = hbm(e["kv_gbs_partition_launch"], read_peak)
    for shape, e in extra.get("head_shapes", {}).items():
        if isinstance(e, dict) and "kv_gbs" in e:  # partition launch + merge
            rows[f"a5_a6_decode_heads_{shape.replace('/', '_')}"] = dict(hbm(e["kv_gbs"], read_peak),
                                                                         partition=e["partition"])
    m = extra.get("mixed", {})
    if "kv_cache_write_gbs" in m:
        rows["a4_kv_cache_write"] = dict(hbm(m["kv_cache_write_gbs"], copy_peak), us=m["kv_cache_write_us"])
        if "kv_cache_write_cold_gbs" in m:
            rows["a4_kv_cache_write"]["cold_caches_gbs"] = m["kv_cache_write_cold_gbs"]
            rows["a4_kv_cache_write"]["cold_frac_of_measured"] = round(m["kv_cache_write_cold_gbs"] / copy_peak, 4)
        if "kv_cache_write_sequential_slots_gbs" in m:
            # the same write into consecutive slots: the kernel without the pool's scatter
            rows["a4_kv_cache_write"]["sequential_slots_gbs"] = m["kv_cache_write_sequential_slots_gbs"]
            rows["a4_kv_cache_write"]["sequential_frac_of_measured"] = round(
                m["kv_cache_write_sequential_slots_gbs"] / copy_peak, 4)
        if "kv_cache_write" in copy_traffic:
            rows["a4_kv_cache_write"]["traffic_over_algorithmic"] = copy_traffic["kv_cache_write"]
    if "prefill_tflops" in m:
        rows["a7_prefill"] = {"achieved_tflops": m["prefill_tflops"], "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "frac": m["prefill_mfma_util"], "us": m["prefill_only_us"]}
    if "attention_us" in m:
        rows["a7_mixed_step"] = {"step_us": m["step_us"], "seqs_per_s": m["seqs_per_s"]}
    for key, row in (("prefill_f16", "a7_prefill_f16"), ("prefill_long", "a7_prefill_long_prompts")):
        # the 13B prompts from an f16 pool (one f16 P operand), and 4 prompts of 8192 tokens (bf16)
        pf = extra.get(key, {})
        if "tflops" in pf:
            rows[row] = {"achieved_tflops": pf["tflops"], "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                         "frac": pf["mfma_util"], "us": pf["median_us"]}
    sp = extra.get("shared_prefix", {})
    if "copy_4096_pairs_gbs" in sp:
        rows["a3_copy_blocks_4096_pairs"] = hbm(sp["copy_4096_pairs_gbs"], copy_peak)
        if "copy_4096_sequential_pairs_gbs" in sp:
            # the same copy between consecutive blocks: the kernel without the pool's scatter
            rows["a3_copy_blocks_4096_pairs"]["sequential_pairs_gbs"] = sp["copy_4096_sequential_pairs_gbs"]
            rows["a3_copy_blocks_4096_pairs"]["sequential_frac_of_measured"] = round(
                sp["copy_4096_sequential_pairs_gbs"] / copy_peak, 4)
        if "copy_blocks" in copy_traffic:
            rows["a3_copy_blocks_4096_pairs"]["traffic_over_algorithmic"] = copy_traffic["copy_blocks"]
        rows["a3_copy_blocks_48_pairs"] = {"us": sp["copy_us"], "bound": "launch latency (24 MiB)"}
    tn = extra.get("tiny", {})
    if "step_us" in tn:
        rows["a4_a5_tiny_step"] = {"us": tn["step_us"], "decode_us": tn["decode_us"],
                                   "bound": "launch latency (315 KB of KV)"}
    sw = extra.get("swap", {})
    if "swap_out_gbs" in sw:
        rows["swap"] = {"out_gbs": sw["swap_out_gbs"], "in_gbs": sw["swap_in_gbs"], "link_gbs": HOST_LINK_GBS,
                        "frac_out": round(sw["swap_out_gbs"] / HOST_LINK_GBS, 4),
                        "frac_in": round(sw["swap_in_gbs"] / HOST_LINK_GBS, 4)}
        for key in ("swap_out", "swap_in"):
            if key in copy_traffic:
                rows["swap"][f"{key}_traffic_over_algorithmic"] = copy_traffic[key]
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--partition", type=int, default=0,
                    help="decode partition size in tokens (default: the library's choice)")
    ap.add_argument("--dense-grid", action="store_true",
                    help="time the dense partition grid (every sequence sized for the longest context) "
                         "instead of the host-built work list")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="only run the prefill kernel on the 13B-shaped step's prompts (profiling target)")
    ap.add_argument("--prefill-dtype", default="bf16", choices=("bf16", "f16"),
                    help="pool dtype of --profile-prefill")
    ap.add_argument("--prefill-prompts", default="",
                    help="LENxCOUNT prompts for --profile-prefill (default: the 13B-shaped step's)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="only run the copy kernel used to calibrate HBM byte counters")
    ap.add_argument("--profile-write", action="store_true",
                    help="only run the cache write of the 13B-shaped mixed step (counter target)")
    ap.add_argument("--layout-study", choices=("head", "token"), default=None,
                    help="GQA decode and cache write with the library PAGEDKV_LIB names, pools in this layout")
    ap.add_argument("--profile-swap", action="store_true",
                    help="only run swap-out then swap-in of 4096 blocks (counter target)")
    ap.add_argument("--profile-heads", default="",
                    help="only run one decode head shape QH/KVH/D (GQA lengths, bf16, B 16): two "
                         "event-timed 20-step windows (counter target)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path has no "
              f"multi-GPU sharding: one GPU runs one shard of the path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.profile_copy:
        profile_copy()
        return
    if args.layout_study:
        layout_study(args.layout_study)
        return
    if args.profile_write:
        profile_write()
        return
    if args.profile_swap:
        profile_swap()
        return
    if args.profile_prefill:
        profile_prefill(args.prefill_dtype, args.prefill_prompts)
        return
    if args.profile_heads:
        profile_heads(args.profile_heads)
        return
    h = run_headline(args)
    w = h["w"]
    log(f"decode kernel avg {h['kern_avg_us']:.1f} us (median {h['kern_med_us']:.1f}), "
        f"{h['achieved']:.0f} GB/s algorithmic, step {h['ms_per_step'] * 1e3:.1f} us")
    result = {
        "metric": "paged decode KV GB/s (% of HBM peak) and seqs/s per step; prefill MFMA util",
        "value": round(h["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"GQA decode step: 256 seqs, 32 q heads / 8 kv heads, head_dim 128, bf16, "
                               f"block_size {w.block_size}, lognormal ctx (median 1024, sigma 1.0, cap 8192), "
                               f"shuffled pool",
                   "seqs": len(w.query_seqs), "block_size": w.block_size,
                   "sum_ctx_first_step": int(sum(w.context_lens)) + len(w.context_lens),
                   "partition_tokens": h["partition"], "mean_ctx_timed": round(h["mean_ctx"], 1),
                   "split_seqs": h["split_seqs"],
                   "partition_launch": "dense grid" if args.dense_grid else "host-built work list"},
        "seqs_per_s": round(h["seqs_per_s"], 1),
        "kv_memory_utilisation": h["util"],
        "pct_hbm_peak_step": round(100 * h["kv_gbs"] / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(h["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(h["achieved"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_decode_kernel<bf16,128,4> (partition launch)",
                     "kernel_avg_us": round(h["kern_avg_us"], 2),
                     "kernel_timing": f"{B2B_LAUNCHES} launches back to back on the last step's inputs, "
                                      f"one event pair around them (after {B2B_WARM} untimed)",
                     "algorithmic_bytes_per_launch": int(h["alg_b2b"]),
                     # the same launches inside the steps, an event pair around each
                     "kernel_avg_us_event_pairs": round(h["kern_ev_avg_us"], 2),
                     "achieved_event_pairs": round(h["achieved_ev"], 1),
                     "algorithmic_bytes_per_launch_event_pairs": int(h["alg_per_launch"]),
                     "merge_launch_avg_us": round(h["merge_avg_us"], 2),
                     "back_to_back_launches": B2B_LAUNCHES, "back_to_back_warm": B2B_WARM},
    }
    tr = load_traffic(w.block_size)
    if tr is not None:
        # The counters' bytes over the algorithmic bytes of the profiled run (the same command's
        # launches), applied to this run's algorithmic bytes per launch.
        result["roofline"]["traffic"] = int(round(tr["ratio"] * h["alg_b2b"]))
        result["roofline"]["traffic_over_algorithmic"] = round(tr["ratio"], 4)
        result["roofline"]["traffic_profile_algorithmic_bytes"] = int(tr["profile_algorithmic_bytes"])
    result["windows"] = h["windows"]
    result["roofline"]["event_timed_launches"] = h["kern_launches"]
    log("streaming read and copy probes")
    read_peak = measured_read_peak()
    copy_peak = measured_copy_peak()
    # Measured ceilings beside the specification: decode is read-bound, so the read probe is its
    # attainable rate; the copy (read + write) probe is the one copy_blocks and swap face.
    result["roofline"]["measured_read_peak"] = round(read_peak, 1)
    result["roofline"]["frac_of_measured_read_peak"] = round(h["achieved"] / read_peak, 4)
    result["roofline"]["measured_copy_peak"] = round(copy_peak, 1)
    # The decode kernel's own access pattern (whole K then V tiles gathered through the tables)
    # without its arithmetic: the attainable rate for this layout and block size.
    gather_peak = measured_gather_peak(h["loop"])
    if gather_peak:
        result["roofline"]["measured_gather_peak"] = round(gather_peak, 1)
        result["roofline"]["frac_of_measured_gather_peak"] = round(h["achieved"] / gather_peak, 4)
    if not args.no_extra:
        extra = {}
        for key, fn in (("head_shapes", run_head_shapes),
                        ("gqa_partition_1024", lambda: run_decode_config("gqa", partition=1024)),
                        ("gqa_partition_512", lambda: run_decode_config("gqa", partition=512)),
                        ("gqa_B32", lambda: run_decode_config("gqa", 32)),
                        ("gqa_B8", lambda: run_decode_config("gqa", 8)),
                        ("llama7b", lambda: run_decode_config("llama7b")),
                        ("tiny", run_tiny),
                        ("shared_prefix", run_shared_prefix),
                        ("swap", run_swap),
                        ("engine", run_engine),
                        ("mixed", run_mixed),
                        ("prefill_f16", lambda: prefill_only("f16")),
                        ("prefill_long", lambda: prefill_only("bf16", reps=10, warm=10, prompts=[8192] * 4))):
            log(f"extra: {key}")
            try:
                extra[key] = fn()
            except Exception as e:  # keep the headline line even if a side measurement fails
                extra[key] = {"error": repr(e)}
        result["extra"] = extra
        result["rows"] = row_rooflines(result, extra, read_peak, copy_peak, load_copy_traffic())
    if not args.no_cpu:
        log("timing the oracle on the host CPU")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
