"""Benchmark of the paged-KV hot path on one MI355X.

A *step* is one decode iteration of the GQA configuration (256 sequences, 32 query heads over 8
KV heads, head_dim 128, bf16, block size 16, lognormal context lengths with median 1024 capped
at 8192, physical blocks in a seeded random order):

  1. host block manager: append one token to every sequence -> slots, copy-on-write pairs,
     block tables (C++ inside libpagedkv.so);
  2. one pinned-memory upload of slots, context lengths and block tables;
  3. copy_blocks for any copy-on-write pairs (none in this workload);
  4. kv_cache_write of the 256 new tokens;
  5. paged decode attention of the 256 query rows over their whole contexts.

Inputs are resident in HBM before timing starts. The JSON line reports whole-step throughput
(KV bytes read by attention per second, and sequences per second), the decode kernel against
the HBM roofline (timed with HIP events on the launch stream), the oracle timed on this host's
CPU on a bounded sample, and secondary measurements of the other workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--block-size 16] [--no-extra]
"""
from __future__ import annotations

import argparse
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


class DecodeLoop:
    """Steady-state decode steps over a resident workload (state advances every step)."""

    def __init__(self, w, steps_total, device="cuda"):
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
        # one pinned staging area per parity of the step: [slots S | ctx S | tables S*MB]
        n = 2 * self.S + self.S * self.max_blocks
        self.host = [torch.empty(n, dtype=torch.int32).pin_memory() for _ in range(2)]
        self.host_np = [h.numpy() for h in self.host]
        self.uploaded = [None, None]
        self.dev = torch.empty(n, dtype=torch.int32, device=device)
        self.slots_d = self.dev[: self.S]
        self.ctx_d = self.dev[self.S: 2 * self.S]
        self.tab_d = self.dev[2 * self.S:].view(self.S, self.max_blocks)
        self.q = R.to_device(w.queries(), w.dtype, device)
        # new-token K/V for the steps (fixed values; only their placement changes per step)
        r = np.random.default_rng([w.seed, 77])
        from workloads import round_to_dtype
        kv = round_to_dtype(r.standard_normal((2, self.S, w.num_kv_heads, w.head_dim), dtype=np.float32), w.dtype)
        self.k_new = R.to_device(kv[0], w.dtype, device)
        self.v_new = R.to_device(kv[1], w.dtype, device)
        self.out = torch.empty_like(self.q)  # pool dtype output, as a serving engine consumes it
        nbytes = pk.decode_workspace_bytes(self.S, w.num_q_heads, self.max_ctx_final, self.st.desc)
        self.ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.partition = pk.decode_partition_size(self.S, w.num_q_heads, self.max_ctx_final, self.st.desc)
        self.step_idx = 0
        self.ctx_history = []
        self.pairs_total = 0

    def step(self, ev=None):
        torch, pk, w = self.torch, self.pk, self.w
        buf = self.step_idx & 1
        if self.uploaded[buf] is not None:
            self.uploaded[buf].synchronize()       # the H2D that last read this buffer is done
        hn = self.host_np[buf]
        slots, pairs = self.st.bm.append(self.seqs, np.ones(self.S, dtype=np.int32))
        hn[: self.S] = slots
        tab = hn[2 * self.S:].reshape(self.S, self.max_blocks)
        self.st.bm.block_tables(self.seqs, self.max_blocks, out=tab, ctx_out=hn[self.S: 2 * self.S])
        self.dev.copy_(self.host[buf], non_blocking=True)
        e = torch.cuda.Event()
        e.record()
        self.uploaded[buf] = e
        if len(pairs):
            self.pairs_total += len(pairs)
            pk.copy_blocks(self.st.k_cache, self.st.v_cache,
                           torch.from_numpy(np.ascontiguousarray(pairs)).to("cuda", non_blocking=False), self.st.desc)
        pk.kv_cache_write(self.k_new, self.v_new, self.st.k_cache, self.st.v_cache, self.slots_d, self.st.desc)
        args = (self.out, self.q, self.st.k_cache, self.st.v_cache, self.tab_d, self.ctx_d, w.scale,
                self.max_ctx_final, self.st.desc, self.ws)
        if ev is not None:
            ev[0].record()
        pk.paged_attention_decode(*args, stage="partitions")
        if ev is not None:
            ev[1].record()
        pk.paged_attention_decode(*args, stage="merge")
        if ev is not None:
            ev[2].record()
        self.ctx_history.append(hn[self.S: 2 * self.S].copy())
        self.step_idx += 1


def run_headline(args):
    import torch
    from workloads import make_workload
    w = make_workload("gqa", "full", block_size=args.block_size)
    ramp_max = 100
    loop = DecodeLoop(w, args.warmup + args.steps + ramp_max)
    for _ in range(args.warmup):
        loop.step()
    torch.cuda.synchronize()
    # keep the GPU busy for a moment so clocks have ramped before the timed steps
    t_ramp = time.perf_counter()
    for _ in range(ramp_max):
        if time.perf_counter() - t_ramp > 0.1:
            break
        loop.step()
        torch.cuda.synchronize()
    loop.ctx_history.clear()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        loop.step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    kern_ms = [a.elapsed_time(b) for a, b, _ in evs]
    merge_ms = [b.elapsed_time(c) for _, b, c in evs]
    kv_total = 0
    alg_total = 0
    for ctx in loop.ctx_history:
        kv, alg = decode_algorithmic_bytes(ctx, w, 2)
        kv_total += kv
        alg_total += alg
    K = args.steps
    ms_per_step = elapsed / K * 1e3
    kv_per_step = kv_total / K
    alg_per_launch = alg_total / K
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    achieved = alg_per_launch / kern_avg_s / 1e9
    return dict(
        w=w, loop=loop, ms_per_step=ms_per_step, seqs_per_s=len(w.query_seqs) / (elapsed / K),
        kv_gbs=kv_per_step / (elapsed / K) / 1e9, kern_avg_us=kern_avg_s * 1e6, kern_med_us=float(np.median(kern_ms)) * 1e3,
        achieved=achieved, alg_per_launch=alg_per_launch, kv_per_step=kv_per_step,
        kern_kv_gbs=kv_per_step / kern_avg_s / 1e9, partition=loop.partition,
        mean_ctx=float(np.mean([c.mean() for c in loop.ctx_history])),
        merge_avg_us=float(np.mean(merge_ms)) * 1e3)


def cpu_baseline(w, budget_s=20.0):
    """The oracle (float64 NumPy, single BLAS thread) on a bounded sample of the workload."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle
    rng = np.random.default_rng(11)
    order = rng.permutation(len(w.query_seqs))
    sample = sorted(order[:32].tolist())
    seqs = [w.query_seqs[i] for i in sample]
    st, _ = oracle.run_workload(w, only_seqs=seqs, attend=False)
    tables, lens = st.bm.padded_tables(seqs, w.max_blocks_per_seq())
    q = w.queries(seqs)
    cu = np.arange(len(seqs) + 1, dtype=np.int32)
    ctx_ctl = threadpool_limits(1) if threadpool_limits else None
    times = []
    try:
        for _ in range(3):
            t = time.perf_counter()
            oracle.paged_ragged(q, cu, lens, tables, st.pool_k, st.pool_v, w.scale, w.block_size, w.dtype)
            times.append(time.perf_counter() - t)
            if sum(times) > budget_s:
                break
    finally:
        if ctx_ctl is not None:
            ctx_ctl.__exit__(None, None, None)
    dt = float(np.median(times))
    kv = int(np.sum(lens)) * w.kv_bytes_per_token()
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seqs_per_s": len(seqs) / dt,
            "sample": f"{len(seqs)} of {len(w.query_seqs)} sequences of {w.name} (seeded pick), "
                      f"sum ctx {int(np.sum(lens))}, median of {len(times)} runs, 1 BLAS thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path has no "
              f"multi-GPU sharding in this build)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
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
                   "partition_tokens": h["partition"], "mean_ctx_timed": round(h["mean_ctx"], 1)},
        "seqs_per_s": round(h["seqs_per_s"], 1),
        "pct_hbm_peak_step": round(100 * h["kv_gbs"] / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(h["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(h["achieved"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_decode_kernel<bf16,128,4> (partition launch)",
                     "kernel_avg_us": round(h["kern_avg_us"], 2),
                     "merge_launch_avg_us": round(h["merge_avg_us"], 2),
                     "algorithmic_bytes_per_launch": int(h["alg_per_launch"])},
    }
    if not args.no_cpu:
        log("timing the oracle on the host CPU")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
