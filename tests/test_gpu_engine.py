"""Multi-step continuous batching through the library: requests join and leave every step,
prompts and decodes share each ragged call, and preemption swaps whole requests to the host pool
and back. Selected steps are replayed through the oracle from the engine's own op log."""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,B,host", [("bf16", 16, 64), ("f16", 8, 0)])
def test_engine_steps_match_oracle(dt, B, host):
    from paged_kv_cache_323_amd.engine import Engine
    rng = np.random.default_rng(7)
    # a pool too small for all requests at once, so admission waits and (with a host pool) swaps
    eng = Engine(num_blocks=28 if host else 200, block_size=B, num_q_heads=4, num_kv_heads=2, head_dim=128,
                 dtype=dt, max_num_seqs=6, max_step_tokens=400, num_host_blocks=host, seed=11, keep_outputs=True)
    for _ in range(14):
        eng.add_request(int(rng.integers(20, 150)), int(rng.integers(3, 25)))
    print(f"[case] engine {dt} B={B} host={host}", flush=True)
    sys.stdout.flush()
    steps = 0
    while eng.has_work() and steps < 200:
        eng.step()
        steps += 1
    print(f"  steps {steps}, stats {eng.stats}", flush=True)
    assert not eng.has_work(), "engine did not drain"
    assert eng.stats.finished == 14
    if host:
        assert eng.stats.preemptions > 0 and eng.stats.resumptions == eng.stats.preemptions
    # replay a spread of steps through the oracle
    picks = sorted(set([0, 1, len(eng.records) // 3, len(eng.records) // 2, len(eng.records) - 1] +
                       [i for i, r in enumerate(eng.records) if any(q > 1 for q in r.q_lens)][:4]))
    for i in picks:
        rec = eng.records[i]
        w = eng.replay_workload(rec)
        _, ref = oracle.run_workload(w)
        got = rec.out.cpu().numpy().astype(np.float64)
        err = float(np.max(np.abs(got - ref)))
        assert err <= 2e-3, (i, err)
