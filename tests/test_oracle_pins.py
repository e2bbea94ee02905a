"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle_pins as P
from workloads import make_workload

SMALL = ["tiny", "llama7b", "gqa", "shared_prefix", "mixed"]


@pytest.mark.parametrize("name", SMALL)
def test_oracle_matches_sdpa(name):
    P.pin_sdpa(make_workload(name, "small"))


def test_oracle_matches_sdpa_gqa_b32():
    P.pin_sdpa(make_workload("gqa", "small", block_size=32))


@pytest.mark.parametrize("name", ["tiny", "gqa", "shared_prefix", "mixed"])
def test_oracle_matches_blockwise_equation(name):
    w = make_workload(name, "small")
    if name == "mixed":       # keep the literal per-row evaluation small
        from workloads.synth import Workload  # noqa: F401
    P.pin_blockwise_equation(w)


@pytest.mark.parametrize("name", SMALL)
def test_oracle_permutation_invariant(name):
    P.pin_permutation_invariance(make_workload(name, "small"))


def test_oracle_brute_force_tiny():
    P.pin_brute_force(make_workload("tiny"))


def test_oracle_brute_force_mixed_rows():
    P.pin_brute_force(make_workload("mixed", "small"), max_rows=40)


def test_oracle_paged_decode_gqa():
    P.pin_paged_decode_gqa()


def test_oracle_closed_forms():
    P.pin_closed_forms()


def test_block_manager_cow_trace():
    P.pin_cow_trace()


def test_block_manager_swap_trace():
    P.pin_swap_trace()


def test_block_manager_fragmentation():
    P.pin_fragmentation()


def test_block_manager_parallel_sampling():
    P.pin_parallel_sampling()


def test_cow_contents():
    P.pin_cow_contents()


def test_block_manager_invariants():
    P.pin_invariants()


def test_block_manager_swap_invariants():
    P.pin_invariants(swap=True, seeds=range(10))


def test_shared_prefix_small_pairs():
    """⌊L/B⌋ shared blocks and n-1 copies per request appear in the config's own script."""
    import oracle
    w = make_workload("shared_prefix", "small")
    st, _ = oracle.run_workload(w, attend=False)
    n_req = len(w.query_seqs) // 4
    assert len(st.pairs_per_append[-2]) == n_req * 3


@pytest.mark.parametrize("seed", range(3))
def test_oracle_matches_sdpa_on_churn(seed):
    """Beam-search-like fork/append/free churn: the paged oracle still equals SDPA over each
    live sequence's contiguous history."""
    from workloads import make_churn_workload
    P.pin_sdpa(make_churn_workload(seed, 8, 4, 2, 64, "f16"))


@pytest.mark.parametrize("seed,B", [(0, 8), (1, 16), (2, 32)])
def test_oracle_swap_round_trip(seed, B):
    """Swapping groups out to the host pool and back (with their GPU blocks reused meanwhile)
    leaves every attention output bit-identical to the same script without swaps, and SDPA
    over the contiguous histories still agrees."""
    import dataclasses
    import numpy as np
    import oracle
    from workloads import make_swap_workload
    w = make_swap_workload(seed, B, 4, 2, 64, "bf16")
    _, out = oracle.run_workload(w)
    twin = dataclasses.replace(w, ops=[op for op in w.ops if type(op).__name__ not in ("SwapOutOp", "SwapInOp")])
    _, out2 = oracle.run_workload(twin)
    assert np.array_equal(out, out2)
    P.pin_sdpa(w)
