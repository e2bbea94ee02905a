"""Plain, slow, CPU reference implementation of the paged-KV hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
anything under ``oracle/``; only the tests, the smoke check and the benchmark's
CPU-baseline leg do. The oracle shares no code with the HIP library: it has its
own block manager, its own pool layout (token-major, deliberately different from
the device layout) and computes attention from the plain softmax definition in
float64 on exactly upcast input values.

Sources (titles of the pages this follows):
  * 「PagedAttention原理」 (scmmm.top): §为什么会有 KV cache (single-query softmax
    attention), §实现一个虚拟内存 (blocks K_j / V_j and the block-wise attention
    equation; block table of physical block + fill count), §解决COW (the five
    copy-on-write steps), §从虚拟内存的启发 (allocate one block at a time),
    §block_size 选取 (expected internal fragmentation (B-1)/2).
  * 「Paged Attention&Orca Paper笔记与解读」 (notion-next): §PagedAttention的方法
    items on parallel sampling (⌊L/B⌋ shared full prompt blocks, partial block
    copied per sample, fork only at the first generated token and none when L
    is a multiple of B) and beam search (reference counts, release at zero);
    §Orca的Solution on selective batching (ragged flattened batches, attention
    split per request and phase).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, a library routine, the page's block-wise equation, physical
permutation invariance, hand-traced copy-on-write fixtures and the
fragmentation expectation). ``paged_decode`` in particular is pinned with one,
two, four and eight query heads per KV head against torch's grouped-query
scaled_dot_product_attention over the contiguous histories, and against
``paged_ragged``; planted mistakes in its head mapping, query row and context
length trip those pins. No function is "parity unpinned".
"""
from .attention import (  # noqa: F401
    upcast,
    gather_kv,
    softmax_attention,
    paged_decode,
    paged_ragged,
)
from .block_manager import BlockManager, NoFreeBlocks, NotResident  # noqa: F401
from .pool import new_pool, write_slots, copy_blocks, copy_between  # noqa: F401
from .run import run_workload, OracleState  # noqa: F401
