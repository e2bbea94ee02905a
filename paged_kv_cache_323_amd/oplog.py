"""The engine's operation log: one record per block-manager operation, in the order they ran.

Plain records, no behaviour. A log can be replayed by anything that understands the six
operation kinds by name (add, append, fork, free, swap out, swap in): the library's own script
runner, or a reference implementation in a test.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List


@dataclass
class AddOp:
    seq: int


@dataclass
class AppendOp:
    seqs: List[int]
    n_tokens: List[int]
    tag: int  # identifies the values appended (the engine's step number plus an offset)


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
