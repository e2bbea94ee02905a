"""Planted mistakes in the oracle (on the CPU) must trip at least one pin.

Each case rewrites one line of an oracle module's source, loads the altered
module and swaps its functions into the oracle package for the duration of the
test, then runs the pins that cover that part. A pin suite that lets a plausible
slip through would make the oracle untrustworthy as a parity reference.
"""
import importlib
import inspect
import types

import pytest

import oracle
import oracle.attention
import oracle.block_manager
import oracle.pool
import oracle.run
import oracle_pins as P
from workloads import make_workload


def _load_mutant(module, old, new, count=None):
    src = inspect.getsource(module)
    assert old in src, f"mutation anchor not found in {module.__name__}: {old!r}"
    src = src.replace(old, new) if count is None else src.replace(old, new, count)
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = module.__file__
    exec(compile(src, module.__file__, "exec"), mod.__dict__)
    return mod


def _install(monkeypatch, module, mutant):
    """Point every binding of the module's public names at the mutant's versions."""
    names = [n for n, v in vars(module).items()
             if (inspect.isfunction(v) or inspect.isclass(v)) and getattr(v, "__module__", "") == module.__name__]
    for n in names:
        orig, new = getattr(module, n), getattr(mutant, n)
        for holder in (module, oracle, oracle.run, oracle.attention, oracle.pool, oracle.block_manager):
            if getattr(holder, n, None) is orig:
                monkeypatch.setattr(holder, n, new)
    # exceptions must stay the real class so pins can catch them
    if hasattr(mutant, "NoFreeBlocks"):
        mutant.NoFreeBlocks = oracle.NoFreeBlocks


def _attention_pins():
    P.pin_closed_forms()
    P.pin_paged_decode_gqa()
    for name in ("tiny", "gqa", "mixed", "shared_prefix"):
        P.pin_sdpa(make_workload(name, "small"))


def _bm_pins():
    P.pin_cow_trace()
    P.pin_fragmentation()
    P.pin_parallel_sampling()
    P.pin_invariants()
    P.pin_sdpa(make_workload("shared_prefix", "small"))


def _swap_pins():
    P.pin_swap_trace()
    P.pin_invariants(swap=True, seeds=range(10))


def _pool_pins():
    P.pin_cow_contents()
    P.pin_sdpa(make_workload("shared_prefix", "small"))
    P.pin_sdpa(make_workload("tiny"))


MUTANTS = [
    # attention
    ("attention", "kh = h // g", "kh = h % hkv", _attention_pins),
    ("attention", "logits = scale * (q @ k.T)", "logits = (q @ k.T)", _attention_pins),
    # the single-query entry point alone (the anchors exist only in paged_decode)
    ("attention", "            kh = h // g\n            out[s, h] = softmax_attention(qs[h:h + 1]",
     "            kh = h % hkv\n            out[s, h] = softmax_attention(qs[h:h + 1]", _attention_pins),
    ("attention", "softmax_attention(qs[h:h + 1], K[:, kh], V[:, kh], scale)",
     "softmax_attention(qs[kh:kh + 1], K[:, kh], V[:, kh], scale)", _attention_pins),
    ("attention", "        if ctx == 0:\n            continue\n        K = upcast(gather_kv(pool_k, block_tables[s], ctx, block_size), dtype)\n        V = upcast(gather_kv(pool_v, block_tables[s], ctx, block_size), dtype)\n        qs = upcast(q[s], dtype)",
     "        if ctx == 0:\n            continue\n        K = upcast(gather_kv(pool_k, block_tables[s], ctx - 1, block_size), dtype)\n        V = upcast(gather_kv(pool_v, block_tables[s], ctx - 1, block_size), dtype)\n        qs = upcast(q[s], dtype)",
     _attention_pins),
    ("attention", "phys = int(table[p // block_size])", "phys = int(table[p % block_size])", _attention_pins),
    ("attention", "rows.append(pool[phys, p % block_size])",
     "rows.append(pool[phys, (p + 1) % block_size])", _attention_pins),
    ("attention", "limits = [ctx - ql + t + 1 for t in range(ql)]",
     "limits = [ctx - ql + t for t in range(ql)]", _attention_pins),
    ("attention", "w = np.exp(logits - logits.max(axis=1, keepdims=True))", "w = np.exp(logits)",
     _attention_pins),
    ("attention", "out[live] = (w / w.sum(axis=1, keepdims=True)) @ v", "out[live] = w @ v", _attention_pins),
    ("attention", "<< np.uint32(16)", "<< np.uint32(15)", _attention_pins),
    ("attention", "V = upcast(gather_kv(pool_v", "V = upcast(gather_kv(pool_k", _attention_pins),
    ("attention", "logits = scale * (q @ k.T)", "logits = scale * (q @ k.T).T.T[:, ::-1]", _attention_pins),
    # block manager
    ("block_manager", "            self.rc[old] -= 1 ", "            pass; ", _bm_pins),
    ("block_manager", "elif self.rc[table[j]] > 1:", "elif self.rc[table[j]] >= 1:", _bm_pins),
    ("block_manager", "                free.append(b)\n        del self.lens[seq]", "                free.appendleft(b)\n        del self.lens[seq]", _bm_pins),
    ("block_manager", "            self.rc[b] += 1", "            pass", _bm_pins),
    ("block_manager", "self.free, self.rc, self.tables, self.lens = saved", "pass", _bm_pins),
    ("block_manager", "b = self.free.popleft()", "b = self.free.pop()", _bm_pins),
    # swap
    ("block_manager", "            src_rc[b] -= refs[b]", "            src_rc[b] = 0", _swap_pins),
    ("block_manager", "            dst_rc[nb] = refs[b]", "            dst_rc[nb] = 1", _swap_pins),
    ("block_manager", "        if len(order) > len(dst_free):", "        if len(order) > len(dst_free) + 1:", _swap_pins),
    # pool
    ("pool", "pool_v[int(dst)] = pool_v[int(src)]", "pass", _pool_pins),
    ("pool", "b, o = divmod(s, B)", "o, b = divmod(s, B)", _pool_pins),
    ("pool", "pool_k[b, o] = k[t]", "pool_k[b, o] = v[t]", _pool_pins),
]


@pytest.mark.parametrize("case", MUTANTS,
                         ids=lambda m: f"{m[0]}:{m[1][:40]}")
def test_pins_catch_planted_mistake(case, monkeypatch):
    modname, old, new, pins = case
    module = importlib.import_module(f"oracle.{modname}")
    mutant = _load_mutant(module, old, new)
    _install(monkeypatch, module, mutant)
    with pytest.raises(Exception):
        pins()


def test_unmutated_pins_pass():
    _attention_pins()
    _bm_pins()
    _pool_pins()
