"""Pins for the oracle allocator's sliding-window trimming (CPU only).

With a window of W positions the newest token and every later one attend
only positions >= len - W, so blocks wholly below that never need to stay
("vLLM：把 KV 缓存当成虚拟内存": sliding windows change how long K/V live).
Checked with a content model (token ids written through the returned slots;
every sequence must read back every position inside its window after every
operation), exact hole positions, pool accounting and invariants under
random operations that mix trims with forks, sharing, swaps and the prefix
cache.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import NO_BLOCK, OracleAllocator, OracleError
from oracle.kvcache import copy_blocks, swap_blocks


class Pools:
    def __init__(self, a, nh=1):
        self.a = a
        self.dev = np.full((a.num_blocks, a.block_size), -1, dtype=np.int64)
        self.host = np.full((max(nh, 1), a.block_size), -1, dtype=np.int64)

    def write(self, slots, pair, ids):
        bs = self.a.block_size
        if pair is not None:
            copy_blocks(self.dev, [pair])
        for s, t in zip(slots, ids):
            self.dev[s // bs, s % bs] = t

    def check(self, toks, window):
        a, bs = self.a, self.a.block_size
        a.check_invariants()
        for s, want in toks.items():
            assert a.lens[s] == len(want)
            if s in a.swapped:
                entries = a.swapped[s]
                where = [(self.host if h else self.dev, i) for h, i in entries]
            else:
                where = [(self.dev, b) for b in a.tables[s]]
            lo = max(len(want) - window, 0) if window else 0
            for p in range(lo, len(want)):
                pool, b = where[p // bs]
                assert b != NO_BLOCK, f"sequence {s}: position {p} inside the window was released"
                assert int(pool[b, p % bs]) == want[p]


def test_worked_trim():
    a = OracleAllocator(10, 4)
    pools = Pools(a)
    s = a.create()
    slots, _ = a.append(s, 17)                    # blocks 0..4, positions 0..16
    pools.write(slots, None, list(range(17)))
    table = list(a.tables[s])
    assert a.trim_window(s, 6) == 2               # positions < 11: blocks 0 and 1
    assert a.tables[s] == [NO_BLOCK, NO_BLOCK] + table[2:]
    assert list(a.free)[-2:] == table[:2]
    assert a.trim_window(s, 6) == 0               # nothing more
    pools.check({s: list(range(17))}, 6)
    slots, _ = a.append(s, 3)                     # len 20: positions < 14 dead -> block 2 too
    pools.write(slots, None, [17, 18, 19])
    assert a.trim_window(s, 6) == 1
    pools.check({s: list(range(20))}, 6)
    c = a.fork(s)                                 # holes are shared as holes
    assert a.tables[c][:3] == [NO_BLOCK] * 3
    with pytest.raises(OracleError):
        a.share_prefix(s, 5)                      # ends in a released block
    with pytest.raises(OracleError):
        a.share_prefix(s, 13)                     # includes released blocks
    d = a.fork(c)
    a.free_seq(s)
    a.free_seq(c)
    a.free_seq(d)
    assert sorted(a.free) == list(range(10))


def test_shared_blocks_stay_for_the_other_holder():
    a = OracleAllocator(8, 4)
    pools = Pools(a)
    s = a.create()
    slots, _ = a.append(s, 12)
    pools.write(slots, None, list(range(12)))
    c = a.fork(s)
    a.trim_window(s, 4)                           # s drops blocks 0, 1
    assert all(a.refcount[b] == 1 for b in a.tables[c][:2])
    pools.check({s: list(range(12))}, 4)
    pools.check({c: list(range(12))}, 0)          # c still reads all of it


ops = st.lists(st.tuples(st.sampled_from(["new", "append", "append", "append", "fork", "share",
                                          "free", "trim", "trim", "out", "in"]),
                         st.integers(0, 1 << 30)), min_size=1, max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4]), nb=st.integers(4, 40), window=st.integers(1, 12))
def test_random_operations_with_trims(ops, bs, nb, window):
    a = OracleAllocator(nb, bs)
    nh = 16
    a.enable_swap(nh)
    pools = Pools(a, nh)
    toks = {}
    for op, r in ops:
        rng = np.random.default_rng(r)
        live = sorted(toks)
        pick = live[r % len(live)] if live else None
        try:
            if op == "new":
                toks[a.create()] = []
            elif op == "append" and pick is not None:
                ids = [int(x) for x in rng.integers(0, 100, rng.integers(1, 6))]
                slots, pair = a.append(pick, len(ids))
                pools.write(slots, pair, ids)
                toks[pick] = toks[pick] + ids
            elif op == "fork" and pick is not None:
                toks[a.fork(pick)] = list(toks[pick])
            elif op == "share" and pick is not None:
                n = int(rng.integers(0, len(toks[pick]) + 1))
                toks[a.share_prefix(pick, n)] = toks[pick][:n]
            elif op == "free" and pick is not None:
                a.free_seq(pick)
                del toks[pick]
            elif op == "trim" and pick is not None:
                a.trim_window(pick, window)
            elif op == "out" and pick is not None:
                swap_blocks(pools.dev, pools.host, a.swap_out(pick))
            elif op == "in" and pick is not None:
                swap_blocks(pools.host, pools.dev, a.swap_in(pick))
        except OracleError as e:
            assert e.code in ("OOM", "SWAPPED", "ARG"), e
        # a sequence never trimmed still reads everything; trims respect the window
        pools.check(toks, window)
    for s in list(toks):
        a.free_seq(s)
    a.check_invariants()
    assert sorted(a.free) == list(range(nb))
