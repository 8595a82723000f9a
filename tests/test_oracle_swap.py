"""Pins for the oracle's block swapping (CPU only).

* The pages' claims: a preempted sequence's KV goes to host memory and comes
  back later, moved block by block, not as one contiguous buffer ("vLLM：把
  KV 缓存当成虚拟内存", section "碎片从哪里来"); an allocator that frees a block
  still in use lets a live sequence read reclaimed memory (same page, the
  accounting paragraph) -- so shared blocks must survive a swap-out.
* A content model: token ids stand in for K/V, written through the returned
  slots and moved through the returned copies (``kvcache.swap_blocks`` and
  ``copy_blocks``); every sequence on the device must read its own tokens
  back through its table after every operation, and a swapped sequence after
  it comes back.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import OracleAllocator, OracleError
from oracle.kvcache import copy_blocks, swap_blocks


class Pools:
    """Token ids per slot on the device and on the host."""

    def __init__(self, a: OracleAllocator, num_host_blocks: int):
        self.a = a
        self.dev = np.full((a.num_blocks, a.block_size), -1, dtype=np.int64)
        self.host = np.full((num_host_blocks, a.block_size), -1, dtype=np.int64)

    def write(self, slots, pair, ids):
        bs = self.a.block_size
        if pair is not None:
            copy_blocks(self.dev, [pair])
        for s, t in zip(slots, ids):
            self.dev[s // bs, s % bs] = t

    def out(self, pairs):
        swap_blocks(self.dev, self.host, pairs)

    def back(self, pairs):
        swap_blocks(self.host, self.dev, pairs)

    def check(self, toks):
        a, bs = self.a, self.a.block_size
        a.check_invariants()
        for s, want in toks.items():
            assert a.lens[s] == len(want)
            if s in a.swapped:
                got = []
                for p in range(len(want)):
                    on_host, i = a.swapped[s][p // bs]
                    got.append(int((self.host if on_host else self.dev)[i, p % bs]))
            else:
                t = a.tables[s]
                got = [int(self.dev[t[p // bs], p % bs]) for p in range(len(want))]
            assert got == list(want), f"sequence {s} reads other tokens"


def test_swap_out_frees_private_blocks_and_keeps_shared_ones():
    a = OracleAllocator(16, 4)
    a.enable_swap(8)
    pools = Pools(a, 8)
    s = a.create()
    ids = list(range(100, 118))                       # 18 tokens: 5 blocks, last partial
    slots, pair = a.append(s, len(ids))
    pools.write(slots, pair, ids)
    c = a.share_prefix(s, 8)                          # blocks 0-1 shared
    free_before = len(a.free)
    table = list(a.tables[s])
    pairs = a.swap_out(s)
    pools.out(pairs)
    assert [d for d, _ in pairs] == table[2:]          # the private blocks, in logical order
    assert len(pairs) == 3 and [h for _, h in pairs] == [0, 1, 2]
    assert len(a.free) == free_before + 3 and len(a.host_free) == 5
    shared = [i for on_host, i in a.swapped[s] if not on_host]
    assert len(shared) == 2 and all(a.refcount[b] == 2 for b in shared)
    pools.check({s: ids, c: ids[:8]})
    # the freed blocks are reused and overwritten by another sequence
    o = a.create()
    slots, pair = a.append(o, 12)
    pools.write(slots, pair, [7] * 12)
    pools.check({s: ids, c: ids[:8], o: [7] * 12})
    back = a.swap_in(s)
    pools.back(back)
    assert [h for h, _ in back] == [0, 1, 2] and len(a.host_free) == 8
    assert a.tables[s][:2] == a.tables[c][:2]         # still shared
    pools.check({s: ids, c: ids[:8], o: [7] * 12})
    # decode continues after the swap-in
    slots, pair = a.append(s, 3)
    pools.write(slots, pair, [1, 2, 3])
    pools.check({s: ids + [1, 2, 3], c: ids[:8], o: [7] * 12})


def test_a_swapped_sequence_is_not_contiguous_after_coming_back():
    """Blocks move one by one: the sequence comes back into whatever blocks
    are free, in any order."""
    a = OracleAllocator(8, 2, [7, 6, 5, 4, 3, 2, 1, 0])
    a.enable_swap(4)
    pools = Pools(a, 4)
    s = a.create()
    slots, _ = a.append(s, 6)
    pools.write(slots, None, [1, 2, 3, 4, 5, 6])
    before = list(a.tables[s])
    pools.out(a.swap_out(s))
    x = a.create()
    a.append(x, 3)                                    # takes two of the released blocks
    pools.back(a.swap_in(s))
    assert a.tables[s] != before
    pools.check({s: [1, 2, 3, 4, 5, 6]})


def test_all_or_nothing_and_errors():
    a = OracleAllocator(6, 2)
    with pytest.raises(OracleError) as e:
        a.swap_out(0)
    assert e.value.code == "ARG"                      # swap is off
    a.enable_swap(2)
    with pytest.raises(OracleError):
        a.enable_swap(2)
    s = a.create()
    a.append(s, 6)                                    # 3 private blocks, 2 host blocks
    snap = a.snapshot()
    with pytest.raises(OracleError) as e:
        a.swap_out(s)
    assert e.value.code == "OOM" and a.snapshot() == snap and len(a.host_free) == 2
    t = a.create()
    a.append(t, 4)
    pools_pairs = a.swap_out(t)
    assert len(pools_pairs) == 2
    for op in (lambda: a.append(t, 1), lambda: a.fork(t), lambda: a.share_prefix(t, 1),
               lambda: a.build_tables([t], 4), lambda: a.swap_out(t)):
        with pytest.raises(OracleError) as e:
            op()
        assert e.value.code == "SWAPPED"
    with pytest.raises(OracleError) as e:
        a.swap_in(s)                                  # not swapped out
    assert e.value.code == "ARG"
    with pytest.raises(OracleError) as e:
        a.swap_in(99)
    assert e.value.code == "NOT_FOUND"
    u = a.create()
    a.append(u, 6)                                    # takes the 2 freed + 1
    with pytest.raises(OracleError) as e:
        a.swap_in(t)                                  # needs 2, 0 free
    assert e.value.code == "OOM" and t in a.swapped
    a.free_seq(t)                                     # a swapped sequence can be freed
    assert len(a.host_free) == 2 and t not in a.swapped
    a.check_invariants()


def test_cached_blocks_swapped_out_stay_hittable():
    a = OracleAllocator(12, 4)
    a.enable_prefix_cache()
    a.enable_swap(8)
    pools = Pools(a, 8)
    prompt = list(range(1, 10))
    s, _ = a.create_prefix(prompt)
    slots, pair = a.append_tokens(s, prompt)
    pools.write(slots, pair, prompt)
    pools.out(a.swap_out(s))                          # its 2 full blocks are cached: evictable
    assert len(a.lru) == 2
    r, hit = a.create_prefix(prompt[:8] + [50])
    assert hit == 8
    slots, pair = a.append_tokens(r, [50])
    pools.write(slots, pair, [50])
    pools.back(a.swap_in(s))
    pools.check({s: prompt, r: prompt[:8] + [50]})
    assert a.tables[s][:2] != a.tables[r][:2]         # the swapped-in copies are private


ops = st.lists(st.tuples(st.sampled_from(["new", "append", "append", "fork", "share", "free",
                                          "out", "out", "in", "in", "serve"]),
                         st.integers(0, 1 << 30)), min_size=1, max_size=50)


@settings(max_examples=200, deadline=None)
@given(ops=ops, bs=st.sampled_from([1, 2, 4]), nb=st.integers(4, 30), nh=st.integers(1, 20),
       cache=st.booleans())
def test_random_operations_keep_contents_and_invariants(ops, bs, nb, nh, cache):
    a = OracleAllocator(nb, bs)
    if cache:
        a.enable_prefix_cache()
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
            elif op == "serve" and cache:
                prompt = [int(x) for x in rng.integers(0, 2, rng.integers(1, 10))]
                s, hit = a.create_prefix(prompt)
                toks[s] = prompt[:hit]
                slots, pair = a.append_tokens(s, prompt[hit:])
                pools.write(slots, pair, prompt[hit:])
                toks[s] = prompt
            elif op == "append" and pick is not None:
                ids = [int(x) for x in rng.integers(0, 2, rng.integers(1, 5))]
                slots, pair = (a.append_tokens(pick, ids) if cache else a.append(pick, len(ids)))
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
            elif op == "out" and pick is not None:
                resident = [x for x in live if x in a.tables] or [pick]
                pools.out(a.swap_out(resident[r % len(resident)]))
            elif op == "in" and pick is not None:
                away = [x for x in live if x in a.swapped] or [pick]
                pools.back(a.swap_in(away[r % len(away)]))
        except OracleError as e:
            assert e.code in ("OOM", "SWAPPED", "ARG"), e
            if e.code == "ARG":
                assert op == "in" and pick in a.tables
            for s in list(toks):
                if s not in a.tables and s not in a.swapped:
                    del toks[s]
        pools.check(toks)
    for s in list(toks):
        a.free_seq(s)
    a.check_invariants()
    assert sorted(a.host_free) == list(range(nh))
    assert sorted(list(a.free) + list(a.lru)) == list(range(nb))
