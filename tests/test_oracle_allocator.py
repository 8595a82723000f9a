"""Pins for the oracle allocator and cache-write/copy (CPU only).

* the pages' worked examples (golden/allocator_examples.json);
* copy-on-write leaves the shared block's bytes untouched;
* random operation sequences keep refcount = in-degree, free <=> refcount 0,
  all-or-nothing OOM, and free-everything restores the pool;
* a contiguous per-sequence model: reading any live sequence back through its
  block table returns exactly the tokens that sequence (or the one it was
  forked or prefix-shared from) wrote, which is what paging must preserve.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import _golden
from oracle import OracleAllocator, OracleError
from oracle.kvcache import copy_blocks, write_slots


class OracleAdapter:
    def __init__(self, nb, bs, order):
        self.a = OracleAllocator(nb, bs, order)

    def create(self):
        return self.a.create()

    def append(self, s, n):
        return self.a.append(s, n)

    def fork(self, s):
        return self.a.fork(s)

    def share(self, s, n):
        return self.a.share_prefix(s, n)

    def free(self, s):
        self.a.free_seq(s)

    def table(self, s):
        return list(self.a.tables[s])

    def refcount(self, b):
        return self.a.refcount[b]

    def free_list(self):
        return list(self.a.free)


EXAMPLES = _golden.load("allocator_examples.json")


@pytest.mark.parametrize("name", [k for k in EXAMPLES if not k.startswith("_")])
def test_worked_examples(name):
    ad, _ = _golden.run_example(EXAMPLES[name], OracleAdapter)
    ad.a.check_invariants()


def test_cow_leaves_parent_block_untouched():
    """Four-score example with token ids as the cached values: after A1
    writes 'fathers', the shared block still reads years/ago/our/[empty] and
    the copy reads years/ago/our/fathers; A2 then writes 'mothers' in place."""
    ex = EXAMPLES["cow_four_score"]
    a = OracleAllocator(ex["num_blocks"], ex["block_size"], ex["initial_free_order"])
    pool = np.zeros((8, 1, 4, 1), dtype=np.uint32)  # one head, one "dim"
    words = {w: i + 1 for i, w in enumerate(
        "Four score and seven years ago our fathers mothers".split())}
    a1 = a.create()
    slots, _ = a.append(a1, 7)
    write_slots(pool, np.array([[[words[w]]] for w in
                                "Four score and seven years ago our".split()], np.uint32), slots)
    a2 = a.fork(a1)
    block1_before = pool[1].copy()
    slots, pair = a.append(a1, 1)
    copy_blocks(pool, [pair])
    write_slots(pool, np.array([[[words["fathers"]]]], np.uint32), slots)
    assert np.array_equal(pool[1], block1_before)
    assert list(pool[3, 0, :, 0]) == [words["years"], words["ago"], words["our"], words["fathers"]]
    slots, pair = a.append(a2, 1)
    assert pair is None
    write_slots(pool, np.array([[[words["mothers"]]]], np.uint32), slots)
    assert list(pool[1, 0, :, 0]) == [words["years"], words["ago"], words["our"], words["mothers"]]
    assert list(pool[3, 0, :, 0]) == [words["years"], words["ago"], words["our"], words["fathers"]]


def test_oom_is_all_or_nothing():
    a = OracleAllocator(4, 4, [3, 2, 1, 0])
    s = a.create()
    a.append(s, 6)            # blocks 3, 2 (block 2 half full)
    t = a.fork(s)             # both share 3 and 2
    a.append(t, 2)            # CoW of block 2 -> 1 ; free = [0]
    before = a.snapshot()
    with pytest.raises(OracleError) as e:
        a.append(s, 7)        # needs 2 new blocks, 1 free
    assert e.value.code == "OOM"
    assert a.snapshot() == before
    a.check_invariants()


def test_errors():
    a = OracleAllocator(8, 4)
    with pytest.raises(OracleError) as e:
        a.append(99, 1)
    assert e.value.code == "NOT_FOUND"
    s = a.create()
    a.append(s, 3)
    with pytest.raises(OracleError) as e:
        a.share_prefix(s, 4)
    assert e.value.code == "ARG"
    with pytest.raises(OracleError):
        OracleAllocator(4, 4, [0, 1, 2, 2])


def test_build_tables_padding():
    a = OracleAllocator(16, 4, list(range(15, -1, -1)))
    s0, s1 = a.create(), a.create()
    a.append(s0, 5)
    a.append(s1, 1)
    tables, lens = a.build_tables([s0, s1], 4)
    assert tables.tolist() == [[15, 14, -1, -1], [13, -1, -1, -1]]
    assert lens.tolist() == [5, 1]
    with pytest.raises(OracleError):
        a.build_tables([s0], 1)


# ------------------------------------------------------------ random operations

OPS = st.lists(
    st.tuples(st.sampled_from(["create", "append", "append", "append", "fork", "share", "free"]),
              st.integers(0, 1000), st.integers(0, 40)),
    min_size=1, max_size=50)


def run_random_ops(make, ops, nb=64, bs=4, seed=0, on_step=None):
    """Drive an allocator (oracle or native, through ``make``) with a random
    operation list while keeping a contiguous per-sequence model of token
    values.  Returns the adapter."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(nb).tolist()
    ad = make(nb, bs, order)
    pool = np.zeros((nb, 1, bs, 1), dtype=np.uint32)
    model = {}          # seq -> list of token values (contiguous view)
    next_val = [1]
    live = []
    for op, pick, n in ops:
        if op == "create" or not live:
            s = ad.create()
            live.append(s)
            model[s] = []
        elif op == "append":
            s = live[pick % len(live)]
            try:
                slots, pair = ad.append(s, n)
            except Exception as e:  # OOM leaves the state unchanged
                assert getattr(e, "code", None) in ("OOM", -4), e
                slots = None
            if slots is not None:
                if pair is not None:
                    copy_blocks(pool, [pair])
                vals = np.arange(next_val[0], next_val[0] + len(slots), dtype=np.uint32)
                next_val[0] += len(slots)
                write_slots(pool, vals.reshape(-1, 1, 1), np.asarray(slots, np.int64))
                model[s].extend(vals.tolist())
        elif op == "fork":
            s = live[pick % len(live)]
            c = ad.fork(s)
            live.append(c)
            model[c] = list(model[s])
        elif op == "share":
            s = live[pick % len(live)]
            k = n % (len(model[s]) + 1)
            c = ad.share(s, k)
            live.append(c)
            model[c] = list(model[s][:k])
        elif op == "free":
            s = live.pop(pick % len(live))
            ad.free(s)
            del model[s]
        # reading back through the tables gives each sequence's own tokens
        for s in live:
            tbl = ad.table(s)
            got = [int(pool[tbl[p // bs], 0, p % bs, 0]) for p in range(len(model[s]))]
            assert got == model[s], (op, s)
        if on_step is not None:
            on_step(ad)
    for s in list(live):
        ad.free(s)
    assert sorted(ad.free_list()) == list(range(nb))
    assert all(ad.refcount(b) == 0 for b in range(nb))
    return ad


@settings(max_examples=150, deadline=None)
@given(OPS, st.integers(0, 3))
def test_random_ops_preserve_contents_and_invariants(ops, seed):
    run_random_ops(OracleAdapter, ops, seed=seed,
                   on_step=lambda ad: ad.a.check_invariants())


@settings(max_examples=40, deadline=None)
@given(OPS)
def test_random_ops_small_pool_hits_oom(ops):
    run_random_ops(OracleAdapter, ops, nb=6, bs=2,
                   on_step=lambda ad: ad.a.check_invariants())


def test_invariant_checker_catches_a_leak():
    a = OracleAllocator(8, 4)
    s = a.create()
    a.append(s, 5)
    a.refcount[a.tables[s][0]] += 1    # planted mistake: a leaked reference
    with pytest.raises(AssertionError):
        a.check_invariants()


def test_free_pool_is_fifo_in_logical_order():
    """The free-pool reading: allocation takes the front; release appends
    each block whose count reaches zero at the back, walking the table in
    logical order."""
    a = OracleAllocator(6, 2, [5, 4, 3, 2, 1, 0])
    s = a.create()
    a.append(s, 5)                       # takes 5, 4, 3
    t = a.create()
    a.append(t, 1)                       # takes 2
    assert list(a.free) == [1, 0]
    a.free_seq(s)
    assert list(a.free) == [1, 0, 5, 4, 3]
    u = a.create()
    a.append(u, 3)
    assert a.tables[u] == [1, 0]
