"""Pins for the oracle allocator's prefix cache (CPU only).

* The pages' numbers: a 1K-token system prompt is 64 blocks (128 MiB at the
  8B shape) and one copy serves 100 concurrent requests ("第 6 章 缓存管理",
  section "一次手算"); a 4096-token system prompt is computed once and the
  next 1000 requests each skip all of it ("放下账簿，打开源码", section "写时复制
  与前缀缓存").
* Least-recently-used eviction ("第 6 章 缓存管理", section "缓存放不下的时候").
* A content model: token ids are written into a pool through the returned
  slots (copy-on-write pairs first), and every sequence must read its own
  tokens back through its table after every operation -- a wrong hit, or a
  write into a shared or cached block, breaks it.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import OracleAllocator, OracleError


class Pool:
    """Token ids per slot: the stand-in for K/V contents."""

    def __init__(self, a: OracleAllocator):
        self.a = a
        self.content = np.full((a.num_blocks, a.block_size), -1, dtype=np.int64)

    def write(self, slots, pair, ids):
        bs = self.a.block_size
        if pair is not None:
            self.content[pair[1]] = self.content[pair[0]]
        for s, t in zip(slots, ids):
            self.content[s // bs, s % bs] = t

    def check(self, seq_tokens):
        a, bs = self.a, self.a.block_size
        a.check_invariants()
        for s, toks in seq_tokens.items():
            t = a.tables[s]
            assert a.lens[s] == len(toks)
            got = [int(self.content[t[p // bs], p % bs]) for p in range(len(toks))]
            assert got == list(toks), f"sequence {s} reads other tokens"


def serve(a, pool, prompt):
    """A request: look its prompt up, append the rest with token ids."""
    s, hit = a.create_prefix(prompt)
    slots, pair = a.append_tokens(s, prompt[hit:])
    pool.write(slots, pair, prompt[hit:])
    return s, hit


def test_one_system_prompt_serves_a_hundred_requests():
    bs, prompt_len = 16, 1024
    a = OracleAllocator(8000, bs)
    a.enable_prefix_cache()
    pool = Pool(a)
    rng = np.random.default_rng(0)
    system = list(rng.integers(0, 50000, prompt_len))
    seqs, toks = [], {}
    for r in range(100):
        user = list(rng.integers(0, 50000, 40 + r))
        s, hit = serve(a, pool, system + user)
        seqs.append(s)
        toks[s] = system + user
        assert hit == (0 if r == 0 else prompt_len)
    pool.check(toks)
    prompt_blocks = a.tables[seqs[0]][:prompt_len // bs]
    assert len(prompt_blocks) == 64                     # 1K tokens = 64 blocks
    assert all(a.tables[s][:64] == prompt_blocks for s in seqs)
    assert all(a.refcount[b] == 100 for b in prompt_blocks)
    # 64 blocks x 2 MiB (16 tokens x 128 KiB per token at the 8B shape) = 128 MiB,
    # held once instead of 100 times
    assert 64 * 16 * 128 * 1024 == 128 * 2 ** 20
    st_ = a.prefix_stats()
    assert st_["hit_tokens"] == 99 * 1024 and st_["pinned_blocks"] >= 64


def test_a_4096_token_prompt_is_computed_once():
    bs = 16
    a = OracleAllocator(2000, bs)
    a.enable_prefix_cache()
    pool = Pool(a)
    system = list(range(4096))
    serve(a, pool, system + [7])
    hits = []
    for r in range(1000):
        s, hit = serve(a, pool, system + [10 ** 6 + r])
        hits.append(hit)
        a.free_seq(s)
    assert hits == [4096] * 1000
    assert a.prefix_stats()["hit_tokens"] == 1000 * 4096


def test_lookup_leaves_one_token_to_compute():
    a = OracleAllocator(64, 16)
    a.enable_prefix_cache()
    pool = Pool(a)
    p = list(range(64))                                  # exactly 4 blocks
    s, _ = serve(a, pool, p)
    a.free_seq(s)
    s2, hit = a.create_prefix(p)
    assert hit == 48                                     # 3 blocks; the last one is recomputed
    s3, hit3 = a.create_prefix(p + [99])
    assert hit3 == 64


def test_least_recently_used_blocks_are_evicted_first():
    bs = 4
    a = OracleAllocator(12, bs)
    a.enable_prefix_cache()
    pool = Pool(a)
    prompts = {k: [100 * (j + 1) + i for i in range(8)] for j, k in enumerate("ABC")}  # 2 blocks
    seqs = {}
    for k in "ABC":
        seqs[k], _ = serve(a, pool, prompts[k] + [0])              # 3 blocks each, last partial
    tables = {k: list(a.tables[seqs[k]]) for k in "ABC"}
    for k in "ABC":                                                 # release A, then B, then C
        a.free_seq(seqs[k])
    # cached: the two full blocks of each; released last block first
    assert list(a.lru) == [tables["A"][1], tables["A"][0], tables["B"][1], tables["B"][0],
                           tables["C"][1], tables["C"][0]]
    assert len(a.free) == 6                                         # 3 free + 3 partial blocks
    s, hit = serve(a, pool, [9] * 31)                               # 8 blocks: 6 free, evict 2
    assert hit == 0 and a.evictions == 2
    assert list(a.lru) == [tables["B"][1], tables["B"][0], tables["C"][1], tables["C"][0]]
    s_a, hit_a = a.create_prefix(prompts["A"] + [1])                # A's prompt is gone
    assert hit_a == 0
    s_c, hit_c = a.create_prefix(prompts["C"] + [1])                # C's is back in use
    assert hit_c == 8 and tables["C"][0] not in a.lru and a.refcount[tables["C"][0]] == 1


def test_a_cached_block_is_never_written_in_place():
    a = OracleAllocator(16, 4)
    a.enable_prefix_cache()
    pool = Pool(a)
    src, _ = serve(a, pool, [1, 2, 3, 4, 5, 6, 7, 8, 9])
    blk = a.tables[src][1]                                          # cached, full: 5 6 7 8
    child = a.share_prefix(src, 6)                                  # ends mid-block
    a.free_seq(src)
    assert a.refcount[blk] == 1
    slots, pair = a.append_tokens(child, [60, 61])
    pool.write(slots, pair, [60, 61])
    assert pair is not None and pair[0] == blk                      # copied, not written
    assert list(pool.content[blk]) == [5, 6, 7, 8] and blk in a.lru
    pool.check({child: [1, 2, 3, 4, 5, 6, 60, 61]})


def test_cache_must_be_enabled_first():
    a = OracleAllocator(8, 4)
    a.create()
    with pytest.raises(OracleError):
        a.enable_prefix_cache()
    with pytest.raises(OracleError):
        a.create_prefix([1, 2, 3])


# ------------------------------------------------------------------ random operations

ops = st.lists(st.tuples(st.sampled_from(["serve", "serve", "append", "append_plain", "fork",
                                          "share", "free", "free"]),
                         st.integers(0, 1 << 30)), min_size=1, max_size=40)


@settings(max_examples=150, deadline=None)
@given(ops=ops, bs=st.sampled_from([2, 4]), nb=st.integers(8, 40))
def test_random_operations_keep_contents_and_invariants(ops, bs, nb):
    a = OracleAllocator(nb, bs)
    a.enable_prefix_cache()
    pool = Pool(a)
    toks = {}
    unknown = set()            # sequences with positions appended without ids
    for op, r in ops:
        rng = np.random.default_rng(r)
        live = sorted(toks)
        try:
            if op == "serve":
                base = [int(x) for x in rng.integers(0, 3, rng.integers(1, 12))]
                prompt = [1, 2, 3, 4, 5, 6][:rng.integers(0, 7)] + base
                if not prompt:
                    continue
                s, hit = a.create_prefix(prompt)
                toks[s] = prompt[:hit]
                ids = prompt[hit:]
                slots, pair = a.append_tokens(s, ids)
                pool.write(slots, pair, ids)
                toks[s] = prompt
            elif op in ("append", "append_plain") and live:
                s = live[r % len(live)]
                ids = [int(x) for x in rng.integers(0, 3, rng.integers(1, 6))]
                if op == "append":
                    slots, pair = a.append_tokens(s, ids)
                else:
                    slots, pair = a.append(s, len(ids))
                    unknown.add(s)
                pool.write(slots, pair, ids)
                toks[s] = toks[s] + ids
            elif op == "fork" and live:
                s = live[r % len(live)]
                c = a.fork(s)
                toks[c] = list(toks[s])
                if s in unknown:
                    unknown.add(c)
            elif op == "share" and live:
                s = live[r % len(live)]
                n = int(rng.integers(0, len(toks[s]) + 1))
                c = a.share_prefix(s, n)
                toks[c] = toks[s][:n]
            elif op == "free" and live:
                s = live[r % len(live)]
                a.free_seq(s)
                del toks[s]
                unknown.discard(s)
        except OracleError as e:
            assert e.code == "OOM"
            for s in list(toks):                 # a failed op changed nothing
                if s not in a.tables:
                    del toks[s]
        pool.check(toks)
    for s in list(toks):
        a.free_seq(s)
    a.check_invariants()
    assert sorted(list(a.free) + list(a.lru)) == list(range(nb))


# ------------------------------------------------------------------ cached prefill

@pytest.mark.parametrize("bs,system_len,suffix", [(16, 100, [1, 5, 16, 17, 40, 3]),
                                                   (4, 13, [1, 2, 7]),
                                                   (16, 64, [1, 30])])
def test_cached_prefill_equals_full_prompt_prefill(bs, system_len, suffix):
    """Skipping the cached prefix changes no output: the suffix rows of a
    prefill over cached blocks equal the same rows of the full prompt's
    prefill without the cache (both in float64 over the same K/V bits), and
    every request after the first hits every full block of the system prompt
    that leaves at least one token to compute."""
    import workloads as W
    from _prefix import run_prompts_oracle
    from oracle.attention import paged_prefill
    ps = W.custom_prompt_set(700 + bs, 8, 2, 32, "bf16", bs, system_len, suffix)
    c = run_prompts_oracle(ps, cached=True)
    u = run_prompts_oracle(ps, cached=False)
    want_hits = [0] + [min(system_len // bs, (system_len + n - 1) // bs) * bs for n in suffix[1:]]
    assert c["hits"].tolist() == want_hits
    oc = paged_prefill(c["q"], c["kp"], c["vp"], c["tables"], c["query_start"], c["lens"],
                       ps.wl.scale, "bf16")
    ou = paged_prefill(u["q"], u["kp"], u["vp"], u["tables"], u["query_start"], u["lens"],
                       ps.wl.scale, "bf16")
    for r in range(ps.requests):
        a, b = c["query_start"][r], c["query_start"][r + 1]
        ua, ub = u["query_start"][r], u["query_start"][r + 1]
        assert b - a == ub - ua - c["hits"][r]
        np.testing.assert_allclose(oc[a:b], ou[ua + c["hits"][r]:ub], rtol=0, atol=1e-12)
    full = system_len // bs
    shared = c["tables"][0, :full]
    for r in range(1, ps.requests):
        k = c["hits"][r] // bs
        assert (c["tables"][r, :k] == shared[:k]).all()
    held_c = len({int(b) for row in c["tables"] for b in row if b >= 0})
    held_u = len({int(b) for row in u["tables"] for b in row if b >= 0})
    assert held_u - held_c == int(c["hits"].sum()) // bs


# ------------------------------------------------------------------ batched decode steps

def _independent(pairs):
    """No pair's destination is another pair's source or destination."""
    return all(d != s2 and d != d2 for i, (_, d) in enumerate(pairs)
               for j, (s2, d2) in enumerate(pairs) if i != j)


def test_a_step_cannot_reuse_a_copied_cached_block():
    """A decode step's copies run together, before its writes (copy, then
    write: "Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统中的应用", section
    4.4).  Two sequences each hold the last reference to a cached partial
    block and must copy it.  With one free block the step does not fit: the
    first copy's source may not serve as the second copy's destination while
    the first still reads it (OOM, nothing changes).  With two free blocks
    the copies are independent, and the copied blocks become evictable
    after the step, in order."""
    for nb in (5, 6):
        a = OracleAllocator(nb, 16)
        a.enable_prefix_cache()
        sharers = []
        for base in (100, 200):
            prompt = list(range(base, base + 32))
            s, _ = a.create_prefix(prompt)
            a.append_tokens(s, prompt)
            sharers.append(a.share_prefix(s, 20))
            a.free_seq(s)
        before = (list(a.free), list(a.lru), list(a.refcount))
        if nb == 5:
            with pytest.raises(OracleError) as e:
                a.append_batch(sharers, 1)
            assert e.value.code == "OOM"
            assert (list(a.free), list(a.lru), list(a.refcount)) == before
            continue
        slots, pairs = a.append_batch(sharers, 1)
        assert len(pairs) == 2 and _independent(pairs)
        assert list(a.lru)[-2:] == [pairs[0][0], pairs[1][0]]
        a.check_invariants()


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 1 << 30), bs=st.sampled_from([2, 4]), nb=st.integers(8, 30))
def test_batched_steps_keep_contents_with_copies_in_any_order(seed, bs, nb):
    """Requests served through the cache, some released (their cached
    blocks evictable), then decode steps of batched appends.  Each step's
    copies are applied in reverse order before its writes: since they are
    independent the order cannot matter, and every live sequence still
    reads its own tokens back."""
    rng = np.random.default_rng(seed)
    a = OracleAllocator(nb, bs, rng.permutation(nb).tolist())
    a.enable_prefix_cache()
    pool = Pool(a)
    live = {}
    for r in range(int(rng.integers(2, 8))):
        prompt = [int(x) for x in rng.integers(0, 2, int(rng.integers(1, 3 * bs + 2)))]
        try:
            s, hit = a.create_prefix(prompt)
            slots, pair = a.append_tokens(s, prompt[hit:])
        except OracleError as e:
            assert e.code == "OOM"
            break
        pool.write(slots, pair, prompt[hit:])
        live[s] = list(prompt)
        if rng.random() < 0.4:
            c = a.share_prefix(s, int(rng.integers(0, len(prompt) + 1)))
            live[c] = live[s][:a.lens[c]]
        if rng.random() < 0.4:
            a.free_seq(s)
            del live[s]
    next_id = 1000
    for _ in range(3):
        seqs = list(live)
        if not seqs:
            break
        try:
            slots, pairs = a.append_batch(seqs, 1)
        except OracleError as e:
            assert e.code == "OOM"
            break
        assert _independent(pairs)
        for src, dst in reversed(pairs):
            pool.content[dst] = pool.content[src]
        for s, slot in zip(seqs, slots):
            pool.content[slot // bs, slot % bs] = next_id
            live[s].append(next_id)
            next_id += 1
        pool.check(live)
