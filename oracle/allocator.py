"""Oracle block allocator (pure Python).  Test infrastructure only.

What it follows:

* Lazy allocation: a sequence records its length and a list of logical
  blocks; a physical block is taken from the pool only when a token position
  first enters that logical block.  Page "Lazy Allocation 与 Copy-on-Write 在
  LLM 推理系统中的应用", section 3.3 (Lazy Allocation 思想的迁移); page
  "放下账簿，打开源码", section "PagedAttention：虚实分离，按需取用" (a block is
  taken when the previous 16 tokens are full).
* Slot of position ``pos``: the block table maps logical block ``pos // BS``
  to a physical block; the slot is that block times BS plus ``pos % BS``
  (same page, same section, block-table example 37/12/88; 0-based).
* Fork: the child gets a copy of the parent's block table and every shared
  block's refcount goes up; no KV bytes move.  Page "vLLM：把 KV 缓存当成虚拟
  内存", section "碎片从哪里来".
* Copy-on-write: a write into a block whose refcount is above one first takes
  a fresh block, copies, drops the old block's count by one, points the
  writer's table at the copy and writes there; the last holder writes in
  place.  Page "Lazy Allocation 与 Copy-on-Write ...", section 4.4 (blocks 7,
  1 and 3); page "放下账簿，打开源码", section "写时复制与前缀缓存" (refcount 4
  -> 3 and 1).
* Prefix sharing and release: a request sharing the first P tokens copies the
  first ceil(P/BS) table entries and their counts go up; ending a request
  drops each count by one and a block whose count reaches zero goes back to
  the free pool.  Page "第 6 章 缓存管理", section "块表长什么样".

Readings where the pages are silent (each one is a documented choice):

* The free pool is a FIFO: allocation pops the front; release walks the
  sequence's table in logical order and appends each block whose count hits
  zero at the back.  ``initial_free_order`` seeds the FIFO.
* One append writes positions ``len .. len+n-1``.  Only its first position
  can land in an existing block; if that block is shared, exactly one CoW
  copy is made.  Full shared blocks are never written.
* An append that cannot get all the blocks it needs (new blocks plus the CoW
  block) fails with ``OOM`` and changes nothing (reject, do not crash:
  "第 6 章 缓存管理", section "缓存放不下的时候").
* Sharing ``n`` tokens copies ``ceil(n / BS)`` entries even when the last one
  holds more of the source's tokens; the sharer's length masks them and its
  first write into that block copies it.

Prefix cache (``enable_prefix_cache``): a prompt prefix that many requests
share stays in memory as cached blocks, marked as cached and kept out of the
free pool, so a later request with the same prefix finds them and skips that
prefill ("vLLM：把 KV 缓存当成虚拟内存", sections "碎片从哪里来" and "KV 的体积
从哪来，页表如何把它切开"; "放下账簿，打开源码", section "写时复制与前缀缓存");
when memory runs out, cached blocks are dropped least recently used first and
recomputed when needed ("第 6 章 缓存管理", section "缓存放不下的时候").
Readings (the pages give no mechanism):

* Only full blocks are cached; a block's identity is the whole token prefix
  up to its end (here the exact tuple of token ids; two requests with the same
  tokens up to there have the same K/V there).  A block is registered when an
  append with known token ids fills it, unless that prefix is already cached
  under another block (the first registration stays).
* A lookup for a new request walks its full blocks from the start and takes
  every cached block (refcount + 1) until the first miss, leaving at least
  one prompt token to compute (the last token's query produces the next
  token).
* A released block whose count reaches zero goes to the back of the free pool
  if it is not cached; a cached one becomes evictable and enters a
  least-recently-used list: the released sequence's cached blocks enter it
  from its last block to its first, so a shared prompt's first blocks are
  the most recently used and are evicted last.  A lookup hit on an evictable
  block takes it out of the list.
* A new block comes from the front of the free pool, or, when that is empty,
  by evicting the least recently used evictable block (its registration is
  dropped).  An append fails with OOM only if both are short.
* A cached block is never written: an append whose first position falls in a
  cached block (possible after sharing a prefix that ends mid-block) copies
  it first, as for a shared block.

Swapping (``enable_swap``): a preempted sequence's KV moves to host memory
and comes back later, block by block rather than as one contiguous buffer
("vLLM：把 KV 缓存当成虚拟内存", section "碎片从哪里来", on preemption; "第 6 章
缓存管理", section "缓存放不下的时候", on moving cold cache to CPU memory).
Readings (the pages name the move, not its bookkeeping):

* The host side is a second pool of ``num_host_blocks`` blocks of the same
  shape, with its own FIFO free list (ids 0.. in order at start).
* Swap-out moves the blocks only this sequence holds (refcount 1) to host
  blocks taken from the front of the host list, in logical order, and
  releases those device blocks as ``free_seq`` does (free pool, or the
  evictable list if cached).  Blocks it shares with other sequences stay on
  the device and it keeps its reference: moving them frees nothing.
  Returns the (device block, host block) copies, which must run before the
  released device blocks are written again.
* A swapped-out sequence can only be swapped in or freed; any other use is
  an error (``SWAPPED``).  Freeing it returns its host blocks to the back of
  the host list in logical order and drops its device references.
* Swap-in takes a device block for each host-resident entry, in logical
  order, the same way an append does (free pool, else eviction), and returns
  the (host block, device block) copies; the host blocks go back to the host
  list in logical order.  The new blocks are private (refcount 1) and not
  cached.
* Both moves are all or nothing: ``OOM`` when the destination is short.

Sliding window (``trim_window``): with a window of W positions, the newest
token (position len - 1) and every later one attend only positions >= len -
W, so a block whose positions all lie below len - W is never read again
("vLLM：把 KV 缓存当成虚拟内存": sliding windows change how long K/V live).
Trimming drops the sequence's reference to each such block (released as
``free_seq`` releases) and leaves a hole (``NO_BLOCK``) in its table, which
keeps its length, so logical block j still maps position j * BS.  Holes are
skipped by every other operation; a fork copies them; sharing a prefix that
includes a hole is refused (ARG): the allocator does not know the sharer's
window, and a prefix without its early blocks is not the whole prefix.
"""
from __future__ import annotations

import copy
from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


NO_BLOCK = -(2 ** 31)  # table entry of a block released by a sliding window


class OracleError(Exception):
    """Allocator error; ``code`` is one of ARG, OOM, REFCOUNT, NOT_FOUND,
    SWAPPED."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class OracleAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise OracleError("ARG", "num_blocks and block_size must be positive")
        if initial_free_order is None:
            order = list(range(num_blocks))
        else:
            order = [int(b) for b in initial_free_order]
            if sorted(order) != list(range(num_blocks)):
                raise OracleError("ARG", "initial_free_order must be a permutation of 0..NB-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.refcount: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self._next_seq = 0
        # counters
        self.lazy_allocs = 0
        self.cow_copies = 0
        # prefix cache (off until enable_prefix_cache)
        self.caching = False
        self.tokens: Dict[int, List[int]] = {}    # known token ids of each sequence
        self.considered: Dict[int, int] = {}       # leading full blocks already offered to the cache
        self.index: Dict[tuple, int] = {}          # token prefix -> cached block
        self.block_key: Dict[int, tuple] = {}      # cached block -> its prefix
        self.lru: "OrderedDict[int, None]" = OrderedDict()  # evictable, least recent first
        self.lookup_tokens = 0
        self.hit_tokens = 0
        self.evictions = 0
        # swapping to a host pool (off until enable_swap)
        self.host_free: Optional[deque] = None
        self.num_host_blocks = 0
        self.swapped: Dict[int, List[Tuple[bool, int]]] = {}  # seq -> (on host, id) per block
        self.swap_outs = 0
        self.swap_ins = 0
        self.blocks_out = 0
        self.blocks_in = 0

    # ------------------------------------------------------------ helpers
    def _seq(self, seq: int) -> List[int]:
        if seq in self.swapped:
            raise OracleError("SWAPPED", f"sequence {seq} is on the host")
        if seq not in self.tables:
            raise OracleError("NOT_FOUND", f"sequence {seq}")
        return self.tables[seq]

    def _release(self, released: List[int]) -> None:
        """Blocks whose count reached zero, in logical order: uncached ones to
        the back of the free pool in that order; cached ones to the back of
        the evictable list, last block first."""
        for b in released:
            if b not in self.block_key:
                self.free.append(b)
        for b in reversed(released):
            if b in self.block_key:
                self.lru[b] = None

    def _new_id(self) -> int:
        s = self._next_seq
        self._next_seq += 1
        return s

    def _available(self) -> int:
        return len(self.free) + len(self.lru)

    def _take(self) -> int:
        """A block for new data: free pool front, else evict the least
        recently used cached block."""
        if self.free:
            return self.free.popleft()
        blk, _ = self.lru.popitem(last=False)
        del self.index[self.block_key.pop(blk)]
        self.evictions += 1
        return blk

    def _register(self, seq: int) -> None:
        """Offer the cache each block of ``seq`` that has become full with
        all of its token ids known: it is cached unless its prefix (or the
        block) already is.  A block is offered once, when it fills."""
        if not self.caching:
            return
        bs = self.block_size
        known = self.tokens[seq]
        table = self.tables[seq]
        full = min(self.lens[seq], len(known)) // bs
        for j in range(self.considered[seq], full):
            key = tuple(known[:(j + 1) * bs])
            blk = table[j]
            if blk != NO_BLOCK and key not in self.index and blk not in self.block_key:
                self.index[key] = blk
                self.block_key[blk] = key
        self.considered[seq] = max(self.considered[seq], full)

    # ------------------------------------------------------------ operations
    def create(self) -> int:
        s = self._new_id()
        self.tables[s] = []
        self.lens[s] = 0
        self.tokens[s] = []
        self.considered[s] = 0
        return s

    def enable_prefix_cache(self) -> None:
        if self.tables:
            raise OracleError("ARG", "enable the prefix cache before creating sequences")
        self.caching = True

    def create_prefix(self, prompt: Sequence[int]) -> Tuple[int, int]:
        """A new sequence for ``prompt``: its longest cached prefix of whole
        blocks (at most len(prompt) - 1 tokens) is shared; returns (seq,
        hit_tokens).  The caller appends prompt[hit_tokens:] next."""
        if not self.caching:
            raise OracleError("ARG", "prefix cache is off")
        prompt = [int(t) for t in prompt]
        bs = self.block_size
        s = self.create()
        hits = 0
        for j in range(max(len(prompt) - 1, 0) // bs):
            blk = self.index.get(tuple(prompt[:(j + 1) * bs]))
            if blk is None:
                break
            if self.refcount[blk] == 0:
                del self.lru[blk]
            self.refcount[blk] += 1
            self.tables[s].append(blk)
            hits += 1
        self.lens[s] = hits * bs
        self.tokens[s] = prompt[:hits * bs]
        self.considered[s] = hits
        self.lookup_tokens += len(prompt)
        self.hit_tokens += hits * bs
        return s, hits * bs

    def append_tokens(self, seq: int, ids: Sequence[int]):
        """``append`` with the token ids of the new positions: full blocks
        whose ids are all known are cached."""
        slots, pair = self.append(seq, len(ids))
        if len(self.tokens[seq]) == self.lens[seq] - len(ids):
            self.tokens[seq].extend(int(t) for t in ids)
        self._register(seq)
        return slots, pair

    def append(self, seq: int, n_tokens: int,
               held: Optional[List[int]] = None) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        """Write positions len..len+n-1.  Returns (slots, cow_pair or None).
        ``held``: see ``append_batch``."""
        table = self._seq(seq)
        if n_tokens < 0:
            raise OracleError("ARG", "n_tokens < 0")
        bs = self.block_size
        start = self.lens[seq]
        end = start + n_tokens
        if n_tokens == 0:
            return [], None
        # is the first position inside an existing block that is shared, or
        # cached (a cached block's contents must not change)?
        needs_cow = start % bs != 0 and (self.refcount[table[start // bs]] > 1
                                         or table[start // bs] in self.block_key)
        new_blocks = _ceil_div(end, bs) - _ceil_div(start, bs)
        if new_blocks + int(needs_cow) > self._available():
            raise OracleError("OOM", f"need {new_blocks + int(needs_cow)}, free {self._available()}")
        pair = None
        if needs_cow:
            src = table[start // bs]
            dst = self._take()
            self.refcount[src] -= 1
            if self.refcount[src] == 0:           # a cached block's last holder copied
                if held is None:
                    self.lru[src] = None
                else:
                    held.append(src)
            self.refcount[dst] = 1
            table[start // bs] = dst
            pair = (src, dst)
            self.cow_copies += 1
        slots = []
        for pos in range(start, end):
            if pos % bs == 0:
                blk = self._take()
                self.refcount[blk] = 1
                table.append(blk)
                self.lazy_allocs += 1
            slots.append(table[pos // bs] * bs + pos % bs)
        self.lens[seq] = end
        return slots, pair

    def append_batch(self, seqs: Sequence[int], n_tokens: int):
        """One decode step: ``append(s, n_tokens)`` for each of ``seqs`` in
        order; returns (all slots, the CoW pairs in order).

        The step's copies are meant to run together, before the step's
        writes (copy, then write: page "Lazy Allocation 与 Copy-on-Write ...",
        section 4.4), so no block may be both read and written by two copies
        of one step.  A cached block whose last holder copies it would
        otherwise become evictable at once, and a later append of the same
        step could take it as its own copy's destination while the first
        copy still reads it.  Such blocks are therefore held back and join
        the evictable list (in the order they were released) only after the
        step's last append.  All or nothing: on OOM (each append must fit
        what is available when it runs, the held blocks excluded) nothing
        changes; a sequence named twice is ARG."""
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise OracleError("ARG", "one append per sequence per step")
        for s in seqs:
            self._seq(s)
        saved = copy.deepcopy(self.__dict__)
        held: List[int] = []
        slots, pairs = [], []
        try:
            for s in seqs:
                sl, pr = self.append(s, n_tokens, held)
                slots += sl
                if pr is not None:
                    pairs.append(pr)
        except OracleError:
            self.__dict__.clear()
            self.__dict__.update(saved)
            raise
        for b in held:
            self.lru[b] = None
        return slots, pairs

    def fork(self, parent: int) -> int:
        table = self._seq(parent)
        child = self._new_id()
        self.tables[child] = list(table)
        self.lens[child] = self.lens[parent]
        self.tokens[child] = list(self.tokens[parent])
        self.considered[child] = self.considered[parent]
        for b in table:
            if b != NO_BLOCK:
                self.refcount[b] += 1
        return child

    def share_prefix(self, src: int, n_tokens: int) -> int:
        table = self._seq(src)
        if n_tokens < 0 or n_tokens > self.lens[src]:
            raise OracleError("ARG", "prefix longer than the source")
        k = _ceil_div(n_tokens, self.block_size)
        if NO_BLOCK in table[:k]:
            raise OracleError("ARG", "part of the prefix was released by a sliding window")
        s = self._new_id()
        self.tables[s] = list(table[:k])
        self.lens[s] = n_tokens
        self.tokens[s] = list(self.tokens[src][:n_tokens])
        self.considered[s] = min(self.considered[src], n_tokens // self.block_size)
        for b in self.tables[s]:
            if b != NO_BLOCK:
                self.refcount[b] += 1
        return s

    def free_seq(self, seq: int) -> None:
        if seq in self.swapped:
            entries = self.swapped.pop(seq)
            released = []
            for on_host, i in entries:
                if on_host:
                    self.host_free.append(i)
                elif i != NO_BLOCK:
                    self.refcount[i] -= 1
                    if self.refcount[i] == 0:
                        released.append(i)
            self._release(released)
            del self.lens[seq]
            del self.tokens[seq]
            del self.considered[seq]
            return
        table = [b for b in self._seq(seq) if b != NO_BLOCK]
        for b in table:
            if self.refcount[b] <= 0:
                raise OracleError("REFCOUNT", f"block {b} already free")
        released = []
        for b in table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                released.append(b)
        self._release(released)
        del self.tables[seq]
        del self.lens[seq]
        del self.tokens[seq]
        del self.considered[seq]

    # ------------------------------------------------------------ sliding window
    def trim_window(self, seq: int, window: int) -> int:
        """Release the blocks of ``seq`` that lie wholly below position
        len - window; returns how many table entries became holes."""
        table = self._seq(seq)
        if window <= 0:
            raise OracleError("ARG", "window must be positive")
        bs = self.block_size
        dead = max(self.lens[seq] - window, 0) // bs     # blocks j with (j + 1) * BS <= len - W
        released, n = [], 0
        for j in range(dead):
            b = table[j]
            if b == NO_BLOCK:
                continue
            table[j] = NO_BLOCK
            n += 1
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                released.append(b)
        self._release(released)
        return n

    # ------------------------------------------------------------ swapping
    def enable_swap(self, num_host_blocks: int) -> None:
        if self.host_free is not None or num_host_blocks <= 0:
            raise OracleError("ARG", "swap already on, or no host blocks")
        self.num_host_blocks = num_host_blocks
        self.host_free = deque(range(num_host_blocks))

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """Move the blocks only ``seq`` holds to host blocks; returns the
        (device, host) copies in logical order."""
        if self.host_free is None:
            raise OracleError("ARG", "swap is off")
        table = self._seq(seq)
        own = [j for j, b in enumerate(table) if b != NO_BLOCK and self.refcount[b] == 1]
        if len(own) > len(self.host_free):
            raise OracleError("OOM", f"need {len(own)} host blocks, free {len(self.host_free)}")
        entries = [(False, b) for b in table]
        pairs, released = [], []
        for j in own:
            h = self.host_free.popleft()
            pairs.append((table[j], h))
            entries[j] = (True, h)
            self.refcount[table[j]] = 0
            released.append(table[j])
        self._release(released)
        del self.tables[seq]
        self.swapped[seq] = entries
        self.swap_outs += 1
        self.blocks_out += len(pairs)
        return pairs

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """Bring a swapped-out sequence back; returns the (host, device)
        copies in logical order."""
        if seq in self.tables:
            raise OracleError("ARG", f"sequence {seq} is not swapped out")
        if seq not in self.swapped:
            raise OracleError("NOT_FOUND", f"sequence {seq}")
        entries = self.swapped[seq]
        on_host = [j for j, (h, _) in enumerate(entries) if h]
        if len(on_host) > self._available():
            raise OracleError("OOM", f"need {len(on_host)}, free {self._available()}")
        table = [i for _, i in entries]
        pairs = []
        for j in on_host:
            d = self._take()
            self.refcount[d] = 1
            pairs.append((entries[j][1], d))
            table[j] = d
        for j in on_host:
            self.host_free.append(entries[j][1])
        del self.swapped[seq]
        self.tables[seq] = table
        self.swap_ins += 1
        self.blocks_in += len(pairs)
        return pairs

    def swap_stats(self) -> Dict[str, int]:
        return dict(swap_outs=self.swap_outs, swap_ins=self.swap_ins, blocks_out=self.blocks_out,
                    blocks_in=self.blocks_in, swapped_seqs=len(self.swapped),
                    host_free=len(self.host_free) if self.host_free is not None else 0)

    def build_tables(self, seqs: Sequence[int], max_blocks: int):
        """Block tables [n][max_blocks] int32 padded with -1, and lengths [n]."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for r, s in enumerate(seqs):
            t = self._seq(s)
            if len(t) > max_blocks:
                raise OracleError("ARG", f"sequence {s} has {len(t)} blocks > {max_blocks}")
            out[r, :len(t)] = t
            lens[r] = self.lens[s]
        return out, lens

    # ------------------------------------------------------------ invariants
    def check_invariants(self) -> None:
        """Refcount = in-degree from all tables; a block is free iff its count
        is zero; the free pool has no duplicates; every table has exactly
        ceil(len / BS) entries."""
        indeg = [0] * self.num_blocks
        for s, t in self.tables.items():
            if len(t) != _ceil_div(self.lens[s], self.block_size):
                raise AssertionError(f"seq {s}: {len(t)} blocks for {self.lens[s]} tokens")
            for b in t:
                if b != NO_BLOCK:
                    indeg[b] += 1
        host_used = []
        for s, entries in self.swapped.items():
            if len(entries) != _ceil_div(self.lens[s], self.block_size):
                raise AssertionError(f"swapped seq {s}: wrong entry count")
            for on_host, i in entries:
                if on_host:
                    host_used.append(i)
                elif i != NO_BLOCK:
                    indeg[i] += 1
        if self.host_free is not None and sorted(list(self.host_free) + host_used) != \
                list(range(self.num_host_blocks)):
            raise AssertionError("host blocks lost or duplicated")
        if indeg != self.refcount:
            raise AssertionError("refcount differs from table in-degree")
        free_set = set(self.free)
        if len(free_set) != len(self.free):
            raise AssertionError("duplicate block in the free pool")
        for b in range(self.num_blocks):
            idle = self.refcount[b] == 0
            cached = b in self.block_key
            if (b in free_set) != (idle and not cached):
                raise AssertionError(f"block {b}: free={b in free_set} refcount={self.refcount[b]}")
            if (b in self.lru) != (idle and cached):
                raise AssertionError(f"block {b}: evictable={b in self.lru} cached={cached}")
        if len(self.index) != len(self.block_key) or any(
                self.block_key.get(b) != k for k, b in self.index.items()):
            raise AssertionError("cache index and block keys differ")
        for k in self.index:
            if len(k) % self.block_size:
                raise AssertionError("a cached key is not a whole number of blocks")

    def snapshot(self):
        """(free FIFO as a list, refcounts, {seq: (table, len)}) for comparisons."""
        return (list(self.free), list(self.refcount),
                {s: (list(t), self.lens[s]) for s, t in self.tables.items()})

    def prefix_stats(self) -> Dict[str, int]:
        return dict(lookup_tokens=self.lookup_tokens, hit_tokens=self.hit_tokens,
                    evictions=self.evictions, cached_blocks=len(self.block_key),
                    evictable_blocks=len(self.lru),
                    pinned_blocks=sum(1 for b in self.block_key if self.refcount[b] > 0))
