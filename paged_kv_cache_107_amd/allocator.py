"""Python handle on libpa's host block allocator (pa_alloc_* / pa_seq_*).

Methods call the C function of the same name; arrays come back as numpy.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import PaError, check, lib, pa_prefix_stats, pa_swap_stats


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int32))


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


class PaAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.num_host_blocks = 0
        h = C.c_void_p()
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
        check("pa_alloc_create", lib().pa_alloc_create(
            self.num_blocks, self.block_size, None if order is None else _i32p(order),
            C.byref(h)))
        self._h = h
        # bumped by every call that can change a block table or a length, so
        # a holder of device copies of tables can tell when they went stale
        self.epoch = 0

    def close(self) -> None:
        if self._h:
            lib().pa_alloc_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ sequences
    def pa_seq_create(self) -> int:
        s = C.c_int64()
        check("pa_seq_create", lib().pa_seq_create(self._h, C.byref(s)))
        return s.value

    def pa_seq_append(self, seq: int, n_tokens: int) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        self.epoch += 1
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        pair = np.zeros(2, dtype=np.int32)
        ncow = C.c_int32()
        check("pa_seq_append", lib().pa_seq_append(self._h, int(seq), int(n_tokens), _i64p(slots),
                                                   _i32p(pair), C.byref(ncow)))
        return slots[:n_tokens], ((int(pair[0]), int(pair[1])) if ncow.value else None)

    def pa_seq_append_batch(self, seqs: Sequence[int], n_tokens: int, with_lens: bool = False):
        """Returns (slots [len(seqs) * n_tokens] int64, pairs [P][2] int32),
        plus the new lengths [len(seqs)] int32 with ``with_lens``."""
        self.epoch += 1
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        slots = np.empty(max(n * n_tokens, 1), dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        lens = np.empty(max(n, 1), dtype=np.int32)
        npairs = C.c_int32()
        check("pa_seq_append_batch", lib().pa_seq_append_batch(
            self._h, _i64p(s), n, int(n_tokens), _i64p(slots), _i32p(pairs), C.byref(npairs),
            _i32p(lens)))
        if with_lens:
            return slots[:n * n_tokens], pairs[:npairs.value], lens[:n]
        return slots[:n * n_tokens], pairs[:npairs.value]

    def append_batch_into(self, seqs_ptr, n: int, n_tokens: int, slots_ptr, pairs_ptr,
                          lens_ptr) -> int:
        """pa_seq_append_batch into caller buffers (raw addresses of int64
        seqs [n], int64 slots [n * n_tokens], int32 pairs [n][2], int32 lens
        [n]); returns the number of pairs."""
        self.epoch += 1
        npairs = C.c_int32()
        check("pa_seq_append_batch", lib().pa_seq_append_batch(
            self._h, C.cast(seqs_ptr, C.POINTER(C.c_int64)), n, n_tokens,
            C.cast(slots_ptr, C.POINTER(C.c_int64)), C.cast(pairs_ptr, C.POINTER(C.c_int32)),
            C.byref(npairs), C.cast(lens_ptr, C.POINTER(C.c_int32))))
        return npairs.value

    def pa_seq_fork(self, parent: int) -> int:
        self.epoch += 1
        c = C.c_int64()
        check("pa_seq_fork", lib().pa_seq_fork(self._h, int(parent), C.byref(c)))
        return c.value

    def pa_seq_share_prefix(self, src: int, n_tokens: int) -> int:
        self.epoch += 1
        c = C.c_int64()
        check("pa_seq_share_prefix",
              lib().pa_seq_share_prefix(self._h, int(src), int(n_tokens), C.byref(c)))
        return c.value

    def pa_seq_free(self, seq: int) -> None:
        self.epoch += 1
        check("pa_seq_free", lib().pa_seq_free(self._h, int(seq)))

    def pa_seq_info(self, seq: int) -> Tuple[int, np.ndarray]:
        length, nblk = C.c_int32(), C.c_int32()
        check("pa_seq_info", lib().pa_seq_info(self._h, int(seq), C.byref(length), None, 0,
                                                C.byref(nblk)))
        table = np.empty(max(nblk.value, 1), dtype=np.int32)
        check("pa_seq_info", lib().pa_seq_info(self._h, int(seq), None, _i32p(table),
                                                table.shape[0], C.byref(nblk)))
        return length.value, table[:nblk.value]

    def pa_build_tables(self, seqs: Sequence[int], max_blocks: int):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.shape[0]
        tables = np.empty((n, max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        check("pa_build_tables", lib().pa_build_tables(self._h, _i64p(s), n, int(max_blocks),
                                                       _i32p(tables), _i32p(lens)))
        return tables, lens

    # ------------------------------------------------------------ pool state
    def pa_alloc_query(self):
        """(free pool front to back, refcounts) as int32 arrays."""
        nf = C.c_int32()
        free = np.empty(self.num_blocks, dtype=np.int32)
        rc = np.empty(self.num_blocks, dtype=np.int32)
        check("pa_alloc_query", lib().pa_alloc_query(self._h, C.byref(nf), _i32p(free), _i32p(rc)))
        return free[:nf.value], rc

    def pa_alloc_stats(self):
        la, cc = C.c_int64(), C.c_int64()
        live, shared = C.c_int32(), C.c_int32()
        check("pa_alloc_stats", lib().pa_alloc_stats(self._h, C.byref(la), C.byref(cc),
                                                     C.byref(live), C.byref(shared)))
        return {"lazy_allocs": la.value, "cow_copies": cc.value, "live_seqs": live.value,
                "shared_blocks": shared.value}

    def pa_alloc_check_invariants(self) -> bool:
        st = lib().pa_alloc_check_invariants(self._h)
        if st not in (0, -5):
            raise PaError("pa_alloc_check_invariants", st)
        return st == 0

    # ------------------------------------------------------------ prefix cache
    def pa_alloc_enable_prefix_cache(self) -> None:
        check("pa_alloc_enable_prefix_cache", lib().pa_alloc_enable_prefix_cache(self._h))

    def pa_seq_create_prefix(self, tokens: Sequence[int]) -> Tuple[int, int]:
        """(sequence, hit_tokens) for a prompt of token ids."""
        self.epoch += 1
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        s, hit = C.c_int64(), C.c_int32()
        check("pa_seq_create_prefix", lib().pa_seq_create_prefix(
            self._h, _i32p(t) if t.size else None, int(t.size), C.byref(s), C.byref(hit)))
        return s.value, hit.value

    def pa_seq_append_tokens(self, seq: int, tokens: Sequence[int]):
        self.epoch += 1
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        n = int(t.size)
        slots = np.empty(max(n, 1), dtype=np.int64)
        pair = np.zeros(2, dtype=np.int32)
        ncow = C.c_int32()
        check("pa_seq_append_tokens", lib().pa_seq_append_tokens(
            self._h, int(seq), _i32p(t) if n else None, n, _i64p(slots), _i32p(pair),
            C.byref(ncow)))
        return slots[:n], ((int(pair[0]), int(pair[1])) if ncow.value else None)

    def pa_prefix_cache_stats(self) -> dict:
        st = pa_prefix_stats()
        check("pa_prefix_cache_stats", lib().pa_prefix_cache_stats(self._h, C.byref(st)))
        return {f: getattr(st, f) for f, _ in pa_prefix_stats._fields_}

    def pa_prefix_cache_query(self) -> np.ndarray:
        """Evictable blocks, least recently used first."""
        n = C.c_int32()
        out = np.empty(self.num_blocks, dtype=np.int32)
        check("pa_prefix_cache_query", lib().pa_prefix_cache_query(self._h, _i32p(out), C.byref(n)))
        return out[:n.value]

    # ------------------------------------------------------------ sliding window
    def pa_seq_trim_window(self, seq: int, window: int) -> int:
        """Release the blocks wholly below position len - window; returns the
        number of table entries that became PA_NO_BLOCK."""
        self.epoch += 1
        n = C.c_int32()
        check("pa_seq_trim_window", lib().pa_seq_trim_window(self._h, int(seq), int(window),
                                                              C.byref(n)))
        return n.value

    # ------------------------------------------------------------ swapping
    def pa_alloc_enable_swap(self, num_host_blocks: int) -> None:
        check("pa_alloc_enable_swap", lib().pa_alloc_enable_swap(self._h, int(num_host_blocks)))
        self.num_host_blocks = int(num_host_blocks)

    def _swap(self, fn: str, seq: int) -> np.ndarray:
        self.epoch += 1
        n = self.pa_seq_info(seq)[1].size
        pairs = np.zeros((max(n, 1), 2), dtype=np.int32)
        num = C.c_int32()
        check(fn, getattr(lib(), fn)(self._h, int(seq), _i32p(pairs), int(n), C.byref(num)))
        return pairs[:num.value]

    def pa_seq_swap_out(self, seq: int) -> np.ndarray:
        """(device block, host block) pairs [P][2] to copy out."""
        return self._swap("pa_seq_swap_out", seq)

    def pa_seq_swap_in(self, seq: int) -> np.ndarray:
        """(host block, device block) pairs [P][2] to copy in."""
        return self._swap("pa_seq_swap_in", seq)

    def pa_swap_query(self):
        """(counters dict, host free list front to back)."""
        st = pa_swap_stats()
        out = np.empty(max(self.num_host_blocks, 1), dtype=np.int32)
        check("pa_swap_query", lib().pa_swap_query(self._h, C.byref(st), _i32p(out)))
        return {f: getattr(st, f) for f, _ in pa_swap_stats._fields_}, out[:st.host_free]

