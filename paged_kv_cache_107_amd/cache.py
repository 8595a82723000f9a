"""A paged KV cache for one attention layer: device pools plus the host
allocator, and the decode step over them.

A step has a host half and a device half:

* ``plan``: the allocator reserves one slot per new token (taking blocks
  lazily, copying shared blocks on write) in one batched call, which writes
  the slots, the copy pairs and the new lengths straight into a pinned
  staging buffer; one asynchronous copy moves them to the device.  The
  block tables stay resident on the device: a step changes a sequence's
  table only in the blocks its new positions fall in (a fresh block, or the
  copied last block), which are the blocks of the new slots, so
  ``pa_update_tables`` patches them from the uploaded slots.  Any other
  change to the batch's tables (a new batch, a fork, a free, a swap, a
  window trim, an append outside ``plan``) rebuilds them once, uploaded
  through the same buffer;
* ``run``: on the device, in order on one stream, the CoW block copies, the
  new tokens' cache write, then decode attention through the tables.

A ``StepPlan`` points into buffers the next ``plan`` reuses: it is valid
until then.  Everything on the device runs in libpa's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from .allocator import PaAllocator
from ._lib import PA_SWAP_IN, PA_SWAP_OUT, check, lib
from .ops import (FP8, _stream, alloc_workspace, pa_copy_blocks, pa_decode,
                  pa_reshape_and_cache, pa_swap_blocks)

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class StepPlan:
    """Device-resident index arrays of one decode step (valid until the
    next ``plan``)."""
    seqs: List[int]
    slots: torch.Tensor         # int64 [T]
    pairs: torch.Tensor         # int32 [P][2]
    tables: torch.Tensor        # int32 [B][max_blocks], -1 past each sequence's blocks
    lens: torch.Tensor          # int32 [B]
    max_context_len: int
    host_lens: np.ndarray
    rebuilt: bool = True        # tables uploaded whole (else patched from the slots)


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


class _Staging:
    """One step's index arrays: a pinned host buffer and its device copy.
    Layout: slots int64 [B*n] | lens int32 [B] | pairs int32 [B][2] |
    tables int32 [B][max_blocks] (rebuilds only)."""

    def __init__(self, n_seqs: int, n_tokens: int, max_blocks: int, device):
        self.n_seqs, self.n_tokens, self.max_blocks = n_seqs, n_tokens, max_blocks
        self.o_lens = _align(8 * max(n_seqs * n_tokens, 1))
        self.o_pairs = self.o_lens + _align(4 * max(n_seqs, 1))
        self.o_tables = self.o_pairs + _align(8 * max(n_seqs, 1))
        self.nbytes = self.o_tables + 4 * max(n_seqs * max_blocks, 1)
        self.host = torch.empty(self.nbytes, dtype=torch.uint8, pin_memory=True)
        self.dev = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.seqs = torch.empty(max(n_seqs, 1), dtype=torch.int64, pin_memory=True)
        h = self.host.numpy()
        self.h_slots = h[:self.o_lens].view(np.int64)
        self.h_lens = h[self.o_lens:self.o_pairs].view(np.int32)
        self.h_pairs = h[self.o_pairs:self.o_tables].view(np.int32).reshape(-1, 2)
        self.h_tables = h[self.o_tables:].view(np.int32)
        base = self.host.data_ptr()
        self.p_seqs = self.seqs.data_ptr()
        self.p_slots, self.p_lens, self.p_pairs = base, base + self.o_lens, base + self.o_pairs
        self.d_slots = self.dev[:self.o_lens].view(torch.int64)
        self.d_lens = self.dev[self.o_lens:self.o_pairs].view(torch.int32)
        self.d_pairs = self.dev[self.o_pairs:self.o_tables].view(torch.int32).view(-1, 2)
        self.d_tables = self.dev[self.o_tables:].view(torch.int32)
        self.done = None            # event after the upload that last read `host`
        self.key = None             # the sequence list `seqs` holds


class PagedKVCache:
    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype: str, initial_free_order: Optional[Sequence[int]] = None,
                 device="cuda", pools: Optional[tuple] = None, kv_dtype: Optional[str] = None,
                 kv_scales=(1.0, 1.0), sliding_window: int = 0):
        """dtype: activations (q, out, new K/V); kv_dtype "fp8_e4m3" stores
        the pools as E4M3 codes with per-pool kv_scales = (k_scale, v_scale);
        sliding_window: positions each query attends (0 = all)."""
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        self.kv_dtype = kv_dtype or dtype
        self.kv_scales = tuple(float(x) for x in kv_scales)
        self.sliding_window = int(sliding_window)
        self.device = torch.device(device)
        self.alloc = PaAllocator(num_blocks, block_size, initial_free_order)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        if pools is None:
            if self.kv_dtype == "fp8_e4m3":  # zero codes, allocated as bytes
                pools = tuple(torch.zeros(shape, dtype=torch.uint8, device=self.device).view(FP8)
                              for _ in range(2))
            else:
                tdt = TORCH_DTYPES[dtype]
                pools = (torch.zeros(shape, dtype=tdt, device=self.device),
                         torch.zeros(shape, dtype=tdt, device=self.device))
        self.k_pool, self.v_pool = pools
        if tuple(self.k_pool.shape) != shape or tuple(self.v_pool.shape) != shape:
            raise ValueError(f"pools must be {shape}")
        # device-resident tables of the last planned batch: (seqs tuple,
        # allocator epoch right after that plan's append, tables [B][cap],
        # lens [B]); any other allocator change since moves the epoch on
        self._resident = None
        self._stages: List[Optional[_Staging]] = [None, None]
        self._turn = 0

    # ------------------------------------------------------------ sequences
    def create(self) -> int:
        return self.alloc.pa_seq_create()

    def fork(self, seq: int) -> int:
        return self.alloc.pa_seq_fork(seq)

    def share_prefix(self, seq: int, n_tokens: int) -> int:
        return self.alloc.pa_seq_share_prefix(seq, n_tokens)

    def free(self, seq: int) -> None:
        self.alloc.pa_seq_free(seq)

    def reserve(self, seq: int, n_tokens: int):
        """Host only: slots for the next n tokens of seq (and a CoW pair)."""
        return self.alloc.pa_seq_append(seq, n_tokens)

    # ------------------------------------------------------------ prefix cache
    def enable_prefix_cache(self) -> None:
        self.alloc.pa_alloc_enable_prefix_cache()

    def create_prefix(self, token_ids: Sequence[int]):
        """A sequence for a prompt: (seq, hit_tokens); the prompt's first
        hit_tokens positions are cached blocks already holding their K/V."""
        return self.alloc.pa_seq_create_prefix(token_ids)

    def reserve_tokens(self, seq: int, token_ids: Sequence[int]):
        """``reserve`` with the new positions' token ids, so that full blocks
        can be cached for later prompts."""
        return self.alloc.pa_seq_append_tokens(seq, token_ids)

    def prefix_stats(self) -> dict:
        return self.alloc.pa_prefix_cache_stats()

    def trim_window(self, seq: int, window: int) -> int:
        """Host only: release seq's blocks that a sliding window of `window`
        positions will never read again."""
        return self.alloc.pa_seq_trim_window(seq, window)

    # ------------------------------------------------------------ swapping
    def enable_swap(self, num_host_blocks: int) -> None:
        """A pinned host pool pair of num_host_blocks blocks for preempted
        sequences."""
        self.alloc.pa_alloc_enable_swap(num_host_blocks)
        shape = (num_host_blocks,) + tuple(self.k_pool.shape[1:])
        self.k_host = torch.empty(shape, dtype=self.k_pool.dtype, pin_memory=True)
        self.v_host = torch.empty(shape, dtype=self.k_pool.dtype, pin_memory=True)

    def swap_out(self, seq: int, stream=None) -> np.ndarray:
        """Move seq's private blocks to the host pool (copies queued on the
        stream before anything else can write the released blocks)."""
        pairs = self.alloc.pa_seq_swap_out(seq)
        if pairs.shape[0]:
            pa_swap_blocks(self.k_pool, self.v_pool, self.k_host, self.v_host,
                           self._dev(pairs, torch.int32), PA_SWAP_OUT, stream)
        return pairs

    def swap_in(self, seq: int, stream=None) -> np.ndarray:
        """Bring seq back into device blocks (copies queued on the stream)."""
        pairs = self.alloc.pa_seq_swap_in(seq)
        if pairs.shape[0]:
            pa_swap_blocks(self.k_pool, self.v_pool, self.k_host, self.v_host,
                           self._dev(pairs, torch.int32), PA_SWAP_IN, stream)
        return pairs

    # ------------------------------------------------------------ device work
    def _dev(self, a: np.ndarray, dtype) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device, dtype)

    def write(self, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor,
              pairs: Optional[torch.Tensor] = None, stream=None) -> None:
        """CoW copies first, then the cache write of the new tokens."""
        if pairs is not None and pairs.shape[0] > 0:
            pa_copy_blocks(self.k_pool, self.v_pool, pairs, stream)
        if slots.shape[0] > 0:
            pa_reshape_and_cache(k, v, slots, self.k_pool, self.v_pool, stream, self.kv_scales)

    def write_host(self, k: torch.Tensor, v: torch.Tensor, slots: np.ndarray, pairs) -> None:
        pr = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
        self.write(k, v, self._dev(slots, torch.int64), self._dev(pr, torch.int32))

    def _stage(self, n: int, n_tokens: int, max_blocks: int) -> _Staging:
        """The staging buffer of this turn (two alternate, so the host fills
        one while the other's upload may still be in flight), grown to fit."""
        st = self._stages[self._turn]
        if st is None or st.n_seqs < n or st.n_tokens < n_tokens or st.max_blocks < max_blocks:
            if st is not None and st.done is not None:
                st.done.synchronize()
            grow = max(max_blocks, 8 if st is None else st.max_blocks)
            st = _Staging(n, n_tokens, grow, self.device)
            self._stages[self._turn] = st
        elif st.done is not None:
            st.done.synchronize()          # its last upload has read the host buffer
        return st

    def plan(self, seqs: Sequence[int], n_tokens: int = 1,
             max_blocks: Optional[int] = None, stream=None) -> StepPlan:
        """Reserve n_tokens per sequence (one batched allocator call) and put
        the step's index arrays on the device: one upload of the staging
        buffer, then either the resident tables patched from the new slots
        (``pa_update_tables``) or, after any other change, rebuilt whole."""
        seqs = [int(s) for s in seqs]
        n = len(seqs)
        key = tuple(seqs)
        res = self._resident
        cap_guess = res[2].shape[1] if res is not None and res[0] == key else 0
        st = self._stage(n, n_tokens, max(cap_guess, max_blocks or 0))
        if st.key != key:
            st.seqs.numpy()[:n] = seqs
            st.key = key
        npairs = self.alloc.append_batch_into(st.p_seqs, n, n_tokens, st.p_slots, st.p_pairs,
                                              st.p_lens) if n else 0
        lens = st.h_lens[:n].copy()
        max_len = int(lens.max(initial=0))
        need = -(-max_len // self.block_size)
        s = torch.cuda.current_stream() if stream is None else stream
        incremental = (res is not None and res[0] == key and res[1] == self.alloc.epoch - 1 and
                       need <= res[2].shape[1] and (max_blocks is None or
                                                    max_blocks == res[2].shape[1]))
        if incremental:
            tables, dlens = res[2], res[3]
            self._resident = (key, self.alloc.epoch, tables, dlens)
            nbytes = st.o_pairs + 8 * npairs
        else:
            cap = max(max_blocks if max_blocks is not None else -(-need // 8) * 8, need, 1)
            if cap > st.max_blocks:       # the rebuilt tables must fit the buffer
                old = st
                st = _Staging(max(n, old.n_seqs), max(n_tokens, old.n_tokens), cap, self.device)
                st.h_slots[:n * n_tokens] = old.h_slots[:n * n_tokens]
                st.h_lens[:n] = old.h_lens[:n]
                st.h_pairs[:npairs] = old.h_pairs[:npairs]
                st.seqs.numpy()[:n] = seqs
                st.key = key
                self._stages[self._turn] = st
            ht = st.h_tables[:n * cap]
            check("pa_build_tables", lib().pa_build_tables(
                self.alloc._h, C.cast(st.p_seqs, C.POINTER(C.c_int64)), n, cap,
                C.cast(ht.ctypes.data, C.POINTER(C.c_int32)),
                C.cast(st.p_lens, C.POINTER(C.c_int32))))
            nbytes = st.o_pairs + 8 * npairs
        with torch.cuda.stream(s):
            st.dev[:nbytes].copy_(st.host[:nbytes], non_blocking=True)
            if incremental:
                check("pa_update_tables", lib().pa_update_tables(
                    st.d_slots.data_ptr(), st.d_lens.data_ptr(), n, n_tokens, self.block_size,
                    tables.data_ptr(), tables.shape[1], dlens.data_ptr(), _stream(s)))
            else:   # new resident tables and lengths, straight from the pinned buffer
                tables = torch.empty((max(n, 1), cap), dtype=torch.int32, device=self.device)[:n]
                dlens = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)[:n]
                host_i32 = st.host[st.o_tables:].view(torch.int32)
                tables.copy_(host_i32[:n * cap].view(n, cap), non_blocking=True)
                dlens.copy_(st.host[st.o_lens:st.o_pairs].view(torch.int32)[:n],
                            non_blocking=True)
                self._resident = (key, self.alloc.epoch, tables, dlens)
            st.done = torch.cuda.Event()
            st.done.record(s)
        self._turn ^= 1
        return StepPlan(seqs, st.d_slots[:n * n_tokens], st.d_pairs[:npairs], tables, dlens,
                        max_len, lens, rebuilt=not incremental)

    def workspace(self, num_seqs: int, num_q_heads: int, max_context_len: int,
                  partition_tokens: int = 0):
        return alloc_workspace(self.k_pool, num_seqs, num_q_heads, max_context_len,
                               partition_tokens)

    def decode(self, plan: StepPlan, q: torch.Tensor, scale: float, out: torch.Tensor,
               workspace: Optional[torch.Tensor], partition_tokens: int = 0, stream=None):
        return pa_decode(q, self.k_pool, self.v_pool, plan.tables, plan.lens, scale, out,
                         workspace, plan.max_context_len, partition_tokens, stream,
                         self.sliding_window, self.kv_scales)

    def run(self, plan: StepPlan, k_new, v_new, q, scale, out, workspace,
            partition_tokens: int = 0, stream=None):
        """The device half of a decode step: copies, cache write, attention."""
        self.write(k_new, v_new, plan.slots, plan.pairs, stream)
        return self.decode(plan, q, scale, out, workspace, partition_tokens, stream)
