"""A paged KV cache for one attention layer: device pools plus the host
allocator, and the decode step over them.

A step has a host half and a device half:

* ``plan``: the allocator reserves one slot per new token (taking blocks
  lazily, copying shared blocks on write) and the block tables and lengths
  of the sequences to decode are built; the small index arrays are copied to
  the device once;
* ``run``: on the device, in order on one stream, the CoW block copies, the
  new tokens' cache write, then decode attention through the tables.

Everything on the device runs in libpa's HIP kernels.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from .allocator import PaAllocator
from ._lib import PA_SWAP_IN, PA_SWAP_OUT
from .ops import (FP8, alloc_workspace, pa_copy_blocks, pa_decode, pa_reshape_and_cache,
                  pa_swap_blocks)

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class StepPlan:
    """Device-resident index arrays of one decode step."""
    seqs: List[int]
    slots: torch.Tensor         # int64 [T]
    pairs: torch.Tensor         # int32 [P][2]
    tables: torch.Tensor        # int32 [B][max_blocks]
    lens: torch.Tensor          # int32 [B]
    max_context_len: int
    host_lens: np.ndarray


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

    def plan(self, seqs: Sequence[int], n_tokens: int = 1,
             max_blocks: Optional[int] = None) -> StepPlan:
        """Reserve n_tokens per sequence and upload the step's index arrays."""
        seqs = [int(s) for s in seqs]
        slots, pairs = self.alloc.pa_seq_append_batch(seqs, n_tokens)
        lens = np.array([self.alloc.pa_seq_info(s)[0] for s in seqs], dtype=np.int32)
        if max_blocks is None:
            max_blocks = int(-(-int(lens.max(initial=0)) // self.block_size))
        tables, lens = self.alloc.pa_build_tables(seqs, max(max_blocks, 1))
        return StepPlan(seqs, self._dev(slots, torch.int64), self._dev(pairs, torch.int32),
                        self._dev(tables, torch.int32), self._dev(lens, torch.int32),
                        int(lens.max(initial=0)), lens)

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
