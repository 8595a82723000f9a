"""Seeded synthetic inputs for the paged-attention decode workloads.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds no step of the method itself: no allocation policy, no cache write,
no attention arithmetic. It only draws lengths, random K/V/q values and the
initial free-block order, and rounds the float32 draws to the element type
the workload names (inputs, not results).

Workloads (shapes follow the pages' model sizes; all are one layer):

* ``tiny``   4 sequences attending {10, 5, 33, 7} tokens, 4 q heads = 4 kv
             heads, head_dim 64, fp32, block 16, 64-block pool.
* ``7b_mha`` 7B-shaped MHA: 32 q = 32 kv heads, head_dim 128, fp16, block 16,
             batch 64, lengths uniform in [128, 2048].  The 7B shape is the one
             whose per-token KV size the page "放下账簿，打开源码"
             (section "KV Cache：推理的工作记忆") works out.
* ``8b_gqa`` 8B GQA: 32 q heads, 8 kv heads, head_dim 128, bf16, block 16,
             batch 256, lengths log-normal (median 1500, sigma 0.8) clipped to
             [16, 8192].  Shape of chapter 6 of the AI-infra book
             ("第 6 章 缓存管理", section "分页：把缓存切成固定大小的块").
* ``cow``    parallel sampling: 32 prompts x 4 branches, 8B-GQA shape, bf16;
             a 1000-token prefix shared by fork, then per-branch tails uniform
             in [0, 256] plus one decode token.
* ``qwen32b_long``  64 q heads, 8 kv heads, head_dim 128, bf16, 32 sequences
             of 2048 tokens plus 4 of 32768, block 16 (``_bs32``: block 32).
* ``prefill_8b``  chunked prefill: 16 sequences, a 512-token chunk each on a
             cached prefix drawn like ``8b_gqa``'s lengths (clipped to [0, 7680]).
* ``prefix_1k``  requests sharing a system prompt (``prompt_set``): 100
             requests, one 1024-token system prompt (64 blocks of 16, the
             size "第 6 章 缓存管理" works through), each followed by its own
             user suffix of uniform [16, 256] tokens; 8B-GQA shape, bf16.

Context lengths here are the number of tokens a decode query attends to,
including the token being decoded (its K/V is written first).

Random streams: the workload's own generator ``default_rng(seed)`` draws the
lengths first and then the initial free-block permutation.  K/V of sequence
(or prompt / branch) ``i`` come from their own child stream so that a single
sequence can be regenerated without drawing the whole batch.
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Dict, List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    partition_tokens: int = 512
    # copy-on-write workload only
    num_prompts: int = 0
    branches: int = 0
    prefix_len: int = 0
    tail_max: int = 0
    # chunked-prefill workload only: sequences and new tokens per sequence
    batch: int = 0
    chunk: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, 4, 4, 64, "f32", 16),
    "7b_mha": Workload("7b_mha", 1, 32, 32, 128, "f16", 16),
    "8b_gqa": Workload("8b_gqa", 2, 32, 8, 128, "bf16", 16),
    "cow": Workload("cow", 3, 32, 8, 128, "bf16", 16, num_prompts=32, branches=4,
                    prefix_len=1000, tail_max=256),
    "qwen32b_long": Workload("qwen32b_long", 4, 64, 8, 128, "bf16", 16),
    "qwen32b_long_bs32": Workload("qwen32b_long_bs32", 4, 64, 8, 128, "bf16", 32),
    "prefill_8b": Workload("prefill_8b", 5, 32, 8, 128, "bf16", 16, batch=16, chunk=512),
}

# Prompt sets (``prompt_set``): requests sharing a system prompt.
PROMPT_WORKLOADS: Dict[str, Workload] = {
    "prefix_1k": Workload("prefix_1k", 6, 32, 8, 128, "bf16", 16, batch=100, prefix_len=1024,
                          tail_max=256),
}


@dataclasses.dataclass
class Draw:
    """Everything random about one workload instance."""
    wl: Workload
    context_lens: np.ndarray          # [B] int64, attended tokens per sequence
    num_blocks: int                   # physical pool size
    free_order: np.ndarray            # [num_blocks] int64 permutation
    tails: Optional[np.ndarray] = None  # cow only: [prompts][branches]
    # new tokens of the step per sequence: None = 1 (decode); else a chunked
    # prefill step whose chunk is the last chunk_lens[i] of ctx_i tokens
    chunk_lens: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def step_lens(self) -> np.ndarray:
        """New tokens per sequence in the step (1 for decode)."""
        if self.chunk_lens is None:
            return np.ones(self.batch, dtype=np.int64)
        return self.chunk_lens

    @property
    def query_start(self) -> np.ndarray:
        """[B+1] offsets of each sequence's query rows in the step."""
        return np.concatenate([[0], np.cumsum(self.step_lens)]).astype(np.int64)


def _blocks_for(n_tokens: np.ndarray, block_size: int) -> int:
    return int(np.sum((n_tokens + block_size - 1) // block_size))


def draw(name: str, batch: Optional[int] = None) -> Draw:
    """Draw lengths, pool size and free order for a named workload.

    ``batch`` truncates the batch (the first draws are kept), for small
    parity cases of the same distribution.
    """
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    tails = None
    if wl.name == "tiny":
        lens = np.array([10, 5, 33, 7], dtype=np.int64)
        nb = 64
    elif wl.name == "7b_mha":
        lens = rng.integers(128, 2048, 64, endpoint=True).astype(np.int64)
    elif wl.name == "8b_gqa":
        lens = np.clip(np.rint(rng.lognormal(math.log(1500.0), 0.8, 256)), 16, 8192).astype(np.int64)
    elif wl.name == "cow":
        tails = rng.integers(0, wl.tail_max, (wl.num_prompts, wl.branches), endpoint=True).astype(np.int64)
        lens = (wl.prefix_len + tails + 1).reshape(-1)
    elif wl.name.startswith("qwen32b_long"):
        lens = np.array([2048] * 32 + [32768] * 4, dtype=np.int64)
    elif wl.name == "prefill_8b":
        # chunked prefill: a 512-token chunk on top of a cached prefix drawn
        # like the decode workload's lengths
        prefix = np.clip(np.rint(rng.lognormal(math.log(1500.0), 0.8, wl.batch)), 0,
                         8192 - wl.chunk).astype(np.int64)
        lens = prefix + wl.chunk
    else:  # pragma: no cover
        raise KeyError(name)
    if batch is not None:
        if tails is not None:
            keep = max(1, batch // wl.branches)
            tails = tails[:keep]
            lens = (wl.prefix_len + tails + 1).reshape(-1)
        else:
            lens = lens[:batch]
    if wl.name != "tiny":
        # pool sized to 1.25x the unshared block demand of the batch
        nb = int(math.ceil(1.25 * _blocks_for(lens, wl.block_size)))
    free_order = rng.permutation(nb).astype(np.int64)
    chunks = np.full(lens.shape[0], wl.chunk, dtype=np.int64) if wl.chunk else None
    return Draw(wl, lens, nb, free_order, tails, chunks)


# ---------------------------------------------------------------- element bits

def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` (round to nearest even) and return
    the raw bit patterns (uint32 for f32, uint16 for f16/bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        return rounded.astype(np.uint16)
    raise ValueError(dtype)


def bits_dtype(dtype: str):
    return np.uint32 if dtype == "f32" else np.uint16


def _normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return to_bits(rng.standard_normal(shape, dtype=np.float32), dtype)


def query_bits(d: Draw) -> np.ndarray:
    """q for the decode step: [B][Hq][D] bits."""
    wl = d.wl
    rng = np.random.default_rng([wl.seed, 3])
    return _normal_bits(rng, (d.batch, wl.num_q_heads, wl.head_dim), wl.dtype)


def prefill_query_bits(d: Draw) -> np.ndarray:
    """q for a chunked-prefill step: [sum of chunk lengths][Hq][D] bits,
    sequence i's rows at query_start[i] .. query_start[i+1]."""
    wl = d.wl
    rng = np.random.default_rng([wl.seed, 5])
    return _normal_bits(rng, (int(d.step_lens.sum()), wl.num_q_heads, wl.head_dim), wl.dtype)


def sequence_kv_bits(d: Draw, i: int):
    """Contiguous K and V of sequence ``i`` for all of its attended tokens:
    two [ctx_i][Hkv][D] bit arrays.  For the copy-on-write workload, the
    first ``prefix_len`` tokens come from the prompt's stream (identical for
    the prompt's branches) and the rest from the branch's own stream."""
    wl = d.wl
    ctx = int(d.context_lens[i])
    shape_tail = (wl.num_kv_heads, wl.head_dim)
    if wl.name == "cow":
        p, b = divmod(i, wl.branches)
        pk, pv = prompt_kv_bits(d, p)
        rng = np.random.default_rng([wl.seed, 2, p, b])
        n = ctx - wl.prefix_len
        tk = _normal_bits(rng, (n,) + shape_tail, wl.dtype)
        tv = _normal_bits(rng, (n,) + shape_tail, wl.dtype)
        return np.concatenate([pk, tk]), np.concatenate([pv, tv])
    rng = np.random.default_rng([wl.seed, 1, i])
    k = _normal_bits(rng, (ctx,) + shape_tail, wl.dtype)
    v = _normal_bits(rng, (ctx,) + shape_tail, wl.dtype)
    return k, v


def prompt_kv_bits(d: Draw, p: int):
    """Copy-on-write workload: K and V of prompt ``p``'s shared prefix."""
    wl = d.wl
    rng = np.random.default_rng([wl.seed, 1, p])
    shape = (wl.prefix_len, wl.num_kv_heads, wl.head_dim)
    return _normal_bits(rng, shape, wl.dtype), _normal_bits(rng, shape, wl.dtype)


def pool_fill_bits(d: Draw, nan: bool = False) -> List[np.ndarray]:
    """Initial contents of the K and V pools before any cache write:
    N(0,1) values, or NaN everywhere when ``nan`` (poisoned-padding runs).
    Returns [k_pool, v_pool], each [NB][Hkv][BS][D] bits."""
    wl = d.wl
    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    if nan:
        nan_bits = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}[wl.dtype]
        return [np.full(shape, nan_bits, dtype=bits_dtype(wl.dtype)) for _ in range(2)]
    rng = np.random.default_rng([wl.seed, 4])
    return [_normal_bits(rng, shape, wl.dtype) for _ in range(2)]


def kv_bytes(d: Draw) -> int:
    """Algorithmic K+V bytes one decode step reads: attended tokens only."""
    wl = d.wl
    return int(d.context_lens.sum()) * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes


# ---------------------------------------------------------------- scenario

def scenario(d: Draw):
    """The order of allocator operations that builds a workload's decode
    step, as phases of ops (structure only):

      ("create", i)              new sequence; ids come out 0, 1, 2, ...
      ("append", i, start, n)    sequence i writes its tokens start..start+n-1
                                 (values: ``sequence_kv_bits(d, i)[start:start+n]``)
      ("fork", parent, child)    child shares parent's blocks

    The last phase is the step: every sequence appends its last attended
    token (position ctx_i - 1), then attends ctx_i tokens; for a chunked
    prefill step it appends its last chunk_lens[i] tokens instead.

    copy-on-write workload: prompt p's first branch (id 4p) writes the
    1000-token prefix and is forked three times; then the branches write
    their tails in branch order; then the decode step.
    """
    wl = d.wl
    lens = d.context_lens
    if wl.name == "cow":
        setup = []
        for p in range(lens.shape[0] // wl.branches):
            base = p * wl.branches
            setup.append(("create", base))
            setup.append(("append", base, 0, wl.prefix_len))
            for b in range(1, wl.branches):
                setup.append(("fork", base, base + b))
        tails = [("append", i, wl.prefix_len, int(lens[i]) - 1 - wl.prefix_len)
                 for i in range(lens.shape[0]) if int(lens[i]) - 1 > wl.prefix_len]
        phases = [setup, tails]
    else:
        setup = []
        new = d.step_lens
        for i in range(lens.shape[0]):
            setup.append(("create", i))
            if lens[i] > new[i]:
                setup.append(("append", i, 0, int(lens[i] - new[i])))
        phases = [setup]
    step = [("append", i, int(lens[i] - d.step_lens[i]), int(d.step_lens[i]))
            for i in range(lens.shape[0])]
    return phases + [step]


def custom(seed: int, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
           block_size: int, lens, spare_blocks: int = 7, chunk_lens=None) -> Draw:
    """A workload of any supported shape with given attended lengths (for
    parity cases beyond the named workloads).  The pool holds every needed
    block plus ``spare_blocks``; the free order is a seeded permutation.
    ``chunk_lens`` makes the step a chunked prefill of that many tokens."""
    wl = Workload(f"custom{seed}", seed, num_q_heads, num_kv_heads, head_dim, dtype, block_size)
    lens = np.asarray(lens, dtype=np.int64)
    nb = _blocks_for(np.maximum(lens, 0), block_size) + spare_blocks
    free_order = np.random.default_rng(seed).permutation(nb).astype(np.int64)
    chunks = None if chunk_lens is None else np.asarray(chunk_lens, dtype=np.int64)
    return Draw(wl, lens, nb, free_order, None, chunks)


# ---------------------------------------------------------------- shared prompts

@dataclasses.dataclass
class PromptSet:
    """Requests that open with one shared system prompt, each followed by its
    own suffix.  Token ids, K/V and q of the system prompt's positions are the
    same for every request (they depend only on the tokens before them); the
    suffix's come from the request's own stream."""
    wl: Workload
    system_len: int
    suffix_lens: np.ndarray           # [R] int64
    num_blocks: int                   # pool for every request unshared, x1.25
    free_order: np.ndarray

    @property
    def requests(self) -> int:
        return int(self.suffix_lens.shape[0])

    @property
    def prompt_lens(self) -> np.ndarray:
        return self.system_len + self.suffix_lens


def prompt_set(name: str = "prefix_1k", requests: Optional[int] = None) -> PromptSet:
    wl = PROMPT_WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    suffix = rng.integers(16, wl.tail_max, wl.batch, endpoint=True).astype(np.int64)
    if requests is not None:
        suffix = suffix[:requests]
    return _prompt_set(wl, wl.prefix_len, suffix, rng)


def custom_prompt_set(seed: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      dtype: str, block_size: int, system_len: int, suffix_lens) -> PromptSet:
    wl = Workload(f"custom{seed}", seed, num_q_heads, num_kv_heads, head_dim, dtype, block_size,
                  prefix_len=system_len)
    return _prompt_set(wl, system_len, np.asarray(suffix_lens, dtype=np.int64),
                       np.random.default_rng(seed))


def _prompt_set(wl: Workload, system_len: int, suffix: np.ndarray, rng) -> PromptSet:
    nb = int(math.ceil(1.25 * _blocks_for(system_len + suffix, wl.block_size))) + 4
    return PromptSet(wl, system_len, suffix, nb, rng.permutation(nb).astype(np.int64))


def prompt_token_ids(ps: PromptSet, r: int) -> List[int]:
    """Token ids of request r's prompt (int32 range)."""
    wl = ps.wl
    system = np.random.default_rng([wl.seed, 6]).integers(0, 50000, ps.system_len)
    own = np.random.default_rng([wl.seed, 7, r]).integers(0, 50000, int(ps.suffix_lens[r]))
    return [int(t) for t in np.concatenate([system, own])]


@functools.lru_cache(maxsize=6)
def _shared_bits(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    out = _normal_bits(np.random.default_rng([seed, stream, 0]), shape, dtype)
    out.flags.writeable = False
    return out


def _shared_then_own(ps: PromptSet, r: int, stream: int, width: int):
    wl = ps.wl
    shared = _shared_bits(wl.seed, stream, (ps.system_len, width, wl.head_dim), wl.dtype)
    own = _normal_bits(np.random.default_rng([wl.seed, stream, 1, r]),
                       (int(ps.suffix_lens[r]), width, wl.head_dim), wl.dtype)
    return np.concatenate([shared, own])


def prompt_kv_bits_of(ps: PromptSet, r: int):
    """K and V of request r's prompt: two [len][Hkv][D] bit arrays."""
    h = ps.wl.num_kv_heads
    return _shared_then_own(ps, r, 8, h), _shared_then_own(ps, r, 9, h)


def prompt_query_bits_of(ps: PromptSet, r: int) -> np.ndarray:
    """q of request r's prompt positions: [len][Hq][D] bits."""
    return _shared_then_own(ps, r, 10, ps.wl.num_q_heads)
