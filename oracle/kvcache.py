"""Oracle cache write and CoW block copy on raw element bits.  Test
infrastructure only.

Pool layout (both pools): [num_blocks][num_kv_heads][block_size][head_dim];
element (block b, head h, offset o, dim d) holds token ``b*BS + o``'s value
for kv head h.  Values are raw bit patterns (uint32 for f32, uint16 for
f16/bf16), so both operations are bit-exact by construction.

* ``write_slots``: decode reads every earlier token's K/V and appends the
  new token's K/V ("Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统中的应用",
  section 2.1); the slot says where: physical block ``slot // BS``, offset
  ``slot % BS`` ("放下账簿，打开源码", section "PagedAttention：虚实分离，按需取用").
  A negative slot means "no write".
* ``copy_blocks``: the copy-on-write copy of a whole shared block before the
  writer's first write ("Lazy Allocation 与 Copy-on-Write ...", section 4.4).
  Pairs are applied in order, all before any write of the same step.
* ``write_slots_fp8``: the cache write into an 8-bit pool: each element is
  quantised (``oracle.fp8.quantize``) with the pool's scale as it is stored.
* ``swap_blocks``: a preempted sequence's blocks moved one by one between the
  device pool and a host pool of the same block shape ("vLLM：把 KV 缓存当成
  虚拟内存", section "碎片从哪里来").
"""
from __future__ import annotations

import numpy as np


def write_slots(pool: np.ndarray, new: np.ndarray, slots: np.ndarray) -> None:
    """pool[slot // BS, :, slot % BS, :] = new[t] for every t with slot >= 0.

    pool: [NB][Hkv][BS][D] bits (modified in place); new: [T][Hkv][D] bits;
    slots: [T] int64.
    """
    bs = pool.shape[2]
    slots = np.asarray(slots, dtype=np.int64)
    for t in range(slots.shape[0]):
        s = int(slots[t])
        if s < 0:
            continue
        pool[s // bs, :, s % bs, :] = new[t]


def copy_blocks(pool: np.ndarray, pairs) -> None:
    """pool[dst] = pool[src] for each (src, dst), in order."""
    for src, dst in pairs:
        pool[int(dst)] = pool[int(src)]


def swap_blocks(src_pool: np.ndarray, dst_pool: np.ndarray, pairs) -> None:
    """dst_pool[d] = src_pool[s] for each (s, d): whole blocks between two
    pools of the same block shape (device -> host or host -> device)."""
    for src, dst in pairs:
        dst_pool[int(dst)] = src_pool[int(src)]


def write_slots_fp8(pool: np.ndarray, new_values: np.ndarray, slots: np.ndarray,
                    scale: float) -> None:
    """``write_slots`` into an E4M3 pool of uint8 codes: new_values [T][Hkv][D]
    are float32 K or V values, quantised with the pool's scale."""
    from .fp8 import quantize
    write_slots(pool, quantize(new_values, scale), slots)

