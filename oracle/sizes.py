"""KV-cache sizes.  Test infrastructure only.

Every layer stores one K and one V vector per kv head per token, so the
cache holds 2 x layers x tokens x kv_heads x head_dim x element bytes x
requests bytes ("Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统中的应用",
section 2.2; "放下账簿，打开源码", section "KV Cache：推理的工作记忆").
"""
from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_cache_bytes(layers: int, seq_len: int, kv_heads: int, head_dim: int,
                   elem_bytes: int, batch: int) -> int:
    return kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes) * seq_len * batch


def blocks_for_tokens(tokens: int, block_size: int) -> int:
    return -(-tokens // block_size)


def pool_bytes(num_blocks: int, block_size: int, kv_heads: int, head_dim: int,
               elem_bytes: int) -> int:
    """Both pools of one layer: K and V, each [NB][Hkv][BS][D]."""
    return 2 * num_blocks * kv_heads * block_size * head_dim * elem_bytes
