"""Requests sharing a system prompt, run through the oracle: allocator with
or without the prefix cache, cache writes of the computed positions, and the
inputs of the one prefill call that computes them."""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import OracleAllocator
from oracle.kvcache import write_slots


def run_prompts_oracle(ps, cached: bool):
    """Every request: look its prompt up (cached) or start empty, append the
    positions to compute with their token ids, write their K/V.  Returns the
    allocator, pools, tables, lengths, hits and the prefill call's q rows
    (the computed positions only) and query_start."""
    wl = ps.wl
    a = OracleAllocator(ps.num_blocks, wl.block_size, ps.free_order)
    if cached:
        a.enable_prefix_cache()
    shape = (ps.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    kp = np.zeros(shape, dtype=W.bits_dtype(wl.dtype))
    vp = np.zeros(shape, dtype=W.bits_dtype(wl.dtype))
    hits, q_rows = [], []
    for r in range(ps.requests):
        ids = W.prompt_token_ids(ps, r)
        if cached:
            s, hit = a.create_prefix(ids)
        else:
            s, hit = a.create(), 0
        slots, pair = a.append_tokens(s, ids[hit:])
        assert s == r and pair is None
        k, v = W.prompt_kv_bits_of(ps, r)
        write_slots(kp, k[hit:], np.asarray(slots))
        write_slots(vp, v[hit:], np.asarray(slots))
        q_rows.append(W.prompt_query_bits_of(ps, r)[hit:])
        hits.append(hit)
    lens = ps.prompt_lens
    max_blocks = int(-(-int(lens.max()) // wl.block_size))
    tables, lens32 = a.build_tables(list(range(ps.requests)), max_blocks)
    hits = np.array(hits, dtype=np.int64)
    qs = np.concatenate([[0], np.cumsum(lens - hits)]).astype(np.int64)
    return dict(alloc=a, kp=kp, vp=vp, tables=tables, lens=lens32, hits=hits,
                q=np.concatenate(q_rows), query_start=qs)
