"""Oracle decode attention in float64.  Test infrastructure only.

Paging changes where K/V rows are stored, not the attention formula: the
kernel follows the block table to find each logical block's physical block,
and the result is plain scaled dot-product attention over the sequence's
tokens (page "vLLM：把 KV 缓存当成虚拟内存", sections "破除误解" and
"跨域连接"; page "放下账簿，打开源码", section "注意力计算的改写", whose dense
form is softmax(Q K^T / sqrt(d_k)) V).

So the oracle (1) walks a sequence's block table in logical order and
concatenates the physical blocks, (2) keeps the first ``ctx`` token rows (the
tokens the sequence has actually produced; slots past them in the last block
are not part of the sequence), (3) decodes the element bits to float64 and
(4) runs textbook softmax attention per query head.

Readings where the pages are silent:

* q head ``h`` reads kv head ``h // (Hq / Hkv)`` (grouped-query attention in
  contiguous groups).
* No mask other than the length: a decode query sees every cached token and
  its own (already written) token.
* The page's block-loop pseudocode leaves its running maximum undefined and
  does not rescale; ``partitioned_decode`` states the standard online-softmax
  merge (running max, rescaled sums) and is pinned to ``paged_decode``.

Variants (the pages list sliding windows and the cache's element type among
the things the paged kernel must follow: "vLLM：把 KV 缓存当成虚拟内存", the
paragraph on variants; no formula is given):

* ``window`` W > 0: a token at position p attends positions max(0, p - W + 1)
  .. p, i.e. its own and the W - 1 before it.  A decode query sits at
  position ctx - 1.
* An 8-bit pool (``kv_dtype="fp8_e4m3"``) holds E4M3 codes; element value =
  code value * k_scale (K) or * v_scale (V); q and outputs keep ``dtype``.
"""
from __future__ import annotations

import math

import numpy as np

from . import fp8


def decode_bits(bits: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Element bit patterns -> float64 values (an 8-bit pool's codes times
    its scale)."""
    if dtype == "fp8_e4m3":
        return fp8.dequantize(bits, scale)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # a bf16 value is the top half of the float32 with the same sign,
        # exponent and leading mantissa bits
        wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):   # signalling-NaN patterns widen to NaN
            return wide.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather_sequence(pool: np.ndarray, table_row, ctx: int, first: int = 0) -> np.ndarray:
    """Reassemble tokens first .. ctx - 1 of one sequence from a pool
    [NB][Hkv][BS][D]: logical block j is physical block table_row[j] (only
    the blocks holding those positions are read); returns [ctx - first][Hkv][D]."""
    bs = pool.shape[2]
    j0 = first // bs
    n_blocks = -(-ctx // bs)
    pieces = []
    for j in range(j0, n_blocks):
        blk = int(table_row[j])
        pieces.append(np.transpose(pool[blk], (1, 0, 2)))  # [BS][Hkv][D]
    rows = np.concatenate(pieces, axis=0)
    return rows[first - j0 * bs:ctx - j0 * bs]


def window_start(pos: int, window: int) -> int:
    """First position a token at ``pos`` attends (0 without a window)."""
    return max(0, pos - window + 1) if window > 0 else 0


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Textbook attention for one decode query.

    q [Hq][D], k and v [ctx][Hkv][D] (float64) -> out [Hq][D]:
    out[h] = sum_t softmax_t(scale * <q[h], k[t, g]>) * v[t, g], g = h // G.
    """
    hq = q.shape[0]
    hkv = k.shape[1]
    group = hq // hkv
    out = np.empty_like(q)
    for h in range(hq):
        g = h // group
        s = scale * (k[:, g, :] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ v[:, g, :]) / p.sum()
    return out


def paged_decode(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
                 scale: float, dtype: str, seqs=None, window: int = 0, kv_dtype=None,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Decode attention for every sequence (or the listed ``seqs``).

    q_bits [B][Hq][D]; pools [NB][Hkv][BS][D]; block_tables [B][max_blocks];
    context_lens [B].  With ``window`` the query (position ctx - 1) attends
    only positions window_start(ctx - 1, window) .. ctx - 1.  ``kv_dtype``
    (default ``dtype``) is the pools' element type.  Returns float64
    [len(seqs)][Hq][D].
    """
    if seqs is None:
        seqs = range(q_bits.shape[0])
    kvt = kv_dtype or dtype
    outs = []
    for i in seqs:
        ctx = int(context_lens[i])
        first = window_start(ctx - 1, window)
        k = decode_bits(gather_sequence(k_pool_bits, block_tables[i], ctx, first), kvt, k_scale)
        v = decode_bits(gather_sequence(v_pool_bits, block_tables[i], ctx, first), kvt, v_scale)
        q = decode_bits(q_bits[i], dtype)
        outs.append(dense_attention(q, k, v, scale))
    return np.stack(outs) if outs else np.zeros((0,) + q_bits.shape[1:])


def partition_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """One partition's softmax state for each q head: running maximum m,
    sum l = sum_t exp(s_t - m) and unnormalised o = sum_t exp(s_t - m) v_t."""
    hq = q.shape[0]
    group = hq // k.shape[1]
    m = np.empty(hq)
    l = np.empty(hq)
    o = np.empty_like(q)
    for h in range(hq):
        g = h // group
        s = scale * (k[:, g, :] @ q[h])
        m[h] = s.max()
        e = np.exp(s - m[h])
        l[h] = e.sum()
        o[h] = e @ v[:, g, :]
    return m, l, o


def merge_partitions(ms, ls, os_):
    """Combine partition states: with M = max_p m_p and w_p = exp(m_p - M),
    out = sum_p w_p o_p / sum_p w_p l_p."""
    ms = np.asarray(ms)
    big_m = ms.max(axis=0)
    w = np.exp(ms - big_m)
    num = np.einsum("ph,phd->hd", w, np.asarray(os_))
    den = np.einsum("ph,ph->h", w, np.asarray(ls))
    return num / den[:, None]


def partitioned_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       partition_tokens: int) -> np.ndarray:
    """Split the sequence into runs of ``partition_tokens`` tokens, compute
    each run's (m, l, o) and merge them (split-K with a log-sum-exp merge)."""
    ctx = k.shape[0]
    n_parts = max(1, math.ceil(ctx / partition_tokens))
    states = [partition_state(q, k[p * partition_tokens:(p + 1) * partition_tokens],
                              v[p * partition_tokens:(p + 1) * partition_tokens], scale)
              for p in range(n_parts)]
    return merge_partitions([s[0] for s in states], [s[1] for s in states],
                            [s[2] for s in states])


def paged_prefill(q_bits, k_pool_bits, v_pool_bits, block_tables, query_start, context_lens,
                  scale: float, dtype: str, window: int = 0, kv_dtype=None, k_scale: float = 1.0,
                  v_scale: float = 1.0) -> np.ndarray:
    """Chunked-prefill attention for a batch of sequences.

    Prefill runs a prompt's tokens through attention and writes their K/V
    into the cache; a long prompt can be cut into chunks that run between
    decode steps (page "附录：Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统中的
    应用" §2.1; page "vLLM：把 KV 缓存当成虚拟内存", section "KV 的体积从哪来，页表
    如何把它切开").  Sequence ``i``'s chunk is the ``n_i = query_start[i+1] -
    query_start[i]`` query rows ``q_bits[query_start[i]:query_start[i+1]]``,
    its tokens at positions ``ctx_i - n_i .. ctx_i - 1`` (``ctx_i`` =
    ``context_lens[i]`` counts the chunk, whose K/V are already written).
    Each token attends to itself and every earlier position of its sequence
    (the autoregressive rule of the same §2.1): chunk token ``j`` sees
    positions ``0 .. ctx_i - n_i + j``.  A token whose position would be
    negative (``ctx_i < n_i``) has an all-zero row.

    With ``window`` token j sees only positions window_start(pos, window) ..
    pos; ``kv_dtype``, ``k_scale``, ``v_scale`` as in ``paged_decode``.

    q_bits [T][Hq][D]; pools [NB][Hkv][BS][D]; block_tables [B][max_blocks];
    query_start [B+1]; context_lens [B].  Returns float64 [T][Hq][D].
    """
    out = np.zeros(q_bits.shape, dtype=np.float64)
    kvt = kv_dtype or dtype
    for i in range(len(context_lens)):
        a, b = int(query_start[i]), int(query_start[i + 1])
        n, ctx = b - a, int(context_lens[i])
        if n <= 0 or ctx <= 0:
            continue
        first = window_start(max(ctx - n, 0), window)   # the first row's window
        k = decode_bits(gather_sequence(k_pool_bits, block_tables[i], ctx, first), kvt, k_scale)
        v = decode_bits(gather_sequence(v_pool_bits, block_tables[i], ctx, first), kvt, v_scale)
        for j in range(n):
            pos = ctx - n + j
            if pos < 0:
                continue
            lo = window_start(pos, window) - first
            q = decode_bits(q_bits[a + j], dtype)
            out[a + j] = dense_attention(q, k[lo:pos + 1 - first], v[lo:pos + 1 - first], scale)
    return out


def paged_prefill_rows_at_once(q_bits, k_pool_bits, v_pool_bits, block_tables, query_start,
                               context_lens, scale: float, dtype: str, window: int = 0,
                               kv_dtype=None, k_scale: float = 1.0, v_scale: float = 1.0,
                               seqs=None) -> np.ndarray:
    """The attention of ``paged_prefill`` with all of a chunk's rows at once,
    for workloads too large for the row-by-row loop.

    Same arguments, readings and result (float64 [T][Hq][D]; rows of
    sequences not in ``seqs``, when given, stay zero).  Per sequence and q
    head h (kv head g = h // (Hq / Hkv)) it is the dense form
    softmax(scale Q K^T + M) V of the pages ("放下账簿，打开源码", section
    "注意力计算的改写") with the mask M written out: M[j, t] = 0 where chunk
    row j (position p = ctx - n + j) may attend key position t
    (window_start(p, W) <= t <= p) and -inf elsewhere; rows with p < 0 are
    zero.  Only the rounding order differs from the row-by-row loop.
    """
    out = np.zeros(q_bits.shape, dtype=np.float64)
    kvt = kv_dtype or dtype
    hq, hkv = q_bits.shape[1], k_pool_bits.shape[1]
    group = hq // hkv
    for i in (range(len(context_lens)) if seqs is None else seqs):
        a, b = int(query_start[i]), int(query_start[i + 1])
        n, ctx = b - a, int(context_lens[i])
        if n <= 0 or ctx <= 0:
            continue
        first = window_start(max(ctx - n, 0), window)
        k = decode_bits(gather_sequence(k_pool_bits, block_tables[i], ctx, first), kvt, k_scale)
        v = decode_bits(gather_sequence(v_pool_bits, block_tables[i], ctx, first), kvt, v_scale)
        pos = ctx - n + np.arange(n)                      # each row's position
        keys = first + np.arange(ctx - first)             # each key's position
        lo = np.array([window_start(int(p), window) for p in pos])
        allowed = (keys[None, :] <= pos[:, None]) & (keys[None, :] >= lo[:, None])
        live = pos >= 0
        q = decode_bits(q_bits[a:b], dtype)               # [n][Hq][D]
        for h in range(hq):
            g = h // group
            s = scale * (q[:, h, :] @ k[:, g, :].T)       # [n][keys]
            s = np.where(allowed, s, -np.inf)
            m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
            p = np.exp(s - m[:, None])
            o = (p @ v[:, g, :]) / np.where(live, p.sum(axis=1), 1.0)[:, None]
            out[a:b, h, :] = np.where(live[:, None], o, 0.0)
    return out
