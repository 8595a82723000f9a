"""Python binding of the libpa kernels: torch tensors in, C ABI calls out.

Each function has the name of the C entry point it calls and only marshals
arguments (shapes, dtypes, device pointers, the current HIP stream); every
step runs in the HIP kernels.  PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from ._lib import (PA_BF16, PA_F16, PA_F32, PA_KV_FP8_E4M3, PA_KV_SAME, check, lib,
                   pa_pool_desc)

_DTYPES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
FP8 = torch.float8_e4m3fn  # 8-bit pool element (E4M3, the OCP "fn" variant)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: Optional[torch.Tensor]) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _need_cuda(name: str, t: torch.Tensor, dtype=None, contiguous=True) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pool_desc(k_pool: torch.Tensor, act_dtype=None, kv_scales=(1.0, 1.0)) -> pa_pool_desc:
    """Descriptor of a [num_blocks][num_kv_heads][block_size][head_dim] pool.
    An 8-bit (float8_e4m3fn) pool needs the activation dtype (q, out, new
    K/V rows; bf16 when only the block size matters) and its (k, v) scales."""
    if k_pool.dim() != 4:
        raise ValueError("pools are [num_blocks][num_kv_heads][block_size][head_dim]")
    nb, hkv, bs, d = k_pool.shape
    if k_pool.dtype == FP8:
        act = act_dtype or torch.bfloat16
        if act not in _DTYPES:
            raise ValueError(f"unsupported activation dtype {act}")
        return pa_pool_desc(nb, bs, hkv, d, _DTYPES[act], PA_KV_FP8_E4M3, float(kv_scales[0]),
                            float(kv_scales[1]))
    if k_pool.dtype not in _DTYPES:
        raise ValueError(f"unsupported pool dtype {k_pool.dtype}")
    if act_dtype is not None and act_dtype != k_pool.dtype:
        raise ValueError(f"activations must be {k_pool.dtype}, got {act_dtype}")
    return pa_pool_desc(nb, bs, hkv, d, _DTYPES[k_pool.dtype], PA_KV_SAME, 1.0, 1.0)


def _check_pools(k_pool, v_pool, act_dtype=None, kv_scales=(1.0, 1.0)):
    _need_cuda("k_pool", k_pool)
    _need_cuda("v_pool", v_pool, k_pool.dtype)
    if v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    return pool_desc(k_pool, act_dtype, kv_scales)


def _act_dtype(k_pool, t):
    """Activation dtype: the pool's, or t's for an 8-bit pool."""
    return t.dtype if k_pool.dtype == FP8 else k_pool.dtype


def pa_decode_workspace_bytes(pool, num_seqs: int, num_q_heads: int, max_context_len: int,
                              partition_tokens: int = 0) -> int:
    """Workspace bytes for pa_decode; `pool` is a pa_pool_desc or the K pool tensor."""
    desc = pool if isinstance(pool, pa_pool_desc) else pool_desc(pool)
    return int(lib().pa_decode_workspace_bytes(C.byref(desc), num_seqs, num_q_heads,
                                               max_context_len, partition_tokens))


def alloc_workspace(k_pool: torch.Tensor, num_seqs: int, num_q_heads: int, max_context_len: int,
                    partition_tokens: int = 0):
    """A workspace tensor sized for pa_decode on this pool (None when none is needed)."""
    n = pa_decode_workspace_bytes(k_pool, num_seqs, num_q_heads, max_context_len,
                                  partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=k_pool.device) if n else None


def _status_ptr(status: Optional[torch.Tensor]) -> C.c_void_p:
    """A device int32 tensor (at least one element) the kernels OR status
    bits into (PA_STATUS_BAD_BLOCK), or None."""
    if status is None:
        return C.c_void_p(0)
    _need_cuda("status", status, torch.int32)
    if status.numel() < 1:
        raise ValueError("status needs at least one element")
    return _ptr(status)


def _decode_call(fn_name, q, k_pool, v_pool, block_tables, context_lens, scale, out,
                 workspace, max_context_len, partition_tokens, stream, sliding_window, kv_scales,
                 status=None):
    act = _act_dtype(k_pool, q)
    desc = _check_pools(k_pool, v_pool, act, kv_scales)
    _need_cuda("q", q, act)
    _need_cuda("out", out, act)
    _need_cuda("block_tables", block_tables, torch.int32)
    _need_cuda("context_lens", context_lens, torch.int32)
    if q.dim() != 3 or q.shape[2] != desc.head_dim or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs][num_q_heads][head_dim]")
    b, hq, _ = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    ws_bytes = 0
    if workspace is not None:
        _need_cuda("workspace", workspace)
        ws_bytes = workspace.numel() * workspace.element_size()
    fn = getattr(lib(), fn_name)
    st = fn(_ptr(q), _ptr(k_pool), _ptr(v_pool), C.byref(desc), _ptr(block_tables),
            int(block_tables.shape[1]), _ptr(context_lens), int(b), int(hq),
            int(max_context_len), float(scale), int(sliding_window), _ptr(out), _ptr(workspace),
            ws_bytes, int(partition_tokens), _status_ptr(status), _stream(stream))
    check(fn_name, st)
    return out


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out, workspace,
              max_context_len, partition_tokens=0, stream=None, sliding_window=0,
              kv_scales=(1.0, 1.0), status=None):
    """Paged decode attention (partition + reduce).  See pa.h.  kv_scales:
    (k_scale, v_scale) of an 8-bit pool."""
    return _decode_call("pa_decode", q, k_pool, v_pool, block_tables, context_lens, scale, out,
                        workspace, max_context_len, partition_tokens, stream, sliding_window,
                        kv_scales, status)


def pa_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale, out,
                      max_context_len, partition_tokens=0, stream=None, sliding_window=0,
                      kv_scales=(1.0, 1.0), status=None):
    """pa_decode with the library's static device scratch as its workspace:
    the call allocates nothing (for callers that cannot).  See pa.h."""
    act = _act_dtype(k_pool, q)
    desc = _check_pools(k_pool, v_pool, act, kv_scales)
    _need_cuda("q", q, act)
    _need_cuda("out", out, act)
    _need_cuda("block_tables", block_tables, torch.int32)
    _need_cuda("context_lens", context_lens, torch.int32)
    if q.dim() != 3 or q.shape[2] != desc.head_dim or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs][num_q_heads][head_dim]")
    b, hq, _ = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != b or context_lens.shape != (b,):
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    st = lib().pa_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), C.byref(desc),
                                 _ptr(block_tables), int(block_tables.shape[1]),
                                 _ptr(context_lens), int(b), int(hq), int(max_context_len),
                                 float(scale), int(sliding_window), _ptr(out),
                                 int(partition_tokens), _status_ptr(status), _stream(stream))
    check("pa_decode_noalloc", st)
    return out


def pa_decode_partition(q, k_pool, v_pool, block_tables, context_lens, scale, out, workspace,
                        max_context_len, partition_tokens=0, stream=None, sliding_window=0,
                        kv_scales=(1.0, 1.0), status=None):
    return _decode_call("pa_decode_partition", q, k_pool, v_pool, block_tables, context_lens,
                        scale, out, workspace, max_context_len, partition_tokens, stream,
                        sliding_window, kv_scales, status)


def pa_decode_reduce(q, k_pool, v_pool, block_tables, context_lens, scale, out, workspace,
                     max_context_len, partition_tokens=0, stream=None, sliding_window=0,
                     kv_scales=(1.0, 1.0), status=None):
    return _decode_call("pa_decode_reduce", q, k_pool, v_pool, block_tables, context_lens,
                        scale, out, workspace, max_context_len, partition_tokens, stream,
                        sliding_window, kv_scales, status)


def pa_prefill(q, k_pool, v_pool, block_tables, query_start, context_lens, scale, out,
               max_query_len, max_context_len, stream=None, sliding_window=0,
               kv_scales=(1.0, 1.0), status=None):
    """Chunked prefill attention over the paged cache.  See pa.h.

    q, out [num_tokens][num_q_heads][head_dim]; query_start int32 [B+1];
    block_tables int32 [B][max_blocks]; context_lens int32 [B]."""
    act = _act_dtype(k_pool, q)
    desc = _check_pools(k_pool, v_pool, act, kv_scales)
    _need_cuda("q", q, act)
    _need_cuda("out", out, act)
    _need_cuda("block_tables", block_tables, torch.int32)
    _need_cuda("query_start", query_start, torch.int32)
    _need_cuda("context_lens", context_lens, torch.int32)
    if q.dim() != 3 or q.shape[2] != desc.head_dim or out.shape != q.shape:
        raise ValueError("q and out must be [num_tokens][num_q_heads][head_dim]")
    t, hq, _ = q.shape
    b = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != b or query_start.shape != (b + 1,):
        raise ValueError("block_tables must be [B][max_blocks], query_start [B+1], "
                         "context_lens [B]")
    st = lib().pa_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), C.byref(desc), _ptr(block_tables),
                          int(block_tables.shape[1]), _ptr(query_start), _ptr(context_lens),
                          int(b), int(t), int(hq), int(max_query_len), int(max_context_len),
                          float(scale), int(sliding_window), _ptr(out), _status_ptr(status),
                          _stream(stream))
    check("pa_prefill", st)
    return out


def pa_set_decode_path(path: int) -> int:
    prev = int(lib().pa_set_decode_path(int(path)))
    if prev < 0:
        raise ValueError(f"bad decode path {path}")
    return prev


def pa_set_decode_balance(on: bool) -> bool:
    """Run-time balance of the stream split on (default) or off; returns the
    previous setting.  See pa.h."""
    prev = int(lib().pa_set_decode_balance(int(bool(on))))
    if prev < 0:
        raise ValueError(f"bad balance setting {on}")
    return bool(prev)


def pa_set_prefill_path(path: int) -> int:
    prev = int(lib().pa_set_prefill_path(int(path)))
    if prev < 0:
        raise ValueError(f"bad prefill path {path}")
    return prev


def pa_reshape_and_cache(k, v, slot_mapping, k_pool, v_pool, stream=None, kv_scales=(1.0, 1.0)):
    """Write new tokens' K/V ([T][Hkv][D]) into their slots (quantised for an
    8-bit pool with kv_scales).  See pa.h."""
    act = _act_dtype(k_pool, k)
    desc = _check_pools(k_pool, v_pool, act, kv_scales)
    _need_cuda("k", k, act)
    _need_cuda("v", v, act)
    _need_cuda("slot_mapping", slot_mapping, torch.int64)
    t = slot_mapping.shape[0]
    shape = (t, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != shape or tuple(v.shape) != shape:
        raise ValueError(f"k and v must be {shape}")
    st = lib().pa_reshape_and_cache(_ptr(k), _ptr(v), _ptr(slot_mapping), int(t), _ptr(k_pool),
                                    _ptr(v_pool), C.byref(desc), _stream(stream))
    check("pa_reshape_and_cache", st)


def pa_copy_blocks(k_pool, v_pool, pairs, stream=None):
    """Copy whole blocks src -> dst for each (src, dst) row of pairs ([P][2] int32)."""
    desc = _check_pools(k_pool, v_pool)
    _need_cuda("pairs", pairs, torch.int32)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [num_pairs][2]")
    st = lib().pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), C.byref(desc), _ptr(pairs),
                              int(pairs.shape[0]), _stream(stream))
    check("pa_copy_blocks", st)


def pa_probe_tile_reads(pool, tile_offsets, tile_bytes: int, num_waves: int = 0, out=None,
                        pool2=None, stream=None):
    """Read the listed tiles of a pool (tile t: tile_bytes bytes at byte offset
    tile_offsets[t], uint32 values in an int32 device tensor), and of pool2 at
    the same offsets when given, with num_waves waves (0: the decode stream
    split's grid) and nothing else.  Returns the per-wave XOR of the words
    read (uint32 values, int32 storage).  See pa.h."""
    _need_cuda("pool", pool)
    nbytes = pool.numel() * pool.element_size()
    if pool2 is not None:
        _need_cuda("pool2", pool2)
        if pool2.numel() * pool2.element_size() != nbytes:
            raise ValueError("pool2 must have the size of pool")
    _need_cuda("tile_offsets", tile_offsets, torch.int32)
    if out is None:
        out = torch.empty(max(int(num_waves), 1024), dtype=torch.int32, device=pool.device)
    _need_cuda("out", out, torch.int32)
    waves = C.c_int32(0)
    st = lib().pa_probe_tile_reads(_ptr(pool), _ptr(pool2), nbytes, _ptr(tile_offsets),
                                   int(tile_offsets.numel()), int(tile_bytes), int(num_waves),
                                   _ptr(out), int(out.numel()), C.byref(waves), _stream(stream))
    check("pa_probe_tile_reads", st)
    return out[:waves.value]


def pa_swap_blocks(k_pool, v_pool, k_host, v_host, pairs, direction: int, stream=None):
    """Copy whole blocks between the device pools and pinned host pools of the
    same block shape: PA_SWAP_OUT copies device p[0] -> host p[1], PA_SWAP_IN
    host p[0] -> device p[1] for each row p of pairs ([P][2] int32, device).
    See pa.h."""
    desc = _check_pools(k_pool, v_pool)
    for name, h in (("k_host", k_host), ("v_host", v_host)):
        if h.device.type != "cpu" or not h.is_pinned() or not h.is_contiguous() \
                or h.dtype != k_pool.dtype or tuple(h.shape[1:]) != tuple(k_pool.shape[1:]):
            raise ValueError(f"{name} must be a contiguous pinned host tensor "
                             f"[NHB]{list(k_pool.shape[1:])} of {k_pool.dtype}")
    if k_host.shape != v_host.shape:
        raise ValueError("k_host and v_host must have the same shape")
    _need_cuda("pairs", pairs, torch.int32)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [num_pairs][2]")
    st = lib().pa_swap_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(k_host), _ptr(v_host),
                              int(k_host.shape[0]), C.byref(desc), _ptr(pairs),
                              int(pairs.shape[0]), int(direction), _stream(stream))
    check("pa_swap_blocks", st)

