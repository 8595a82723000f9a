"""Paged KV-cache decode for AMD MI355X (gfx950).

The product is ``libpa.so`` (C ABI declared in ``include/pa.h``): HIP kernels
for paged decode attention (partition + split-K reduce), chunked prefill
attention, the new-token cache write, the copy-on-write block copy and block
swapping to pinned host pools, plus a host block allocator with a FIFO free
pool, refcounts, fork, prefix sharing, a prefix cache and swap bookkeeping.
This package is the thin Python binding: ``ops`` (kernels on torch device
tensors), ``allocator`` and ``cache`` (a per-layer driver of both).
"""
from ._lib import (LIB_PATH, PA_BF16, PA_F16, PA_F32, PA_KV_FP8_E4M3, PA_KV_SAME,  # noqa: F401
                   PA_NO_BLOCK, PA_PATH_AUTO, PA_PATH_MFMA, PA_PATH_MFMA_GRID, PA_PATH_VALU,
                   PA_PREFILL_AUTO, PA_PREFILL_DMA, PA_PREFILL_LDS,
                   PA_STATUS_BAD_BLOCK, PA_SWAP_IN, PA_SWAP_OUT, SIGNATURES, PaError, lib)
from .allocator import PaAllocator  # noqa: F401
from .ops import (FP8, alloc_workspace, pa_copy_blocks, pa_decode, pa_decode_noalloc,  # noqa: F401
                  pa_decode_partition, pa_decode_reduce, pa_decode_workspace_bytes, pa_prefill, pa_reshape_and_cache,
                  pa_probe_tile_reads, pa_set_decode_balance, pa_set_decode_path,
                  pa_set_prefill_path, pa_swap_blocks, pool_desc)
