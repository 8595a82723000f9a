"""CPU oracle for the paged-attention decode path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``paged_kv_cache_107_amd``) and never imports it; the only module both sides
use is ``workloads`` (seeded input draws, none of the method's arithmetic).

Contents, each written from the pages' statement of the method:

* ``allocator``  lazy block allocation, fork, copy-on-write, prefix sharing
                 and release over a FIFO free list with per-block refcounts.
* ``kvcache``    the cache write through a slot mapping and the CoW block copy,
                 on raw element bits (bit-exact by construction).
* ``attention``  decode and chunked-prefill attention: walk each block
                 table, reassemble K/V contiguously, then textbook softmax
                 attention in float64 (optionally over a sliding window, on
                 an 8-bit pool); plus the partitioned (split-K) form used to
                 pin the merge.
* ``sizes``      KV-cache byte counts.
* ``fp8``        the E4M3 8-bit float of a quantised KV pool (encode with
                 round-to-nearest-even and saturation, decode, scales).

Every function is pinned by tests against values the pages print, closed
forms, invariants or an independent library routine (see ``tests/``).
"""
from .allocator import OracleAllocator, OracleError  # noqa: F401
from . import attention, fp8, kvcache, sizes  # noqa: F401
