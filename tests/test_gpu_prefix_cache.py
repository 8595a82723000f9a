"""Prefill through the prefix cache on the GPU against the oracle, via the C ABI.

Requests sharing a system prompt go through the native allocator with the
prefix cache on: the cached blocks are looked up, only the positions after
the hit are appended, written by the cache kernel and computed by one
pa_prefill call.  Checked: hits and tables equal the oracle allocator's, both
pools bit for bit, outputs within 2e-2 (16-bit inputs) of the oracle's
prefill over its own pools, and the suffix rows within the same bound of the
GPU's own prefill of the full prompts without the cache.
"""
import numpy as np
import pytest

import workloads as W
from _prefix import run_prompts_oracle
from _scenario import TOL, from_device_bits, max_abs_err, to_device, to_f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; never a fallback
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="needs a GPU")]

import paged_kv_cache_107_amd as pa  # noqa: E402
from oracle.attention import paged_prefill, paged_prefill_rows_at_once  # noqa: E402


def run_prompts_gpu(ps, cached: bool):
    """The oracle runner's steps on the HIP path: native allocator, one
    cache write of every computed position, one pa_prefill call."""
    from paged_kv_cache_107_amd.cache import PagedKVCache
    wl = ps.wl
    cache = PagedKVCache(ps.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype,
                         ps.free_order)
    if cached:
        cache.enable_prefix_cache()
    slots, ks, vs, qs, hits = [], [], [], [], []
    for r in range(ps.requests):
        ids = W.prompt_token_ids(ps, r)
        s, hit = cache.create_prefix(ids) if cached else (cache.create(), 0)
        sl, pair = cache.reserve_tokens(s, ids[hit:])
        assert s == r and pair is None
        k, v = W.prompt_kv_bits_of(ps, r)
        slots.append(sl)
        ks.append(k[hit:])
        vs.append(v[hit:])
        qs.append(W.prompt_query_bits_of(ps, r)[hit:])
        hits.append(hit)
    cache.write_host(to_device(np.concatenate(ks), wl.dtype),
                     to_device(np.concatenate(vs), wl.dtype), np.concatenate(slots), [])
    lens = ps.prompt_lens
    tables, lens32 = cache.alloc.pa_build_tables(list(range(ps.requests)),
                                                 int(-(-int(lens.max()) // wl.block_size)))
    hits = np.array(hits, dtype=np.int64)
    qstart = np.concatenate([[0], np.cumsum(lens - hits)]).astype(np.int32)
    q = to_device(np.concatenate(qs), wl.dtype)
    out = torch.full_like(q, float("nan"))
    pa.pa_prefill(q, cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(),
                  torch.from_numpy(qstart).cuda(), torch.from_numpy(lens32).cuda(), wl.scale,
                  out, int((lens - hits).max()), int(lens.max()))
    torch.cuda.synchronize()
    return dict(cache=cache, out=out, tables=tables, hits=hits, query_start=qstart)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bs", [16, 32])
def test_cached_prefill_matches_oracle(dtype, bs):
    ps = W.custom_prompt_set(800 + bs, 32, 8, 128, dtype, bs, 300,
                             [1, 5, 16, 17, 40, 3, 100, 64, 2])
    o = run_prompts_oracle(ps, cached=True)
    g = run_prompts_gpu(ps, cached=True)
    assert g["hits"].tolist() == o["hits"].tolist()
    assert (g["hits"][1:] > 0).all()
    assert np.array_equal(g["tables"], o["tables"])
    assert np.array_equal(from_device_bits(g["cache"].k_pool, dtype), o["kp"])
    assert np.array_equal(from_device_bits(g["cache"].v_pool, dtype), o["vp"])
    want = paged_prefill(o["q"], o["kp"], o["vp"], o["tables"], o["query_start"], o["lens"],
                         ps.wl.scale, dtype)
    err = max_abs_err(g["out"], want)
    print(f"cached prefill {dtype} BS={bs} hits={g['hits'].tolist()} max_abs_err={err:.3e}",
          flush=True)
    assert err <= TOL[dtype]
    st = g["cache"].prefix_stats()
    assert st == o["alloc"].prefix_stats()

    u = run_prompts_gpu(ps, cached=False)
    for r in range(ps.requests):
        a, b = g["query_start"][r], g["query_start"][r + 1]
        ua, ub = u["query_start"][r], u["query_start"][r + 1]
        full = to_f64(u["out"][ua + g["hits"][r]:ub])
        assert max_abs_err(g["out"][a:b], full) <= TOL[dtype]


def test_system_prompt_workload_full_size():
    """100 requests on one 1024-token system prompt: the 99 later requests
    hit all 64 of its blocks; every computed row of every request against
    the oracle (the matrix form of its chunked prefill)."""
    ps = W.prompt_set("prefix_1k")
    o = run_prompts_oracle(ps, cached=True)
    g = run_prompts_gpu(ps, cached=True)
    assert g["hits"].tolist() == [0] + [1024] * 99
    assert np.array_equal(g["tables"], o["tables"])
    assert np.array_equal(from_device_bits(g["cache"].k_pool, "bf16"), o["kp"])
    assert np.array_equal(from_device_bits(g["cache"].v_pool, "bf16"), o["vp"])
    want = paged_prefill_rows_at_once(o["q"], o["kp"], o["vp"], o["tables"], o["query_start"],
                                      o["lens"], ps.wl.scale, "bf16")
    err = max_abs_err(g["out"], want)
    print(f"prefix_1k {want.shape[0]} rows max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
