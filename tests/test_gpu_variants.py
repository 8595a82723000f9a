"""Sliding windows and 8-bit (E4M3) pools on the GPU against the oracle,
through the C ABI.

* Window: decode on every kernel path (vector, matrix-core grid and stream
  splits) and chunked prefill, for windows below, at and above the lengths
  and on both sides of tile and block edges, against the oracle's windowed
  attention; with the allocator's trims applied and every released block
  poisoned with NaN (the kernels never read them).
* 8-bit pools: the quantising cache write is bit-exact against the oracle's
  E4M3 encoding (every bf16 value in range, saturation, signed zero); decode
  (grid and stream splits, G 1-16) and prefill on 8-bit pools against the
  oracle on the same codes; copies of 8-bit blocks bit-exact; windows and
  8-bit pools together (full-size workloads: test_gpu_full_size.py).
Tolerance: max-abs error <= 2e-2 (16-bit activations, fp32 accumulation), as
for 16-bit pools: the codes are exact inputs on both sides.
"""
import numpy as np
import pytest

import workloads as W
from _scenario import (KV, TOL, from_device_bits, max_abs_err, run_gpu, run_oracle, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; never a fallback
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="needs a GPU")]

import paged_kv_cache_107_amd as pa  # noqa: E402
from oracle import OracleAllocator, fp8  # noqa: E402
from oracle.attention import decode_bits, paged_decode, paged_prefill  # noqa: E402
from oracle.kvcache import copy_blocks, write_slots_fp8  # noqa: E402

PATHS = {"valu": pa.PA_PATH_VALU, "grid": pa.PA_PATH_MFMA_GRID, "stream": pa.PA_PATH_MFMA}
SCALES = (0.05, 0.03)


@pytest.fixture
def decode_path():
    prev = pa.pa_set_decode_path(pa.PA_PATH_AUTO)
    yield lambda p: pa.pa_set_decode_path(PATHS[p])
    pa.pa_set_decode_path(prev)


def decode_gpu(cache, seqs, q, scale, window=0, kv_scales=(1.0, 1.0), max_blocks=None):
    lens = np.array([cache.alloc.pa_seq_info(s)[0] for s in seqs])
    mb = max_blocks or int(-(-lens.max() // cache.block_size))
    tables, lens32 = cache.alloc.pa_build_tables(seqs, mb)
    out = torch.full_like(q, float("nan"))
    ws = cache.workspace(len(seqs), q.shape[1], int(lens.max()))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_decode(q, cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(),
                 torch.from_numpy(lens32).cuda(), scale, out, ws, int(lens.max()),
                 sliding_window=window, kv_scales=kv_scales, status=status)
    torch.cuda.synchronize()
    # holes a window trim left below the window are never read: no report
    assert int(status.item()) == 0
    return out, tables, lens32


# ------------------------------------------------------------------ windows

WINDOW_LENS = [1, 15, 16, 17, 33, 100, 511, 512, 513, 1024, 1100, 2000]


@pytest.mark.parametrize("path", ["valu", "grid", "stream"])
@pytest.mark.parametrize("window", [1, 15, 16, 17, 100, 512, 1000, 5000])
def test_windowed_decode_every_path(path, window, decode_path):
    d = W.custom(1000 + window, 32, 8, 128, "bf16", 16, WINDOW_LENS)
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    g = run_gpu(d, kv, decode=False)
    decode_path(path)
    q = g["q"] if "q" in g else to_device(W.query_bits(d), "bf16")
    out, tables, lens = decode_gpu(g["cache"], list(range(d.batch)), q, d.wl.scale, window)
    want = paged_decode(W.query_bits(d), o["kp"], o["vp"], o["tables"], o["lens"], d.wl.scale,
                        "bf16", window=window)
    err = max_abs_err(out, want)
    print(f"window={window} path={path} max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("shape", [("f16", 16, 8, 128, 4), ("bf16", 32, 2, 128, 8),
                                   ("f32", 16, 4, 64, 1), ("bf16", 16, 32, 128, 1)])
def test_windowed_decode_shapes_with_trims_and_poison(shape):
    """Trim every sequence to the window, poison every released block with
    NaN: the windowed output is unchanged (the auto-chosen kernel)."""
    dtype, bs, hkv, dh, g = shape
    window = 40
    d = W.custom(1100 + bs + dh, hkv * g, hkv, dh, dtype, bs, WINDOW_LENS[:9])
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    gg = run_gpu(d, kv, decode=False)
    cache = gg["cache"]
    free_before = set(cache.alloc.pa_alloc_query()[0].tolist())
    released = sum(cache.trim_window(s, window) for s in range(d.batch))
    freed = sorted(set(cache.alloc.pa_alloc_query()[0].tolist()) - free_before)
    assert released == len(freed) > 0
    nan = float("nan")
    idx = torch.tensor(freed, dtype=torch.long, device="cuda")
    cache.k_pool[idx] = nan
    cache.v_pool[idx] = nan
    q = to_device(W.query_bits(d), dtype)
    out, tables, _ = decode_gpu(cache, list(range(d.batch)), q, d.wl.scale, window,
                                max_blocks=o["tables"].shape[1])
    assert (tables == pa.PA_NO_BLOCK).any()
    want = paged_decode(W.query_bits(d), o["kp"], o["vp"], o["tables"], o["lens"], d.wl.scale,
                        dtype, window=window)
    err = max_abs_err(out, want)
    print(f"{shape} trimmed window={window} released={released} max_abs_err={err:.3e}",
          flush=True)
    assert err <= TOL[dtype]


@pytest.fixture(params=["lds", "dma"])
def prefill_kernel(request):
    """The 16-bit prefill tests run on both prefill kernels."""
    path = {"lds": pa.PA_PREFILL_LDS, "dma": pa.PA_PREFILL_DMA}[request.param]
    prev = pa.pa_set_prefill_path(path)
    yield request.param
    pa.pa_set_prefill_path(prev)


@pytest.mark.parametrize("window", [1, 7, 16, 40, 200])
@pytest.mark.parametrize("g", [1, 4, 16])
def test_windowed_prefill(window, g, prefill_kernel):
    chunks = [1, 17, 64, 65, 100, 33]
    prefixes = [0, 40, 16, 300, 3, 1000]
    lens = [c + p for c, p in zip(chunks, prefixes)]
    d = W.custom(1200 + g + window, 2 * g, 2, 128, "bf16", 16, lens, chunk_lens=chunks)
    from test_gpu_prefill import run_gpu_prefill
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    gp = run_gpu_prefill(d, kv)
    out = torch.full_like(gp["q"], float("nan"))
    pa.pa_prefill(gp["q"], gp["cache"].k_pool, gp["cache"].v_pool, gp["tables"], gp["qs"],
                  gp["lens"], d.wl.scale, out, gp["max_q"], gp["max_ctx"], sliding_window=window)
    torch.cuda.synchronize()
    want = paged_prefill(W.prefill_query_bits(d), o["kp"], o["vp"], o["tables"], d.query_start,
                         o["lens"], d.wl.scale, "bf16", window=window)
    err = max_abs_err(out, want)
    print(f"prefill window={window} G={g} max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("window", [7, 40])
@pytest.mark.parametrize("g", [1, 4])
def test_windowed_prefill_after_trims(window, g, prefill_kernel):
    """Blocks no chunk row's window reaches are released (each sequence is
    trimmed to window + its chunk length, so the chunk's first row keeps its
    whole window), the released blocks are poisoned with NaN and the tables
    rebuilt with their holes: the windowed prefill output is unchanged."""
    chunks = [1, 17, 64, 65, 100, 33]
    prefixes = [0, 400, 160, 300, 90, 1000]
    lens = [c + p for c, p in zip(chunks, prefixes)]
    d = W.custom(1300 + g + window, 2 * g, 2, 128, "bf16", 16, lens, chunk_lens=chunks)
    from test_gpu_prefill import run_gpu_prefill
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    gp = run_gpu_prefill(d, kv)
    cache = gp["cache"]
    free_before = set(cache.alloc.pa_alloc_query()[0].tolist())
    released = sum(cache.trim_window(s, window + c) for s, c in enumerate(chunks))
    freed = sorted(set(cache.alloc.pa_alloc_query()[0].tolist()) - free_before)
    assert released == len(freed) > 0
    idx = torch.tensor(freed, dtype=torch.long, device="cuda")
    cache.k_pool[idx] = float("nan")
    cache.v_pool[idx] = float("nan")
    tables, _ = cache.alloc.pa_build_tables(list(range(d.batch)), gp["host_tables"].shape[1])
    assert (tables == pa.PA_NO_BLOCK).any()
    out = torch.full_like(gp["q"], float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_prefill(gp["q"], cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(),
                  gp["qs"], gp["lens"], d.wl.scale, out, gp["max_q"], gp["max_ctx"],
                  sliding_window=window, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0          # the released blocks are below every window
    want = paged_prefill(W.prefill_query_bits(d), o["kp"], o["vp"], o["tables"], d.query_start,
                         o["lens"], d.wl.scale, "bf16", window=window)
    err = max_abs_err(out, want)
    print(f"trimmed prefill window={window} G={g} released={released} max_abs_err={err:.3e}",
          flush=True)
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ 8-bit pools

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [1.0, 0.05, 3.0])
def test_fp8_cache_write_bitexact(dtype, scale):
    """Every 16-bit value that is finite, through the quantising write, equals
    the oracle's E4M3 encoding (with saturation beyond 448 * scale)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    if dtype == "bf16":
        vals = (bits << np.uint32(16)).view(np.float32)
        src = bits.astype(np.uint16)
    else:
        src = bits.astype(np.uint16)
        vals = src.view(np.float16).astype(np.float32)
    keep = np.isfinite(vals)
    src, vals = src[keep], vals[keep]
    n = (src.size // 128) * 128
    src, vals = src[:n], vals[:n]
    hkv, dh, bs = 1, 128, 16
    t = n // (hkv * dh)
    nb = -(-t // bs)
    kp = torch.zeros((nb, hkv, bs, dh), dtype=torch.uint8, device="cuda").view(pa.FP8)
    vp = torch.zeros_like(kp)
    k = to_device(src.reshape(t, hkv, dh), dtype)
    slots = torch.arange(t, dtype=torch.int64, device="cuda")
    pa.pa_reshape_and_cache(k, k, slots, kp, vp, kv_scales=(scale, scale))
    torch.cuda.synchronize()
    got = kp.view(torch.uint8).cpu().numpy().reshape(nb * bs, dh)[:t].reshape(-1)
    want = fp8.quantize(vals, scale)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad[:5], vals[bad[:5]], got[bad[:5]], want[bad[:5]])
    assert np.array_equal(vp.view(torch.uint8).cpu().numpy(), kp.view(torch.uint8).cpu().numpy())


def run_fp8_scenario(d, kv, scales):
    """The workload's allocator scenario on both sides with 8-bit pools: the
    oracle quantises each append (write_slots_fp8) and copies CoW blocks; the
    HIP path runs the native allocator, pa_copy_blocks and the quantising
    pa_reshape_and_cache per phase."""
    from paged_kv_cache_107_amd.cache import PagedKVCache
    wl = d.wl
    a = OracleAllocator(d.num_blocks, wl.block_size, d.free_order)
    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    okp, ovp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    cache = PagedKVCache(d.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype,
                         d.free_order, kv_dtype="fp8_e4m3", kv_scales=scales)
    for phase in W.scenario(d):
        slots, pairs, ks, vs = [], [], [], []
        for op in phase:
            if op[0] == "create":
                assert a.create() == op[1] == cache.create()
            elif op[0] == "fork":
                assert a.fork(op[1]) == op[2] == cache.fork(op[1])
            else:
                i, start, n = op[1:]
                so, po = a.append(i, n)
                sg, pg = cache.reserve(i, n)
                assert list(so) == sg.tolist() and po == pg
                if po is not None:
                    copy_blocks(okp, [po])
                    copy_blocks(ovp, [po])
                    pairs.append(po)
                k, v = kv(i)
                k, v = k[start:start + n], v[start:start + n]
                write_slots_fp8(okp, decode_bits(k, wl.dtype).astype(np.float32), so, scales[0])
                write_slots_fp8(ovp, decode_bits(v, wl.dtype).astype(np.float32), so, scales[1])
                slots.append(sg)
                ks.append(k)
                vs.append(v)
        if slots:
            cache.write_host(to_device(np.concatenate(ks), wl.dtype),
                             to_device(np.concatenate(vs), wl.dtype), np.concatenate(slots), pairs)
    torch.cuda.synchronize()
    mb = int(-(-int(d.context_lens.max()) // wl.block_size))
    tables, lens = a.build_tables(list(range(d.batch)), mb)
    return dict(alloc=a, kp=okp, vp=ovp, tables=tables, lens=lens), cache


def fp8_bits(t):
    return t.view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("path", ["grid", "stream"])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_fp8_decode(path, g, decode_path):
    d = W.custom(1300 + g, 2 * g, 2, 128, "bf16", 16, WINDOW_LENS)
    kv = KV(d)
    o, cache = run_fp8_scenario(d, kv, SCALES)
    assert np.array_equal(fp8_bits(cache.k_pool), o["kp"])
    assert np.array_equal(fp8_bits(cache.v_pool), o["vp"])
    decode_path(path)
    q = to_device(W.query_bits(d), "bf16")
    for window in (0, 100):
        out, _, _ = decode_gpu(cache, list(range(d.batch)), q, d.wl.scale, window, SCALES)
        want = paged_decode(W.query_bits(d), o["kp"], o["vp"], o["tables"], o["lens"],
                            d.wl.scale, "bf16", window=window, kv_dtype="fp8_e4m3",
                            k_scale=SCALES[0], v_scale=SCALES[1])
        err = max_abs_err(out, want)
        print(f"fp8 decode path={path} G={g} window={window} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_cow_workload_and_copies(dtype):
    """Forks, CoW copies of 8-bit blocks and their decode (the parallel
    sampling workload's structure at a small size)."""
    d = W.draw("cow", batch=16)
    if dtype == "f16":
        d = W.custom(1400, 32, 8, 128, "f16", 16, list(d.context_lens[:12]))
    kv = KV(d)
    o, cache = run_fp8_scenario(d, kv, SCALES)
    assert np.array_equal(fp8_bits(cache.k_pool), o["kp"])
    assert np.array_equal(fp8_bits(cache.v_pool), o["vp"])
    q = to_device(W.query_bits(d), d.wl.dtype)
    out, _, _ = decode_gpu(cache, list(range(d.batch)), q, d.wl.scale, 0, SCALES)
    want = paged_decode(W.query_bits(d), o["kp"], o["vp"], o["tables"], o["lens"], d.wl.scale,
                        d.wl.dtype, kv_dtype="fp8_e4m3", k_scale=SCALES[0], v_scale=SCALES[1])
    assert max_abs_err(out, want) <= TOL[d.wl.dtype]


@pytest.mark.parametrize("window,g,dtype", [(0, 1, "bf16"), (0, 4, "bf16"), (0, 8, "bf16"),
                                            (50, 1, "bf16"), (50, 4, "bf16"), (50, 8, "bf16"),
                                            (0, 4, "f16"), (50, 16, "f16")])
@pytest.mark.parametrize("kernel", ["lds", "dma"])
def test_fp8_prefill(window, g, dtype, kernel):
    """8-bit pools on both prefill kernels: codes widened in registers on the
    way into LDS (lds), or loaded straight into LDS and widened there (dma)."""
    prev = pa.pa_set_prefill_path({"lds": pa.PA_PREFILL_LDS, "dma": pa.PA_PREFILL_DMA}[kernel])
    try:
        fp8_prefill_case(window, g, dtype, kernel)
    finally:
        pa.pa_set_prefill_path(prev)


def fp8_prefill_case(window, g, dtype, kernel):
    chunks = [1, 17, 64, 65, 100]
    prefixes = [0, 40, 16, 300, 3]
    lens = [c + p for c, p in zip(chunks, prefixes)]
    d = W.custom(1500 + g, 2 * g, 2, 128, dtype, 16, lens, chunk_lens=chunks)
    kv = KV(d)
    o, cache = run_fp8_scenario(d, kv, SCALES)
    tables, lens32 = cache.alloc.pa_build_tables(list(range(d.batch)), o["tables"].shape[1])
    q = to_device(W.prefill_query_bits(d), dtype)
    out = torch.full_like(q, float("nan"))
    pa.pa_prefill(q, cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(),
                  torch.from_numpy(d.query_start.astype(np.int32)).cuda(),
                  torch.from_numpy(lens32).cuda(), d.wl.scale, out, int(max(chunks)),
                  int(lens32.max()), sliding_window=window, kv_scales=SCALES)
    torch.cuda.synchronize()
    want = paged_prefill(W.prefill_query_bits(d), o["kp"], o["vp"], o["tables"], d.query_start,
                         o["lens"], d.wl.scale, dtype, window=window, kv_dtype="fp8_e4m3",
                         k_scale=SCALES[0], v_scale=SCALES[1])
    err = max_abs_err(out, want)
    print(f"fp8 prefill {kernel} {dtype} G={g} window={window} max_abs_err={err:.3e}",
          flush=True)
    assert err <= TOL[dtype]
