"""Every output row of the benchmarked workloads at full size, on the GPU,
against the oracle, through the C ABI, in the launch configurations the
benchmark times.

* Chunked prefill, 16 sequences x 512-token chunks on cached prefixes (8192
  rows, 32 q / 8 kv heads, head_dim 128, bf16): without a window and with a
  1024-position window, on both prefill kernels; and, on both kernels, on
  8-bit E4M3 pools holding the quantised contents of the 16-bit pools (codes
  written by the
  quantising cache write and checked bit for bit against the oracle's
  encoding of the oracle's own pools).
* Decode of the 8B batch (256 sequences): a 1024-position window on the
  16-bit pools, and the 8-bit pools (quantised contents) without and with
  the window: all 256 x 32 rows.
The prefill expectation is ``paged_prefill_rows_at_once`` (the matrix form of
the oracle's chunked prefill, pinned to the row-by-row loop and to SDPA on
the CPU); each oracle result is computed once per module.
Tolerance: max-abs error <= 2e-2 (16-bit activations, fp32 accumulation).
"""
import functools

import numpy as np
import pytest

import workloads as W
from _scenario import KV, TOL, from_device_bits, max_abs_err, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; never a fallback
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="needs a GPU")]

import paged_kv_cache_107_amd as pa  # noqa: E402
from oracle import fp8  # noqa: E402
from oracle.attention import decode_bits, paged_decode, paged_prefill_rows_at_once  # noqa: E402

WINDOW = 1024
SCALES = (0.05, 0.05)
KERNELS = {"lds": pa.PA_PREFILL_LDS, "dma": pa.PA_PREFILL_DMA}


def quantise_device(k_pool, v_pool):
    """Every slot of both pools through the quantising cache write."""
    nb, hkv, bs, dh = k_pool.shape
    flat = lambda p: p.permute(0, 2, 1, 3).reshape(nb * bs, hkv, dh).contiguous()
    k8 = torch.zeros_like(k_pool, dtype=torch.uint8).view(pa.FP8)
    v8 = torch.zeros_like(k8)
    slots = torch.arange(nb * bs, dtype=torch.int64, device="cuda")
    pa.pa_reshape_and_cache(flat(k_pool), flat(v_pool), slots, k8, v8, kv_scales=SCALES)
    torch.cuda.synchronize()
    return k8, v8


def quantise_oracle(bits, dtype, scale):
    return fp8.quantize(decode_bits(bits, dtype).astype(np.float32), scale)


def fp8_bits(t):
    return t.view(torch.uint8).cpu().numpy()


# ------------------------------------------------------------------ prefill

@functools.lru_cache(maxsize=1)
def prefill_state():
    """The prefill workload built on both sides (pools bit-equal), with the
    device tables and the call's arguments."""
    from test_gpu_prefill import run_gpu_prefill
    d = W.draw("prefill_8b")
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    g = run_gpu_prefill(d, kv)
    assert np.array_equal(from_device_bits(g["cache"].k_pool, "bf16"), o["kp"])
    assert np.array_equal(from_device_bits(g["cache"].v_pool, "bf16"), o["vp"])
    return d, o, g


@functools.lru_cache(maxsize=None)
def prefill_want(window: int, eight_bit: bool):
    d, o, _ = prefill_state()
    kw = dict(window=window)
    kp, vp = o["kp"], o["vp"]
    if eight_bit:
        kp, vp = prefill_codes()[2:]
        kw.update(kv_dtype="fp8_e4m3", k_scale=SCALES[0], v_scale=SCALES[1])
    return paged_prefill_rows_at_once(W.prefill_query_bits(d), kp, vp, o["tables"],
                                      d.query_start, o["lens"], d.wl.scale, "bf16", **kw)


@functools.lru_cache(maxsize=1)
def prefill_codes():
    _, o, g = prefill_state()
    k8, v8 = quantise_device(g["cache"].k_pool, g["cache"].v_pool)
    return k8, v8, quantise_oracle(o["kp"], "bf16", SCALES[0]), \
        quantise_oracle(o["vp"], "bf16", SCALES[1])


def run_prefill(k_pool, v_pool, window=0, kv_scales=(1.0, 1.0)):
    d, _, g = prefill_state()
    out = torch.full_like(g["q"], float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_prefill(g["q"], k_pool, v_pool, g["tables"], g["qs"], g["lens"], d.wl.scale, out,
                  g["max_q"], g["max_ctx"], sliding_window=window, kv_scales=kv_scales,
                  status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out


@pytest.fixture(params=sorted(KERNELS))
def prefill_kernel(request):
    prev = pa.pa_set_prefill_path(KERNELS[request.param])
    yield request.param
    pa.pa_set_prefill_path(prev)


@pytest.mark.parametrize("window", [0, WINDOW])
def test_prefill_every_row(window, prefill_kernel):
    print(f"prefill_8b full size: window={window} kernel={prefill_kernel}", flush=True)
    _, _, g = prefill_state()
    out = run_prefill(g["cache"].k_pool, g["cache"].v_pool, window)
    err = max_abs_err(out, prefill_want(window, False))
    print(f"  8192 rows max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_prefill_every_row_on_quantised_pools(prefill_kernel):
    print(f"prefill_8b full size on 8-bit pools: kernel={prefill_kernel}", flush=True)
    k8, v8, ck, cv = prefill_codes()
    assert np.array_equal(fp8_bits(k8), ck) and np.array_equal(fp8_bits(v8), cv)
    out = run_prefill(k8, v8, 0, SCALES)
    err = max_abs_err(out, prefill_want(0, True))
    print(f"  8192 rows max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ decode

@functools.lru_cache(maxsize=1)
def decode_state():
    d = W.draw("8b_gqa")
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    g = run_gpu(d, kv, decode=False)
    kp, vp = o["kp"], o["vp"]
    assert np.array_equal(from_device_bits(g["cache"].k_pool, "bf16"), kp)
    assert np.array_equal(from_device_bits(g["cache"].v_pool, "bf16"), vp)
    k8, v8 = quantise_device(g["cache"].k_pool, g["cache"].v_pool)
    ck, cv = quantise_oracle(kp, "bf16", SCALES[0]), quantise_oracle(vp, "bf16", SCALES[1])
    assert np.array_equal(fp8_bits(k8), ck) and np.array_equal(fp8_bits(v8), cv)
    return d, o, g, (k8, v8, ck, cv)


@pytest.mark.parametrize("name,window,eight_bit", [("window_1024", WINDOW, False),
                                                   ("fp8_e4m3", 0, True),
                                                   ("fp8_e4m3_window_1024", WINDOW, True)])
def test_decode_variant_every_row(name, window, eight_bit):
    print(f"8b_gqa full size decode: {name}", flush=True)
    d, o, g, (k8, v8, ck, cv) = decode_state()
    wl, plan = d.wl, g["plan"]
    kp, vp = (k8, v8) if eight_bit else (g["cache"].k_pool, g["cache"].v_pool)
    scales = SCALES if eight_bit else (1.0, 1.0)
    q = to_device(W.query_bits(d), wl.dtype)
    out = torch.full_like(q, float("nan"))
    ws = g["cache"].workspace(d.batch, wl.num_q_heads, plan.max_context_len)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the benchmark's call: library-chosen partition size and kernel
    pa.pa_decode(q, kp, vp, plan.tables, plan.lens, wl.scale, out, ws, plan.max_context_len, 0,
                 None, window, scales, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    kw = dict(window=window)
    okp, ovp = o["kp"], o["vp"]
    if eight_bit:
        okp, ovp = ck, cv
        kw.update(kv_dtype="fp8_e4m3", k_scale=SCALES[0], v_scale=SCALES[1])
    want = paged_decode(W.query_bits(d), okp, ovp, o["tables"], o["lens"], wl.scale, wl.dtype,
                        **kw)
    err = max_abs_err(out, want)
    print(f"  {d.batch} sequences max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
