"""Pins for the oracle's attention variants: sliding windows and an 8-bit
(E4M3) KV pool (CPU only).

Window: against torch's scaled_dot_product_attention (float64, CPU) with an
explicit band mask on the contiguous K/V, closed forms (W = 1 returns the
last V row; W >= ctx changes nothing), decode = one-token prefill with the
same window, and blocks below the window never read (NaN contents and
released table entries change nothing).

E4M3: decode of all 256 codes and encode of every bfloat16 value in range
against torch's float8_e4m3fn conversion; the format's closed-form points;
round trip of every finite code; the quantisation error bound; attention on
an 8-bit pool against SDPA on the dequantised values.
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8
from oracle.attention import decode_bits, paged_decode, paged_prefill, paged_prefill_rows_at_once
from oracle.kvcache import write_slots, write_slots_fp8

torch = pytest.importorskip("torch")
F = torch.nn.functional


def contiguous_case(seed, hq, hkv, d, dtype, ctx, bs=16):
    """One sequence written through a shuffled block table; returns the
    pools, table, the contiguous K/V and the q bits."""
    rng = np.random.default_rng(seed)
    nb = -(-ctx // bs) + 3
    k = W.to_bits(rng.standard_normal((ctx, hkv, d), dtype=np.float32), dtype)
    v = W.to_bits(rng.standard_normal((ctx, hkv, d), dtype=np.float32), dtype)
    kp = np.zeros((nb, hkv, bs, d), dtype=k.dtype)
    vp = np.zeros_like(kp)
    table = rng.permutation(nb)[: -(-ctx // bs)]
    slots = np.array([table[p // bs] * bs + p % bs for p in range(ctx)])
    write_slots(kp, k, slots)
    write_slots(vp, v, slots)
    tables = np.full((1, nb), -1, dtype=np.int64)
    tables[0, :len(table)] = table
    return kp, vp, tables, k, v


def sdpa(q, k, v, scale, mask):
    """q [T][Hq][D], k/v [S][Hkv][D] float64, mask [T][S] bool -> [T][Hq][D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask),
                                       scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("ctx,window", [(100, 1), (100, 17), (100, 64), (100, 99), (37, 16),
                                        (513, 256)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_windowed_decode_equals_sdpa_on_the_band(ctx, window, dtype):
    kp, vp, tables, k, v = contiguous_case(ctx + window, 8, 2, 64, dtype, ctx)
    q = W.to_bits(np.random.default_rng(1).standard_normal((1, 8, 64), dtype=np.float32), dtype)
    got = paged_decode(q, kp, vp, tables, [ctx], 0.125, dtype, window=window)
    mask = np.zeros((1, ctx), dtype=bool)
    mask[0, max(0, ctx - window):] = True
    want = sdpa(decode_bits(q, dtype), decode_bits(k, dtype), decode_bits(v, dtype), 0.125, mask)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_window_closed_forms():
    ctx = 70
    kp, vp, tables, k, v = contiguous_case(3, 4, 2, 64, "bf16", ctx)
    q = W.to_bits(np.random.default_rng(2).standard_normal((1, 4, 64), dtype=np.float32), "bf16")
    one = paged_decode(q, kp, vp, tables, [ctx], 0.125, "bf16", window=1)
    last = decode_bits(v[ctx - 1], "bf16")                  # [Hkv][D]
    np.testing.assert_array_equal(one[0], last[[0, 0, 1, 1]])
    full = paged_decode(q, kp, vp, tables, [ctx], 0.125, "bf16")
    for w in (ctx, ctx + 1, 10 ** 6):
        assert np.array_equal(paged_decode(q, kp, vp, tables, [ctx], 0.125, "bf16", window=w), full)


def test_blocks_below_the_window_are_never_read():
    ctx, window, bs = 200, 40, 16
    kp, vp, tables, k, v = contiguous_case(4, 8, 2, 64, "bf16", ctx, bs)
    q = W.to_bits(np.random.default_rng(3).standard_normal((1, 8, 64), dtype=np.float32), "bf16")
    want = paged_decode(q, kp, vp, tables, [ctx], 0.125, "bf16", window=window)
    dead = (ctx - window) // bs                            # blocks wholly below the window
    kp2, vp2, t2 = kp.copy(), vp.copy(), tables.copy()
    for j in range(dead):
        kp2[t2[0, j]] = 0x7FC0                              # NaN
        vp2[t2[0, j]] = 0x7FC0
        t2[0, j] = -1                                       # released
    got = paged_decode(q, kp2, vp2, t2, [ctx], 0.125, "bf16", window=window)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fn", [paged_prefill, paged_prefill_rows_at_once])
@pytest.mark.parametrize("window", [1, 5, 16, 33, 1000])
def test_windowed_prefill_equals_sdpa_band_and_decode(window, fn):
    ctx, n = 90, 30
    kp, vp, tables, k, v = contiguous_case(5 + window, 8, 2, 64, "bf16", ctx)
    qb = W.to_bits(np.random.default_rng(6).standard_normal((n, 8, 64), dtype=np.float32), "bf16")
    got = fn(qb, kp, vp, tables, [0, n], [ctx], 0.125, "bf16", window=window)
    i = np.arange(ctx - n, ctx)[:, None]
    j = np.arange(ctx)[None, :]
    mask = (j <= i) & (j > i - window)
    want = sdpa(decode_bits(qb, "bf16"), decode_bits(k, "bf16"), decode_bits(v, "bf16"), 0.125,
                mask)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the chunk's last row is the decode step at that length
    dec = paged_decode(qb[-1:], kp, vp, tables, [ctx], 0.125, "bf16", window=window)
    if fn is paged_prefill:
        np.testing.assert_array_equal(got[-1], dec[0])
    else:   # the matrix form rounds in another order
        np.testing.assert_allclose(got[-1], dec[0], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ E4M3

def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode_e4m3(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])
    assert np.isnan(ours[[0x7F, 0xFF]]).all() and np.isnan(ours).sum() == 2


def test_encode_every_bf16_in_range_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    ours = fp8.encode_e4m3(x)
    theirs = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_closed_form_points():
    enc = lambda v: int(fp8.encode_e4m3(np.array([v], dtype=np.float32))[0])
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(2.0 ** -9) == 0x01 and enc(2.0 ** -10) == 0x00       # tie to even (zero)
    assert enc(3 * 2.0 ** -10) == 0x02                               # tie to even (2)
    assert enc(1.0) == 0x38 and enc(1.0625) == 0x38 and enc(1.1875) == 0x3A
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80 and enc(float("nan")) == 0x7F
    q = fp8.quantize(np.array([1000.0, -1000.0, 1.0], dtype=np.float32), 0.5)
    assert q.tolist() == [0x7E, 0xFE, enc(2.0)]                     # saturated; 1 / 0.5 = 2


def test_round_trip_and_error_bound():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[~np.isnan(fp8.decode_e4m3(codes))]
    assert np.array_equal(fp8.encode_e4m3(fp8.decode_e4m3(finite).astype(np.float32)), finite)
    rng = np.random.default_rng(0)
    for scale in (1.0, 0.05, 3.0):
        x = (rng.standard_normal(20000) * 4 * scale).astype(np.float32)
        back = fp8.dequantize(fp8.quantize(x, scale), scale)
        inside = np.abs(x) <= 448 * scale
        err = np.abs(back - x)[inside]
        assert np.all(err <= 2.0 ** -4 * np.abs(x[inside]) + 2.0 ** -10 * scale * 1.0001)


def test_attention_on_an_fp8_pool_equals_sdpa_on_dequantised_values():
    rng = np.random.default_rng(9)
    ctx, bs, hkv, hq, d = 77, 16, 2, 8, 128
    ks, vs = 0.02, 0.05
    k = (rng.standard_normal((ctx, hkv, d)) * 0.3).astype(np.float32)
    v = rng.standard_normal((ctx, hkv, d)).astype(np.float32)
    nb = 8
    kp = np.zeros((nb, hkv, bs, d), dtype=np.uint8)
    vp = np.zeros_like(kp)
    table = np.array([5, 2, 7, 0, 3])
    slots = np.array([table[p // bs] * bs + p % bs for p in range(ctx)])
    write_slots_fp8(kp, k, slots, ks)
    write_slots_fp8(vp, v, slots, vs)
    tables = np.full((1, 6), -1)
    tables[0, :5] = table
    qb = W.to_bits(rng.standard_normal((1, hq, d), dtype=np.float32), "bf16")
    for window in (0, 20):
        got = paged_decode(qb, kp, vp, tables, [ctx], 0.09, "bf16", window=window,
                           kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs)
        kd = fp8.dequantize(fp8.quantize(k, ks), ks)
        vd = fp8.dequantize(fp8.quantize(v, vs), vs)
        mask = np.zeros((1, ctx), dtype=bool)
        mask[0, (ctx - window if window else 0):] = True
        want = sdpa(decode_bits(qb, "bf16"), kd, vd, 0.09, mask)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # quantisation error stays small next to the bf16 path on these values
    ref = sdpa(decode_bits(qb, "bf16"), k.astype(np.float64), v.astype(np.float64), 0.09,
               np.ones((1, ctx), dtype=bool))
    assert np.max(np.abs(paged_decode(qb, kp, vp, tables, [ctx], 0.09, "bf16",
                                      kv_dtype="fp8_e4m3", k_scale=ks, v_scale=vs) - ref)) < 0.05
