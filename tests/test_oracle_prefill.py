"""Pins for the oracle's chunked-prefill attention (CPU only).

* paged == dense: every chunk row equals torch's scaled_dot_product_attention
  (float64, CPU, grouped-query heads) on the contiguous K/V with an explicit
  mask that lets a token see its own and earlier positions;
* a one-token chunk is the decode step: it equals ``paged_decode``;
* the same positions give the same rows whatever the chunk boundary;
* closed forms: a prompt's first token returns its own V row; equal keys give
  the running mean of the V rows;
* a token whose position would be negative gets a zero row;
* ``paged_prefill_rows_at_once`` (the matrix form for full-size workloads)
  passes the SDPA pin above and equals the row-by-row loop within rounding on
  windows, 8-bit pools, negative positions and sequence subsets.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import decode_bits, paged_decode, paged_prefill, paged_prefill_rows_at_once
from test_oracle_attention import page_sequences


def chunk_case(rng, ctxs, chunks, hq, hkv, d, dtype, bs):
    ks = [W.to_bits(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype) for n in ctxs]
    vs = [W.to_bits(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype) for n in ctxs]
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = W.to_bits(rng.standard_normal((int(qs[-1]), hq, d), dtype=np.float32), dtype)
    nb = sum(-(-n // bs) for n in ctxs) + 3
    kp, vp, tables, lens = page_sequences(ks, vs, nb, bs, rng.permutation(nb))
    return q, ks, vs, qs, kp, vp, tables, lens


def sdpa_chunk(q64, k64, v64, scale):
    """torch SDPA for one sequence's chunk: q [n][Hq][D], k/v [ctx][Hkv][D];
    chunk row j sits at position ctx - n + j and sees positions <= it."""
    n, ctx = q64.shape[0], k64.shape[0]
    allowed = torch.arange(ctx)[None, :] <= (ctx - n + torch.arange(n))[:, None]
    qt = torch.from_numpy(np.ascontiguousarray(q64.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k64.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v64.transpose(1, 0, 2)))[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                           scale=scale, enable_gqa=True)
    return out[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("fn", [paged_prefill, paged_prefill_rows_at_once])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [16, 4])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_prefill_equals_dense_sdpa_with_causal_mask(dtype, bs, hq, hkv, fn):
    rng = np.random.default_rng(21)
    ctxs, chunks = [40, 17, 64, 5, 33], [40, 9, 20, 1, 16]   # full prompt, tails, a 1-token step
    d = 32
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, ctxs, chunks, hq, hkv, d, dtype, bs)
    scale = 1 / math.sqrt(d)
    out = fn(q, kp, vp, tables, qs, lens, scale, dtype)
    for i in range(len(ctxs)):
        a, b = qs[i], qs[i + 1]
        ref = sdpa_chunk(decode_bits(q[a:b], dtype), decode_bits(ks[i], dtype),
                         decode_bits(vs[i], dtype), scale)
        np.testing.assert_allclose(out[a:b], ref, rtol=0, atol=1e-12)


def test_one_token_chunks_are_the_decode_step():
    rng = np.random.default_rng(22)
    ctxs = [1, 30, 77]
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, ctxs, [1, 1, 1], 8, 2, 16, "bf16", 16)
    got = paged_prefill(q, kp, vp, tables, qs, lens, 0.25, "bf16")
    want = paged_decode(q, kp, vp, tables, lens, 0.25, "bf16")
    assert np.array_equal(got, want)


def test_rows_do_not_depend_on_the_chunk_boundary():
    rng = np.random.default_rng(23)
    ctx, d = 50, 16
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, [ctx], [30], 4, 2, d, "f32", 16)
    full = paged_prefill(q, kp, vp, tables, qs, lens, 0.3, "f32")       # positions 20..49
    tail = paged_prefill(q[20:], kp, vp, tables, np.array([0, 10]), lens, 0.3, "f32")  # 40..49
    assert np.array_equal(full[20:], tail)


def test_first_prompt_token_returns_its_value_row():
    rng = np.random.default_rng(24)
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, [12], [12], 4, 2, 16, "bf16", 4)
    out = paged_prefill(q, kp, vp, tables, qs, lens, 0.25, "bf16")
    v0 = decode_bits(vs[0][0], "bf16")                      # [Hkv][D]
    assert np.array_equal(out[0], np.repeat(v0, 2, axis=0))


def test_equal_keys_give_running_means():
    rng = np.random.default_rng(25)
    ctx, n, hkv, d = 20, 8, 1, 8
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, [ctx], [n], 2, hkv, d, "f32", 4)
    k_same = np.repeat(ks[0][:1], ctx, axis=0)
    kp2, vp2, tables2, lens2 = page_sequences([k_same], vs, kp.shape[0], 4, np.arange(kp.shape[0]))
    out = paged_prefill(q, kp2, vp2, tables2, qs, lens2, 0.5, "f32")
    v64 = decode_bits(vs[0], "f32")[:, 0, :]
    for j in range(n):
        pos = ctx - n + j
        want = v64[:pos + 1].mean(axis=0)
        np.testing.assert_allclose(out[j], np.stack([want, want]), rtol=0, atol=1e-12)


def test_negative_positions_give_zero_rows():
    rng = np.random.default_rng(26)
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, [6], [6], 4, 2, 16, "f32", 4)
    qs2 = np.array([0, 9])                                  # 9 rows for a 6-token sequence
    q2 = np.concatenate([q[:3], q])                         # rows 3.. are q again
    out = paged_prefill(q2, kp, vp, tables, qs2, lens, 0.25, "f32")
    assert not out[:3].any()                                 # positions -3..-1
    np.testing.assert_array_equal(out[3:], paged_prefill(q, kp, vp, tables, qs, lens, 0.25, "f32"))


def test_workload_scenario_builds_the_chunks():
    d = W.draw("prefill_8b")
    assert d.batch == 16 and int(d.step_lens.sum()) == 16 * 512
    step = W.scenario(d)[-1]
    assert step == [("append", i, int(d.context_lens[i]) - 512, 512) for i in range(16)]
    assert d.query_start[-1] == 8192 and W.prefill_query_bits(d).shape == (8192, 32, 128)


@pytest.mark.parametrize("window", [0, 1, 7, 40])
@pytest.mark.parametrize("kv_dtype", [None, "fp8_e4m3"])
def test_rows_at_once_equals_the_row_loop(window, kv_dtype):
    rng = np.random.default_rng(27)
    ctxs, chunks = [40, 17, 64, 5, 33, 3], [40, 9, 20, 1, 16, 5]   # the last: 2 negative rows
    q, ks, vs, qs, kp, vp, tables, lens = chunk_case(rng, ctxs, chunks, 8, 2, 32, "bf16", 4)
    if kv_dtype:   # arbitrary finite E4M3 codes in both pools
        kp = rng.integers(0, 0x7F, kp.shape).astype(np.uint8) | (rng.integers(0, 2, kp.shape) << 7).astype(np.uint8)
        vp = rng.integers(0, 0x7F, vp.shape).astype(np.uint8)
    kw = dict(window=window, kv_dtype=kv_dtype, k_scale=0.3, v_scale=0.7)
    want = paged_prefill(q, kp, vp, tables, qs, lens, 0.2, "bf16", **kw)
    got = paged_prefill_rows_at_once(q, kp, vp, tables, qs, lens, 0.2, "bf16", **kw)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)   # 8-bit values reach ~300
    assert not got[qs[5]:qs[5] + 2].any() and got[qs[5] + 2:].any()
    sub = paged_prefill_rows_at_once(q, kp, vp, tables, qs, lens, 0.2, "bf16", seqs=[1, 4], **kw)
    for i in range(len(ctxs)):
        rows = slice(qs[i], qs[i + 1])
        np.testing.assert_array_equal(sub[rows], got[rows] if i in (1, 4) else 0.0)
