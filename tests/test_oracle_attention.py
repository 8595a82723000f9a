"""Pins for the oracle's decode attention (CPU only).

* paged == dense: the paged oracle equals torch's scaled_dot_product_attention
  (float64, CPU, grouped-query heads) run on the contiguous K/V;
* relabelling physical blocks and changing the block size leave the output
  bit-identical;
* closed forms: one token, zero query, equal keys, one dominant key;
* split-K: the partitioned log-sum-exp merge equals direct softmax;
* poisoned padding: NaN in every slot the sequences do not own and a huge
  id in table padding change nothing;
* brute force: pure-Python loops on the tiny workload;
* element decoding matches torch's own bf16/f16 views.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import OracleAllocator
from oracle.attention import (decode_bits, dense_attention, gather_sequence,
                              merge_partitions, paged_decode, partition_state,
                              partitioned_decode)
from oracle.kvcache import write_slots


def page_sequences(k_seqs, v_seqs, nb, bs, order, fill=None):
    """Oracle state: allocate each sequence's tokens lazily and write them."""
    a = OracleAllocator(nb, bs, order)
    hkv, d = k_seqs[0].shape[1:]
    dt = k_seqs[0].dtype
    kp = np.zeros((nb, hkv, bs, d), dt) if fill is None else fill[0].copy()
    vp = np.zeros((nb, hkv, bs, d), dt) if fill is None else fill[1].copy()
    seqs = []
    for k, v in zip(k_seqs, v_seqs):
        s = a.create()
        slots, _ = a.append(s, k.shape[0])
        write_slots(kp, k, np.asarray(slots))
        write_slots(vp, v, np.asarray(slots))
        seqs.append(s)
    maxb = max(-(-k.shape[0] // bs) for k in k_seqs)
    tables, lens = a.build_tables(seqs, maxb)
    return kp, vp, tables, lens


def random_case(rng, lens, hq, hkv, d, dtype="f32"):
    ks = [W.to_bits(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype) for n in lens]
    vs = [W.to_bits(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype) for n in lens]
    q = W.to_bits(rng.standard_normal((len(lens), hq, d), dtype=np.float32), dtype)
    return q, ks, vs


def sdpa_reference(q64, k64, v64, scale):
    """torch SDPA on contiguous K/V: q [Hq][D], k/v [ctx][Hkv][D]."""
    qt = torch.from_numpy(q64)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k64.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v64.transpose(1, 0, 2)))[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale,
                                                           enable_gqa=True)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bs", [16, 32, 4])
def test_paged_equals_dense_sdpa(dtype, bs):
    rng = np.random.default_rng(11)
    lens = [1, 17, 40, 64, 3]
    hq, hkv, d = 8, 2, 32
    q, ks, vs = random_case(rng, lens, hq, hkv, d, dtype)
    nb = sum(-(-n // bs) for n in lens) + 5
    kp, vp, tables, ctx = page_sequences(ks, vs, nb, bs, rng.permutation(nb))
    scale = 1 / math.sqrt(d)
    out = paged_decode(q, kp, vp, tables, ctx, scale, dtype)
    for i in range(len(lens)):
        ref = sdpa_reference(decode_bits(q[i], dtype), decode_bits(ks[i], dtype),
                             decode_bits(vs[i], dtype), scale)
        np.testing.assert_allclose(out[i], ref, rtol=0, atol=1e-12)


def test_gqa_head_mapping_is_contiguous_groups():
    """q heads 0..G-1 read kv head 0: with kv head 1 made of zeros in V, the
    first group's output is non-zero and the second group's is zero."""
    rng = np.random.default_rng(3)
    q, ks, vs = random_case(rng, [20], 4, 2, 8)
    vs[0][:, 1, :] = W.to_bits(np.zeros((20, 8), np.float32), "f32")
    kp, vp, tables, ctx = page_sequences(ks, vs, 4, 16, [2, 0, 1, 3])
    out = paged_decode(q, kp, vp, tables, ctx, 0.3, "f32")[0]
    assert np.all(np.abs(out[:2]).sum(axis=1) > 0)
    assert np.all(out[2:] == 0)


def test_block_permutation_invariance_bit_exact():
    rng = np.random.default_rng(5)
    lens = [33, 16, 1, 50]
    q, ks, vs = random_case(rng, lens, 4, 4, 16)
    nb = 20
    kp, vp, tables, ctx = page_sequences(ks, vs, nb, 16, rng.permutation(nb))
    out = paged_decode(q, kp, vp, tables, ctx, 0.25, "f32")
    pi = rng.permutation(nb)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    tables2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1)
    out2 = paged_decode(q, kp2, vp2, tables2, ctx, 0.25, "f32")
    assert np.array_equal(out, out2)


def test_block_size_invariance_bit_exact():
    rng = np.random.default_rng(6)
    lens = [70, 5, 32]
    q, ks, vs = random_case(rng, lens, 2, 1, 16, "bf16")
    a = page_sequences(ks, vs, 12, 16, rng.permutation(12))
    b = page_sequences(ks, vs, 6, 32, rng.permutation(6))
    oa = paged_decode(q, *a, 0.25, "bf16")
    ob = paged_decode(q, *b, 0.25, "bf16")
    assert np.array_equal(oa, ob)


def test_closed_forms():
    rng = np.random.default_rng(7)
    d, hkv = 16, 2
    # one token: out is that token's V exactly
    q = rng.standard_normal((4, d))
    k = rng.standard_normal((1, hkv, d))
    v = rng.standard_normal((1, hkv, d))
    out = dense_attention(q, k, v, 0.5)
    assert np.array_equal(out[:2], np.repeat(v[:, 0], 2, axis=0))
    assert np.array_equal(out[2:], np.repeat(v[:, 1], 2, axis=0))
    # zero query, or all keys equal: the plain mean of the V rows
    k = rng.standard_normal((37, hkv, d))
    v = rng.standard_normal((37, hkv, d))
    out = dense_attention(np.zeros((4, d)), k, v, 0.5)
    np.testing.assert_allclose(out[0], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[3], v[:, 1].mean(axis=0), rtol=0, atol=1e-14)
    keq = np.repeat(rng.standard_normal((1, hkv, d)), 37, axis=0)
    out = dense_attention(q, keq, v, 0.5)
    np.testing.assert_allclose(out[1], v[:, 0].mean(axis=0), rtol=0, atol=1e-14)
    # one key aligned with the query and much larger: out -> that V row
    k = rng.standard_normal((37, hkv, d))
    k[21, 0] = 200.0 * q[0] / np.linalg.norm(q[0])
    out = dense_attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0], v[21, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("ptok", [16, 512])
@pytest.mark.parametrize("ctx", [1, 511, 512, 513, 32768])
def test_split_k_merge_equals_direct(ptok, ctx):
    rng = np.random.default_rng(ctx + ptok)
    hq, hkv, d = 2, 1, 8
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((ctx, hkv, d)) * 2
    v = rng.standard_normal((ctx, hkv, d))
    direct = dense_attention(q, k, v, 0.7)
    split = partitioned_decode(q, k, v, 0.7, ptok)
    np.testing.assert_allclose(split, direct, rtol=0, atol=1e-12)


def test_merge_of_one_partition_is_normalisation():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((9, 1, 4))
    v = rng.standard_normal((9, 1, 4))
    m, l, o = partition_state(q, k, v, 1.0)
    np.testing.assert_allclose(merge_partitions([m], [l], [o]), o / l[:, None], rtol=1e-15)


def test_poisoned_padding_changes_nothing():
    rng = np.random.default_rng(9)
    lens = [33, 7, 16]
    q, ks, vs = random_case(rng, lens, 4, 2, 16, "bf16")
    nb = 12
    order = rng.permutation(nb)
    clean = page_sequences(ks, vs, nb, 16, order)
    nan = np.full((nb, 2, 16, 16), 0x7FC0, np.uint16)
    poisoned = page_sequences(ks, vs, nb, 16, order, fill=(nan, nan))
    tables = poisoned[2].copy()
    tables[tables < 0] = 1 << 30
    oc = paged_decode(q, *clean, 0.25, "bf16")
    op = paged_decode(q, poisoned[0], poisoned[1], tables, poisoned[3], 0.25, "bf16")
    assert np.all(np.isfinite(op))
    assert np.array_equal(oc, op)


def brute_force_attention(q, k_rows, v_rows, scale):
    """Pure-Python loops: q [D] list, k_rows/v_rows lists of [D] lists."""
    scores = [scale * sum(a * b for a, b in zip(q, kr)) for kr in k_rows]
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = sum(w)
    d = len(q)
    return [sum(w[t] * v_rows[t][j] for t in range(len(w))) / tot for j in range(d)]


def test_brute_force_tiny_workload():
    d = W.draw("tiny")
    wl = d.wl
    q = W.query_bits(d)
    ks, vs = zip(*[W.sequence_kv_bits(d, i) for i in range(d.batch)])
    kp, vp, tables, ctx = page_sequences(list(ks), list(vs), d.num_blocks, wl.block_size,
                                         d.free_order)
    out = paged_decode(q, kp, vp, tables, ctx, wl.scale, wl.dtype)
    for i in range(d.batch):
        kf = ks[i].view(np.float32).tolist()
        vf = vs[i].view(np.float32).tolist()
        qf = q[i].view(np.float32).tolist()
        for h in range(wl.num_q_heads):
            g = h // wl.group
            ref = brute_force_attention(qf[h], [kr[g] for kr in kf], [vr[g] for vr in vf], wl.scale)
            np.testing.assert_allclose(out[i, h], ref, rtol=0, atol=1e-12)


def test_gather_follows_logical_order():
    pool = np.arange(4 * 1 * 2 * 1).reshape(4, 1, 2, 1)   # token id = 2*block + offset
    rows = gather_sequence(pool, [3, 0, 2], 5)
    assert rows[:, 0, 0].tolist() == [6, 7, 0, 1, 4]


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_decode_bits_matches_torch(dtype, tdt):
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    ours = decode_bits(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16)).view(tdt).double().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_decode_bits_f32():
    x = np.array([0.0, -1.5, 3.25e-20, np.inf], np.float32)
    assert decode_bits(x.view(np.uint32), "f32").tolist() == [0.0, -1.5, float(np.float32(3.25e-20)), math.inf]


def test_bf16_rounding_of_inputs_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000, dtype=np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 1.0 + 2 ** -9]  # ties and near-ties
    ours = W.to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
