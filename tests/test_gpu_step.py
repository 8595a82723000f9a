"""Decode steps through ``PagedKVCache.plan`` with device-resident block
tables, against the oracle, on the GPU.

A step's plan makes one batched allocator call, uploads the slots, copy
pairs and new lengths once, and patches the resident tables on the device
from the slots (``pa_update_tables``); any other table change (here a fork
that adds a sequence to the batch) rebuilds them.  After every step: slots
and pairs equal the oracle's batched append, the device tables equal the
oracle's tables entry for entry (-1 past each sequence's blocks), the
lengths are equal, and decode through the device tables is within tolerance
of the oracle's; at the end both pools are bit-identical.
"""
import numpy as np
import pytest

import workloads as W
from _scenario import KV, TOL, from_device_bits, max_abs_err, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; never a fallback
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="needs a GPU")]

import paged_kv_cache_107_amd as pa  # noqa: E402
from oracle.attention import paged_decode  # noqa: E402
from oracle.kvcache import copy_blocks, write_slots  # noqa: E402


@pytest.mark.parametrize("name,batch", [("cow", 32), ("8b_gqa", 40), ("tiny", None),
                                        ("qwen32b_long_bs32", 6)])
def test_resident_tables_follow_the_oracle(name, batch):
    d = W.draw(name, batch=batch)
    wl = d.wl
    print(f"step planner: {name} B={d.batch}", flush=True)
    kv = KV(d)
    o = run_oracle(d, kv, compute_out=False)
    g = run_gpu(d, kv, decode=False)
    cache, oa, kp, vp = g["cache"], o["alloc"], o["kp"], o["vp"]
    assert g["plan"].rebuilt
    seqs = list(range(d.batch))
    rng = np.random.default_rng(1234)
    bits = np.uint32 if wl.dtype == "f32" else np.uint16
    # steps: (tokens per sequence, fork the first sequence before the step)
    schedule = [(1, False), (1, False), (3, False), (1, True), (1, False), (2, False)]
    patched = 0
    for k, (n_tok, fork) in enumerate(schedule):
        if fork:
            child = cache.fork(seqs[0])
            assert oa.fork(seqs[0]) == child
            seqs = seqs + [child]
        shared_partial = fork and oa.lens[seqs[0]] % wl.block_size != 0
        plan = cache.plan(seqs, n_tok)
        o_slots, o_pairs = oa.append_batch(seqs, n_tok)
        if fork:
            assert plan.rebuilt              # the batch changed
        patched += not plan.rebuilt
        assert plan.slots.cpu().tolist() == o_slots
        assert [tuple(p) for p in plan.pairs.cpu().tolist()] == o_pairs
        if shared_partial:
            assert len(o_pairs) >= 1          # parent and child share the partial block
        shape = (len(seqs) * n_tok, wl.num_kv_heads, wl.head_dim)
        k_new = W.to_bits(rng.standard_normal(shape, dtype=np.float32), wl.dtype)
        v_new = W.to_bits(rng.standard_normal(shape, dtype=np.float32), wl.dtype)
        copy_blocks(kp, o_pairs)
        copy_blocks(vp, o_pairs)
        write_slots(kp, k_new, np.asarray(o_slots))
        write_slots(vp, v_new, np.asarray(o_slots))
        q_bits = W.to_bits(rng.standard_normal((len(seqs), wl.num_q_heads, wl.head_dim),
                                               dtype=np.float32), wl.dtype)
        q = to_device(q_bits, wl.dtype)
        out = torch.full_like(q, float("nan"))
        ws = cache.workspace(len(seqs), wl.num_q_heads, plan.max_context_len)
        cache.run(plan, to_device(k_new, wl.dtype), to_device(v_new, wl.dtype), q, wl.scale, out,
                  ws)
        torch.cuda.synchronize()
        tables_o, lens_o = oa.build_tables(seqs, plan.tables.shape[1])
        assert np.array_equal(plan.tables.cpu().numpy(), tables_o), f"step {k}: tables differ"
        assert np.array_equal(plan.lens.cpu().numpy(), lens_o)
        assert plan.host_lens.tolist() == lens_o.tolist()
        assert plan.max_context_len == int(lens_o.max())
        want = paged_decode(q_bits, kp, vp, tables_o, lens_o, wl.scale, wl.dtype)
        err = max_abs_err(out, want)
        print(f"  step {k}: n={n_tok} rebuilt={plan.rebuilt} pairs={len(o_pairs)} "
              f"max_abs_err={err:.2e}", flush=True)
        assert err <= TOL[wl.dtype], (k, err)
    assert patched >= 3, "the incremental path ran too rarely to be tested"
    assert np.array_equal(from_device_bits(cache.k_pool, wl.dtype), kp.view(bits))
    assert np.array_equal(from_device_bits(cache.v_pool, wl.dtype), vp.view(bits))
    free, rc = cache.alloc.pa_alloc_query()
    assert free.tolist() == list(oa.free) and rc.tolist() == oa.refcount


def test_update_tables_kernel_skips_out_of_range_entries():
    """pa_update_tables on hand-made rows: negative slots and positions past
    max_blocks_per_seq are skipped, every other entry is the slot's block,
    and every length is written."""
    bs, maxb, n_tok = 16, 3, 4
    lens = np.array([4, 20, 49, 3], dtype=np.int32)          # 3 rows x 4 new positions (row 3: 3)
    slots = np.array([[160, 161, 162, 163],                   # positions 0..3 -> block 10
                      [300, 301, -1, 303],                    # 16..19: block 18, one skipped
                      [900, 901, 902, 903],                   # 45..48: pos 48 is block 3 >= maxb
                      [-5, 7, 8, 9]], dtype=np.int64)         # positions -1..2: -1 skipped
    tables = np.full((4, maxb), 77, dtype=np.int32)
    want = tables.copy()
    for i in range(4):
        for t in range(n_tok):
            pos = int(lens[i]) - n_tok + t
            if slots[i, t] >= 0 and pos >= 0 and pos // bs < maxb:
                want[i, pos // bs] = slots[i, t] // bs
    dt = torch.from_numpy(tables).cuda()
    dl = torch.zeros(4, dtype=torch.int32, device="cuda")
    ds = torch.from_numpy(slots.reshape(-1)).cuda()
    dn = torch.from_numpy(lens).cuda()
    st = pa.lib().pa_update_tables(ds.data_ptr(), dn.data_ptr(), 4, n_tok, bs, dt.data_ptr(),
                                   maxb, dl.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    assert dt.cpu().numpy().tolist() == want.tolist()
    assert dl.cpu().numpy().tolist() == lens.tolist()
