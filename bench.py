"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b_gqa]

A step is one pass of the whole device path over one batch: the step's CoW
block copies, the cache write of every sequence's new token, decode attention
through the block tables (partition kernel, then the split-K reduce).  The
host half of the step (allocator reservations, block tables, their upload)
is timed once and reported beside it; the inputs of the timed steps are
already resident in HBM.

Default workload: 8B-shaped GQA decode, one layer, batch 256 (32 q heads,
8 kv heads, head_dim 128, bf16, block 16, log-normal lengths with median
1500 and sigma 0.8 clipped to [16, 8192]), synthetic N(0,1) data.

Printed (one JSON line): sequences/s of the whole step, KV GB/s and its
fraction of the HBM peak, the partition kernel's roofline (algorithmic bytes
over its average duration, timed with HIP events on the launch stream), the
CPU oracle timed on a bounded sample of the same workload, and, apart from the
timed step, the chunked-prefill kernel on its own workload with its
matrix-core roofline, and the prefill of requests sharing a system prompt
with and without the prefix cache (hit rate, pinned blocks, blocks held,
device time of the prefill pass, host time per request), and swapping every
8th decode sequence out to pinned host memory and back (host-link rate of
the swap kernel beside a plain copy of the same size), and the decode of the
same batch with a 1024-position sliding window and on 8-bit E4M3 pools.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "paged decode-attn KV GB/s (% of HBM peak) + sequences/s, 8B-GQA batch 256"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 matrix-core peak
KERNEL_SOURCES = ["paged_kv_cache_107_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_107_amd/csrc/pa_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_pa_decode_partition.json")

DESCRIPTIONS = {
    "8b_gqa": "8B GQA decode, 1 layer: B=256, 32 q / 8 kv heads, head_dim 128, bf16, block 16, "
              "lengths lognormal(median 1500, sigma 0.8) clipped to [16, 8192], seed 2",
    "7b_mha": "7B MHA decode, 1 layer: B=64, 32 q = 32 kv heads, head_dim 128, fp16, block 16, "
              "lengths uniform [128, 2048], seed 1",
    "cow": "parallel-sampling CoW, 8B GQA shape, bf16: 32 prompts x 4 branches, 1000-token "
           "shared prefix, tails uniform [0, 256], seed 3",
    "qwen32b_long": "Qwen3-32B-shaped long context, 1 layer: 64 q / 8 kv heads, head_dim 128, "
                    "bf16, block 16, 32 x 2048 + 4 x 32768 tokens",
    "qwen32b_long_bs32": "as qwen32b_long with block 32",
    "tiny": "tiny: 4 sequences {10, 5, 33, 7}, 4 heads, head_dim 64, fp32, block 16",
}
PREFILL_DESCRIPTION = ("8B GQA chunked prefill, 1 layer: 16 sequences x 512-token chunks on "
                       "cached prefixes lognormal(median 1500, sigma 0.8) clipped to [0, 7680], "
                       "32 q / 8 kv heads, head_dim 128, bf16, block 16, seed 5")


# Split-K partition size per workload: the long-context workload is stated
# with 512-token partitions; for the others the size with the shortest
# measured partition + reduce time on MI355X.
DEFAULT_PARTITION = {"8b_gqa": 2048, "7b_mha": 512, "cow": 2048, "qwen32b_long": 512,
                     "qwen32b_long_bs32": 512, "tiny": 512}
# the decode workloads measured, in the order they are listed
CONFIG_WORKLOADS = ["tiny", "7b_mha", "8b_gqa", "cow", "qwen32b_long", "qwen32b_long_bs32"]


def calibration_copy(pairs: int, wl, log):
    """pa_copy_blocks of `pairs` disjoint whole blocks (K and V) on a scratch
    pool: reads and writes exactly pairs * 2 * Hkv * BS * D * b bytes each."""
    import torch
    import paged_kv_cache_107_amd as pa
    from paged_kv_cache_107_amd.cache import TORCH_DTYPES
    shape = (2 * pairs, wl.num_kv_heads, wl.block_size, wl.head_dim)
    kp = torch.zeros(shape, dtype=TORCH_DTYPES[wl.dtype], device="cuda")
    vp = torch.zeros_like(kp)
    pr = torch.stack([torch.arange(pairs), torch.arange(pairs, 2 * pairs)], 1).int().cuda()
    pa.pa_copy_blocks(kp, vp, pr)
    torch.cuda.synchronize()
    nbytes = 2 * pairs * wl.num_kv_heads * wl.block_size * wl.head_dim * wl.elem_bytes
    log(f"calibration copy: {pairs} block pairs, {nbytes} bytes read and {nbytes} written")
    del kp, vp


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, part_tokens: int):
    """HBM bytes per partition-kernel launch from the committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_sha256") != kernel_source_hash():
        return None
    if entry.get("partition_tokens", 512) != part_tokens:
        return None
    return entry.get("traffic_bytes")


# ------------------------------------------------------------------ setup

def build_state(d, part_tokens: int, log):
    """Pool population (prefill-size cache writes) and the step's plan."""
    import torch
    from paged_kv_cache_107_amd.cache import TORCH_DTYPES, PagedKVCache
    wl = d.wl
    signed = np.int32 if wl.dtype == "f32" else np.int16
    tdt = TORCH_DTYPES[wl.dtype]

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits.view(signed))).cuda().view(tdt)

    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    pools = tuple(torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(tdt)
                  for _ in range(2))
    cache = PagedKVCache(d.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype,
                         d.free_order, pools=pools)
    phases = W.scenario(d)
    kv_cache = {}

    def kv(i):
        if i not in kv_cache:
            kv_cache[i] = W.sequence_kv_bits(d, i)
        return kv_cache[i]

    t0 = time.perf_counter()
    for phase in phases[:-1]:
        slots, pairs, ks, vs, n_tok = [], [], [], [], 0
        for op in phase:
            if op[0] == "create":
                cache.create()
            elif op[0] == "fork":
                cache.fork(op[1])
            else:
                i, start, n = op[1:]
                s, pair = cache.reserve(i, n)
                # copies of earlier reservations must land before later writes
                if pair is not None:
                    pairs.append(pair)
                slots.append(s)
                k, v = kv(i)
                ks.append(k[start:start + n])
                vs.append(v[start:start + n])
                n_tok += n
            if n_tok > (1 << 18):
                cache.write_host(dev(np.concatenate(ks)), dev(np.concatenate(vs)),
                                 np.concatenate(slots), pairs)
                slots, pairs, ks, vs, n_tok = [], [], [], [], 0
        if slots or pairs:
            cache.write_host(dev(np.concatenate(ks)), dev(np.concatenate(vs)),
                             np.concatenate(slots), pairs)
    step = phases[-1]
    k_new = dev(np.stack([kv(op[1])[0][op[2]] for op in step]))
    v_new = dev(np.stack([kv(op[1])[1][op[2]] for op in step]))
    kv_cache.clear()
    torch.cuda.synchronize()
    log(f"pool populated in {time.perf_counter() - t0:.1f}s")
    plan = cache.plan([op[1] for op in step], 1)
    torch.cuda.synchronize()
    q = dev(W.query_bits(d))
    out = torch.empty_like(q)
    ws = cache.workspace(d.batch, wl.num_q_heads, plan.max_context_len, part_tokens)
    return cache, plan, q, out, ws, k_new, v_new


def populate_device(d, part_tokens: int, seed_stream: int = 11):
    """Pool population for a timing-only record: the workload's allocator
    scenario, with every written token's K/V drawn on the device (torch's
    seeded generator, N(0,1) rounded to the dtype) and written by
    pa_reshape_and_cache; CoW copies first within each batch of writes.
    Returns the step's state like build_state."""
    import torch
    from paged_kv_cache_107_amd.cache import TORCH_DTYPES, PagedKVCache
    wl = d.wl
    tdt = TORCH_DTYPES[wl.dtype]
    gen = torch.Generator(device="cuda").manual_seed(1000 * wl.seed + seed_stream)
    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    pools = tuple(torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(tdt)
                  for _ in range(2))
    cache = PagedKVCache(d.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype,
                         d.free_order, pools=pools)

    def rows(n):
        return torch.randn((n, wl.num_kv_heads, wl.head_dim), generator=gen, device="cuda",
                           dtype=torch.float32).to(tdt)

    phases = W.scenario(d)
    for phase in phases[:-1]:
        slots, pairs, n_tok = [], [], 0

        def flush():
            if slots:
                cache.write_host(rows(n_tok), rows(n_tok), np.concatenate(slots), pairs)

        for op in phase:
            if op[0] == "create":
                cache.create()
            elif op[0] == "fork":
                cache.fork(op[1])
            else:
                sl, pair = cache.reserve(op[1], op[3])
                if pair is not None:
                    pairs.append(pair)
                slots.append(sl)
                n_tok += op[3]
                if n_tok > (1 << 18):
                    flush()
                    slots, pairs, n_tok = [], [], 0
        flush()
    step = phases[-1]
    plan = cache.plan([op[1] for op in step], 1)
    n = len(step)
    k_new, v_new = rows(n), rows(n)
    q = torch.randn((n, wl.num_q_heads, wl.head_dim), generator=gen, device="cuda",
                    dtype=torch.float32).to(tdt)
    out = torch.empty_like(q)
    ws = cache.workspace(n, wl.num_q_heads, plan.max_context_len, part_tokens)
    torch.cuda.synchronize()
    return cache, plan, q, out, ws, k_new, v_new


def time_step(cache, plan, q, out, ws, k_new, v_new, wl, part_tokens: int, reps: int):
    """`reps` decode steps on the launch stream, each pass between its own
    HIP events: mean microseconds per pass and of the whole step (first
    event to last)."""
    import torch
    import paged_kv_cache_107_amd as pa
    stream = torch.cuda.current_stream()
    args = (q, cache.k_pool, cache.v_pool, plan.tables, plan.lens, wl.scale, out, ws,
            plan.max_context_len, part_tokens)
    fns = []
    if plan.pairs.shape[0]:
        fns.append(("copy_blocks", lambda: pa.pa_copy_blocks(cache.k_pool, cache.v_pool,
                                                               plan.pairs)))
    fns += [("reshape_and_cache", lambda: pa.pa_reshape_and_cache(
                k_new, v_new, plan.slots, cache.k_pool, cache.v_pool)),
            ("decode_partition", lambda: pa.pa_decode_partition(*args)),
            ("decode_reduce", lambda: pa.pa_decode_reduce(*args))]
    for _ in range(5):
        for _, f in fns:
            f()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        for j, (_, f) in enumerate(fns):
            f()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    res = {name: 1e3 * float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
           for j, (name, _) in enumerate(fns)}
    res["step"] = 1e3 * float(np.mean([e[0].elapsed_time(e[-1]) for e in ev]))
    return res


def measure_configs(names, reps: int, log):
    """Each listed decode workload, each on its own freshly
    populated cache (device-drawn contents): the decode step's passes timed
    with HIP events on the launch stream, sequences/s of the step, KV GB/s
    and the partition kernel's HBM roofline."""
    import torch
    res = {}
    for name in names:
        d = W.draw(name)
        wl = d.wl
        pt = DEFAULT_PARTITION[name]
        t0 = time.perf_counter()
        state = populate_device(d, pt)
        cache, plan = state[0], state[1]
        t = time_step(*state, wl, pt, reps)
        ctx = d.context_lens.astype(np.int64)
        eb = wl.elem_bytes
        row = 2 * wl.num_kv_heads * wl.head_dim * eb          # K + V bytes of one token
        kv = int(ctx.sum()) * row
        # K/V of the distinct blocks the batch attends: a block shared by
        # several sequences is one block of memory, read for each of them;
        # the roofline counts it once (its tokens: the most any sharer uses)
        used = {}
        tables = plan.tables.cpu().numpy()
        for i, c in enumerate(ctx.tolist()):
            for j in range(-(-c // wl.block_size)):
                b = int(tables[i, j])
                used[b] = max(used.get(b, 0), min(wl.block_size, c - j * wl.block_size))
        kv_unique = sum(used.values()) * row
        alg = (kv_unique + 2 * d.batch * wl.num_q_heads * wl.head_dim * eb +
               int(np.sum(-(-ctx // wl.block_size))) * 4 + 4 * d.batch)
        part = t["decode_partition"]
        gbps = alg / (part * 1e-6) / 1e9
        rec = {"workload": DESCRIPTIONS[name], "dtype": wl.dtype, "batch": d.batch,
               "attended_tokens": int(ctx.sum()), "partition_tokens": pt,
               "cow_pairs": int(plan.pairs.shape[0]), "kv_bytes": kv,
               "kv_bytes_distinct_blocks": kv_unique, "algorithmic_bytes": alg,
               "step_us": round(t["step"], 2),
               "passes_us": {k: round(v, 2) for k, v in t.items() if k != "step"},
               "seq_per_s": round(d.batch / (t["step"] * 1e-6), 1),
               "kv_gbps_step": round(kv / (t["step"] * 1e-6) / 1e9, 1),
               "roofline": {"bound": "hbm", "kernel": "pa_decode_partition",
                            "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None}}
        if name == "cow":
            rec["note"] = ("branches share their prefix blocks: kv_bytes counts them per "
                           "sequence, the roofline once (kv_bytes_distinct_blocks)")
        if name == "tiny":
            rec["note"] = "latency-bound (110 KiB of K/V): no bandwidth claim"
        res[name] = rec
        log(f"config {name}: step {t['step']:.1f} us, partition {part:.1f} us "
            f"({gbps:.0f} GB/s, {gbps / HBM_PEAK_GBPS:.1%}), {rec['seq_per_s']:.0f} seq/s, "
            f"{rec['cow_pairs']} CoW pairs, populated in {time.perf_counter() - t0:.1f}s")
        del state, cache, plan
        torch.cuda.empty_cache()
    return res


def measure_e2e(cache, plan, q, out, ws, k_new, v_new, d, part_tokens: int, steps: int, log):
    """Real decode steps back to back: each step plans (one batched
    allocator call, one upload, the resident tables patched on the device)
    and runs (copies, cache write, attention), so every sequence grows by
    one token per step.  The host's planning of step k+1 overlaps the
    device's work of step k.  Reports the host time of a plan (median) and
    the wall time per step."""
    import torch
    wl = d.wl
    seqs = plan.seqs
    # the host half alone: each plan timed with the device idle (nothing to
    # wait for), then its step run
    host = []
    for _ in range(steps):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        p = cache.plan(seqs, 1)
        host.append(time.perf_counter() - h0)
        cache.run(p, k_new, v_new, q, wl.scale, out, ws, part_tokens)
    # pipelined: the host plans step k + 1 while the device runs step k
    rebuilt = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        p = cache.plan(seqs, 1)
        rebuilt += p.rebuilt
        cache.run(p, k_new, v_new, q, wl.scale, out, ws, part_tokens)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    host_ms = 1e3 * float(np.median(host))
    log(f"e2e: {steps} steps, {1e3 * wall:.3f} ms per step ({d.batch / wall:.0f} seq/s), host "
        f"plan {host_ms:.3f} ms median (device idle), {rebuilt} table rebuilds")
    return {"steps": steps, "ms_per_step": round(1e3 * wall, 4),
            "seq_per_s": round(d.batch / wall, 1), "host_plan_ms_median": round(host_ms, 4),
            "host_plan_ms_p90": round(1e3 * float(np.percentile(host, 90)), 4),
            "table_rebuilds": rebuilt}


def measure_prefill(reps: int, log):
    """pa_prefill on the chunked-prefill workload: every sequence's prefix and
    chunk K/V written through the allocator and the cache kernels, then `reps`
    timed calls (HIP events on the launch stream)."""
    import torch
    import paged_kv_cache_107_amd as pa
    from paged_kv_cache_107_amd.cache import TORCH_DTYPES, PagedKVCache
    d = W.draw("prefill_8b")
    wl = d.wl
    tdt = TORCH_DTYPES[wl.dtype]

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits.view(np.int16))).cuda().view(tdt)

    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    pools = tuple(torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(tdt)
                  for _ in range(2))
    cache = PagedKVCache(d.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.dtype,
                         d.free_order, pools=pools)
    for phase in W.scenario(d):
        slots, ks, vs = [], [], []
        for op in phase:
            if op[0] == "create":
                cache.create()
            else:
                i, start, n = op[1:]
                s, pair = cache.reserve(i, n)
                assert pair is None
                k, v = W.sequence_kv_bits(d, i)
                slots.append(s)
                ks.append(k[start:start + n])
                vs.append(v[start:start + n])
        cache.write_host(dev(np.concatenate(ks)), dev(np.concatenate(vs)),
                         np.concatenate(slots), [])
    seqs = list(range(d.batch))
    lens = d.context_lens
    tables, lens_i = cache.alloc.pa_build_tables(seqs, int(-(-lens.max() // wl.block_size)))
    q = dev(W.prefill_query_bits(d))
    out = torch.empty_like(q)
    qs = torch.from_numpy(d.query_start.astype(np.int32)).cuda()
    args = (q, cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(), qs,
            torch.from_numpy(lens_i).cuda(), wl.scale, out, int(d.step_lens.max()),
            int(lens.max()))
    stream = torch.cuda.current_stream()

    def timed(window: int, call_args=args, **kw) -> float:
        for _ in range(3):
            pa.pa_prefill(*call_args, sliding_window=window, **kw)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            pa.pa_prefill(*call_args, sliding_window=window, **kw)
            b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))

    def attended(window: int) -> int:
        # row at position p attends p + 1 keys, at most `window` with a window
        pos1 = [(L - c) + np.arange(c) + 1 for L, c in zip(lens, d.step_lens)]
        return sum(int((np.minimum(p, window) if window > 0 else p).sum()) for p in pos1)

    us = timed(0)
    # 2 flops per multiply-add in each of Q K^T and P V
    flops = 4 * wl.head_dim * wl.num_q_heads * attended(0)
    tflops = flops / (us * 1e-6) / 1e12
    tokens = int(d.step_lens.sum())
    log(f"prefill: {us:.1f} us, {tflops:.1f} TFLOP/s, {tokens / (us * 1e-6):.0f} tokens/s")
    us_w = timed(VARIANT_WINDOW)
    flops_w = 4 * wl.head_dim * wl.num_q_heads * attended(VARIANT_WINDOW)
    tflops_w = flops_w / (us_w * 1e-6) / 1e12
    log(f"prefill window_{VARIANT_WINDOW}: {us_w:.1f} us, {tflops_w:.1f} TFLOP/s")
    # 8-bit E4M3 pools holding the quantised contents of the 16-bit pools
    # (every slot through the quantising pa_reshape_and_cache), same attended keys
    codes = quantised_pools(cache.k_pool, cache.v_pool)
    us_8 = timed(0, (q, *codes) + args[3:], kv_scales=FP8_SCALES)
    tflops_8 = flops / (us_8 * 1e-6) / 1e12
    log(f"prefill fp8_e4m3: {us_8:.1f} us, {tflops_8:.1f} TFLOP/s")
    del codes
    return {
        "workload": PREFILL_DESCRIPTION,
        "kernel_us": round(us, 2),
        "tokens_per_s": round(tokens / (us * 1e-6), 1),
        "roofline": {"bound": "mfma", "kernel": "pa_prefill", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops": flops},
        f"window_{VARIANT_WINDOW}": {
            "kernel_us": round(us_w, 2), "achieved": round(tflops_w, 1), "unit": "TFLOP/s",
            "frac": round(tflops_w / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops_w},
        "fp8_e4m3": {
            "kernel_us": round(us_8, 2), "achieved": round(tflops_8, 1), "unit": "TFLOP/s",
            "frac": round(tflops_8 / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops},
    }


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, per direction
VARIANT_WINDOW = 1024
FP8_SCALES = (0.05, 0.05)


def decode_tile_offsets(plan, d):
    """Byte offsets, in the pool, of every 16-token tile the decode step
    reads, in the stream split's flat order (kv head, sequence, tile)."""
    wl = d.wl
    tables = plan.tables.cpu().numpy().astype(np.int64)
    lens = plan.lens.cpu().numpy().astype(np.int64)
    row = wl.head_dim * wl.elem_bytes
    blk = wl.num_kv_heads * wl.block_size * row
    offs = []
    for g in range(wl.num_kv_heads):
        for i in range(d.batch):
            pos = np.arange(-(-int(lens[i]) // 16), dtype=np.int64) * 16
            offs.append(tables[i, pos // wl.block_size] * blk + g * wl.block_size * row +
                        (pos % wl.block_size) * row)
    return np.concatenate(offs)


def measure_read_probe(cache, plan, d, part_us: float, reps: int, log):
    """The read ceiling of the decode access pattern: pa_probe_tile_reads over
    the step's tiles, each (block, kv head)'s K and V tile read together as
    the partition kernel reads them, `reps` back-to-back calls between two
    HIP events, (a) with the decode stream kernel's work split (one run per
    wave, 4 waves per CU), set beside the partition kernel, and (b) with one
    tile per wave."""
    import torch
    import paged_kv_cache_107_amd as pa
    offs = decode_tile_offsets(plan, d)
    offs_d = torch.from_numpy(offs.astype(np.uint32).view(np.int32)).cuda()
    tile_bytes = 16 * d.wl.head_dim * d.wl.elem_bytes
    per_tile = 4 * (-(-len(offs) // 4))
    out = torch.empty(per_tile, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    nbytes = 2 * len(offs) * tile_bytes
    rec = {"tiles_per_pool": int(len(offs)), "tile_bytes": tile_bytes, "bytes": nbytes}
    for name, waves in (("decode_split", 0), ("one_tile_per_wave", per_tile)):
        for _ in range(3):
            pa.pa_probe_tile_reads(cache.k_pool, offs_d, tile_bytes, waves, out, cache.v_pool)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            pa.pa_probe_tile_reads(cache.k_pool, offs_d, tile_bytes, waves, out, cache.v_pool)
        b.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / reps
        rate = nbytes / (us * 1e-6) / 1e9
        rec[name] = {"us_k_and_v": round(us, 2), "gbps": round(rate, 1),
                     "frac_of_hbm_peak": round(rate / HBM_PEAK_GBPS, 4),
                     "partition_frac_of_probe_rate": round(us / part_us, 4)}
        log(f"read probe ({name}): {len(offs)} K and V tiles ({nbytes / 1e9:.3f} GB) in "
            f"{us:.1f} us = {rate:.0f} GB/s ({rate / HBM_PEAK_GBPS:.1%} of peak); the partition "
            f"kernel reads the same tiles at {us / part_us:.1%} of that rate")
    return rec


def quantised_pools(k_pool, v_pool):
    """8-bit E4M3 copies of both pools: every slot written once by the
    quantising pa_reshape_and_cache (scales FP8_SCALES)."""
    import torch
    import paged_kv_cache_107_amd as pa
    n_blocks, hkv, bs, dh = k_pool.shape
    flat = lambda p: p.permute(0, 2, 1, 3).reshape(n_blocks * bs, hkv, dh).contiguous()
    k8 = torch.zeros_like(k_pool, dtype=torch.uint8).view(pa.FP8)
    v8 = torch.zeros_like(k8)
    slots = torch.arange(n_blocks * bs, dtype=torch.int64, device="cuda")
    pa.pa_reshape_and_cache(flat(k_pool), flat(v_pool), slots, k8, v8, kv_scales=FP8_SCALES)
    torch.cuda.synchronize()
    return k8, v8


def measure_variants(cache, plan, q, d, reps: int, log):
    """Decode of the same 8B batch (same block tables, same q) in the
    attention variants: a sliding window of 1024 positions on the 16-bit
    pools, and 8-bit E4M3 pools holding the quantised contents of the 16-bit
    pools (written by the quantising pa_reshape_and_cache), with and without
    the window.  Each: partition and reduce kernels timed with HIP events on
    the launch stream; the partition kernel's algorithmic bytes are the
    attended K/V (at the pool's element size), q, out and the table entries
    of the attended blocks."""
    import torch
    import paged_kv_cache_107_amd as pa
    wl = d.wl
    ctx = d.context_lens.astype(np.int64)
    n_blocks, hkv, bs, dh = cache.k_pool.shape
    k8, v8 = quantised_pools(cache.k_pool, cache.v_pool)
    out = torch.empty_like(q)
    ws = cache.workspace(d.batch, wl.num_q_heads, plan.max_context_len)
    stream = torch.cuda.current_stream()
    res = {}
    for name, kp, vp, window, scales, eb in (
            ("window_1024", cache.k_pool, cache.v_pool, VARIANT_WINDOW, (1.0, 1.0), wl.elem_bytes),
            ("fp8_e4m3", k8, v8, 0, FP8_SCALES, 1),
            ("fp8_e4m3_window_1024", k8, v8, VARIANT_WINDOW, FP8_SCALES, 1)):
        args = (q, kp, vp, plan.tables, plan.lens, wl.scale, out, ws, plan.max_context_len, 0,
                None, window, scales)
        for _ in range(3):
            pa.pa_decode(*args)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in ev:
            e[0].record(stream)
            pa.pa_decode_partition(*args)
            e[1].record(stream)
            pa.pa_decode_reduce(*args)
            e[2].record(stream)
        torch.cuda.synchronize()
        part = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        whole = 1e3 * float(np.mean([e[0].elapsed_time(e[2]) for e in ev]))
        att = np.minimum(ctx, window) if window else ctx
        first = ctx - att
        tiles = -(-ctx // 16) - first // 16
        kv = int(att.sum()) * 2 * hkv * dh * eb
        alg = kv + 2 * d.batch * wl.num_q_heads * dh * wl.elem_bytes + int(tiles.sum()) * 4 // (
            bs // 16) + 4 * d.batch
        gbps = alg / (part * 1e-6) / 1e9
        res[name] = {"window": window, "kv_dtype": "fp8_e4m3" if eb == 1 else wl.dtype,
                     "attended_tokens": int(att.sum()), "kv_bytes": kv, "algorithmic_bytes": alg,
                     "partition_us": round(part, 2), "decode_us": round(whole, 2),
                     "seq_per_s": round(d.batch / (whole * 1e-6), 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1),
                                  "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                  "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None}}
        log(f"{name}: partition {part:.1f} us ({gbps:.0f} GB/s, {gbps / HBM_PEAK_GBPS:.1%}), "
            f"decode {whole:.1f} us, {d.batch / (whole * 1e-6):.0f} seq/s")
        if name == "fp8_e4m3":
            # the read ceiling of the 8-bit step's tiles (2 KiB each, K with
            # its V), as for the 16-bit pools in the main record
            offs = decode_tile_offsets(plan, d) // wl.elem_bytes
            offs_d = torch.from_numpy(offs.astype(np.uint32).view(np.int32)).cuda()
            pout = torch.empty(1024, dtype=torch.int32, device="cuda")
            for _ in range(3):
                pa.pa_probe_tile_reads(k8, offs_d, 2048, 0, pout, v8)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                pa.pa_probe_tile_reads(k8, offs_d, 2048, 0, pout, v8)
            b.record(stream)
            torch.cuda.synchronize()
            pus = 1e3 * a.elapsed_time(b) / reps
            res[name]["read_probe"] = {"us_k_and_v": round(pus, 2),
                                       "gbps": round(2 * len(offs) * 2048 / (pus * 1e-6) / 1e9, 1),
                                       "partition_frac_of_probe_rate": round(pus / part, 4)}
            log(f"{name}: read probe over the same 2 KiB K and V tiles {pus:.1f} us; the "
                f"partition kernel at {pus / part:.1%} of that rate")
    del k8, v8
    torch.cuda.empty_cache()
    return res
SWAP_DESCRIPTION = ("preemption on the 8B GQA decode batch: every 8th of the 256 sequences "
                    "swapped out to pinned host pools and back, 32 q / 8 kv heads, head_dim 128, "
                    "bf16, block 16")


def measure_swap(cache, d, reps: int, log):
    """Swap-out and swap-in of every 8th sequence of the decode batch on its
    populated cache: the allocator's host work, then pa_swap_blocks (device
    pools <-> pinned host pools), timed with HIP events on the launch stream.
    Beside it, a plain copy of the same byte count between a contiguous
    device buffer and pinned host memory (the DMA engines' rate)."""
    import torch
    import paged_kv_cache_107_amd as pa
    wl = d.wl
    victims = list(range(0, d.batch, 8))
    blocks = sum(int(cache.alloc.pa_seq_info(s)[1].size) for s in victims)
    cache.enable_swap(blocks + 64)
    block_bytes = wl.num_kv_heads * wl.block_size * wl.head_dim * wl.elem_bytes
    stream = torch.cuda.current_stream()
    out_us, in_us, host_out, host_in, moved = [], [], [], [], []
    for _ in range(reps + 1):
        t0 = time.perf_counter()
        pairs_out = [cache.alloc.pa_seq_swap_out(s) for s in victims]
        host_out.append(time.perf_counter() - t0)
        p_out = torch.from_numpy(np.concatenate(pairs_out)).cuda()
        t0 = time.perf_counter()
        pairs_in = [cache.alloc.pa_seq_swap_in(s) for s in victims]
        host_in.append(time.perf_counter() - t0)
        p_in = torch.from_numpy(np.concatenate(pairs_in)).cuda()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        pa.pa_swap_blocks(cache.k_pool, cache.v_pool, cache.k_host, cache.v_host, p_out,
                          pa.PA_SWAP_OUT)
        ev[1].record(stream)
        pa.pa_swap_blocks(cache.k_pool, cache.v_pool, cache.k_host, cache.v_host, p_in,
                          pa.PA_SWAP_IN)
        ev[2].record(stream)
        torch.cuda.synchronize()
        out_us.append(1e3 * ev[0].elapsed_time(ev[1]))
        in_us.append(1e3 * ev[1].elapsed_time(ev[2]))
        moved.append(int(p_out.shape[0]))
    out_us, in_us, host_out, host_in = out_us[1:], in_us[1:], host_out[1:], host_in[1:]
    nbytes = 2 * moved[-1] * block_bytes
    dev_buf = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    host_buf = torch.empty(nbytes // 2, dtype=torch.int16, pin_memory=True)
    dma = {"out": [], "in": []}
    for _ in range(reps + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        host_buf.copy_(dev_buf, non_blocking=True)
        ev[1].record(stream)
        dev_buf.copy_(host_buf, non_blocking=True)
        ev[2].record(stream)
        torch.cuda.synchronize()
        dma["out"].append(1e3 * ev[0].elapsed_time(ev[1]))
        dma["in"].append(1e3 * ev[1].elapsed_time(ev[2]))
    del dev_buf, host_buf
    o_us, i_us = float(np.mean(out_us)), float(np.mean(in_us))
    d_out, d_in = float(np.mean(dma["out"][1:])), float(np.mean(dma["in"][1:]))
    gbps = {k: nbytes / (u * 1e-6) / 1e9 for k, u in
            (("out", o_us), ("in", i_us), ("dma_out", d_out), ("dma_in", d_in))}
    log(f"swap: {moved[-1]} blocks ({nbytes / 1e6:.1f} MB) out {o_us:.0f} us "
        f"({gbps['out']:.1f} GB/s), in {i_us:.0f} us ({gbps['in']:.1f} GB/s); plain copy "
        f"{gbps['dma_out']:.1f} / {gbps['dma_in']:.1f} GB/s; host "
        f"{1e6 * np.mean(host_out) / len(victims):.1f} / {1e6 * np.mean(host_in) / len(victims):.1f}"
        f" us per sequence")
    return {
        "workload": SWAP_DESCRIPTION,
        "sequences": len(victims),
        "blocks": moved[-1],
        "bytes_per_direction": nbytes,
        "swap_out_us": round(o_us, 1),
        "swap_in_us": round(i_us, 1),
        "roofline": {"bound": "host link", "kernel": "pa_swap_blocks", "unit": "GB/s",
                     "peak": HOST_LINK_PEAK_GBPS,
                     "achieved_out": round(gbps["out"], 2), "achieved_in": round(gbps["in"], 2),
                     "frac_out": round(gbps["out"] / HOST_LINK_PEAK_GBPS, 4),
                     "frac_in": round(gbps["in"] / HOST_LINK_PEAK_GBPS, 4), "traffic": None},
        "plain_copy_gbps": {"out": round(gbps["dma_out"], 2), "in": round(gbps["dma_in"], 2)},
        "host_us_per_sequence": {"out": round(1e6 * float(np.mean(host_out)) / len(victims), 2),
                                 "in": round(1e6 * float(np.mean(host_in)) / len(victims), 2)},
    }


PREFIX_DESCRIPTION = ("8B GQA prompts sharing a system prompt, 1 layer: 100 requests, one "
                      "1024-token system prompt + per-request suffix uniform [16, 256] tokens, "
                      "32 q / 8 kv heads, head_dim 128, bf16, block 16, seed 6")


def measure_prefix_cache(reps: int, log):
    """The prefill of 100 requests that share a system prompt, with the
    prefix cache and without it.  Host: the allocator's lookups and appends
    (with token ids) for every request.  Device: one pass of the prefill path
    over the positions left to compute -- the cache write of their K/V and
    pa_prefill through the block tables -- timed with HIP events on the
    launch stream, `reps` passes per variant."""
    import torch
    import paged_kv_cache_107_amd as pa
    from paged_kv_cache_107_amd.cache import TORCH_DTYPES, PagedKVCache
    ps = W.prompt_set("prefix_1k")
    wl = ps.wl
    tdt = TORCH_DTYPES[wl.dtype]

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits.view(np.int16))).cuda().view(tdt)

    prompts = [W.prompt_token_ids(ps, r) for r in range(ps.requests)]
    res = {}
    for variant in ("cached", "uncached"):
        cache = PagedKVCache(ps.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                             wl.dtype, ps.free_order)
        if variant == "cached":
            cache.enable_prefix_cache()
        t0 = time.perf_counter()
        slots, hits = [], []
        for r, ids in enumerate(prompts):
            s, hit = cache.create_prefix(ids) if variant == "cached" else (cache.create(), 0)
            sl, _ = cache.reserve_tokens(s, ids[hit:])
            slots.append(sl)
            hits.append(hit)
        host_s = time.perf_counter() - t0
        hits = np.array(hits, dtype=np.int64)
        kv = [W.prompt_kv_bits_of(ps, r) for r in range(ps.requests)]
        k_new = dev(np.concatenate([k[h:] for (k, _), h in zip(kv, hits)]))
        v_new = dev(np.concatenate([v[h:] for (_, v), h in zip(kv, hits)]))
        del kv
        q = dev(np.concatenate([W.prompt_query_bits_of(ps, r)[h:] for r, h in enumerate(hits)]))
        out = torch.empty_like(q)
        slot_t = torch.from_numpy(np.concatenate(slots)).cuda()
        lens = ps.prompt_lens
        tables, lens32 = cache.alloc.pa_build_tables(list(range(ps.requests)),
                                                     int(-(-int(lens.max()) // wl.block_size)))
        qs = torch.from_numpy(np.concatenate([[0], np.cumsum(lens - hits)]).astype(np.int32)).cuda()
        args = (q, cache.k_pool, cache.v_pool, torch.from_numpy(tables).cuda(), qs,
                torch.from_numpy(lens32).cuda(), wl.scale, out, int((lens - hits).max()),
                int(lens.max()))

        def one_pass():
            pa.pa_reshape_and_cache(k_new, v_new, slot_t, cache.k_pool, cache.v_pool)
            pa.pa_prefill(*args)

        for _ in range(3):
            one_pass()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            one_pass()
            b.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in ev]))
        held = int(np.unique(tables[tables >= 0]).size)
        res[variant] = dict(us=us, held=held, host_s=host_s, computed=int((lens - hits).sum()),
                            stats=cache.prefix_stats() if variant == "cached" else None)
        del cache, k_new, v_new, q, out
        torch.cuda.empty_cache()
    c, u = res["cached"], res["uncached"]
    st = c["stats"]
    block_bytes = 2 * wl.num_kv_heads * wl.block_size * wl.head_dim * wl.elem_bytes
    lookups_per_s = ps.requests / c["host_s"]
    log(f"prefix cache: hit rate {st['hit_tokens'] / st['lookup_tokens']:.3f}, "
        f"prefill pass {c['us']:.1f} us cached vs {u['us']:.1f} us uncached "
        f"({u['us'] / c['us']:.2f}x), blocks held {c['held']} vs {u['held']}, "
        f"host {1e6 * c['host_s'] / ps.requests:.1f} us per request")
    return {
        "workload": PREFIX_DESCRIPTION,
        "hit_rate": round(st["hit_tokens"] / st["lookup_tokens"], 4),
        "pinned_blocks": st["pinned_blocks"],
        "cached_blocks": st["cached_blocks"],
        "tokens_computed": {"cached": c["computed"], "uncached": u["computed"]},
        "prefill_pass_us": {"cached": round(c["us"], 2), "uncached": round(u["us"], 2)},
        "prefill_speedup": round(u["us"] / c["us"], 3),
        "blocks_held": {"cached": c["held"], "uncached": u["held"]},
        "kv_bytes_saved_per_layer": (u["held"] - c["held"]) * block_bytes,
        "host_us_per_request": {"cached": round(1e6 * c["host_s"] / ps.requests, 2),
                                "uncached": round(1e6 * u["host_s"] / ps.requests, 2)},
        "host_lookups_per_s": round(lookups_per_s, 1),
    }


# ------------------------------------------------------------------ CPU oracle

def cpu_baseline(d, gpu_out, budget_s: float, log):
    """The oracle (as it stands) on the first sequences of the same workload,
    timed on the host; also checks those outputs against the GPU's."""
    from oracle import OracleAllocator
    from oracle.attention import paged_decode
    from oracle.kvcache import write_slots
    wl = d.wl
    q_all = W.query_bits(d)
    # probe one sequence, then size the sample to the time budget
    n_target = d.batch
    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    kp = np.full(shape, 0, W.bits_dtype(wl.dtype))
    vp = np.full(shape, 0, W.bits_dtype(wl.dtype))
    a = OracleAllocator(d.num_blocks, wl.block_size, d.free_order)
    wall = cpu = 0.0
    outs = []
    done = 0
    for i in range(n_target):
        k, v = W.sequence_kv_bits(d, i)
        s = a.create()
        slots, _ = a.append(s, k.shape[0])
        write_slots(kp, k, np.asarray(slots))
        write_slots(vp, v, np.asarray(slots))
        tables, lens = a.build_tables([s], -(-k.shape[0] // wl.block_size))
        c0, t0 = time.process_time(), time.perf_counter()
        outs.append(paged_decode(q_all[i:i + 1], kp, vp, tables, lens, wl.scale, wl.dtype)[0])
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        done += 1
        if wall >= budget_s:
            break
    ref = np.stack(outs)
    got = gpu_out[:done].float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - ref)))
    tokens = int(d.context_lens[:done].sum())
    log(f"oracle: {done} sequences ({tokens} tokens) in {wall:.2f}s wall, {cpu:.2f}s cpu; "
        f"max |gpu - oracle| = {err:.2e}")
    return {"value": done / wall, "unit": "seq/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"first {done} of {d.batch} sequences ({tokens} attended tokens), fp64 "
                      f"numpy oracle attention timed alone; host has {os.cpu_count()} logical "
                      f"CPUs; max abs diff vs GPU output on the sample {err:.2e}"}


# ------------------------------------------------------------------ main

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="8b_gqa", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="split-K partition size (0 = the workload's default)")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="PAIRS",
                    help="before warmup, copy PAIRS whole blocks once with pa_copy_blocks on a "
                         "scratch pool (a plain copy of known size for counter calibration)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--prefill-reps", type=int, default=20,
                    help="timed pa_prefill calls on the chunked-prefill workload (0 = skip)")
    ap.add_argument("--variant-reps", type=int, default=50,
                    help="timed decode calls per attention variant (window, 8-bit pools; 0 = "
                         "skip)")
    ap.add_argument("--swap-reps", type=int, default=10,
                    help="timed swap-out + swap-in cycles of every 8th decode sequence "
                         "(0 = skip)")
    ap.add_argument("--prefix-reps", type=int, default=10,
                    help="timed prefill passes per variant on the shared-system-prompt "
                         "workload, with and without the prefix cache (0 = skip)")
    ap.add_argument("--probe-reps", type=int, default=20,
                    help="read-ceiling probe passes over the step's K and V tiles (0 = skip)")
    ap.add_argument("--config-reps", type=int, default=30,
                    help="timed decode steps on each other named workload (0 = skip)")
    ap.add_argument("--e2e-steps", type=int, default=50,
                    help="real decode steps (plan + run) at the end, timing the host "
                         "planner (0 = skip)")
    ap.add_argument("--decode-balance", type=int, choices=(0, 1), default=1,
                    help="run-time balance of the decode stream split's XCD chunks (1, the "
                         "library default) or the even cut (0)")
    ap.add_argument("--only-configs", nargs="*", metavar="NAME", default=None,
                    help="time the other named workloads only, or just the NAMEs given (for a "
                         "profiler run)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        return 2

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import torch
    import paged_kv_cache_107_amd as pa
    torch.cuda.set_device(0)
    pa.lib()
    pa.pa_set_decode_balance(bool(args.decode_balance))
    others = [n for n in CONFIG_WORKLOADS if n != args.workload]
    if args.only_configs is not None:
        names = args.only_configs or others
        unknown = [n for n in names if n not in CONFIG_WORKLOADS]
        if unknown:
            print(f"unknown workloads {unknown}; named: {list(CONFIG_WORKLOADS)}", file=sys.stderr)
            return 2
        print(json.dumps({"configs": measure_configs(names, max(args.config_reps, 1), log)}),
              flush=True)
        return 0
    d = W.draw(args.workload)
    wl = d.wl
    pt = args.partition_tokens or DEFAULT_PARTITION[args.workload]
    log(f"workload {args.workload}: B={d.batch} sum(ctx)={int(d.context_lens.sum())} "
        f"pool={d.num_blocks} blocks")
    cache, plan, q, out, ws, k_new, v_new = build_state(d, pt, log)
    if args.calibration_copy:
        calibration_copy(args.calibration_copy, wl, log)
    stream = torch.cuda.current_stream()
    dec_args = (q, cache.k_pool, cache.v_pool, plan.tables, plan.lens, wl.scale, out, ws,
                plan.max_context_len, pt)

    def step(ev=None):
        """One decode step; with `ev`, each pass is bracketed by its own pair
        of HIP events on the launch stream."""
        def timed(name, fn):
            if ev is None:
                fn()
            else:
                ev[name][0].record(stream)
                fn()
                ev[name][1].record(stream)
        if plan.pairs.shape[0]:
            timed("copy_blocks", lambda: pa.pa_copy_blocks(cache.k_pool, cache.v_pool, plan.pairs))
        timed("reshape_and_cache", lambda: pa.pa_reshape_and_cache(
            k_new, v_new, plan.slots, cache.k_pool, cache.v_pool))
        timed("decode_partition", lambda: pa.pa_decode_partition(*dec_args))
        timed("decode_reduce", lambda: pa.pa_decode_reduce(*dec_args))

    for _ in range(args.warmup):
        step()
    # Timed region: K whole steps back to back, bracketed by synchronisations
    # (HIP events between the kernels would add a pipeline drain to each step).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # The same K steps again with HIP events around every pass on the launch
    # stream: the partition kernel's mean duration for the roofline, and the
    # other passes' durations.
    passes = ["copy_blocks", "reshape_and_cache", "decode_partition", "decode_reduce"]
    events = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for n in passes} for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    passes_us = {}
    for n in passes:
        if n == "copy_blocks" and not plan.pairs.shape[0]:
            passes_us[n] = 0.0
            continue
        passes_us[n] = round(1e3 * float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in events])), 2)
    part_ms = [e["decode_partition"][0].elapsed_time(e["decode_partition"][1]) for e in events]
    part_us = 1e3 * float(np.mean(part_ms))
    log(f"step {ms_per_step * 1e3:.1f} us, partition kernel mean {part_us:.1f} us "
        f"(median {1e3 * float(np.median(part_ms)):.1f}, min {1e3 * float(np.min(part_ms)):.1f}); "
        f"passes {passes_us}")

    ctx = d.context_lens.astype(np.int64)
    eb = wl.elem_bytes
    kv_bytes = int(ctx.sum()) * 2 * wl.num_kv_heads * wl.head_dim * eb
    qo_bytes = 2 * d.batch * wl.num_q_heads * wl.head_dim * eb
    table_bytes = int(np.sum(-(-ctx // wl.block_size))) * 4 + 4 * d.batch
    alg_bytes = kv_bytes + qo_bytes + table_bytes
    achieved = alg_bytes / (part_us * 1e-6) / 1e9
    traffic = measured_traffic(args.workload, pt)
    seq_per_s = d.batch / (ms_per_step * 1e-3)
    kv_gbps_step = kv_bytes / (ms_per_step * 1e-3) / 1e9

    probe = None
    if args.probe_reps > 0:
        probe = measure_read_probe(cache, plan, d, part_us, args.probe_reps, log)
    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(d, out, args.cpu_budget, log)
    prefill = None
    if args.prefill_reps > 0:
        prefill = measure_prefill(args.prefill_reps, log)
    prefix = None
    if args.prefix_reps > 0:
        prefix = measure_prefix_cache(args.prefix_reps, log)
    variants = None
    if args.variant_reps > 0 and args.workload == "8b_gqa":
        variants = measure_variants(cache, plan, q, d, args.variant_reps, log)
    configs = None
    if args.config_reps > 0:
        configs = measure_configs(others, args.config_reps, log)
    swap = None
    if args.swap_reps > 0 and args.workload == "8b_gqa":
        swap = measure_swap(cache, d, args.swap_reps, log)
    # Last (it grows the sequences and patches the step's tables): real
    # steps, planned and run back to back.
    e2e = None
    if args.e2e_steps > 0:
        e2e = measure_e2e(cache, plan, q, out, ws, k_new, v_new, d, pt, args.e2e_steps, log)

    rec = {
        "metric": METRIC,
        "value": round(seq_per_s, 1),
        "unit": "seq/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS[args.workload],
            "global_batch": d.batch,
            "attended_tokens": int(ctx.sum()),
            "partition_tokens": pt,
            "decode_balance": "run-time XCD balance" if args.decode_balance else "even cut",
            "parallelism": "none (1 GPU)",
        },
        "kv_gbps": round(kv_gbps_step, 1),
        "kv_frac_of_hbm_peak": round(kv_gbps_step / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode_partition",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg_bytes,
            "kernel_us": round(part_us, 2),
        },
        "passes_us": passes_us,
        "read_probe": probe,
        "host_step_ms": None if e2e is None else e2e["host_plan_ms_median"],
        "e2e": e2e,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "prefix_cache": prefix,
        "variants": variants,
        "configs": configs,
        "swap": swap,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
