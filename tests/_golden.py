"""Runs the worked allocator examples of ``golden/allocator_examples.json``
against any allocator exposing the small adapter interface below, so the
oracle allocator and the native one are held to the same printed values."""
from __future__ import annotations

import json
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def full_free_order(example) -> list:
    nb = example["num_blocks"]
    if "initial_free_order" in example:
        return list(example["initial_free_order"])
    head = list(example["initial_free_order_head"])
    return head + [b for b in range(nb) if b not in head]


def run_example(example, make_adapter):
    """make_adapter(num_blocks, block_size, free_order) -> adapter with
    create(), append(seq, n) -> (slots, pair|None), fork(seq), share(seq, n),
    free(seq), table(seq) -> list, refcount(block) -> int, free_list() -> list."""
    a = make_adapter(example["num_blocks"], example["block_size"], full_free_order(example))
    names = {}
    for step in example["steps"]:
        op = step["op"]
        if op == "create":
            names[step["as"]] = a.create()
        elif op == "append":
            slots, pair = a.append(names[step["seq"]], step["n"])
            if "expect_slots" in step:
                assert list(slots) == step["expect_slots"], (step, slots)
            if "expect_pair" in step:
                exp = step["expect_pair"]
                assert (None if pair is None else list(pair)) == exp, (step, pair)
            for pos, slot in step.get("expect_slot_at", {}).items():
                assert slots[int(pos)] == slot, (step, pos, slots[int(pos)])
        elif op == "fork":
            names[step["as"]] = a.fork(names[step["parent"]])
        elif op == "share":
            names[step["as"]] = a.share(names[step["src"]], step["n"])
        elif op == "free":
            a.free(names[step["seq"]])
        else:  # pragma: no cover
            raise ValueError(op)
        seq = names.get(step.get("seq", step.get("as")))
        if "expect_table" in step:
            assert a.table(seq) == step["expect_table"], (step, a.table(seq))
        if "expect_table_len" in step:
            assert len(a.table(seq)) == step["expect_table_len"]
        if "expect_table_head" in step:
            h = step["expect_table_head"]
            assert a.table(seq)[:len(h)] == h
        for nm, tbl in step.get("expect_tables", {}).items():
            assert a.table(names[nm]) == tbl, (step, nm, a.table(names[nm]))
        for nm, n in step.get("expect_table_len_of", {}).items():
            assert len(a.table(names[nm])) == n
        for nm, k in step.get("expect_shared_entries", {}).items():
            src = names[step["src"]]
            assert a.table(names[nm])[:k] == a.table(src)[:k]
        for blk, rc in step.get("expect_refcounts", {}).items():
            assert a.refcount(int(blk)) == rc, (step, blk, a.refcount(int(blk)))
        if "expect_refcount_first_k" in step:
            e = step["expect_refcount_first_k"]
            for b in a.table(names[e["seq"]])[:e["k"]]:
                assert a.refcount(b) == e["value"], (step, b)
        if "free_contains" in step:
            fl = set(a.free_list())
            for b in step["free_contains"]:
                assert b in fl, (step, b)
        if "expect_num_free" in step:
            assert len(a.free_list()) == step["expect_num_free"]
    return a, names
