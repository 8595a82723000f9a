"""Size pins: the pages' printed KV byte counts against oracle.sizes, and
the pool footprint of every workload."""
import numpy as np
import pytest

import _golden
import workloads as W
from oracle import sizes

G = _golden.load("sizes.json")


def test_per_token_7b():
    c = G["per_token_7b"]
    per = sizes.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"])
    assert per == c["per_token"]
    assert sizes.kv_cache_bytes(c["layers"], c["tokens"], c["kv_heads"], c["head_dim"],
                                c["elem_bytes"], 1) == c["request_bytes"]


def test_per_token_8b_gqa_and_capacity():
    c = G["per_token_8b_gqa"]
    per = sizes.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"])
    assert per == c["per_token"]
    assert per * c["block_size"] == c["per_block"]
    assert per * c["tokens"] == c["request_bytes"]
    assert sizes.blocks_for_tokens(c["tokens"], c["block_size"]) == c["request_blocks"]
    blocks = c["kv_budget_bytes"] // c["per_block"]
    assert blocks == c["budget_blocks"]
    assert blocks * c["block_size"] == c["budget_tokens"]
    assert blocks * c["block_size"] // c["mean_request_tokens"] == c["budget_requests"]


def test_qwen_batch_and_long_context():
    c = G["qwen3_32b_batch"]
    assert sizes.kv_cache_bytes(c["layers"], c["tokens"], c["kv_heads"], c["head_dim"],
                                c["elem_bytes"], c["batch"]) == c["cache_bytes"]
    c = G["long_context_128k"]
    assert sizes.kv_cache_bytes(c["layers"], c["tokens"], c["kv_heads"], c["head_dim"],
                                c["elem_bytes"], 1) == c["cache_bytes"]


def test_prefix_blocks():
    c = G["prefix_1k"]
    n = sizes.blocks_for_tokens(c["tokens"], c["block_size"])
    assert n == c["blocks"]
    per = sizes.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"])
    assert n * c["block_size"] * per == c["bytes"]


def test_reservation_waste():
    c = G["reservation_waste"]
    assert (c["reserved"] - c["used"]) / c["reserved"] == c["waste_fraction"]
    assert c["a_reserved"] - c["a_used"] == c["a_waste"]
    assert c["b_reserved"] - c["b_used"] == c["b_waste"]


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_pool_bytes_match_layout(name):
    d = W.draw(name)
    wl = d.wl
    shape = (d.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    expect = 2 * int(np.prod(shape)) * wl.elem_bytes
    assert sizes.pool_bytes(d.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim,
                            wl.elem_bytes) == expect
    # one layer of KV for the attended tokens is the per-token size times tokens
    per = sizes.kv_bytes_per_token(1, wl.num_kv_heads, wl.head_dim, wl.elem_bytes)
    assert W.kv_bytes(d) == per * int(d.context_lens.sum())


def test_qwen_long_batch_is_one_layer_of_the_page_figure():
    """The 32 x 2048 part of the long-context workload is one layer (of 64)
    of the page's 16 GiB batch."""
    d = W.draw("qwen32b_long")
    per = sizes.kv_bytes_per_token(1, 8, 128, 2)
    assert per * 32 * 2048 * 64 == G["qwen3_32b_batch"]["cache_bytes"]
    assert W.kv_bytes(d) == per * (32 * 2048 + 4 * 32768)
