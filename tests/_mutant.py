"""pytest plugin for the oracle mutation check (``test_oracle_mutations``).

With ``PA_ORACLE_MUTANT`` naming one entry of ``MUTANTS``, it plants that
mistake into the oracle's source before any test module imports the oracle:
the named module's source is edited (the original text must occur exactly
once) and executed again in the module's own namespace, and the ``oracle``
package is reloaded so that its re-exports follow.  The test files listed
with the mutant then run against the planted mistake and must fail.

Each entry: (oracle module, original text, planted text, test files that
must catch it).  Only the CPU oracle is touched; nothing here runs on a GPU.
"""
from __future__ import annotations

import importlib
import inspect
import os
import sys

ATT = ["tests/test_oracle_attention.py"]
PRE = ["tests/test_oracle_prefill.py"]
ALLOC = ["tests/test_oracle_allocator.py"]
PFX = ["tests/test_oracle_prefix_cache.py"]
SWAP = ["tests/test_oracle_swap.py"]
VAR = ["tests/test_oracle_variants.py"]
WIN = ["tests/test_oracle_window_alloc.py"]

MUTANTS = {
    # attention
    "gqa_index": ("oracle.attention", "        g = h // group\n        s = scale * (k[:, g, :] @ q[h])\n        p = np.exp",
                  "        g = h % hkv\n        s = scale * (k[:, g, :] @ q[h])\n        p = np.exp", ATT),
    "missing_transpose": ("oracle.attention", "np.transpose(pool[blk], (1, 0, 2))",
                          "pool[blk].reshape(pool.shape[2], pool.shape[1], pool.shape[3])", ATT),
    "dropped_scale": ("oracle.attention", "        s = scale * (k[:, g, :] @ q[h])\n        p = np.exp",
                      "        s = (k[:, g, :] @ q[h])\n        p = np.exp", ATT),
    "missing_truncation": ("oracle.attention", "return rows[first - j0 * bs:ctx - j0 * bs]",
                           "return rows[first - j0 * bs:]", ATT),
    "merge_weight": ("oracle.attention", 'den = np.einsum("ph,ph->h", w, np.asarray(ls))',
                     'den = np.einsum("ph,ph->h", np.ones_like(w), np.asarray(ls))', ATT),
    "bf16_shift": ("oracle.attention", "<< np.uint32(16)", "<< np.uint32(15)", ATT),
    # prefill
    "causal_limit": ("oracle.attention", "k[lo:pos + 1 - first], v[lo:pos + 1 - first]",
                     "k[lo:pos + 2 - first], v[lo:pos + 2 - first]", PRE),
    "position_offset": ("oracle.attention", "            pos = ctx - n + j\n",
                        "            pos = ctx - n + j - 1\n", PRE),
    "negative_guard": ("oracle.attention", "            if pos < 0:\n                continue\n            lo",
                       "            lo", PRE),
    # prefill, matrix form
    "rows_causal_limit": ("oracle.attention", "allowed = (keys[None, :] <= pos[:, None])",
                          "allowed = (keys[None, :] < pos[:, None])", PRE),
    "rows_window_limit": ("oracle.attention", "& (keys[None, :] >= lo[:, None])",
                          "& (keys[None, :] > lo[:, None])", PRE + VAR),
    "rows_gqa_index": ("oracle.attention", "            g = h // group\n            s = scale * (q[:, h, :]",
                       "            g = h % hkv\n            s = scale * (q[:, h, :]", PRE),
    "rows_norm": ("oracle.attention", "np.where(live, p.sum(axis=1), 1.0)",
                  "np.where(live, p.sum(axis=1) + 1e-9, 1.0)", PRE),
    # allocator
    "cow_no_decrement": ("oracle.allocator",
                         "            self.refcount[src] -= 1\n            if self.refcount[src] == 0:",
                         "            if self.refcount[src] == 0:", ALLOC),
    "lifo_pool": ("oracle.allocator", "return self.free.popleft()", "return self.free.pop()", ALLOC),
    "cow_disabled": ("oracle.allocator", "needs_cow = start % bs != 0 and (",
                     "needs_cow = False and (", ALLOC),
    "share_floor": ("oracle.allocator",
                    "k = _ceil_div(n_tokens, self.block_size)\n        if NO_BLOCK in table[:k]:",
                    "k = n_tokens // self.block_size\n        if NO_BLOCK in table[:k]:", ALLOC),
    "slot_off_by_one": ("oracle.allocator", "slots.append(table[pos // bs] * bs + pos % bs)",
                        "slots.append(table[pos // bs] * bs + (pos + 1) % bs)", ALLOC),
    # cache write, sizes
    "write_offset": ("oracle.kvcache", "pool[s // bs, :, s % bs, :] = new[t]",
                     "pool[s // bs, :, (s + 1) % bs, :] = new[t]", ALLOC + ATT),
    "size_no_2x": ("oracle.sizes", "return 2 * layers * kv_heads * head_dim * elem_bytes",
                   "return layers * kv_heads * head_dim * elem_bytes",
                   ["tests/test_oracle_sizes.py"]),
    # prefix cache
    "lru_release_order": ("oracle.allocator", "for b in reversed(released):",
                          "for b in released:", PFX),
    "evict_most_recent": ("oracle.allocator", "blk, _ = self.lru.popitem(last=False)",
                          "blk, _ = self.lru.popitem(last=True)", PFX),
    "batch_no_hold": ("oracle.allocator",
                      "                if held is None:\n                    self.lru[src] = None\n"
                      "                else:\n                    held.append(src)",
                      "                self.lru[src] = None", PFX),
    # swapping
    "swap_shared_blocks": ("oracle.allocator",
                           "if b != NO_BLOCK and self.refcount[b] == 1]",
                           "if b != NO_BLOCK and self.refcount[b] >= 1]", SWAP),
    "swap_in_reversed": ("oracle.allocator", "pairs.append((entries[j][1], d))",
                         "pairs.append((d, entries[j][1]))", SWAP),
    # variants: window and 8-bit pools
    "window_off_by_one": ("oracle.attention",
                          "return max(0, pos - window + 1) if window > 0 else 0",
                          "return max(0, pos - window) if window > 0 else 0", VAR),
    "trim_partial_block": ("oracle.allocator",
                           "dead = max(self.lens[seq] - window, 0) // bs",
                           "dead = -(-max(self.lens[seq] - window, 0) // bs)", WIN),
    "fp8_ties_to_odd": ("oracle.fp8", "((d_hi == d_lo) & (hi % 2 == 0))",
                        "((d_hi == d_lo) & (hi % 2 == 1))", VAR),
    "fp8_subnormal_exponent": ("oracle.fp8", "out[code] = s * (m / 8.0) * 2.0 ** -6",
                               "out[code] = s * (m / 8.0) * 2.0 ** -7", VAR),
}


def plant(name: str) -> None:
    mod_name, old, new, _ = MUTANTS[name]
    mod = importlib.import_module(mod_name)
    src = inspect.getsource(mod)
    if src.count(old) != 1:
        raise RuntimeError(f"mutant {name}: the original text occurs {src.count(old)} times")
    exec(compile(src.replace(old, new), mod.__file__, "exec"), mod.__dict__)
    importlib.reload(sys.modules["oracle"])


def pytest_configure(config):
    name = os.environ.get("PA_ORACLE_MUTANT")
    if name:
        plant(name)
