"""The decode stream split's run-time balance on the GPU, through the C ABI.

The stream split cuts the flat tile order into one chunk per XCD; with
balancing on, each partition pass records per chunk its tiles, and per wave
its time, in the workspace's balance header, and the next reduce pass moves
the cut towards the chunks' measured rates.  Checked against the oracle
(max-abs error <= 2e-2, 16-bit inputs): decode under hand-set skewed cuts
(shares 1/16 .. 3/16, the extremes the header allows) and after several
adapting calls, including the full 8B batch; the header after each call is
a valid cut (magic, cum[0] = 0, cum[8] = 2^16, shares in range) with the
record marked used; an unrecognised header means the even cut; with balancing
off the cut is even whatever the header says (bit-identical outputs).
"""
import numpy as np
import pytest

import workloads as W
from _scenario import KV, TOL, max_abs_err, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU suite deselects these; never a fallback
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="needs a GPU")]

import paged_kv_cache_107_amd as pa  # noqa: E402

MAGIC, ONE = 0x6C614257, 1 << 16
# header words: magic, stamped, 2 pad, cum[12], tiles[8], then per-wave times
CUM, TILES = 4, 16


def header(ws):
    return ws[:256].view(torch.int32).cpu().numpy().view(np.uint32)


def set_cut(ws, shares):
    cum = np.concatenate([[0], np.cumsum(shares)]).astype(np.uint32)
    assert cum[-1] == ONE
    h = np.zeros(64, dtype=np.uint32)
    h[0] = MAGIC
    h[CUM:CUM + 9] = cum
    ws[:256].copy_(torch.from_numpy(h.view(np.uint8)).cuda())


def check_header(h):
    assert h[0] == MAGIC
    cum = h[CUM:CUM + 9].astype(np.int64)
    d = np.diff(cum)
    assert cum[0] == 0 and cum[8] == ONE
    assert (d >= ONE // 16).all() and (d <= 3 * ONE // 16).all(), d
    assert h[1] == 0                                   # the record was used
    return d


@pytest.fixture(scope="module")
def case():
    d = W.draw("8b_gqa", batch=128)     # > 80 tiles per wave: the balanced size
    kv = KV(d)
    o = run_oracle(d, kv)
    g = run_gpu(d, kv)
    return d, o, g


@pytest.fixture
def balance():
    prev = pa.pa_set_decode_balance(True)
    yield
    pa.pa_set_decode_balance(prev)


def run(d, g, ws):
    out = torch.full_like(g["q"], float("nan"))
    plan, cache = g["plan"], g["cache"]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.pa_decode(g["q"], cache.k_pool, cache.v_pool, plan.tables, plan.lens, d.wl.scale, out,
                 ws, plan.max_context_len, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return out


SKEWS = {
    "low_high": [ONE // 16] * 4 + [3 * ONE // 16] * 4,
    "alternate": [ONE // 16, 3 * ONE // 16] * 4,
    "one_light": [ONE // 16] + [8777] * 6 + [ONE - ONE // 16 - 6 * 8777],
    "ragged": [5000, 9000, 12000, 4200, 11000, 7336, 8000, 9000],
}


@pytest.mark.usefixtures("balance")
@pytest.mark.parametrize("skew", sorted(SKEWS))
def test_skewed_cuts_match_the_oracle(case, skew):
    d, o, g = case
    ws = g["cache"].workspace(d.batch, d.wl.num_q_heads, g["plan"].max_context_len)
    set_cut(ws, np.array(SKEWS[skew], dtype=np.int64))
    out = run(d, g, ws)
    err = max_abs_err(out, o["out"])
    print(f"cut {skew}: max_abs_err={err:.3e}, next shares {check_header(header(ws)).tolist()}",
          flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.usefixtures("balance")
def test_adapting_calls_stay_correct(case):
    d, o, g = case
    ws = g["cache"].workspace(d.batch, d.wl.num_q_heads, g["plan"].max_context_len)
    ws[:256].fill_(0x55)                               # not a header: the even cut first
    for k in range(6):
        out = run(d, g, ws)
        err = max_abs_err(out, o["out"])
        shares = check_header(header(ws))
        print(f"call {k}: max_abs_err={err:.3e} shares={shares.tolist()}", flush=True)
        assert err <= TOL["bf16"]
        if k == 0:
            assert shares.tolist() == [ONE // 8] * 8   # initialised, nothing measured yet


def test_balance_off_uses_the_even_cut(case, even_cut):
    d, o, g = case
    ws = g["cache"].workspace(d.batch, d.wl.num_q_heads, g["plan"].max_context_len)
    ws[:256].fill_(0x55)
    even = run(d, g, ws)
    set_cut(ws, np.array(SKEWS["low_high"], dtype=np.int64))
    skewed_header = run(d, g, ws)
    assert torch.equal(even.view(torch.int16), skewed_header.view(torch.int16))
    assert max_abs_err(even, o["out"]) <= TOL["bf16"]


@pytest.mark.usefixtures("balance")
def test_full_batch_after_adapting():
    """The 8B batch at full size (256 sequences), every row, after five
    adapting calls on one workspace (the benchmark's setting)."""
    d = W.draw("8b_gqa")
    kv = KV(d)
    o = run_oracle(d, kv)
    g = run_gpu(d, kv)
    ws = g["ws"]
    for _ in range(5):
        out = run(d, g, ws)
    shares = check_header(header(ws))
    err = max_abs_err(out, o["out"])
    print(f"8b_gqa full: shares={shares.tolist()} max_abs_err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
