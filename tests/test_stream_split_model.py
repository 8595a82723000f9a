"""Model check of the stream split's arithmetic (CPU only).

The decode kernel's stream split cuts a flat order of T tiles into one
chunk per XCD (the device's count, at most 8: equal chunks, or, with 8,
chunks sized by the balance state's cut) and
each chunk evenly over its waves; a (kv head, sequence) pair cut between
waves leaves one partial per wave in workspace slot (pair index + wave
rank), merged by the pair's first wave's rank.  This file restates that
integer arithmetic in Python and checks, over random sizes and cuts, the
properties the kernels rely on:

* runs tile the order: lo(0) = 0, lo(N) = T, non-decreasing;
* rank_of(t) is the rank whose run holds t;
* dense() holds exactly when every run is non-empty;
* slots never collide: the slots of different pairs are disjoint;
* a weighted cut at the sizes where weights apply (80 tiles per wave) is
  always dense, so the reduce pass never needs the cut;
* the balance update keeps every share within [1/16, 3/16] and the cut
  summing to 2^16, moves shares towards the measured rates, and leaves the
  cut alone when the chunks end within 1/64 of each other.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

K_WAVES, K_XCDS, ONE = 4, 8, 1 << 16
SHARE_MIN, SHARE_MAX = ONE // 16, 3 * ONE // 16


class Split:
    def __init__(self, T, nwg, cut=None, xcds=K_XCDS):
        self.T, self.nwg, self.cut, self.xcds = T, nwg, cut, xcds

    def chunks(self):
        return min(self.xcds, K_XCDS, self.nwg)

    def wgs_of(self, x):
        c = self.chunks()
        return self.nwg // c + (1 if x < self.nwg % c else 0)

    def base(self, x):
        c = self.chunks()
        return K_WAVES * (x * (self.nwg // c) + min(x, self.nwg % c))

    def chunk_lo(self, x):
        return self.cut[x] if self.cut is not None else self.T * x // self.chunks()

    def lo(self, r):
        if r >= K_WAVES * self.nwg:
            return self.T
        x = 0
        while x + 1 < self.chunks() and self.base(x + 1) <= r:
            x += 1
        c0 = self.chunk_lo(x)
        return c0 + (self.chunk_lo(x + 1) - c0) * (r - self.base(x)) // (K_WAVES * self.wgs_of(x))

    def dense(self):
        c = self.chunks()
        if self.cut is None:
            return self.T // c >= K_WAVES * ((self.nwg + c - 1) // c)
        return all(self.chunk_lo(x + 1) - self.chunk_lo(x) >= K_WAVES * self.wgs_of(x)
                   for x in range(c))

    def rank_of(self, t):
        c = self.chunks()
        if self.cut is not None:
            x = 0
            while x + 1 < c and self.chunk_lo(x + 1) <= t:
                x += 1
        else:
            x = ((t + 1) * c - 1) // self.T
        c0 = self.chunk_lo(x)
        tx = self.chunk_lo(x + 1) - c0
        return self.base(x) + ((t - c0 + 1) * (K_WAVES * self.wgs_of(x)) - 1) // tx


def cut_of(T, shares):
    cum = np.concatenate([[0], np.cumsum(shares)])
    return [int((T * int(c)) >> 16) for c in cum]


def random_shares(rng):
    """Integer shares in [1/16, 3/16] summing to 2^16."""
    while True:
        s = rng.integers(SHARE_MIN, SHARE_MAX + 1, K_XCDS - 1)
        last = ONE - int(s.sum())
        if SHARE_MIN <= last <= SHARE_MAX:
            return np.concatenate([s, [last]])


def check_split(sp, pair_tiles):
    n = K_WAVES * sp.nwg
    los = [sp.lo(r) for r in range(n + 1)]
    assert los[0] == 0 and los[-1] == sp.T
    assert all(a <= b for a, b in zip(los, los[1:]))
    assert sp.dense() == all(a < b for a, b in zip(los, los[1:]))
    owner = np.repeat(np.arange(n), np.diff(los))        # rank of every tile
    for t in range(0, sp.T, max(1, sp.T // 97)):
        assert sp.rank_of(t) == owner[t]
    assert sp.rank_of(sp.T - 1) == owner[-1]
    # pairs in flat order; slot = pair + rank for every rank whose run
    # touches the pair
    used = set()
    start = 0
    for p, nt in enumerate(pair_tiles):
        if nt == 0:
            continue
        ranks = set(owner[start:start + nt].tolist())
        slots = {p + r for r in ranks}
        assert not (slots & used)
        used |= slots
        start += nt


@settings(max_examples=150, deadline=None)
@given(nwg=st.integers(1, 64), seed=st.integers(0, 2**31), weighted=st.booleans(),
       pairs=st.integers(1, 300), xcds=st.integers(1, K_XCDS))
def test_runs_ranks_and_slots(nwg, seed, weighted, pairs, xcds):
    rng = np.random.default_rng(seed)
    pair_tiles = rng.integers(0, 40, pairs)
    T = int(pair_tiles.sum())
    if T == 0:
        return
    # weights only with all eight dies
    cut = cut_of(T, random_shares(rng)) if weighted and nwg >= K_XCDS and xcds == K_XCDS else None
    check_split(Split(T, nwg, cut, xcds), pair_tiles)


@settings(max_examples=100, deadline=None)
@given(nwg=st.integers(8, 256), extra=st.integers(0, 10**6), seed=st.integers(0, 2**31))
def test_weighted_cut_is_dense_where_weights_apply(nwg, extra, seed):
    rng = np.random.default_rng(seed)
    T = 80 * K_WAVES * nwg + extra                      # balanced_size()
    for shares in (random_shares(rng), np.array([SHARE_MIN] * 4 + [SHARE_MAX] * 4)):
        assert Split(T, nwg, cut_of(T, shares)).dense()


def update(cum, tiles, dur):
    """The reduce pass's balance update (same arithmetic, float32 steps
    approximated in float64): shares halfway to the measured rates, clamped
    to [0.0675, 0.1825] over 4 rounds of renormalisation, then rounded."""
    rate = np.asarray(tiles, float) / np.asarray(dur, float)
    if max(dur) - min(dur) <= max(dur) // 64:     # balanced: the cut stays
        return list(cum)
    cur = np.diff(cum) / ONE
    sh = 0.5 * cur + 0.5 * rate / rate.sum()
    for _ in range(4):
        sh = np.clip(sh / sh.sum(), 0.0675, 0.1825)
    run = np.cumsum(sh) / sh.sum()
    nxt = [0] + [int(np.rint(r * ONE)) for r in run[:-1]] + [ONE]
    d = np.diff(nxt)
    if (d >= SHARE_MIN).all() and (d <= SHARE_MAX).all():
        return nxt
    return list(cum)


@settings(max_examples=200, deadline=None)
@given(seed=st.integers(0, 2**31))
def test_balance_update_stays_valid_and_moves_towards_rates(seed):
    rng = np.random.default_rng(seed)
    cum = [0] + np.cumsum(random_shares(rng)).tolist()
    speed = rng.uniform(0.5, 2.0, K_XCDS)                 # tiles per tick of each die
    for _ in range(12):
        tiles = np.diff(cum) * 1000
        dur = np.maximum(1, np.rint(tiles / speed))
        new = update(cum, tiles, dur)
        d = np.diff(new)
        assert new[0] == 0 and new[-1] == ONE
        assert (d >= SHARE_MIN).all() and (d <= SHARE_MAX).all()
        cum = new
    # shares end near the speeds' proportions where those are inside the clamp
    want = speed / speed.sum()
    got = np.diff(cum) / ONE
    inside = (want > 0.07) & (want < 0.18)
    assert np.all(np.abs(got - want)[inside] < 0.02) or not inside.all()


def test_equal_rates_keep_the_even_cut():
    cum = [ONE // 8 * x for x in range(9)]
    assert update(cum, [1000] * 8, [500] * 8) == cum
