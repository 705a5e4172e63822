"""A host model of the single-launch merge protocol (PA_FLAG_SINGLE_LAUNCH), run on the
CPU before any GPU use: the even split of units over workgroups, the bands that cross
workgroup boundaries, and the arrival counters, simulated under random completion orders.

The protocol, as the decode kernel runs it at the end of each workgroup x:
  * x holds a piece of up to two crossing bands: the band holding its first unit if that
    band started in an earlier workgroup o (a 'covering' band, piece on side 0), and the
    band holding its last unit if that band starts in x and goes on (x owns it; piece on
    the side the records give).  A band owned by o has participants o .. o + n - 1.
  * Participants are grouped by 16 from the owner: group g = (x - o) // 16, leader
    L = o + 16 g.  Each participant increments its group's counter (the leader's
    group-counter slot: 2 L + 1 when L is the owner, else 2 L); the one that sees
    group size - 1 is the group's merger.  It folds the group's pieces into the
    leader's piece slot (or, for a band of one group, into the output) and resets the
    counter.
  * With more than one group, each group merger then increments the band counter
    (slot o); the one that sees groups - 1 folds the group triples into the output and
    resets it.
Checked here, for the five workloads and random shapes: every band is finished exactly
once; every fold reads only slots that a participant of that band (or a group merger)
wrote, after they wrote them; no two bands or groups share a counter in one call; every
counter ends at zero.  The model is test-side bookkeeping, not the oracle.
"""
import math
import random

import numpy as np
import pytest

GROUP = 16


def split_of(ctx, query_heads, kv_heads, n_wg):
    """Units, bands and the even split, as the plan and the decode kernel compute them."""
    group = query_heads // kv_heads
    hp = max(h for h in range(1, 9) if group % h == 0)
    streams = kv_heads * (group // hp)
    spw = math.gcd(streams, 12)
    if len(ctx) * (streams // spw) < 32 and spw % 2 == 0:
        spw //= 2
    bands = streams // spw
    tiles = [(c + 15) // 16 for c in ctx]
    pref = [0]
    for t in tiles:
        pref.append(pref[-1] + t)
    N = bands * pref[-1]

    def split_point(x):
        return x * N // n_wg

    def wg_of(u):
        return min(((u + 1) * n_wg - 1) // N, n_wg - 1)

    def locate(u):
        b = next(i for i in range(len(ctx)) if bands * pref[i + 1] > u)
        Tb = pref[b + 1] - pref[b]
        off = u - bands * pref[b]
        return b, off // Tb, Tb

    records = []
    for x in range(n_wg):
        g0, g1 = split_point(x), split_point(x + 1)
        own = cov = None
        if g1 > g0:
            b, band, Tb = locate(g1 - 1)
            S0 = bands * pref[b] + band * Tb
            if S0 + Tb > g1 and S0 >= g0:
                own = dict(owner=x, n=wg_of(S0 + Tb - 1) - x + 1, side=0 if S0 == g0 else 1, key=(b, band))
        if g0 < N:
            b, band, Tb = locate(g0)
            S0 = bands * pref[b] + band * Tb
            if S0 < g0:
                o = wg_of(S0)
                cov = dict(owner=o, n=wg_of(S0 + Tb - 1) - o + 1,
                           side=0 if S0 == split_point(o) else 1, key=(b, band))
        records.append((own, cov))
    return records


def simulate(records, n_wg, rng):
    """Run the protocol over one random completion order; return the events seen."""
    band_cnt = [0] * n_wg
    grp_cnt = [0] * (2 * n_wg)
    written = {}            # (slot x, side) -> (band key, what)
    finished = []
    order = list(range(n_wg))
    rng.shuffle(order)
    # the pieces a workgroup writes before arriving
    for x in order:
        own, cov = records[x]
        if cov is not None:
            written[(x, 0)] = (cov["key"], "piece")
        if own is not None:
            written[(x, own["side"])] = (own["key"], "piece")
        for rec in (cov, own):
            if rec is None:
                continue
            o, n = rec["owner"], rec["n"]
            assert o <= x < o + n, (x, rec)
            g = (x - o) // GROUP
            L = o + GROUP * g
            sg = min(GROUP, n - GROUP * g)
            ng = (n + GROUP - 1) // GROUP
            gslot = 2 * L + (1 if L == o else 0)
            old = grp_cnt[gslot]
            grp_cnt[gslot] += 1
            if old != sg - 1:
                continue
            # group merger: every participant of the group has written its piece
            for p in range(sg):
                xp = L + p
                side = rec["side"] if xp == o else 0
                assert written.get((xp, side), (None,))[0] == rec["key"], ("unwritten piece", xp, rec)
            grp_cnt[gslot] = 0
            if ng == 1:
                finished.append(rec["key"])
                continue
            lead_side = rec["side"] if L == o else 0
            written[(L, lead_side)] = (rec["key"], "group")
            old = band_cnt[o]
            band_cnt[o] += 1
            if old != ng - 1:
                continue
            for gg in range(ng):
                Lg = o + GROUP * gg
                side = rec["side"] if Lg == o else 0
                assert written.get((Lg, side)) == (rec["key"], "group"), ("unmerged group", Lg, rec)
            band_cnt[o] = 0
            finished.append(rec["key"])
    assert not any(band_cnt) and not any(grp_cnt), "a counter was left non-zero"
    return finished


def crossing_bands(records):
    keys = set()
    for own, cov in records:
        for r in (own, cov):
            if r is not None:
                keys.add(r["key"])
    return keys


def check(ctx, qh, kvh, n_wg=256, orders=4, seed=0):
    records = split_of(list(ctx), qh, kvh, n_wg)
    # every participant of a band agrees on owner, count and side
    seen = {}
    for own, cov in records:
        for r in (own, cov):
            if r is not None:
                t = (r["owner"], r["n"], r["side"])
                assert seen.setdefault(r["key"], t) == t, r
    # a workgroup owns at most one band and covers at most one, never the same one
    for x, (own, cov) in enumerate(records):
        if own is not None and cov is not None:
            assert own["key"] != cov["key"]
    rng = random.Random(seed)
    want = crossing_bands(records)
    for _ in range(orders):
        done = simulate(records, n_wg, rng)
        assert sorted(done) == sorted(want), "a band finished twice or never"
    return max((r["n"] for own, cov in records for r in (own, cov) if r), default=0)


WORKLOAD_SHAPES = {
    "tiny": ([37, 100], 8, 2),
    "small_batch": (list(np.random.Generator(np.random.PCG64(1002)).integers(1, 4097, size=8)), 32, 8),
    "long100k": ([100000], 24, 4),
    "batch64": (list(np.random.Generator(np.random.PCG64(1003)).integers(512, 2049, size=64)), 32, 8),
}


@pytest.mark.parametrize("name", list(WORKLOAD_SHAPES))
def test_protocol_on_workload_shapes(name):
    ctx, qh, kvh = WORKLOAD_SHAPES[name]
    span = check(ctx, qh, kvh)
    print(name, "largest band span", span)


def test_protocol_on_random_shapes():
    rng = np.random.default_rng(77)
    for i in range(40):
        B = int(rng.integers(1, 40))
        kvh = int(rng.choice([1, 2, 4, 8]))
        qh = kvh * int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        kind = i % 4
        if kind == 0:
            ctx = rng.integers(0, 5000, size=B)
        elif kind == 1:
            ctx = np.clip(np.rint(np.exp(rng.normal(6.5, 1.5, size=B))), 0, 60000)
        elif kind == 2:
            ctx = rng.integers(1, 40, size=B)
            ctx[0] = int(rng.integers(20000, 120000))
        else:
            ctx = rng.integers(0, 3, size=B)
        if int(np.sum(ctx)) == 0:
            ctx[0] = 1
        n_wg = int(rng.choice([80, 128, 256, 304]))
        check(ctx.astype(int).tolist(), qh, kvh, n_wg=n_wg, orders=2, seed=i)


def test_long_bands_use_two_levels():
    """The long-context shape has bands of 128 pieces: 8 groups and a band merge."""
    records = split_of([100000], 24, 4, 256)
    spans = {r["n"] for own, cov in records for r in (own, cov) if r}
    assert max(spans) > GROUP
