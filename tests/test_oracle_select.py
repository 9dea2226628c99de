"""Pins of the oracle's keep-list selection (CPU only).

* Rank definition by brute force: a middle position p is kept iff fewer than `take` middle
  positions outrank it (q outranks p when its score is larger, or equal with q < p; NaN is outranked
  by every number), counted by pairwise comparison with no sorting.
* Invariants: ascending, unique, in range, the count formula, sinks and recent always kept, every
  kept middle score >= every dropped one.
* Special cases: keep >= n keeps everything; keep <= sinks + recent keeps only those; all-equal
  scores keep the lowest middle positions; n smaller than sinks; +-0 tie; +-inf; NaN last.
"""
import numpy as np
import pytest

from oracle import select as sel


def _brute(s, n, sinks, recent, keep):
    lo = min(sinks, n)
    hi = max(lo, n - recent)
    fixed = lo + (n - hi)
    take = max(0, keep - fixed)
    kept = list(range(lo)) + list(range(hi, n))
    for p in range(lo, hi):
        beats = 0
        for q in range(lo, hi):
            if q == p:
                continue
            sp, sq = float(s[p]), float(s[q])
            if np.isnan(sq):
                continue  # a NaN outranks nobody
            if np.isnan(sp) or sq > sp or (sq == sp and q < p):
                beats += 1
        if beats < take:
            kept.append(p)
    return sorted(kept)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 40))
    sinks, recent = int(g.integers(0, 6)), int(g.integers(0, 6))
    keep = int(g.integers(0, n + 3))
    kind = seed % 4
    if kind == 0:
        s = g.standard_normal(n).astype(np.float32)
    elif kind == 1:  # heavy ties
        s = g.integers(-2, 3, n).astype(np.float32)
    elif kind == 2:  # specials
        s = g.choice(np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan], np.float32), n)
    else:
        s = (g.standard_normal(n) * 1e-38).astype(np.float32)  # subnormals and zeros
    got = sel.keep_positions(s, n, sinks, recent, keep).tolist()
    assert got == _brute(s, n, sinks, recent, keep)
    assert len(got) == sel.keep_count(n, sinks, recent, keep)


def test_invariants_large():
    g = np.random.default_rng(7)
    n, sinks, recent, keep = 20000, 64, 256, 5000
    s = g.standard_normal(n).astype(np.float32)
    k = sel.keep_positions(s, n, sinks, recent, keep)
    assert k.size == keep and np.all(np.diff(k) > 0) and k[0] == 0 and k[-1] == n - 1
    assert set(range(64)) <= set(k.tolist()) and set(range(n - 256, n)) <= set(k.tolist())
    mid = np.zeros(n, bool)
    mid[64:n - 256] = True
    kept = np.zeros(n, bool)
    kept[k] = True
    assert s[mid & kept].min() >= s[mid & ~kept].max()


def test_special_cases():
    s = np.arange(10, dtype=np.float32)
    assert sel.keep_positions(s, 10, 2, 2, 100).tolist() == list(range(10))
    assert sel.keep_positions(s, 10, 2, 2, 3).tolist() == [0, 1, 8, 9]
    assert sel.keep_positions(np.ones(10, np.float32), 10, 2, 2, 6).tolist() == [0, 1, 2, 3, 8, 9]
    assert sel.keep_positions(s[:3], 3, 5, 5, 1).tolist() == [0, 1, 2]
    z = np.array([0.0, -0.0, 0.0, -0.0], np.float32)
    assert sel.keep_positions(z, 4, 0, 0, 2).tolist() == [0, 1]
    sp = np.array([np.nan, -np.inf, 1.0, np.inf, np.nan], np.float32)
    assert sel.keep_positions(sp, 5, 0, 0, 3).tolist() == [1, 2, 3]
    assert sel.keep_positions(sp, 5, 0, 0, 4).tolist() == [0, 1, 2, 3]
    assert sel.keep_count(100000, 64, 256, 25000) == 25000
