"""Keep-list selection of the token-dropping drafter (CPU oracle).

Token-dropping compressors keep only part of the cached positions: some always keep the attention
sinks (the first tokens) and the most recent tokens, others score the cached entries and evict the
least useful ones ("VeriCache: making lossy KV compression exact", The Tradeoff VeriCache Is Trying
to Escape). VeriCache drives any such compressor through one interface that exposes only which
positions are dropped ("VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key
Contributions), and assumes the same number of dropped tokens in every (layer, head) (same page,
Limitations).

Readings where the pages are silent (the pages give no scoring rule, no counts and no tie rule):
* the kept set of one (batch row, kv head) over positions 0..n-1 is the first `sinks` positions,
  the last `recent` positions, and the `take` highest-scoring positions of the middle
  [lo, hi) = [min(sinks, n), max(lo, n - recent)), take = max(0, keep - fixed), capped at the
  middle's size; the list is ascending;
* scores are float32; equal scores prefer the lower position; -0.0 equals +0.0; a NaN score ranks
  below every number (NaNs among themselves by position).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def bounds(n: int, sinks: int, recent: int, keep: int):
    """(lo, hi, take): the middle [lo, hi) and how many of its positions are selected by score."""
    lo = min(max(sinks, 0), n)
    hi = max(lo, n - max(recent, 0))
    fixed = lo + (n - hi)
    take = min(max(0, keep - fixed), hi - lo)
    return lo, hi, take


def keep_count(n: int, sinks: int, recent: int, keep: int) -> int:
    lo, hi, take = bounds(n, sinks, recent, keep)
    return lo + (n - hi) + take


def keep_positions(scores, n: int, sinks: int, recent: int, keep: int) -> np.ndarray:
    """Ascending kept positions (int64) of one row of `n` float32 scores.

    Rank order of the middle: NaN last; otherwise by descending score, equal scores by ascending
    position (a stable sort on the key (is NaN, -score, position)).
    """
    s = np.asarray(scores, np.float32).reshape(-1)[:n]
    assert s.size == n
    lo, hi, take = bounds(n, sinks, recent, keep)
    mid = s[lo:hi].astype(np.float64)
    isnan = np.isnan(mid)
    neg = np.where(isnan, 0.0, -mid)  # -0.0 and +0.0 compare equal in the sort
    order = np.lexsort((np.arange(mid.size), neg, isnan))  # last key is primary
    chosen = lo + np.sort(order[:take])
    return np.concatenate([np.arange(0, lo), chosen, np.arange(hi, n)]).astype(np.int64)
