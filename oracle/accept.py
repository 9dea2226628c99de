"""Greedy accept of one verification round (CPU oracle).

The rule ("VeriCache: making lossy KV compression exact", The Core Idea, the accept step, its
Figure 1, the worked example and the round's code listing): compare the x drafted tokens with
the verifier's predictions from left to right; keep the matching prefix; at the first mismatch
emit the verifier's token there and drop the rest; if every draft matches, emit all drafts plus
the verifier's extra (x+1-th) prediction. The verifier's predictions are greedy, i.e. the argmax
of each row of logits (the guarantee is stated for greedy decoding; Final Takeaways).

Reading where the pages are silent: argmax ties go to the lowest token id; logits are finite.
"""
from __future__ import annotations

import numpy as np


def argmax_rows(Z: np.ndarray) -> np.ndarray:
    """Per-row argmax, lowest index on ties (np.argmax returns the first maximum)."""
    Z = np.asarray(Z)
    assert np.all(np.isfinite(Z)), "logits must be finite"
    return np.argmax(Z, axis=-1).astype(np.int64)


def top2_gap(Z: np.ndarray) -> np.ndarray:
    """Per-row gap between the largest and second-largest logit (0 on an exact tie)."""
    Z = np.asarray(Z, np.float64)
    part = -np.partition(-Z, 1, axis=-1)
    return part[..., 0] - part[..., 1]


def accept(drafts, verified):
    """drafts: x ids; verified: x+1 greedy predictions of the same positions plus one.

    Returns (a, next, emitted): a = number of accepted drafts (the first position where draft and
    verifier disagree, or x when they never do), next = verified[a] (the correction at the first
    disagreement, or the bonus prediction when all x drafts stand), emitted = drafts[:a] + [next].
    """
    d = np.asarray(drafts, np.int64).reshape(-1)
    v = np.asarray(verified, np.int64).reshape(-1)
    x = d.size
    assert v.size == x + 1
    disagree = np.flatnonzero(d != v[:x])
    a = int(disagree[0]) if disagree.size else x
    nxt = int(v[a])
    return a, nxt, [int(t) for t in d[:a]] + [nxt]
