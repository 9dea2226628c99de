"""Pins of the oracle's accept rule and the draft/verify loop (CPU only).

* The pages' worked example (golden fixture with its citation).
* Brute force over every draft / prediction sequence with ids in {0,1,2} and x <= 4, against the
  properties that define the output: the emitted tokens are the drafts up to the first
  disagreement followed by the verifier's token there, every emitted token equals the verifier's
  prediction at its position, and one to x+1 tokens are emitted.
* The pages' guarantee on a tiny random decoder: whatever the drafter proposes, the loop emits
  exactly the full-cache greedy sequence; an uncompressed drafter is accepted in full every round.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept as acc
from oracle import loop

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_worked_example():
    g = json.load(open(GOLDEN))
    ids = g["token_ids"]
    drafts = [ids[t] for t in g["drafts"]]
    printed = [ids[t] for t in g["verified_printed"]]
    x = len(drafts)
    # The verifier's predictions after X are not printed ("..."): the result must not depend on them.
    for tail in itertools.product([0, 5, 6, 7, 23], repeat=x + 1 - len(printed)):
        a, nxt, emitted = acc.accept(drafts, printed + list(tail))
        assert a == g["expected"]["accepted"]
        assert nxt == ids[g["expected"]["next"]]
        assert emitted == [ids[t] for t in g["expected"]["emitted"]]


@pytest.mark.parametrize("x", [1, 2, 3, 4])
def test_brute_force_defining_properties(x):
    for d in itertools.product(range(3), repeat=x):
        for v in itertools.product(range(3), repeat=x + 1):
            a, nxt, em = acc.accept(d, v)
            assert 0 <= a <= x and len(em) == a + 1
            assert list(em[:a]) == list(d[:a])
            assert all(em[i] == v[i] for i in range(a + 1))      # each emitted token is verified
            assert nxt == v[a] and em[-1] == nxt
            if a < x:
                assert d[a] != v[a]
            assert all(d[i] == v[i] for i in range(a))


def test_argmax_lowest_index_on_ties_and_gap():
    Z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [0.0, -1.0, 0.5, 0.25]])
    assert acc.argmax_rows(Z).tolist() == [1, 0, 2]
    assert acc.top2_gap(Z).tolist() == [0.0, 0.0, 0.25]


MODEL = loop.TinyModel(seed=3)
PROMPT = [1, 4, 2, 7, 7, 0, 3]
DRAFTERS = {
    "exact": loop.drafter_exact,
    "quant": loop.drafter_quant,
    "drop": loop.drafter_drop,
    "wrong": loop.drafter_wrong,
    "random": loop.drafter_random,
}


@pytest.fixture(scope="module")
def reference():
    return loop.greedy(MODEL, PROMPT, 24)


@pytest.mark.parametrize("x", [1, 3, 6])
@pytest.mark.parametrize("name", list(DRAFTERS))
def test_loop_emits_full_cache_greedy_output(reference, name, x):
    out, rounds = loop.vericache(MODEL, PROMPT, 24, x, DRAFTERS[name])
    assert out == reference
    assert all(1 <= e <= x + 1 for _, e in rounds)
    if name == "exact":
        assert all(a == x for a, _ in rounds)
    if name == "wrong":
        assert all(a == 0 and e == 1 for a, e in rounds)


def test_lossy_drafters_do_get_rejected_sometimes(reference):
    """The lossy drafters are really lossy here (otherwise the test above would prove little)."""
    _, rq = loop.vericache(MODEL, PROMPT, 24, 6, loop.drafter_quant)
    _, rd = loop.vericache(MODEL, PROMPT, 24, 6, loop.drafter_drop)
    assert any(a < 6 for a, _ in rq + rd)
