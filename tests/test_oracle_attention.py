"""Pins of the oracle's attention, verify, merge, drafter key sets and keep lists (CPU only).

Pinned against closed forms (one key, two keys, equal keys, a dominant key, weights summing to
one), an independent library routine (torch's scaled_dot_product_attention on the CPU in
float64, causal block with an offset), an independent masked-matrix formulation of the verify
block, causality, split-merge algebra, and special cases that reduce one drafter to full
attention exactly.
"""
import numpy as np
import pytest
import torch

from kv_cache_compressed_amd import synth
from oracle import select as sel
from oracle import attention as A
from oracle.quant import KiviLayer

RNG = np.random.default_rng(11)


def _rand(*shape):
    return RNG.standard_normal(shape)


def test_weights_sum_to_one():
    for S in (1, 2, 7, 300):
        q, K = _rand(16), _rand(S, 16)
        o, _ = A.decode(q, K, np.ones((S, 3)), 0.3)
        assert np.allclose(o, 1.0, rtol=0, atol=1e-12)


def test_one_key_gives_its_value():
    q, K, V = _rand(8), _rand(1, 8), _rand(1, 8)
    o, lse = A.decode(q, K, V, 0.5)
    assert np.array_equal(o, V[0])
    assert lse == pytest.approx(float(K[0] @ q) * 0.5, abs=1e-14)


def test_two_keys_closed_form():
    for _ in range(50):
        q, K, V = _rand(8), _rand(2, 8), _rand(2, 8)
        s0, s1 = (K @ q) * 0.2
        sig = 1.0 / (1.0 + np.exp(-(s0 - s1)))
        o, lse = A.decode(q, K, V, 0.2)
        assert np.allclose(o, sig * V[0] + (1 - sig) * V[1], atol=1e-13)
        assert lse == pytest.approx(np.logaddexp(s0, s1), abs=1e-13)


def test_equal_keys_give_mean_value():
    k = _rand(16)
    K = np.tile(k, (9, 1))
    V = _rand(9, 16)
    o, lse = A.decode(_rand(16), K, V, 0.1)
    assert np.allclose(o, V.mean(axis=0), atol=1e-13)


def test_dominant_key_gives_its_value():
    q = np.ones(8)
    K = _rand(50, 8) * 0.01
    K[17] = 100.0
    V = _rand(50, 8)
    o, _ = A.decode(q, K, V, 1.0)
    assert np.allclose(o, V[17], atol=1e-12)


@pytest.mark.parametrize("n,L,d", [(0, 1, 8), (5, 3, 16), (37, 9, 32), (200, 31, 128)])
def test_verify_matches_torch_sdpa(n, L, d):
    """Row i at position n+i against keys 0..n+i == torch SDPA with a causal-offset mask."""
    Q = _rand(L, d)
    Kp, Vp, Kb, Vb = _rand(n, d), _rand(n, d), _rand(L, d), _rand(L, d)
    O, lse = A.verify_block(Q, Kp, Vp, Kb, Vb, 1 / np.sqrt(d))
    K = torch.from_numpy(np.concatenate([Kp, Kb]))
    V = torch.from_numpy(np.concatenate([Vp, Vb]))
    mask = torch.arange(n + L)[None, :] <= (n + torch.arange(L))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None, None], K[None, None], V[None, None], attn_mask=mask[None, None],
        scale=1 / np.sqrt(d))[0, 0].numpy()
    assert np.allclose(O, ref, atol=1e-12, rtol=0)


def test_verify_matches_masked_matrix_form():
    """An independent formulation: one L x (n+L) score matrix, -inf above the causal diagonal."""
    n, L, d = 60, 31, 128
    Q, Kp, Vp, Kb, Vb = _rand(L, d), _rand(n, d), _rand(n, d), _rand(L, d), _rand(L, d)
    O, lse = A.verify_block(Q, Kp, Vp, Kb, Vb)
    K = np.concatenate([Kp, Kb])
    V = np.concatenate([Vp, Vb])
    S = (Q @ K.T) * A.SM_SCALE_F32
    S[np.arange(n + L)[None, :] > (n + np.arange(L))[:, None]] = -np.inf
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    ref = (P @ V) / P.sum(axis=1, keepdims=True)
    assert np.allclose(O, ref, atol=1e-12, rtol=0)
    assert np.allclose(lse, m[:, 0] + np.log(P.sum(axis=1)), atol=1e-12)


def test_verify_row_is_decode_and_causal():
    n, L, d = 40, 9, 128
    Q, Kp, Vp, Kb, Vb = _rand(L, d), _rand(n, d), _rand(n, d), _rand(L, d), _rand(L, d)
    O, lse = A.verify_block(Q, Kp, Vp, Kb, Vb)
    for i in range(L):
        o, l = A.decode(Q[i], np.concatenate([Kp, Kb[: i + 1]]), np.concatenate([Vp, Vb[: i + 1]]))
        assert np.array_equal(O[i], o) and lse[i] == l
        Kb2, Vb2 = Kb.copy(), Vb.copy()
        Kb2[i + 1:] += 5.0
        Vb2[i + 1:] -= 3.0
        O2, _ = A.verify_block(Q, Kp, Vp, Kb2, Vb2)
        assert np.array_equal(O2[i], O[i])
    O1, _ = A.verify_block(Q[:1], Kp, Vp, Kb[:1], Vb[:1])
    assert np.array_equal(O1[0], O[0])


def test_gqa_head_map():
    assert [A.kv_head(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.kv_head(h, 8, 8) for h in range(8)] == list(range(8))
    assert A.kv_head(63, 64, 8) == 7


@pytest.mark.parametrize("trial", range(8))
def test_split_merge_equals_unsplit(trial):
    g = np.random.default_rng(100 + trial)
    S = int(g.integers(1, 400))
    q, K, V = g.standard_normal(64), g.standard_normal((S, 64)) * 2, g.standard_normal((S, 64))
    o, lse = A.decode(q, K, V, 0.125)
    cuts = np.sort(g.integers(0, S + 1, size=int(g.integers(0, 12))))
    bounds = [0, *cuts.tolist(), S]
    parts = [A.partial(q, K[a:b], V[a:b], 0.125) for a, b in zip(bounds[:-1], bounds[1:])]
    om, lm = A.lse_merge(parts)
    assert np.allclose(om, o, atol=1e-12, rtol=0) and abs(lm - lse) < 1e-12
    om2, lm2 = A.lse_merge(parts[::-1])
    assert np.allclose(om2, om, atol=1e-12, rtol=0) and abs(lm2 - lm) < 1e-12
    one = [A.partial(q, K[i:i + 1], V[i:i + 1], 0.125) for i in range(S)]
    om3, lm3 = A.lse_merge(one)
    assert np.allclose(om3, o, atol=1e-12, rtol=0) and abs(lm3 - lse) < 1e-12


def test_kivi_with_nothing_quantised_is_full_attention():
    g = np.random.default_rng(12)
    K, V = g.standard_normal((70, 128)).astype(np.float32), g.standard_normal((70, 128)).astype(np.float32)
    q = g.standard_normal(128)
    lay = KiviLayer(K, V, n_q=0, bits=2, meta_dtype="f16", res_dtype="f32")
    o1, l1 = A.decode(q, lay.keys(70), lay.values(70))
    o2, l2 = A.decode(q, K.astype(np.float64), V.astype(np.float64))
    assert np.array_equal(o1, o2) and l1 == l2


def test_drop_keep_all_is_full_attention():
    g = np.random.default_rng(13)
    K, V, q = g.standard_normal((90, 128)), g.standard_normal((90, 128)), g.standard_normal(128)
    o1, l1 = A.drop_draft(q, K, V, np.arange(90))
    o2, l2 = A.decode(q, K, V)
    assert np.array_equal(o1, o2) and l1 == l2


def test_keep_list_recipe_of_the_dropping_workload():
    """The dropping workload's recipe through the oracle's selection: 25% kept, sinks and recent
    included, every kept middle score >= every dropped one."""
    w = synth.WORKLOADS["c3"].with_(n=5000, B=2, Hkv=2, Hq=4)
    for b in range(2):
        for h in range(2):
            s = synth.scores(w, 0, b, h)
            idx = sel.keep_positions(s, w.n, w.sinks, w.recent, w.keep)
            assert idx.size == w.keep == 1250
            assert np.all(np.diff(idx) > 0)
            assert set(range(64)) <= set(idx.tolist())
            assert set(range(w.n - 256, w.n)) <= set(idx.tolist())
            mid = np.zeros(w.n, bool)
            mid[64:w.n - 256] = True
            kept = np.zeros(w.n, bool)
            kept[idx] = True
            assert s[mid & kept].min() >= s[mid & ~kept].max()


def test_keep_list_ties_prefer_lower_position():
    w = synth.WORKLOADS["c3"].with_(n=400, keep_frac=0.9)   # keep 360: 64 + 256 + 40 of 80
    idx = sel.keep_positions(np.zeros(w.n, np.float32), w.n, w.sinks, w.recent, w.keep)
    assert idx.tolist() == list(range(64)) + list(range(64, 104)) + list(range(144, 400))
