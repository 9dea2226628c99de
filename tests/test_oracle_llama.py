"""Pins of the oracle's Llama-style layer stack (oracle/loop.py: rms_norm, rope, silu, LlamaModel)
against properties the mathematics fixes: the rotary embedding as complex multiplication, its
relative-position property and inverse, the norm's unit root mean square, the gated unit's odd
part, causality, the head's closed form when every block adds nothing, and invariance of the
logits under a shift of all positions (rotary positions are relative)."""
import numpy as np
import pytest

from oracle.loop import LlamaModel, greedy_llama, rms_norm, rope, silu


def test_rope_is_complex_rotation():
    g = np.random.default_rng(0)
    d, pos, theta = 16, 37.0, 500000.0
    X = g.standard_normal((5, d))
    half = d // 2
    z = (X[:, :half] + 1j * X[:, half:]) * np.exp(1j * pos * theta ** (-np.arange(0, d, 2) / d))
    np.testing.assert_allclose(rope(X, pos, theta), np.concatenate([z.real, z.imag], axis=1),
                               rtol=0, atol=1e-12)


def test_rope_relative_identity_and_inverse():
    g = np.random.default_rng(1)
    q, k = g.standard_normal(128), g.standard_normal(128)
    for m, n, s in ((5, 2, 11), (0, 40, 1000), (300, 299, 7)):
        a = rope(q, m) @ rope(k, n)
        b = rope(q, m + s) @ rope(k, n + s)
        assert abs(a - b) < 1e-9 * (1 + abs(a))
    np.testing.assert_array_equal(rope(q, 0), q)
    np.testing.assert_allclose(rope(rope(q, 123.0), -123.0), q, atol=1e-12)
    assert abs(np.linalg.norm(rope(q, 77)) - np.linalg.norm(q)) < 1e-12


def test_rms_norm_and_silu():
    g = np.random.default_rng(2)
    X = g.standard_normal((4, 64)) * np.array([[0.1], [1.0], [10.0], [1e3]])
    Y = rms_norm(X, np.ones(64), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(Y * Y, axis=1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(Y, X / np.linalg.norm(X, axis=1, keepdims=True) * 8.0, rtol=1e-12)
    np.testing.assert_allclose(rms_norm(X, np.full(64, 3.0), eps=0.0), 3.0 * Y, rtol=1e-12)
    x = np.linspace(-20, 20, 81)
    np.testing.assert_allclose(silu(x) - silu(-x), x, atol=1e-12)   # x * (s(x) + s(-x)) = x
    assert silu(np.array([0.0]))[0] == 0.0


def test_llama_model_causal_shift_invariant_and_head():
    m = LlamaModel(seed=3, vocab=17, dm=16, d=8, Hq=4, Hkv=2, layers=2, F=24)
    g = np.random.default_rng(3)
    toks = [int(t) for t in g.integers(0, 17, 12)]
    z = m.logits_all(toks)
    # causal: changing later tokens leaves earlier rows alone
    other = toks[:7] + [(t + 1) % 17 for t in toks[7:]]
    np.testing.assert_array_equal(m.logits_all(other)[:7], z[:7])
    assert not np.allclose(m.logits_all(other)[7:], z[7:])
    # rotary positions are relative: shifting every position changes nothing
    np.testing.assert_allclose(m.logits_all(toks, pos0=1000), z, rtol=1e-9, atol=1e-9)
    # blocks that add nothing (Wo = W2 = 0): logits are the head of the normed embedding
    for l in range(m.nl):
        m.Wo[l] = np.zeros_like(m.Wo[l])
        m.W2[l] = np.zeros_like(m.W2[l])
    E = m.E[np.asarray(toks)]
    head = (E / np.sqrt(np.mean(E * E, axis=1, keepdims=True) + 1e-5) * m.g_f) @ m.Wlm.T
    np.testing.assert_allclose(m.logits_all(toks), head, rtol=1e-12, atol=1e-12)


def test_llama_model_sensitive_to_rotation_and_mlp():
    """The rotation and the MLP both act: switching either off changes the logits."""
    m = LlamaModel(seed=4, vocab=17, dm=16, d=8, Hq=4, Hkv=2, layers=2, F=24)
    toks = [3, 1, 4, 1, 5, 9, 2, 6]
    z = m.logits_all(toks)
    m0 = LlamaModel(seed=4, vocab=17, dm=16, d=8, Hq=4, Hkv=2, layers=2, F=24, theta=1e30)
    assert not np.allclose(m0.logits_all(toks), z)       # other rotation frequencies
    for l in range(m.nl):
        m.W2[l] = np.zeros_like(m.W2[l])
    assert not np.allclose(m.logits_all(toks), z)
    assert len(greedy_llama(m, toks, 3)) == 3
