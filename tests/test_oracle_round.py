"""Round-level pins of the oracle on small workloads (CPU only).

An uncompressed drafter must be accepted in full (the pages' same-weights argument: the drafter
and verifier then compute the same thing), for both drafter kinds; and verify row j must equal an
uncompressed draft step j exactly.
"""
import numpy as np

from kv_cache_compressed_amd import synth
from oracle.round import Round


def _inputs(w, seed=0):
    K, V = synth.kv_past(w, seed)
    Kn, Vn = synth.kv_new(w, seed)
    return K, V, Kn, Vn, synth.q_new(w, seed), synth.projection(w, seed)


def test_uncompressed_kivi_drafter_accepts_everything():
    # R >= n: nothing is quantised, the residual holds every token at fp32.
    w = synth.WORKLOADS["c1"].with_(n=300, R=400, x=5, B=1, Hq=8, Hkv=2, vocab=64)
    rnd = Round(w, *_inputs(w))
    assert rnd.n_q == 0
    res = rnd.run(0)
    assert res["a"] == w.x and res["next"] == res["verified"][-1]
    assert np.array_equal(res["drafts"], res["verified"][:-1])


def test_keep_all_drop_drafter_accepts_everything():
    w = synth.WORKLOADS["c3"].with_(n=500, x=4, B=1, Hq=8, Hkv=2, vocab=64, keep_frac=1.0,
                                    kv_dtype="bf16")
    K, V, Kn, Vn, Q, W = _inputs(w)
    idx = [[np.arange(w.n) for _ in range(w.Hkv)]]
    rnd = Round(w, K, V, Kn, Vn, Q, W, idx=idx)
    res = rnd.run(0)
    assert res["a"] == w.x
    for j in range(w.x):
        O, _ = rnd.draft_step(0, j)
        Ov, _ = rnd.verify(0)
        assert np.array_equal(O, Ov[:, j, :])


def test_compressed_round_is_well_formed():
    w = synth.WORKLOADS["c2"].with_(n=700, B=1, x=6, vocab=128)
    rnd = Round(w, *_inputs(w))
    res = rnd.run(0)
    assert 0 <= res["a"] <= w.x and len(res["emitted"]) == res["a"] + 1
    assert np.all(np.isfinite(res["draft_logits"])) and np.all(res["draft_gap"] >= 0)


def test_bf16_rounding_of_the_tiny_model():
    """The oracle's bf16 rounding (8 significant bits): exact bf16 values are kept, halfway cases go
    to the neighbour with the even last bit, others to the nearest."""
    from oracle.loop import bf16
    cases = [
        (1.0, 1.0),                          # exact
        (1.0 + 2 ** -8, 1.0),                # halfway between 1 and 1 + 2^-7: 1 is even
        (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),  # halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
        (1.0 + 2 ** -9, 1.0),                # below halfway
        (1.0 + 2 ** -8 + 2 ** -12, 1.0 + 2 ** -7),  # above halfway
        (-2.5, -2.5),
        (3.0 + 2 ** -7, 3.0),                # spacing 2^-6 in [2, 4): halfway, 3 is even
        (3.0 + 3 * 2 ** -7, 3.0 + 2 ** -5),  # halfway between 3 + 2^-6 (odd) and 3 + 2^-5 (even)
    ]
    x = np.array([c[0] for c in cases], np.float32)
    assert bf16(x).tolist() == [c[1] for c in cases]
    g = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    r = bf16(g)
    assert np.all(np.abs(r - g) <= np.abs(g) * 2.0 ** -8)                 # within half a bf16 ulp
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)   # representable in bf16


def test_layered_model_one_layer_is_the_tiny_model_and_causal():
    from oracle.loop import LayeredModel, TinyModel, full_cache
    lm = LayeredModel(seed=2, vocab=13, dm=16, d=8, Hq=4, Hkv=2, layers=1, max_pos=64)
    tm = TinyModel(seed=9, vocab=13, dm=16, d=8, Hq=4, Hkv=2, max_pos=64)
    for k in ("E", "P", "Wlm"):
        setattr(tm, k, getattr(lm, k))
    tm.Wq, tm.Wk, tm.Wv, tm.Wo = lm.Wq[0], lm.Wk[0], lm.Wv[0], lm.Wo[0]
    toks = list(np.random.default_rng(0).integers(0, 13, 20))
    Z = lm.logits_all(toks)
    for p in (0, 7, 19):
        K, V = full_cache(tm, toks[: p + 1])
        assert np.allclose(Z[p], tm.next_logits(toks[p], p, K, V), rtol=1e-12, atol=1e-12)
    # causality: later tokens do not change earlier logits (two layers)
    lm2 = LayeredModel(seed=3, vocab=13, dm=16, d=8, Hq=4, Hkv=2, layers=2, max_pos=64)
    a = lm2.logits_all(toks)
    b = lm2.logits_all(toks[:12] + [(t + 1) % 13 for t in toks[12:]])
    assert np.array_equal(a[:12], b[:12]) and not np.allclose(a[12:], b[12:])


def test_logits_select_the_concatenated_head_channel():
    """z = W concat_heads(O) with heads in order and channels contiguous within a head: an output
    that is zero except at (head h, channel c) picks column h*d + c of W, and a W whose row v is the
    indicator of slot (h_v, c_v) reads back O[h_v, c_v] (a transposed or head-interleaved concat
    fails both)."""
    from oracle.round import logits

    Hq, d, V = 4, 128, 37
    g = np.random.default_rng(3)
    W = g.standard_normal((V, Hq * d)).astype(np.float32)
    for h, c in ((0, 0), (2, 5), (3, 127), (1, 64)):
        O = np.zeros((Hq, d), np.float32)
        O[h, c] = 1.0
        assert np.array_equal(logits(W, O), W[:, h * d + c].astype(np.float64))
    O = g.standard_normal((Hq, d)).astype(np.float32)
    slots = [(int(g.integers(0, Hq)), int(g.integers(0, d))) for _ in range(V)]
    Wi = np.zeros((V, Hq * d), np.float32)
    for v, (h, c) in enumerate(slots):
        Wi[v, h * d + c] = 1.0
    assert np.array_equal(logits(Wi, O), np.array([O[h, c] for h, c in slots], np.float64))
    # linear in O: two heads' contributions add
    O2 = np.zeros((Hq, d), np.float32)
    O2[1, 3], O2[3, 9] = 2.0, -0.5
    W64 = W.astype(np.float64)
    assert np.allclose(logits(W, O2), 2.0 * W64[:, d + 3] - 0.5 * W64[:, 3 * d + 9], rtol=0, atol=1e-12)
