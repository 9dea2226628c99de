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
    assert w.n_q == 0
    rnd = Round(w, *_inputs(w))
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
