"""The draft-then-verify loop on a tiny random decoder (CPU oracle, float64).

Used only to pin the accept rule and the round semantics against the pages' central claim: the
loop emits exactly what greedy decoding over the full cache emits, whatever the drafter proposes
("VeriCache: making lossy KV compression exact", The Core Idea and Verifying Without Giving Back
the Speedup; "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Abstract and
Results). The drafter and the verifier share the model weights and differ only in the cache they
read (Methodology).

The model: one attention layer with grouped-query heads over token + position embeddings, a
residual connection and an untied output head. Keys/values of a position depend only on its token
and position, so both caches are functions of the committed tokens; the compressed cache is rebuilt
from the committed prefix each round (reading: the compressed copy tracks the committed prefix and
draft-time entries are discarded after the round).
"""
from __future__ import annotations

import numpy as np

from .accept import accept
from .attention import decode
from .quant import quantize_groups


def bf16(a):
    """float32 values rounded to the nearest bfloat16 (ties to even), as float64."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class TinyModel:
    """kv_bf16: queries, keys and values are stored at bfloat16 precision (rounded from their fp32
    values), as a cache kept in bf16 holds them."""

    def __init__(self, seed=0, vocab=11, dm=16, d=8, Hq=4, Hkv=2, max_pos=128, kv_bf16=False):
        self.kv_bf16 = kv_bf16
        g = np.random.default_rng(seed)
        self.V, self.dm, self.d, self.Hq, self.Hkv = vocab, dm, d, Hq, Hkv
        self.E = g.standard_normal((vocab, dm))
        self.P = 0.5 * g.standard_normal((max_pos, dm))
        self.Wq = g.standard_normal((Hq * d, dm)) / np.sqrt(dm)
        self.Wk = g.standard_normal((Hkv * d, dm)) / np.sqrt(dm)
        self.Wv = g.standard_normal((Hkv * d, dm)) / np.sqrt(dm)
        self.Wo = g.standard_normal((dm, Hq * d)) / np.sqrt(Hq * d)
        self.Wlm = 3.0 * g.standard_normal((vocab, dm)) / np.sqrt(dm)
        self.scale = 1.0 / np.sqrt(d)

    def _x(self, tok, pos):
        return self.E[tok] + self.P[pos]

    def _r(self, a):
        return bf16(a) if self.kv_bf16 else a

    def kv(self, tok, pos):
        x = self._x(tok, pos)
        return (self._r(self.Wk @ x).reshape(self.Hkv, self.d),
                self._r(self.Wv @ x).reshape(self.Hkv, self.d))

    def next_logits(self, tok, pos, K, V):
        """Logits after token `tok` at `pos`, attending over K/V [Hkv][S, d] (S includes pos)."""
        x = self._x(tok, pos)
        q = self._r(self.Wq @ x).reshape(self.Hq, self.d)
        G = self.Hq // self.Hkv
        o = np.concatenate([decode(q[h], K[h // G], V[h // G], self.scale)[0]
                            for h in range(self.Hq)])
        return self.Wlm @ (x + self.Wo @ o)


def full_cache(model, tokens):
    """Per kv head: keys/values of every position of `tokens`, float64 [Hkv][len, d]."""
    kvs = [model.kv(t, p) for p, t in enumerate(tokens)]
    K = [np.stack([k[h] for k, _ in kvs]) for h in range(model.Hkv)]
    V = [np.stack([v[h] for _, v in kvs]) for h in range(model.Hkv)]
    return K, V


def greedy(model, prompt, steps):
    """Plain greedy decoding over the full cache."""
    toks = list(prompt)
    out = []
    while len(out) < steps:
        K, V = full_cache(model, toks)
        z = model.next_logits(toks[-1], len(toks) - 1, K, V)
        t = int(np.argmax(z))
        out.append(t)
        toks.append(t)
    return out


# ---- drafters: each maps (model, committed tokens, x) -> x proposed tokens -----------------

def _draft_with_cache(model, toks, x, compress):
    """Autoregressive drafting: the committed positions come from compress(full cache); the
    draft's own positions are appended exactly."""
    K, V = full_cache(model, toks)
    K, V = compress(K, V)
    K = [k.copy() for k in K]
    V = [v.copy() for v in V]
    seq = list(toks)
    draft = []
    for _ in range(x):
        z = model.next_logits(seq[-1], len(seq) - 1, K, V)
        t = int(np.argmax(z))
        draft.append(t)
        seq.append(t)
        k, v = model.kv(t, len(seq) - 1)
        K = [np.vstack([K[h], k[h]]) for h in range(model.Hkv)]
        V = [np.vstack([V[h], v[h]]) for h in range(model.Hkv)]
    return draft


def drafter_exact(model, toks, x):
    return _draft_with_cache(model, toks, x, lambda K, V: (K, V))


def drafter_quant(model, toks, x, bits=2):
    """Per-token min/max quantisation of every committed key and value row (lossy)."""
    def comp(K, V):
        def q(A):
            c, s, m = quantize_groups(A.astype(np.float32), bits, "f32")
            return c.astype(np.float64) * s[:, None] + m[:, None]
        return [q(k) for k in K], [q(v) for v in V]
    return _draft_with_cache(model, toks, x, comp)


def drafter_drop(model, toks, x, sinks=2, recent=3):
    """Keep the first `sinks` and last `recent` committed positions (lossy)."""
    def comp(K, V):
        n = K[0].shape[0]
        keep = sorted(set(range(min(sinks, n))) | set(range(max(0, n - recent), n)))
        return [k[keep] for k in K], [v[keep] for v in V]
    return _draft_with_cache(model, toks, x, comp)


def drafter_wrong(model, toks, x):
    """Always proposes tokens the full-cache model would not pick first."""
    K, V = full_cache(model, toks)
    z = model.next_logits(toks[-1], len(toks) - 1, K, V)
    return [(int(np.argmax(z)) + 1) % model.V] * x


def drafter_random(model, toks, x, seed=0):
    g = np.random.default_rng(seed + len(toks))
    return [int(t) for t in g.integers(0, model.V, size=x)]


def verify(model, toks, draft):
    """One pass over the full cache: predictions after the last committed token and after each
    draft token, x + 1 in all (each position attends causally over everything before it)."""
    seq = list(toks) + list(draft)
    K, V = full_cache(model, seq)
    n = len(toks)
    preds = []
    for i in range(len(draft) + 1):
        p = n - 1 + i
        Kp = [k[: p + 1] for k in K]
        Vp = [v[: p + 1] for v in V]
        preds.append(int(np.argmax(model.next_logits(seq[p], p, Kp, Vp))))
    return preds


def vericache(model, prompt, steps, x, drafter):
    """Repeat draft / verify / accept until `steps` tokens are emitted; returns (tokens, rounds)
    with rounds = [(a, emitted count)]."""
    toks = list(prompt)
    out, rounds = [], []
    while len(out) < steps:
        draft = drafter(model, toks, x)
        a, _, emitted = accept(draft, verify(model, toks, draft))
        emitted = emitted[: steps - len(out)]
        rounds.append((a, len(emitted)))
        out += emitted
        toks += emitted
    return out, rounds


class LayeredModel:
    """`layers` attention layers stacked on the residual stream: x_0 = E[tok] + P[pos];
    x_{l+1} = x_l + Wo_l attention_l(Wq_l x_l; keys Wk_l x_l and values Wv_l x_l of positions
    0..p); logits = Wlm x_L. With one layer it is TinyModel (the drafter and the verifier again
    share every weight). Layers above the first see keys/values that depend on the attention below,
    so a drafter's keys/values of its own positions differ from the verifier's there.
    kv_bf16 as in TinyModel. Weights drawn like TinyModel's, per layer."""

    def __init__(self, seed=0, vocab=11, dm=16, d=8, Hq=4, Hkv=2, layers=2, max_pos=128,
                 kv_bf16=False):
        g = np.random.default_rng(seed)
        self.V, self.dm, self.d, self.Hq, self.Hkv, self.nl = vocab, dm, d, Hq, Hkv, layers
        self.kv_bf16 = kv_bf16
        self.E = g.standard_normal((vocab, dm))
        self.P = 0.5 * g.standard_normal((max_pos, dm))
        self.Wq, self.Wk, self.Wv, self.Wo = [], [], [], []
        for _ in range(layers):
            self.Wq.append(g.standard_normal((Hq * d, dm)) / np.sqrt(dm))
            self.Wk.append(g.standard_normal((Hkv * d, dm)) / np.sqrt(dm))
            self.Wv.append(g.standard_normal((Hkv * d, dm)) / np.sqrt(dm))
            self.Wo.append(g.standard_normal((dm, Hq * d)) / np.sqrt(Hq * d) / np.sqrt(layers))
        self.Wlm = 3.0 * g.standard_normal((vocab, dm)) / np.sqrt(dm)
        self.scale = 1.0 / np.sqrt(d)

    def _r(self, a):
        return bf16(a) if self.kv_bf16 else a

    def logits_all(self, tokens):
        """Causal forward over every position of `tokens`: logits [len, V] (float64)."""
        n = len(tokens)
        X = self.E[np.asarray(tokens)] + self.P[:n]
        G = self.Hq // self.Hkv
        for l in range(self.nl):
            Q = self._r(X @ self.Wq[l].T).reshape(n, self.Hq, self.d)
            K = self._r(X @ self.Wk[l].T).reshape(n, self.Hkv, self.d)
            Vv = self._r(X @ self.Wv[l].T).reshape(n, self.Hkv, self.d)
            O = np.zeros((n, self.Hq, self.d))
            for p in range(n):
                for h in range(self.Hq):
                    O[p, h] = decode(Q[p, h], K[: p + 1, h // G], Vv[: p + 1, h // G], self.scale)[0]
            X = X + O.reshape(n, -1) @ self.Wo[l].T
        return X @ self.Wlm.T


def greedy_layered(model, prompt, steps):
    """Plain greedy decoding over the full cache of a LayeredModel."""
    toks = list(prompt)
    out = []
    while len(out) < steps:
        t = int(np.argmax(model.logits_all(toks)[-1]))
        out.append(t)
        toks.append(t)
    return out


# ---- a Llama-style layer stack (norms, rotary positions, gated MLP) ---------------------------
# The pages evaluate Llama-, Mistral- and Qwen-family models ("VeriCache: Turning Lossy KV Cache
# into Lossless LLM Inference", Results) without describing their layers; the layer below is the
# published Llama form (pre-norm RMSNorm, rotary position embedding on queries and keys, SwiGLU
# MLP, a final RMSNorm before the output head). Reading: keys are cached after the rotation, as a
# KV cache of such a model holds them; the rotation pairs channel i with channel i + d/2.

def rms_norm(X, g, eps=1e-5):
    """Each row of X divided by its root mean square (eps inside the root), times the gain g."""
    X = np.asarray(X, np.float64)
    return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps) * g


def rope(X, pos, theta=500000.0):
    """Rotary position embedding of rows X [..., d] at positions pos (broadcast over the leading
    axes): channel pair (i, i + d/2) is turned by the angle pos * theta^(-2i/d)."""
    X = np.asarray(X, np.float64)
    half = X.shape[-1] // 2
    ang = np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * np.arange(half) / X.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    a, b = X[..., :half], X[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(X):
    return X / (1.0 + np.exp(-X))


class LlamaModel:
    """`layers` pre-norm blocks on the residual stream: x_0 = E[tok];
    h = rms_norm(x_l) g_att_l; q, k = rope(Wq_l h), rope(Wk_l h) at the row's position; v = Wv_l h;
    x' = x_l + Wo_l attention(q; k, v of positions 0..p);
    x_{l+1} = x' + W2_l (silu(W1_l h') * (W3_l h')) with h' = rms_norm(x') g_mlp_l;
    logits = Wlm rms_norm(x_L) g_f. kv_bf16 rounds q, k (after the rotation) and v to bfloat16.
    Gains are drawn near 1, projections at the scales of LayeredModel, the MLP width F."""

    def __init__(self, seed=0, vocab=11, dm=16, d=8, Hq=4, Hkv=2, layers=2, F=32, kv_bf16=False,
                 theta=500000.0):
        g = np.random.default_rng(seed)
        self.V, self.dm, self.d, self.Hq, self.Hkv, self.nl, self.F = vocab, dm, d, Hq, Hkv, layers, F
        self.kv_bf16, self.theta = kv_bf16, theta
        self.E = g.standard_normal((vocab, dm))
        gain = lambda: 1.0 + 0.1 * g.standard_normal(dm)
        self.g_att, self.Wq, self.Wk, self.Wv, self.Wo = [], [], [], [], []
        self.g_mlp, self.W1, self.W3, self.W2 = [], [], [], []
        for _ in range(layers):
            self.g_att.append(gain())
            self.Wq.append(g.standard_normal((Hq * d, dm)) / np.sqrt(dm))
            self.Wk.append(g.standard_normal((Hkv * d, dm)) / np.sqrt(dm))
            self.Wv.append(g.standard_normal((Hkv * d, dm)) / np.sqrt(dm))
            self.Wo.append(g.standard_normal((dm, Hq * d)) / np.sqrt(Hq * d) / np.sqrt(layers))
            self.g_mlp.append(gain())
            self.W1.append(g.standard_normal((F, dm)) / np.sqrt(dm))
            self.W3.append(g.standard_normal((F, dm)) / np.sqrt(dm))
            self.W2.append(g.standard_normal((dm, F)) / np.sqrt(F) / np.sqrt(layers))
        self.g_f = gain()
        self.Wlm = 3.0 * g.standard_normal((vocab, dm)) / np.sqrt(dm)
        self.scale = 1.0 / np.sqrt(d)

    def _r(self, a):
        return bf16(a) if self.kv_bf16 else a

    def logits_all(self, tokens, pos0=0):
        """Causal forward over every position of `tokens` (the first at position pos0): logits
        [len, V] (float64)."""
        n = len(tokens)
        X = self.E[np.asarray(tokens)].copy()
        pos = pos0 + np.arange(n)
        G = self.Hq // self.Hkv
        for l in range(self.nl):
            H = rms_norm(X, self.g_att[l])
            Q = self._r(rope((H @ self.Wq[l].T).reshape(n, self.Hq, self.d), pos[:, None], self.theta))
            K = self._r(rope((H @ self.Wk[l].T).reshape(n, self.Hkv, self.d), pos[:, None], self.theta))
            Vv = self._r((H @ self.Wv[l].T).reshape(n, self.Hkv, self.d))
            O = np.zeros((n, self.Hq, self.d))
            for p in range(n):
                for h in range(self.Hq):
                    O[p, h] = decode(Q[p, h], K[: p + 1, h // G], Vv[: p + 1, h // G], self.scale)[0]
            X = X + O.reshape(n, -1) @ self.Wo[l].T
            H2 = rms_norm(X, self.g_mlp[l])
            X = X + (silu(H2 @ self.W1[l].T) * (H2 @ self.W3[l].T)) @ self.W2[l].T
        return rms_norm(X, self.g_f) @ self.Wlm.T


def greedy_llama(model, prompt, steps):
    """Plain greedy decoding over the full cache of a LlamaModel."""
    toks = list(prompt)
    out = []
    while len(out) < steps:
        t = int(np.argmax(model.logits_all(toks)[-1]))
        out.append(t)
        toks.append(t)
    return out
