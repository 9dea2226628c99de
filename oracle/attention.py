"""Attention over the KV cache, as the draft and verify passes use it (CPU oracle, float64).

The method runs the *same* model on both sides; only the KV source differs ("VeriCache: making
lossy KV compression exact", The Core Idea; "VeriCache: Turning Lossy KV Cache into Lossless LLM
Inference", Methodology). So one attention definition serves every step here, and the draft /
verify variants differ only in which keys and values they are handed:

* draft, quantised drafter: the dequantised prefix plus the full-precision residual
  (the compressed cache the drafter reads from GPU memory; Key Contributions, first item);
* draft, token-dropping drafter: only the kept positions (the uniform compressor interface
  exposes dropped-token positions; Key Contributions, third item);
* verify: every position of the full cache. The verifier scores all drafted positions in one
  pass and returns one more prediction than there are drafts (The Core Idea); row i of that
  pass sees the cached context plus block rows 0..i.

Readings taken where the pages are silent: the attention is textbook scaled dot-product
softmax attention with scale 1/sqrt(128) passed in; a query at position p sees keys 0..p
inclusive; query head h reads kv head h // (Hq/Hkv). Split-K partials and their log-sum-exp
merge are not part of the definition (they are a faster route to the same numbers); the merge is
written out below only so that its algebra can be pinned.
"""
from __future__ import annotations

import numpy as np

SM_SCALE_F32 = float(np.float32(1.0 / np.sqrt(128.0)))


def decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float = SM_SCALE_F32):
    """One query against a key/value list.

    s_t = (q . k_t) * scale;  w = exp(s - max s) / sum exp(s - max s);  o = sum_t w_t v_t;
    lse = max s + ln sum exp(s - max s).  Returns (o [d], lse) in float64.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = (K @ q) * sm_scale
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    o = (e @ V) / l
    return o, m + np.log(l)


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Grouped-query head map: contiguous groups of Hq/Hkv query heads share one kv head."""
    return h // (Hq // Hkv)


def verify_block(Q: np.ndarray, K_past: np.ndarray, V_past: np.ndarray, K_blk: np.ndarray,
                 V_blk: np.ndarray, sm_scale: float = SM_SCALE_F32):
    """Rows i = 0..L-1 of one query head against the full cache, causally.

    Row i is decode attention at position n + i over keys 0..n-1 (cached) and n..n+i (block).
    Q [L, d]; K_past/V_past [n, d]; K_blk/V_blk [L, d]. Returns (O [L, d], lse [L]).
    """
    L = Q.shape[0]
    O = np.zeros((L, Q.shape[1]))
    lse = np.zeros(L)
    for i in range(L):
        K = np.concatenate([K_past, K_blk[: i + 1]], axis=0)
        V = np.concatenate([V_past, V_blk[: i + 1]], axis=0)
        O[i], lse[i] = decode(Q[i], K, V, sm_scale)
    return O, lse


def drop_draft(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
               sm_scale: float = SM_SCALE_F32):
    """Decode attention over the kept positions only: keys K[idx], values V[idx]."""
    idx = np.asarray(idx, np.int64)
    return decode(q, K[idx], V[idx], sm_scale)


def partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float = SM_SCALE_F32):
    """Unnormalised partial of one key subset: (o_s = sum e_t v_t, m_s, l_s = sum e_t)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf, 0.0
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64)) * sm_scale
    m = s.max()
    e = np.exp(s - m)
    return e @ np.asarray(V, np.float64), m, e.sum()


def lse_merge(parts):
    """Merge split partials (o_s, m_s, l_s): m = max m_s, w_s = l_s e^{m_s - m},
    o = sum o_s e^{m_s - m} / sum w_s, lse = m + ln sum w_s. Empty splits (l_s = 0) add nothing."""
    live = [p for p in parts if p[2] > 0]
    if not live:
        return np.zeros_like(parts[0][0], dtype=np.float64), -np.inf
    m = max(p[1] for p in live)
    num = sum(p[0] * np.exp(p[1] - m) for p in live)
    den = sum(p[2] * np.exp(p[1] - m) for p in live)
    return num / den, m + np.log(den)
