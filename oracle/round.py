"""One single-layer draft/verify round on a synthetic workload (CPU oracle, float64).

The round ("VeriCache: making lossy KV compression exact", The Core Idea): the drafter runs x
sequential decode steps over the compressed cache, each at the next position; the verifier then
scores all x drafted positions plus one more over the full cache in one pass; the accept rule
keeps the agreeing prefix and appends the verifier's token.

Readings taken where the pages are silent:
  * single layer, no embedding: the queries/keys/values of positions n..n+x are drawn inputs,
    so draft step j and verify row j use the same query and the same new key/value, and token ids
    only enter the accept step;
  * the draft-round keys/values are appended to the drafter's cache (to the quantised drafter's
    full-precision residual, or to the dropped drafter's kept list) before the step reads them;
  * logits are a random fp32 projection of the concatenated head outputs, z = W o.
"""
from __future__ import annotations

import numpy as np

from . import accept as acc
from .attention import SM_SCALE_F32, decode, kv_head, verify_block
from .quant import KiviLayer, quantised_prefix


def logits(W: np.ndarray, O: np.ndarray) -> np.ndarray:
    """z = W @ concat_heads(O); W [V, Hq*d], O [Hq, d] -> z [V] (float64)."""
    return np.asarray(W, np.float64) @ np.asarray(O, np.float64).reshape(-1)


class Round:
    """Inputs of one round: K_past/V_past [B,Hkv,n,d], K_new/V_new [B,Hkv,L,d], Q [B,Hq,L,d],
    W [V, Hq*d] (float32 arrays holding the exact input values), and for the dropping drafter the
    kept lists idx[b][h] (ascending positions < n)."""

    def __init__(self, w, K_past, V_past, K_new, V_new, Q, W, idx=None, sm_scale=SM_SCALE_F32):
        self.w, self.K_past, self.V_past = w, K_past, V_past
        self.K_new, self.V_new, self.Q, self.W, self.idx = K_new, V_new, Q, W, idx
        self.sm = sm_scale
        self._kivi = {}
        # quantised prefix after prefill (whole groups before a residual of at least R tokens)
        self.n_q = quantised_prefix(w.n, w.R, w.group) if w.drafter == "kivi" else 0

    # ---- drafter caches -------------------------------------------------------------------
    def kivi(self, b: int, h: int) -> KiviLayer:
        key = (b, h)
        if key not in self._kivi:
            w = self.w
            lay = KiviLayer(self.K_past[b, h], self.V_past[b, h], self.n_q, w.bits, w.meta_dtype,
                            w.res_dtype)
            for j in range(w.x):
                lay.append(self.K_new[b, h, j], self.V_new[b, h, j])
            self._kivi[key] = lay
        return self._kivi[key]

    def draft_head(self, b: int, hq: int, j: int):
        """Draft step j (position n+j) of query head hq: (o [d], lse)."""
        w = self.w
        h = kv_head(hq, w.Hq, w.Hkv)
        q = self.Q[b, hq, j]
        if w.drafter == "kivi":
            lay = self.kivi(b, h)
            r = (w.n - self.n_q) + j + 1
            return decode(q, lay.keys(r), lay.values(r), self.sm)
        K = np.concatenate([self.K_past[b, h][self.idx[b][h]], self.K_new[b, h, : j + 1]])
        V = np.concatenate([self.V_past[b, h][self.idx[b][h]], self.V_new[b, h, : j + 1]])
        return decode(q, K, V, self.sm)

    def draft_step(self, b: int, j: int):
        """All query heads of draft step j for batch row b: (O [Hq, d], lse [Hq])."""
        w = self.w
        O = np.zeros((w.Hq, w.d))
        lse = np.zeros(w.Hq)
        for hq in range(w.Hq):
            O[hq], lse[hq] = self.draft_head(b, hq, j)
        return O, lse

    # ---- verifier ----------------------------------------------------------------------
    def verify_head(self, b: int, hq: int):
        """All L rows of query head hq over the full cache: (O [L, d], lse [L])."""
        h = kv_head(hq, self.w.Hq, self.w.Hkv)
        return verify_block(self.Q[b, hq], self.K_past[b, h], self.V_past[b, h],
                            self.K_new[b, h], self.V_new[b, h], self.sm)

    def verify(self, b: int):
        w = self.w
        O = np.zeros((w.Hq, w.L, w.d))
        lse = np.zeros((w.Hq, w.L))
        for hq in range(w.Hq):
            O[hq], lse[hq] = self.verify_head(b, hq)
        return O, lse

    # ---- whole round ---------------------------------------------------------------------
    def run(self, b: int):
        """Draft tokens, verifier predictions, gaps and the accept result for batch row b."""
        w = self.w
        dz = np.stack([logits(self.W, self.draft_step(b, j)[0]) for j in range(w.x)])
        drafts = acc.argmax_rows(dz)
        Ov, _ = self.verify(b)
        vz = np.stack([logits(self.W, Ov[:, i, :]) for i in range(w.L)])
        verified = acc.argmax_rows(vz)
        a, nxt, emitted = acc.accept(drafts, verified)
        return dict(draft_logits=dz, drafts=drafts, draft_gap=acc.top2_gap(dz),
                    verify_logits=vz, verified=verified, verify_gap=acc.top2_gap(vz),
                    a=a, next=nxt, emitted=emitted)
