"""Seeded synthetic inputs for the draft/verify attention path.

This module only *draws* inputs. It holds no step of the method: no quantisation, no
attention, no softmax, no accept rule. The tests, the benchmark and the CPU checker all take
their inputs from here, so every side sees the same values.

Generator: NumPy ``PCG64`` seeded with ``SeedSequence([seed, workload_id, tag, b, h])``;
values are float32 ``standard_normal``; bf16 tensors are the float32 draws rounded to the
nearest bf16 (ties to even). Slicing per (b, h) lets multi-GB tensors be drawn in parallel
pieces.

The workload shapes follow the pages' setting: Llama-3.1-8B- and Llama-70B-shaped attention
layers, contexts up to ~500K tokens, draft length 30 and 4x compression ("VeriCache: Turning
Lossy KV Cache into Lossless LLM Inference", Methodology and Results). The KIVI parameters
(group 32, 2/4-bit, residual length and dtype), the outlier-channel recipe (1% of the
(kv head, channel) slots scaled by 8) and the keep-list recipe (64 sinks + 256 recent +
top-scoring middle tokens, 25% kept; the scores are drawn here, the selection is the method's)
are the workload recipes of the study, since the pages give none of them.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

# Fixed tensor tags of the seed sequence.
TAG_K_PAST, TAG_V_PAST, TAG_Q_NEW, TAG_K_NEW, TAG_V_NEW = 0, 1, 3, 4, 5
TAG_W, TAG_SCORES, TAG_OUTLIERS, TAG_Q_PROMPT = 6, 7, 8, 9

_POOL_WORKERS = 8


@dataclass(frozen=True)
class Workload:
    """One synthetic single-layer draft/verify round.

    n is the number of cached tokens before the round; the round drafts x tokens and verifies
    L = x + 1 query rows at positions n .. n + x.
    """

    name: str
    wid: int                  # workload id mixed into every seed
    B: int
    Hq: int
    Hkv: int
    n: int
    x: int
    kv_dtype: str             # "f32" | "bf16" (also the dtype of q)
    drafter: str              # "kivi" | "drop"
    d: int = 128
    bits: int = 0             # KIVI code width (2 or 4)
    group: int = 32           # KIVI group size
    R: int = 0                # KIVI full-precision residual length after prefill
    res_dtype: str = "f32"    # KIVI residual storage dtype
    meta_dtype: str = "f32"   # KIVI (scale, min) storage dtype
    res_cap: int = 0          # KIVI residual ring capacity (multiple of group)
    keep_frac: float = 0.0    # drop drafter: kept fraction of the context
    sinks: int = 64           # drop drafter: leading tokens always kept
    recent: int = 256         # drop drafter: trailing tokens always kept
    outlier_frac: float = 0.0  # fraction of (kv head, channel) slots scaled up
    outlier_scale: float = 8.0
    vocab: int = 2048         # width of the random fp32 logits projection
    past_on_host: bool = False
    chunk_tokens: int = 0

    @property
    def L(self) -> int:
        return self.x + 1

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def keep(self) -> int:
        return int(round(self.keep_frac * self.n))

    @property
    def tok_cap(self) -> int:
        """Token capacity of the full-KV store (context plus the round's block), group aligned."""
        t = self.n + self.L
        return ((t + 31) // 32) * 32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the study. 1-4 are single attention layers; 5 (the end-to-end loop
# on a 4-layer decoder) is not a single-layer round and is not listed here.
WORKLOADS = {
    "c1": Workload("c1", 1, B=1, Hq=32, Hkv=8, n=2048, x=8, kv_dtype="f32", drafter="kivi",
                   bits=4, R=32, res_dtype="f32", meta_dtype="f32", res_cap=128),
    "c2": Workload("c2", 2, B=8, Hq=32, Hkv=8, n=32768, x=30, kv_dtype="bf16", drafter="kivi",
                   bits=2, R=128, res_dtype="f16", meta_dtype="f16", res_cap=256,
                   outlier_frac=0.01),
    "c3": Workload("c3", 3, B=4, Hq=64, Hkv=8, n=100000, x=30, kv_dtype="bf16", drafter="drop",
                   keep_frac=0.25),
    "c4": Workload("c4", 4, B=1, Hq=32, Hkv=8, n=500000, x=30, kv_dtype="bf16", drafter="kivi",
                   bits=4, R=128, res_dtype="f16", meta_dtype="f16", res_cap=256,
                   past_on_host=True, chunk_tokens=65536),
}


def generator(seed: int, wid: int, tag: int, b: int = 0, h: int = 0,
              extra: int | None = None) -> np.random.Generator:
    ent = [seed, wid, tag, b, h] + ([] if extra is None else [extra])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ent)))


def normal(seed: int, wid: int, tag: int, b: int, h: int, shape, extra: int | None = None) -> np.ndarray:
    return generator(seed, wid, tag, b, h, extra).standard_normal(shape, dtype=np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 holding the bf16 value."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def outlier_slots(w: Workload, seed: int = 0) -> np.ndarray:
    """(kv head, channel) slots scaled by outlier_scale; drawn without replacement."""
    nslots = int(round(w.outlier_frac * w.Hkv * w.d))
    if nslots == 0:
        return np.zeros((0, 2), np.int64)
    flat = generator(seed, w.wid, TAG_OUTLIERS).choice(w.Hkv * w.d, size=nslots, replace=False)
    flat = np.sort(flat)
    return np.stack([flat // w.d, flat % w.d], axis=1)


def _kv_slice(w: Workload, seed: int, tag: int, b: int, h: int, ntok: int, slots,
              extra: int | None = None) -> np.ndarray:
    x = normal(seed, w.wid, tag, b, h, (ntok, w.d), extra)
    if w.kv_dtype == "bf16":
        x = round_bf16(x)
    for hh, c in slots:
        if hh == h:
            x[:, c] *= np.float32(w.outlier_scale)  # exact: power of two
    return x


def _fill(fn, items):
    with ThreadPoolExecutor(_POOL_WORKERS) as ex:
        return list(ex.map(fn, items))


def kv_past(w: Workload, seed: int = 0):
    """Cached keys/values of positions 0..n-1: float32 arrays [B, Hkv, n, d] (bf16-valued for bf16)."""
    slots = outlier_slots(w, seed)
    K = np.empty((w.B, w.Hkv, w.n, w.d), np.float32)
    V = np.empty_like(K)

    def one(bh):
        b, h = bh
        K[b, h] = _kv_slice(w, seed, TAG_K_PAST, b, h, w.n, slots)
        V[b, h] = _kv_slice(w, seed, TAG_V_PAST, b, h, w.n, slots)

    _fill(one, [(b, h) for b in range(w.B) for h in range(w.Hkv)])
    return K, V


def kv_new(w: Workload, seed: int = 0, round_index: int = 0):
    """Keys/values of the round's positions n..n+x: float32 arrays [B, Hkv, L, d]. Round t > 0 of
    a multi-round decode draws its own block (positions that a round drafted but did not commit
    get new values in the next round, as they would once the token there changes)."""
    slots = outlier_slots(w, seed)
    extra = None if round_index == 0 else round_index
    K = np.empty((w.B, w.Hkv, w.L, w.d), np.float32)
    V = np.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            K[b, h] = _kv_slice(w, seed, TAG_K_NEW, b, h, w.L, slots, extra)
            V[b, h] = _kv_slice(w, seed, TAG_V_NEW, b, h, w.L, slots, extra)
    return K, V


def q_new(w: Workload, seed: int = 0, round_index: int = 0) -> np.ndarray:
    """Queries of positions n..n+x: float32 [B, Hq, L, d] (bf16-valued for bf16 workloads); round
    t > 0 of a multi-round decode draws its own."""
    extra = None if round_index == 0 else round_index
    Q = np.empty((w.B, w.Hq, w.L, w.d), np.float32)
    for b in range(w.B):
        for h in range(w.Hq):
            Q[b, h] = normal(seed, w.wid, TAG_Q_NEW, b, h, (w.L, w.d), extra)
    if w.kv_dtype == "bf16":
        Q = round_bf16(Q)
    return Q


def q_prompt(w: Workload, seed: int = 0) -> np.ndarray:
    """Queries of a prompt's positions 0..n-1: float32 [B, Hq, n, d] (bf16-valued for bf16
    workloads), for the prefill pass."""
    Q = np.empty((w.B, w.Hq, w.n, w.d), np.float32)
    for b in range(w.B):
        for h in range(w.Hq):
            Q[b, h] = normal(seed, w.wid, TAG_Q_PROMPT, b, h, (w.n, w.d))
    if w.kv_dtype == "bf16":
        Q = round_bf16(Q)
    return Q


def projection(w: Workload, seed: int = 0) -> np.ndarray:
    """Random fp32 logits projection W [vocab, Hq*d]; logits z = W @ concat_heads(o)."""
    return normal(seed, w.wid, TAG_W, 0, 0, (w.vocab, w.Hq * w.d))


def scores(w: Workload, seed: int, b: int, h: int) -> np.ndarray:
    """Seeded per-(b, kv head) importance scores over positions 0..n-1 (float32 N(0,1))."""
    return normal(seed, w.wid, TAG_SCORES, b, h, (w.n,))
