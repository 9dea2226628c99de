"""KIVI-style quantisation of one attention layer's KV cache (CPU oracle).

The pages name quantisation as one of the two compressor families: every cached position is
kept, each entry is stored with fewer bits ("VeriCache: making lossy KV compression exact",
"The Tradeoff VeriCache Is Trying to Escape"), and KIVI is one of the quantising compressors
the uniform interface accepts, which exposes only bits-per-element ("VeriCache: Turning Lossy
KV Cache into Lossless LLM Inference", Key Contributions). Uniform bit width across the cache
is part of the stated scope (same page, Limitations). The pages give no KIVI parameters; the
workload recipe fixes: keys per channel over 32-token groups, values per token over
32-channel groups, 2- or 4-bit codes, a full-precision residual of the most recent tokens.

Readings taken where the pages are silent:
  * asymmetric min/max per group, codes = round-half-even((x - min) / scale) clamped to
    [0, 2^b - 1], scale = (max - min) / (2^b - 1), every step one IEEE float32 operation;
  * a constant group (scale 0) stores code 0 and reconstructs its value exactly;
  * with float16 metadata the stored min is rounded *down* and the scale *up* to float16, so
    the half-step error bound holds against the stored values;
  * dequantisation x_hat = code * scale + min, evaluated here in float64 (exact).

The packed code layout is the library's documented format (include/vc.h); this module
implements it from that description, independently of the library's code.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def f16_round_down(x32: np.ndarray) -> np.ndarray:
    """Largest float16 value <= x (x float32)."""
    x32 = np.asarray(x32, np.float32)
    h = x32.astype(np.float16)
    over = h.astype(np.float32) > x32
    with np.errstate(over="ignore"):
        h = np.where(over, np.nextafter(h, np.float16(-np.inf)), h)
    return h


def f16_round_up(x32: np.ndarray) -> np.ndarray:
    """Smallest float16 value >= x (x float32)."""
    x32 = np.asarray(x32, np.float32)
    h = x32.astype(np.float16)
    under = h.astype(np.float32) < x32
    with np.errstate(over="ignore"):
        h = np.where(under, np.nextafter(h, np.float16(np.inf)), h)
    return h


def quantize_groups(X: np.ndarray, bits: int, meta_dtype: str):
    """Quantise groups laid along the last axis of X (float32 values).

    Returns (codes uint8 same shape as X, scale float32 [...], min float32 [...]); scale and
    min are the *stored* values (float16-representable when meta_dtype == "f16").
    """
    X = np.asarray(X, np.float32)
    levels = np.float32(2 ** bits - 1)
    lo = X.min(axis=-1)
    hi = X.max(axis=-1)
    if meta_dtype == "f16":
        mn = f16_round_down(lo).astype(np.float32)
    elif meta_dtype == "f32":
        mn = lo.astype(np.float32)
    else:
        raise ValueError(meta_dtype)
    rng = (hi - mn).astype(np.float32)              # one float32 subtraction
    sc = (rng / levels).astype(np.float32)          # one float32 division
    if meta_dtype == "f16":
        sc = f16_round_up(sc).astype(np.float32)
    diff = (X - mn[..., None]).astype(np.float32)   # one float32 subtraction per element
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / sc[..., None]).astype(np.float32)  # one float32 division per element
    q = np.clip(np.rint(t), 0, levels)              # round half to even, then clamp
    q = np.where(sc[..., None] == 0, 0, q)
    return q.astype(np.uint8), sc, mn


def quantize_k(K: np.ndarray, bits: int, meta_dtype: str):
    """Keys [T, d] (T a multiple of 32): per channel, over 32-token groups.

    Returns codes [T, d], scale [T/32, d], min [T/32, d].
    """
    T, d = K.shape
    assert T % GROUP == 0
    Xg = K.reshape(T // GROUP, GROUP, d).transpose(0, 2, 1)       # [g, d, 32]
    q, sc, mn = quantize_groups(Xg, bits, meta_dtype)
    return q.transpose(0, 2, 1).reshape(T, d), sc, mn


def quantize_v(V: np.ndarray, bits: int, meta_dtype: str):
    """Values [T, d]: per token, over 32-channel groups.

    Returns codes [T, d], scale [T, d/32], min [T, d/32].
    """
    T, d = V.shape
    assert d % GROUP == 0
    q, sc, mn = quantize_groups(V.reshape(T, d // GROUP, GROUP), bits, meta_dtype)
    return q.reshape(T, d), sc, mn


def dequantize_k(codes: np.ndarray, sc: np.ndarray, mn: np.ndarray) -> np.ndarray:
    T, d = codes.shape
    c = codes.astype(np.float64).reshape(T // GROUP, GROUP, d)
    return (c * sc.astype(np.float64)[:, None, :] + mn.astype(np.float64)[:, None, :]).reshape(T, d)


def dequantize_v(codes: np.ndarray, sc: np.ndarray, mn: np.ndarray) -> np.ndarray:
    T, d = codes.shape
    c = codes.astype(np.float64).reshape(T, d // GROUP, GROUP)
    return (c * sc.astype(np.float64)[..., None] + mn.astype(np.float64)[..., None]).reshape(T, d)


# --------------------------------------------------------------------------------------------
# Packed layout (as documented in include/vc.h).
#
# Codes are stored per block of 32 tokens x 128 channels. A block is 64 "lanes" of 2*bits
# 32-bit words; word u of lane l sits at word index l*(2*bits) + u of the block. Each word holds
# two 16-bit halves hf in {0, 1}; half hf holds 16/bits slots s, slot s occupying bits
# [16*hf + bits*s, 16*hf + bits*s + bits). With i = l % 16, gq = l // 16:
#   keys,   2-bit: token = 16*(u//2) + i,  kb = 2*(u%2) + s//4, p = s%4
#   keys,   4-bit: token = 16*(u//4) + i,  kb = u%4,            p = s
#                  channel = 32*kb + 8*gq + 2*p + hf
#   values, 2-bit: tile = 2*u + s//4, p = s%4
#   values, 4-bit: tile = u,          p = s
#                  channel = 16*tile + i,  token = 16*(p//2) + 4*gq + 2*(p%2) + hf
# --------------------------------------------------------------------------------------------

def _slot_map(bits: int, kind: str):
    """For every (lane, word, half, slot): the (token, channel) it stores. Plain loops."""
    words = 2 * bits
    slots = 16 // bits
    tok = np.zeros((64, words, 2, slots), np.int64)
    ch = np.zeros_like(tok)
    for lane in range(64):
        i, gq = lane % 16, lane // 16
        for u in range(words):
            for hf in range(2):
                for s in range(slots):
                    if kind == "k":
                        if bits == 2:
                            t, kb, p = 16 * (u // 2) + i, 2 * (u % 2) + s // 4, s % 4
                        else:
                            t, kb, p = 16 * (u // 4) + i, u % 4, s
                        c = 32 * kb + 8 * gq + 2 * p + hf
                    else:
                        if bits == 2:
                            tile, p = 2 * u + s // 4, s % 4
                        else:
                            tile, p = u, s
                        c = 16 * tile + i
                        t = 16 * (p // 2) + 4 * gq + 2 * (p % 2) + hf
                    tok[lane, u, hf, s] = t
                    ch[lane, u, hf, s] = c
    return tok, ch


_MAPS: dict = {}


def _maps(bits: int, kind: str):
    key = (bits, kind)
    if key not in _MAPS:
        _MAPS[key] = _slot_map(bits, kind)
    return _MAPS[key]


def pack_codes(codes: np.ndarray, bits: int, kind: str) -> np.ndarray:
    """codes [T, 128] (T multiple of 32) -> packed bytes [T, 128*bits/8] in the block layout.

    Row t of the result is simply the t-th 128*bits/8-byte slice of the packed blocks (block
    g occupies rows 32g..32g+31), matching the library's [tok][row_bytes] buffer.
    """
    T, d = codes.shape
    assert d == 128 and T % GROUP == 0 and kind in ("k", "v")
    tok, ch = _maps(bits, kind)
    words = np.zeros((T // GROUP, 64, 2 * bits), np.uint32)
    slots = 16 // bits
    blocks = codes.reshape(T // GROUP, GROUP, d).astype(np.uint32)
    for hf in range(2):
        for s in range(slots):
            shift = np.uint32(16 * hf + bits * s)
            vals = blocks[:, tok[:, :, hf, s], ch[:, :, hf, s]]    # [g, 64, words]
            words |= vals << shift
    return words.reshape(-1).view(np.uint8).reshape(T, d * bits // 8)


def unpack_codes(packed: np.ndarray, bits: int, kind: str) -> np.ndarray:
    """Inverse of pack_codes: packed [T, 128*bits/8] -> codes [T, 128] uint8."""
    T = packed.shape[0]
    tok, ch = _maps(bits, kind)
    words = np.ascontiguousarray(packed).reshape(-1).view(np.uint32).reshape(T // GROUP, 64, 2 * bits)
    out = np.zeros((T // GROUP, GROUP, 128), np.uint8)
    mask = np.uint32(2 ** bits - 1)
    slots = 16 // bits
    for hf in range(2):
        for s in range(slots):
            shift = np.uint32(16 * hf + bits * s)
            out[:, tok[:, :, hf, s], ch[:, :, hf, s]] = ((words >> shift) & mask).astype(np.uint8)
    return out.reshape(T, 128)


def quantised_prefix(n: int, R: int, group: int = GROUP) -> int:
    """Tokens held as codes once n tokens are cached with a full-precision residual of R tokens.

    The pages give no residual rule; the workload recipe keeps the most recent tokens in full
    precision (the last 32 in fp32 for the fp32 layer, a 128-token fp16 residual for the bf16
    layers). Reading taken: quantise the longest prefix of whole `group`-token groups that leaves
    at least R tokens unquantised, i.e. group * floor(max(0, n - R) / group); nothing is quantised
    while n <= R.
    """
    if n < 0 or R < 0 or group <= 0:
        raise ValueError((n, R, group))
    spare = n - R
    if spare <= 0:
        return 0
    return group * (spare // group)


class KiviLayer:
    """Oracle KIVI cache of one (batch, kv-head) slice after prefill.

    Tokens 0..n_q-1 are quantised; tokens n_q.. live in the residual at the residual dtype.
    """

    def __init__(self, K: np.ndarray, V: np.ndarray, n_q: int, bits: int, meta_dtype: str,
                 res_dtype: str):
        self.bits, self.meta_dtype, self.res_dtype, self.n_q = bits, meta_dtype, res_dtype, n_q
        self.d = K.shape[1]
        K32 = np.asarray(K, np.float32)
        V32 = np.asarray(V, np.float32)
        self.kc, self.ks, self.km = quantize_k(K32[:n_q], bits, meta_dtype)
        self.vc, self.vs, self.vm = quantize_v(V32[:n_q], bits, meta_dtype)
        self.res_k = [to_res(r, res_dtype) for r in K32[n_q:]]
        self.res_v = [to_res(r, res_dtype) for r in V32[n_q:]]

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        """Append one position's key/value to the residual (stored at the residual dtype)."""
        self.res_k.append(to_res(np.asarray(k, np.float32), self.res_dtype))
        self.res_v.append(to_res(np.asarray(v, np.float32), self.res_dtype))

    def keys(self, r: int) -> np.ndarray:
        """Dequantised keys 0..n_q-1 followed by the first r residual keys, float64."""
        parts = [dequantize_k(self.kc, self.ks, self.km)] if self.n_q else []
        parts.append(np.array(self.res_k[:r], np.float64).reshape(r, self.d))
        return np.concatenate(parts, axis=0)

    def values(self, r: int) -> np.ndarray:
        parts = [dequantize_v(self.vc, self.vs, self.vm)] if self.n_q else []
        parts.append(np.array(self.res_v[:r], np.float64).reshape(r, self.d))
        return np.concatenate(parts, axis=0)


def to_res(x32: np.ndarray, res_dtype: str) -> np.ndarray:
    """Residual storage rounding: float32 kept as is, float16 by round-half-even."""
    if res_dtype == "f32":
        return np.asarray(x32, np.float32).astype(np.float64)
    if res_dtype == "f16":
        return np.asarray(x32, np.float32).astype(np.float16).astype(np.float64)
    raise ValueError(res_dtype)
