"""Thin ctypes binding of libvc (include/vc.h): the same entry points, argument marshalling only.

Every step of the draft/verify path runs in libvc's HIP kernels. This module only turns torch
tensors into pointers, sizes and dtype codes, passes the current HIP stream, and raises on a
non-OK status. It never computes anything itself and has no fallback: if libvc.so is missing it
raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("VC_LIB") or os.path.join(PKG, "libvc.so")  # VC_LIB: another build
HEADER = os.path.join(os.path.dirname(PKG), "include", "vc.h")

VC_OK, VC_ERR_INVALID, VC_ERR_UNSUPPORTED, VC_ERR_WORKSPACE, VC_ERR_HIP = 0, 1, 2, 3, 4
VC_F32, VC_F16, VC_BF16 = 0, 1, 2
VC_PAST_DEVICE, VC_PAST_HOST, VC_PAST_HOST_PREFETCHED = 0, 1, 2
VC_OP_DRAFT_QUANT, VC_OP_DRAFT_DROP, VC_OP_VERIFY, VC_OP_PROJECT, VC_OP_DECODER, VC_OP_PREFILL = 1, 2, 3, 4, 5, 6
VC_DEC_STORE, VC_DEC_ADD, VC_DEC_ROPE, VC_DEC_SWIGLU = 0, 1, 2, 3
_TORCH_DT = {torch.float32: VC_F32, torch.float16: VC_F16, torch.bfloat16: VC_BF16}

_lib = None


class VcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class vc_kivi(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("meta_dtype", ctypes.c_int32),
        ("res_dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("res_cap", ctypes.c_int32), ("tok_cap", ctypes.c_int64),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p), ("k_meta", ctypes.c_void_p),
        ("v_meta", ctypes.c_void_p), ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
    ]


_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_KP = ctypes.POINTER(vc_kivi)
_SIGS = {
    "vc_quantize_kv": [_KP, _P, _P, _I32, _I64, _I64, _I64, _P],
    "vc_kivi_append": [_KP, _P, _P, _I32, _I64, _I64, _I64, _P],
    "vc_draft_attn_quant": [_KP, _I64, _I32, _P, _P, _I32, _I64, _P, _I32, _I32, _F, _P, _P, _P, _SZ, _P],
    "vc_draft_quant_workspace": [_KP, _I64, _I32, _I32, ctypes.POINTER(_SZ)],
    "vc_draft_attn_quant_rows": [_KP, _P, _P, _I32, _I64, _I32, _P, _P, _I32, _I64, _I64, _P, _I32, _I32,
                                 _F, _P, _P, _P, _SZ, _P],
    "vc_draft_attn_quant_noalloc": [_KP, _I64, _I32, _P, _P, _I32, _I64, _P, _I32, _I32, _F, _P, _P, _P],
    "vc_draft_attn_drop": [_P, _P, _I32, _I32, _I32, _I64, _P, _I64, _I64, _P, _I32, _F, _P, _P, _P,
                           _SZ, _P],
    "vc_draft_drop_workspace": [_I32, _I32, _I32, _I64, ctypes.POINTER(_SZ)],
    "vc_verify_attn": [_P, _P, _P, _I32, _P, _P, _I64, _I64, _I32, _I64, _I32, _I32, _I32, _I32, _F,
                       _P, _P, _P, _SZ, _P, _P],
    "vc_verify_workspace": [_I32, _I32, _I32, _I32, _I64, _I32, _I64, _I32, ctypes.POINTER(_SZ)],
    "vc_verify_prefetch": [_P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P, _P],
    "vc_lse_merge": [_P, _P, _I64, _I32, _I32, _P, _P, _P],
    "vc_accept": [_P, _P, _I32, _I32, _I32, _P, _P, _P, _P],
    "vc_logit_margins": [_P, _I64, _I32, _P, _P],
    "vc_hbm_read_stream": [_P, _SZ, _P, _I32, _P],
    "vc_project_workspace": [_I32, _I32, _I32, ctypes.POINTER(_SZ)],
    "vc_project_logits": [_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _P, _I64, _P, _SZ, _P],
    "vc_select_keep": [_P, _I64, _I32, _I64, _I64, _I64, _I64, _P, _I64, ctypes.POINTER(_I64), _P],
    "vc_verify_stream_copies": [_P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P, _SZ, _P],
    "vc_workspace_bytes": [_I32, ctypes.POINTER(_I64), _I32, ctypes.POINTER(_SZ)],
    "vc_decoder_gemv": [_I32, _P, _I32, _I32, _I32, _P, _I32, _P, _F, _P, _P, _P, _P, _I32, _I32, _I32,
                        _P, _P, _I32, _P, _I32, _P, _SZ, _P],
    "vc_decoder_gemv_workspace": [_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
    "vc_prefill_attn": [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _P],
    "vc_prefill_workspace": [_I32, _I32, _I32, _I64, ctypes.POINTER(_SZ)],
    "vc_rmsnorm": [_P, _P, _F, _I32, _I32, _P, _P],
    "vc_embed_rows": [_P, _I32, _I32, _P, _I64, _I32, _P, _P],
    "vc_status_string": [_I32],
    "vc_last_error": [],
    "vc_abi_version": [],
}


def lib():
    """Load libvc.so (built in-tree by kv_cache_compressed_amd.build); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_compressed_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        l.vc_status_string.restype = ctypes.c_char_p
        l.vc_last_error.restype = ctypes.c_char_p
        _lib = l
    return _lib


def header_symbols() -> list[str]:
    """Names of every function include/vc.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:vc_status|const char \*|int32_t)\s*(vc_\w+)\s*\(", text, re.M)))


def _check(st: int):
    if st != VC_OK:
        l = lib()
        raise VcError(st, f"{l.vc_status_string(st).decode()}: {l.vc_last_error().decode()}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def dtype_code(t: torch.Tensor) -> int:
    return _TORCH_DT[t.dtype]


# ------------------------------------------------------------------------------------------
# KIVI cache storage (device tensors) and its C descriptor
# ------------------------------------------------------------------------------------------
class KiviCache:
    """Device buffers of one layer's KIVI cache, laid out as include/vc.h describes."""

    def __init__(self, B, Hkv, tok_cap, bits, meta_dtype, res_dtype, res_cap, device="cuda", d=128):
        assert tok_cap % 32 == 0 and res_cap % 32 == 0 and d == 128
        self.B, self.Hkv, self.tok_cap, self.bits, self.res_cap, self.d = B, Hkv, tok_cap, bits, res_cap, d
        self.meta_dtype, self.res_dtype = meta_dtype, res_dtype
        row = d * bits // 8
        mdt = torch.float16 if meta_dtype == VC_F16 else torch.float32
        rdt = torch.float16 if res_dtype == VC_F16 else torch.float32
        cap = max(tok_cap, 32)
        self.k_codes = torch.zeros(B, Hkv, cap, row, dtype=torch.uint8, device=device)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_meta = torch.zeros(B, Hkv, cap // 32, 2, d, dtype=mdt, device=device)  # scales, mins
        self.v_meta = torch.zeros(B, Hkv, cap, d // 32, 2, dtype=mdt, device=device)
        self.k_res = torch.zeros(B, Hkv, res_cap, d, dtype=rdt, device=device)
        self.v_res = torch.zeros_like(self.k_res)

    _BUFFERS = ("k_codes", "v_codes", "k_meta", "v_meta", "k_res", "v_res")

    def __setattr__(self, name, value):
        if name in self._BUFFERS:  # a replaced buffer invalidates the cached descriptor
            object.__setattr__(self, "_desc", None)
        object.__setattr__(self, name, value)

    def row(self, b: int) -> "KiviCache":
        """Batch row b as a one-row cache over this cache's storage (a request's own appends,
        flushes and quantisation in a batched cache)."""
        v = object.__new__(KiviCache)
        for name in ("Hkv", "tok_cap", "bits", "res_cap", "d", "meta_dtype", "res_dtype"):
            object.__setattr__(v, name, getattr(self, name))
        object.__setattr__(v, "B", 1)
        for name in self._BUFFERS:
            setattr(v, name, getattr(self, name)[b:b + 1])
        return v

    def desc(self) -> vc_kivi:
        """The C descriptor, built on first use and rebuilt after a buffer is replaced."""
        if getattr(self, "_desc", None) is None:
            self._desc = vc_kivi(self.bits, 32, self.meta_dtype, self.res_dtype, self.B, self.Hkv,
                                 self.d, self.res_cap, self.tok_cap, _ptr(self.k_codes),
                                 _ptr(self.v_codes), _ptr(self.k_meta), _ptr(self.v_meta),
                                 _ptr(self.k_res), _ptr(self.v_res))
        return self._desc


class Workspace:
    """A reusable device workspace, grown on demand."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=self.device)
        return self.buf


# ------------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ------------------------------------------------------------------------------------------
def vc_quantize_kv(cache: KiviCache, k, v, t0: int, ntok: int, src_bh_stride: int | None = None,
                   stream=None):
    """k, v: device tensors whose (b, h) slices start src_bh_stride elements apart (default: a
    contiguous [B, Hkv, ntok, 128] tensor)."""
    stride = k.stride(1) if src_bh_stride is None else src_bh_stride
    d = cache.desc()
    _check(lib().vc_quantize_kv(ctypes.byref(d), _ptr(k), _ptr(v), dtype_code(k), stride, t0, ntok,
                                _stream(stream)))


def vc_kivi_append(cache: KiviCache, k, v, t0: int, ntok: int, src_bh_stride: int | None = None,
                   stream=None):
    stride = k.stride(1) if src_bh_stride is None else src_bh_stride
    d = cache.desc()
    _check(lib().vc_kivi_append(ctypes.byref(d), _ptr(k), _ptr(v), dtype_code(k), stride, t0, ntok,
                                _stream(stream)))


def vc_draft_quant_workspace(cache: KiviCache, n_q: int, r: int, Hq: int) -> int:
    n = _SZ(0)
    d = cache.desc()
    _check(lib().vc_draft_quant_workspace(ctypes.byref(d), n_q, r, Hq, ctypes.byref(n)))
    return n.value


def vc_draft_attn_quant(cache: KiviCache, n_q: int, r: int, q, out, lse, ws: torch.Tensor,
                        sm_scale: float, stream=None, k_new=None, v_new=None):
    """k_new, v_new: None, or the step's own key/value [B, Hkv, 128] (any (b, kv head) row stride,
    channels contiguous), stored as residual token n_q + r - 1 before attending."""
    d = cache.desc()
    stride, ndt = 0, 0
    if k_new is not None:
        assert k_new.shape == v_new.shape and k_new.stride() == v_new.stride() and k_new.dim() == 3
        assert k_new.stride(2) == 1 and (k_new.shape[0] == 1 or
                                         k_new.stride(0) == k_new.shape[1] * k_new.stride(1))
        stride, ndt = k_new.stride(1), dtype_code(k_new)
    _check(lib().vc_draft_attn_quant(ctypes.byref(d), n_q, r, _ptr(k_new), _ptr(v_new), ndt, stride,
                                     _ptr(q), dtype_code(q), q.shape[1], sm_scale, _ptr(out), _ptr(lse),
                                     _ptr(ws), ws.numel(), _stream(stream)))


def vc_draft_attn_quant_rows(cache: KiviCache, n_q, r, r_add: int, n_q_max: int, r_max: int, q, out, lse,
                             ws: torch.Tensor, sm_scale: float, stream=None, k_new=None, v_new=None):
    """vc_draft_attn_quant with per-batch-row lengths: n_q (int64) and r (int32) device tensors of B
    entries, row b's residual count r[b] + r_add; n_q_max, r_max host bounds. k_new/v_new
    [B, Hkv, 128] views with any batch-row stride (channels contiguous)."""
    d = cache.desc()
    assert n_q.dtype == torch.int64 and r.dtype == torch.int32 and n_q.numel() == r.numel() == cache.B
    bs, hs, ndt = 0, 0, 0
    if k_new is not None:
        assert k_new.shape == v_new.shape and k_new.stride() == v_new.stride() and k_new.dim() == 3
        assert k_new.stride(2) == 1
        bs, hs, ndt = k_new.stride(0), k_new.stride(1), dtype_code(k_new)
    _check(lib().vc_draft_attn_quant_rows(ctypes.byref(d), _ptr(n_q), _ptr(r), r_add, n_q_max, r_max,
                                          _ptr(k_new), _ptr(v_new), ndt, bs, hs, _ptr(q), dtype_code(q),
                                          q.shape[1], sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                          _stream(stream)))


def vc_draft_attn_quant_noalloc(cache: KiviCache, n_q: int, r: int, q, out, lse, sm_scale: float,
                                stream=None, k_new=None, v_new=None):
    """vc_draft_attn_quant without a workspace (the library's per-device scratch; nothing allocated)."""
    d = cache.desc()
    stride, ndt = 0, 0
    if k_new is not None:
        assert k_new.shape == v_new.shape and k_new.stride() == v_new.stride() and k_new.dim() == 3
        assert k_new.stride(2) == 1 and (k_new.shape[0] == 1 or
                                         k_new.stride(0) == k_new.shape[1] * k_new.stride(1))
        stride, ndt = k_new.stride(1), dtype_code(k_new)
    _check(lib().vc_draft_attn_quant_noalloc(ctypes.byref(d), n_q, r, _ptr(k_new), _ptr(v_new), ndt, stride,
                                             _ptr(q), dtype_code(q), q.shape[1], sm_scale, _ptr(out),
                                             _ptr(lse), _stream(stream)))


def vc_draft_drop_workspace(B: int, Hkv: int, Hq: int, n_keep: int) -> int:
    n = _SZ(0)
    _check(lib().vc_draft_drop_workspace(B, Hkv, Hq, n_keep, ctypes.byref(n)))
    return n.value


def vc_draft_attn_drop(k, v, idx, n_keep: int, q, out, lse, ws: torch.Tensor, sm_scale: float,
                       stream=None):
    """k, v: [B, Hkv, tok_cap, 128]; idx: int32 [B, Hkv, idx_cap]; q: [B, Hq, 128]."""
    B, Hkv, tok_cap, _ = k.shape
    _check(lib().vc_draft_attn_drop(_ptr(k), _ptr(v), dtype_code(k), B, Hkv, tok_cap, _ptr(idx),
                                    n_keep, idx.shape[2], _ptr(q), q.shape[1], sm_scale, _ptr(out),
                                    _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def vc_verify_workspace(B, Hq, Hkv, L, n, past_on_host, chunk_tokens, dtype) -> int:
    nb = _SZ(0)
    _check(lib().vc_verify_workspace(B, Hq, Hkv, L, n, int(past_on_host), chunk_tokens, dtype,
                                     ctypes.byref(nb)))
    return nb.value


def vc_prefill_workspace(B: int, Hq: int, Hkv: int, n: int) -> int:
    b = _SZ(0)
    _check(lib().vc_prefill_workspace(B, Hq, Hkv, n, ctypes.byref(b)))
    return b.value


def vc_prefill_attn(q, k, v, n: int, out, lse, ws: torch.Tensor, sm_scale: float, kv_stride: int | None = None,
                    stream=None):
    """q [B, Hq, n, 128] bf16; k, v [B, Hkv, >= n, 128] bf16 (kv_stride = their token dimension);
    out [B, Hq, n, 128] fp32; lse [B, Hq, n] or None. Causal self-attention of the n rows."""
    B, Hq = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    stride = k.shape[2] if kv_stride is None else kv_stride
    _check(lib().vc_prefill_attn(_ptr(q), _ptr(k), _ptr(v), stride, n, B, Hq, Hkv, sm_scale, _ptr(out),
                                 _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def vc_verify_prefetch(k_past, v_past, n: int, ws: torch.Tensor, B: int, Hq: int, Hkv: int, L: int,
                       chunk_tokens: int, past_stride: int | None = None, stream=None, copy_stream=None):
    """Issue the first two streamed chunks' copies of a later vc_verify_attn(...,
    past_on_host=VC_PAST_HOST_PREFETCHED) with the same past, sizes and workspace."""
    stride = k_past.shape[2] if past_stride is None else past_stride
    comp = _stream(stream)
    cp = _stream(copy_stream) if copy_stream is not None else comp
    _check(lib().vc_verify_prefetch(_ptr(k_past), _ptr(v_past), stride, n, chunk_tokens, B, Hq, Hkv, L,
                                    _ptr(ws), ws.numel() * ws.element_size(), comp, cp))


def vc_verify_attn(q, k_blk, v_blk, k_past, v_past, n: int, out, lse, ws: torch.Tensor,
                   sm_scale: float, past_stride: int | None = None, past_on_host: int = VC_PAST_DEVICE,
                   chunk_tokens: int = 0, stream=None, copy_stream=None):
    """q [B, Hq, L, 128]; k_blk/v_blk [B, Hkv, L, 128]; k_past/v_past [B, Hkv, >=n, 128].
    past_on_host: VC_PAST_DEVICE (or False), VC_PAST_HOST (or True), VC_PAST_HOST_PREFETCHED."""
    B, Hq, L, _ = q.shape
    Hkv = k_blk.shape[1]
    stride = k_past.shape[2] if past_stride is None else past_stride
    comp = _stream(stream)
    cp = _stream(copy_stream) if copy_stream is not None else comp
    _check(lib().vc_verify_attn(_ptr(q), _ptr(k_blk), _ptr(v_blk), L, _ptr(k_past), _ptr(v_past),
                                stride, n, int(past_on_host), chunk_tokens, dtype_code(q), B, Hq, Hkv,
                                sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), comp, cp))


def vc_verify_stream_copies(k_past, v_past, n: int, ws: torch.Tensor, B: int, Hq: int, Hkv: int,
                            L: int, chunk_tokens: int, past_stride: int | None = None, copy_stream=None):
    """Only the chunk copies a host-streamed vc_verify_attn with these arguments issues (no compute)."""
    stride = k_past.shape[2] if past_stride is None else past_stride
    _check(lib().vc_verify_stream_copies(_ptr(k_past), _ptr(v_past), stride, n, chunk_tokens, B, Hq, Hkv,
                                         L, _ptr(ws), ws.numel() * ws.element_size(), _stream(copy_stream)))


def vc_workspace_bytes(op: int, dims) -> int:
    """Workspace bytes of operation `op` (VC_OP_*) for its size arguments `dims`."""
    arr = (_I64 * max(1, len(dims)))(*dims)
    n = _SZ(0)
    _check(lib().vc_workspace_bytes(op, arr, len(dims), ctypes.byref(n)))
    return n.value


def vc_lse_merge(part_o, part_ml, out, lse, stream=None):
    """part_o [rows, S, 128], part_ml [rows, S, 2] -> out [rows, 128], lse [rows]."""
    rows, S, d = part_o.shape
    _check(lib().vc_lse_merge(_ptr(part_o), _ptr(part_ml), rows, S, d, _ptr(out), _ptr(lse),
                              _stream(stream)))


def vc_accept(logits, drafts, accept_len, next_token, argmax=None, stream=None):
    """logits [B, L, V] fp32; drafts [B, L-1] int32 (or None when L == 1)."""
    B, L, V = logits.shape
    _check(lib().vc_accept(_ptr(logits), _ptr(drafts), B, L, V, _ptr(accept_len), _ptr(next_token),
                           _ptr(argmax), _stream(stream)))


def vc_logit_margins(logits, gap, stream=None):
    """gap[r] = best - second best of logits row r (logits [..., V] fp32 contiguous; gap has one
    entry per row)."""
    V = logits.shape[-1]
    rows = logits.numel() // V
    assert logits.is_contiguous() and gap.numel() == rows and gap.dtype == torch.float32
    _check(lib().vc_logit_margins(_ptr(logits), rows, V, _ptr(gap), _stream(stream)))


def vc_hbm_read_stream(src, sink, blocks: int, stream=None):
    """Read all of `src` (device tensor, bytes a multiple of 16) once; sink: int32 device tensor of
    blocks * 256 entries."""
    nbytes = src.numel() * src.element_size()
    assert sink.numel() >= blocks * 256
    _check(lib().vc_hbm_read_stream(_ptr(src), nbytes, _ptr(sink), blocks, _stream(stream)))


def vc_project_workspace(B: int, L: int, V: int) -> int:
    n = _SZ()
    _check(lib().vc_project_workspace(B, L, V, ctypes.byref(n)))
    return n.value


def vc_project_logits(W, o, logits=None, argmax=None, argmax_b_stride: int | None = None,
                      ws: torch.Tensor | None = None, stream=None):
    """W [V, Hq*128] fp32 or bf16; o [B, Hq, L, 128] (or [B, Hq, 128] for L == 1) fp32 -> logits
    [B, L, V] and/or argmax (row (b, i) at argmax.flat[b * argmax_b_stride + i]; default stride L)."""
    V = W.shape[0]
    B, Hq = o.shape[0], o.shape[1]
    L = o.shape[2] if o.dim() == 4 else 1
    if argmax_b_stride is None:
        argmax_b_stride = L
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().vc_project_logits(_ptr(W), dtype_code(W), V, _ptr(o), B, Hq, L, _ptr(logits), _ptr(argmax),
                                   argmax_b_stride, _ptr(ws), nb, _stream(stream)))


def vc_select_keep(scores, n: int, sinks: int, recent: int, keep: int, idx, stream=None) -> int:
    """Kept positions of every row of `scores` (fp32 [..., stride] on the device, rows = all
    leading dims, row stride = the last dim) into `idx` (int32 [..., idx_stride]); returns the
    kept count per row."""
    assert scores.dtype == torch.float32 and idx.dtype == torch.int32
    assert scores.stride(-1) == 1 and idx.stride(-1) == 1
    rows = scores.numel() // scores.shape[-1]
    assert idx.numel() // idx.shape[-1] == rows
    out = ctypes.c_int64(0)
    _check(lib().vc_select_keep(_ptr(scores), scores.shape[-1] if scores.dim() == 1 else scores.stride(-2),
                                rows, n, sinks, recent, keep, _ptr(idx),
                                idx.shape[-1] if idx.dim() == 1 else idx.stride(-2), ctypes.byref(out),
                                _stream(stream)))
    return int(out.value)



def vc_decoder_gemv(epilogue: int, W, X, out=None, norm_gain=None, eps: float = 1e-5, q_out=None,
                    k_out=None, v_out=None, Hq: int = 0, Hkv: int = 0, cos_t=None, sin_t=None,
                    pos=None, pos_add: int = 0, ws=None, stream=None):
    """W [N, K] fp32/bf16; X [M, K] fp32 (contiguous rows); see include/vc.h for the epilogues.
    ws: None (vector form) or a zero-filled uint8 device buffer of vc_decoder_gemv_workspace()
    bytes (matrix-core form where it applies)."""
    N, K = W.shape
    M = X.shape[0]
    assert X.is_contiguous() and X.shape[1] == K and W.is_contiguous()
    odt = dtype_code(q_out) if q_out is not None else VC_F32
    n_pos = cos_t.shape[0] if cos_t is not None else 0
    _check(lib().vc_decoder_gemv(epilogue, _ptr(W), dtype_code(W), N, K, _ptr(X), M, _ptr(norm_gain), eps,
                                 _ptr(out), _ptr(q_out), _ptr(k_out), _ptr(v_out), odt, Hq, Hkv,
                                 _ptr(cos_t), _ptr(sin_t), n_pos, _ptr(pos), pos_add, _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def vc_decoder_gemv_workspace(epilogue: int, w_dtype: int, N: int, K: int, M: int) -> int:
    """Bytes of the matrix-core form's workspace (0 where it does not apply)."""
    n = _SZ(0)
    _check(lib().vc_decoder_gemv_workspace(epilogue, w_dtype, N, K, M, ctypes.byref(n)))
    return n.value


def vc_rmsnorm(X, g, Y, eps: float = 1e-5, stream=None):
    """Y[m] = X[m] * g / sqrt(mean(X[m]^2) + eps); X, Y [M, K] fp32."""
    M, K = X.shape
    _check(lib().vc_rmsnorm(_ptr(X), _ptr(g), eps, M, K, _ptr(Y), _stream(stream)))


def vc_embed_rows(E, tok, out, stream=None):
    """out[m] = E[tok[m]] for a 1-D int32 device view `tok` (any stride); E [V, K] fp32."""
    V, K = E.shape
    assert tok.dim() == 1 and tok.dtype == torch.int32 and out.shape == (tok.shape[0], K)
    _check(lib().vc_embed_rows(_ptr(E), V, K, _ptr(tok), tok.stride(0), tok.shape[0], _ptr(out),
                               _stream(stream)))
