"""C-ABI checks that need no GPU: libvc.so loads, exports every function include/vc.h declares,
and rejects invalid arguments on the host with the documented status (nothing is enqueued: these
calls never reach a HIP launch). Pointers are fake but 16-byte aligned; validation never
dereferences them.
"""
import ctypes

import pytest

from kv_cache_compressed_amd import vc

P = 0x10000  # a fake, aligned "device" pointer
BAD = 0x10004  # misaligned


@pytest.fixture(scope="module")
def L():
    return vc.lib()


def test_every_header_symbol_is_exported(L):
    names = vc.header_symbols()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(vc._SIGS) == set(names)


def test_version_and_strings(L):
    assert L.vc_abi_version() == 1
    assert L.vc_status_string(0) == b"VC_OK"
    assert L.vc_status_string(4) == b"VC_ERR_HIP"
    assert L.vc_status_string(99) == b"VC_ERR_UNKNOWN"


def _kivi(**kw):
    d = dict(bits=2, group=32, meta_dtype=vc.VC_F16, res_dtype=vc.VC_F16, B=2, Hkv=2, d=128,
             res_cap=256, tok_cap=1024, k_codes=P, v_codes=P, k_meta=P, v_meta=P, k_res=P, v_res=P)
    d.update(kw)
    return vc.vc_kivi(*[d[f] for f, _ in vc.vc_kivi._fields_])


def _err(L):
    return L.vc_last_error().decode()


@pytest.mark.parametrize("field,val,msg", [
    ("bits", 3, "bits"), ("bits", 8, "bits"), ("group", 64, "group"), ("d", 64, "head dim"),
    ("meta_dtype", vc.VC_BF16, "meta_dtype"), ("res_dtype", 7, "res_dtype"), ("res_cap", 40, "res_cap"),
    ("tok_cap", 33, "tok_cap"), ("k_codes", 0, "k_codes"), ("v_meta", BAD, "aligned"), ("B", 0, "B"),
])
def test_quantize_rejects_bad_descriptor(L, field, val, msg):
    k = _kivi(**{field: val})
    st = L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 1024 * 128, 0, 64, None)
    assert st == vc.VC_ERR_INVALID and msg in _err(L)


def test_quantize_rejects_bad_ranges(L):
    k = _kivi()
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 1 << 20, 16, 32, None) == vc.VC_ERR_INVALID
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 1 << 20, 0, 48, None) == vc.VC_ERR_INVALID
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 1 << 20, 992, 64, None) == vc.VC_ERR_INVALID
    assert "tok_cap" in _err(L)
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 100, 0, 64, None) == vc.VC_ERR_INVALID
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, 9, 1 << 20, 0, 64, None) == vc.VC_ERR_INVALID
    assert L.vc_quantize_kv(None, P, P, vc.VC_BF16, 1 << 20, 0, 64, None) == vc.VC_ERR_INVALID
    # ntok == 0 is a valid no-op that enqueues nothing
    assert L.vc_quantize_kv(ctypes.byref(k), P, P, vc.VC_BF16, 1 << 20, 0, 0, None) == vc.VC_OK


def test_append_rejects(L):
    k = _kivi()
    assert L.vc_kivi_append(ctypes.byref(k), P, P, vc.VC_BF16, 128, 0, 0, None) == vc.VC_ERR_INVALID
    assert L.vc_kivi_append(ctypes.byref(k), P, P, vc.VC_BF16, 1 << 20, 0, 257, None) == vc.VC_ERR_INVALID
    assert L.vc_kivi_append(ctypes.byref(k), P, BAD, vc.VC_BF16, 1 << 20, 0, 1, None) == vc.VC_ERR_INVALID


def test_draft_quant_rejects(L):
    k = _kivi()
    call = lambda **a: L.vc_draft_attn_quant(
        ctypes.byref(a.get("kivi", k)), a.get("n_q", 512), a.get("r", 100), a.get("k_new", None),
        a.get("v_new", None), a.get("new_dtype", vc.VC_BF16), a.get("new_stride", 128), a.get("q", P),
        vc.VC_BF16, a.get("Hq", 8), 0.088, a.get("out", P), None, a.get("ws", P), a.get("ws_bytes", 1 << 30),
        None)
    assert call(n_q=500) == vc.VC_ERR_INVALID
    assert call(n_q=2048) == vc.VC_ERR_INVALID
    assert call(r=300) == vc.VC_ERR_INVALID
    assert call(n_q=0, r=0) == vc.VC_ERR_INVALID and "no keys" in _err(L)
    assert call(Hq=7) == vc.VC_ERR_INVALID
    assert call(q=0) == vc.VC_ERR_INVALID
    assert call(out=BAD) == vc.VC_ERR_INVALID
    assert call(Hq=2 * 9) == vc.VC_ERR_UNSUPPORTED
    assert call(kivi=_kivi(res_cap=1024)) == vc.VC_ERR_UNSUPPORTED
    assert call(k_new=P) == vc.VC_ERR_INVALID                      # v_new missing
    assert call(k_new=P, v_new=P, r=0) == vc.VC_ERR_INVALID         # the step's token is n_q + r - 1
    assert call(k_new=P, v_new=P, new_dtype=7) == vc.VC_ERR_INVALID
    assert call(k_new=P, v_new=P, new_stride=64) == vc.VC_ERR_INVALID
    assert call(ws=0) == vc.VC_ERR_WORKSPACE
    assert call(ws_bytes=100) == vc.VC_ERR_WORKSPACE
    n = ctypes.c_size_t(0)
    assert L.vc_draft_quant_workspace(ctypes.byref(k), 512, 100, 8, ctypes.byref(n)) == vc.VC_OK
    assert n.value > 4096
    assert call(ws_bytes=n.value - 1) == vc.VC_ERR_WORKSPACE


def test_draft_drop_rejects(L):
    call = lambda **a: L.vc_draft_attn_drop(
        P, P, a.get("dt", vc.VC_BF16), 2, 2, 5000, a.get("idx", P), a.get("n_keep", 100),
        a.get("idx_cap", 200), P, a.get("Hq", 8), 0.088, P, None, a.get("ws", P), a.get("ws_bytes", 1 << 30), None)
    assert call(idx=0) == vc.VC_ERR_INVALID
    assert call(n_keep=0) == vc.VC_ERR_INVALID
    assert call(n_keep=300) == vc.VC_ERR_INVALID
    assert call(Hq=5) == vc.VC_ERR_INVALID
    assert call(dt=vc.VC_F32) == vc.VC_ERR_UNSUPPORTED
    assert call(ws_bytes=10) == vc.VC_ERR_WORKSPACE


def test_verify_rejects(L):
    call = lambda **a: L.vc_verify_attn(
        P, P, P, a.get("L", 31), a.get("kp", P), P, a.get("stride", 4096), a.get("n", 4000),
        a.get("host", 0), a.get("chunk", 0), a.get("dt", vc.VC_BF16), 2, a.get("Hq", 8), 2, 0.088, P,
        None, P, a.get("ws_bytes", 1 << 34), None, None)
    assert call(L=0) == vc.VC_ERR_INVALID
    assert call(L=33) == vc.VC_ERR_INVALID and "L must be" in _err(L)
    assert call(stride=100) == vc.VC_ERR_INVALID
    assert call(kp=0) == vc.VC_ERR_INVALID
    assert call(dt=vc.VC_F16) == vc.VC_ERR_INVALID
    assert call(Hq=5) == vc.VC_ERR_INVALID
    assert call(Hq=18) == vc.VC_ERR_UNSUPPORTED
    assert call(dt=vc.VC_F32, host=1, chunk=1024) == vc.VC_ERR_UNSUPPORTED
    assert call(host=1, chunk=16) == vc.VC_ERR_INVALID
    assert call(ws_bytes=64) == vc.VC_ERR_WORKSPACE
    # one bf16 source per (b, kv head) is limited to 8388607 tokens (256 B each, 32-bit buffer range)
    assert call(n=8388608, stride=8388608) == vc.VC_ERR_UNSUPPORTED and "resident" in _err(L)
    assert call(n=8388608, stride=8388608, host=1, chunk=8388608) == vc.VC_ERR_UNSUPPORTED
    assert call(host=3, chunk=1024) == vc.VC_ERR_INVALID and "past_on_host must be" in _err(L)


def test_verify_prefetch_rejects(L):
    """Argument checks of the prefetch (all before any HIP call)."""
    call = lambda **a: L.vc_verify_prefetch(
        a.get("kp", P), P, a.get("stride", 4096), a.get("n", 4000), a.get("chunk", 1024), 2,
        a.get("Hq", 8), 2, a.get("L", 31), P, 1 << 34, None, None)
    assert call(L=0) == vc.VC_ERR_INVALID
    assert call(L=33) == vc.VC_ERR_INVALID and "L must be" in _err(L)
    assert call(n=0) == vc.VC_ERR_INVALID and "n >= 1" in _err(L)
    assert call(stride=100) == vc.VC_ERR_INVALID
    assert call(kp=0) == vc.VC_ERR_INVALID
    assert call(chunk=16) == vc.VC_ERR_INVALID
    assert call(Hq=5) == vc.VC_ERR_INVALID
    assert call(Hq=18) == vc.VC_ERR_UNSUPPORTED
    assert call(n=8388608, stride=8388608, chunk=8388608) == vc.VC_ERR_UNSUPPORTED


def test_merge_and_accept_reject(L):
    assert L.vc_lse_merge(P, P, 10, 0, 128, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_lse_merge(P, P, 10, 5000, 128, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_lse_merge(P, P, 10, 4, 64, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_lse_merge(P, BAD, 10, 4, 128, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_accept(P, P, 1, 65, 10, P, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_accept(P, None, 1, 9, 10, P, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_accept(P, P, 0, 9, 10, P, P, None, None) == vc.VC_ERR_INVALID
    assert L.vc_accept(P, P, 1, 9, 0, P, P, None, None) == vc.VC_ERR_INVALID


def test_project_rejects_and_sizes(L):
    """Projection: argument checks (nothing enqueued) and the workspace size (ticket counters,
    one per 8-row tile, rounded to 256 B, then one 8-byte argmax slot per row)."""
    n = ctypes.c_size_t()
    assert L.vc_project_workspace(8, 1, 2048, ctypes.byref(n)) == vc.VC_OK
    assert n.value == 256 + 8 * 8
    assert L.vc_project_workspace(8, 31, 2048, ctypes.byref(n)) == vc.VC_OK
    assert n.value == 256 + 8 * 31 * 8
    assert L.vc_project_workspace(0, 1, 2048, ctypes.byref(n)) == vc.VC_ERR_INVALID
    call = lambda **a: L.vc_project_logits(a.get("W", P), a.get("wdt", vc.VC_F32), a.get("V", 2048), a.get("o", P), a.get("B", 8),
                                           a.get("Hq", 32), a.get("L", 1), a.get("z", P), a.get("idx", P),
                                           a.get("stride", 1), a.get("ws", P), a.get("ws_bytes", 1 << 20), None)
    assert call(W=0) == vc.VC_ERR_INVALID
    assert call(wdt=vc.VC_F16) == vc.VC_ERR_INVALID and "w_dtype" in _err(L)
    assert call(o=BAD) == vc.VC_ERR_INVALID
    assert call(V=0) == vc.VC_ERR_INVALID
    assert call(Hq=0) == vc.VC_ERR_INVALID
    assert call(z=None, idx=None) == vc.VC_ERR_INVALID and "nothing to write" in _err(L)
    assert call(L=4, stride=3) == vc.VC_ERR_INVALID                # argmax row stride < L
    assert call(ws=None) == vc.VC_ERR_WORKSPACE
    assert call(ws_bytes=100) == vc.VC_ERR_WORKSPACE


def test_workspace_queries_grow_with_work(L):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.vc_verify_workspace(8, 32, 8, 31, 32768, 0, 0, vc.VC_BF16, ctypes.byref(a)) == vc.VC_OK
    assert L.vc_verify_workspace(1, 32, 8, 31, 500000, 1, 65536, vc.VC_BF16, ctypes.byref(b)) == vc.VC_OK
    assert b.value > 2 * 8 * 65536 * 128 * 2 * 2  # two chunk stages of keys + values
    assert L.vc_draft_drop_workspace(4, 8, 64, 25000, ctypes.byref(a)) == vc.VC_OK and a.value > 4096


def test_kivi_descriptor_follows_replaced_buffers():
    """Replicas share one residual ring by replacing their ring tensors: the cached C descriptor
    must then point at the new buffers."""
    import torch

    c = vc.KiviCache(1, 2, 64, 2, vc.VC_F16, vc.VC_F16, 64, device="cpu")
    before = c.desc().k_res
    ring = torch.zeros(1, 2, 64, 128, dtype=torch.float16)
    c.k_res, c.v_res = ring, ring.clone()
    d = c.desc()
    assert d.k_res == ring.data_ptr() != before
    assert d.v_res == c.v_res.data_ptr()
    assert d.k_codes == c.k_codes.data_ptr()


def test_select_keep_rejects(L):
    out = ctypes.c_int64(-1)
    ok = dict(scores=P, stride=1000, rows=4, n=1000, sinks=64, recent=256, keep=400, idx=P, istride=400)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.vc_select_keep(a["scores"], a["stride"], a["rows"], a["n"], a["sinks"], a["recent"],
                                a["keep"], a["idx"], a["istride"], ctypes.byref(out), None)

    # every case fails validation (a valid call would launch kernels on the fake pointers)
    for kw, msg in [(dict(scores=0), "scores"), (dict(scores=BAD), "aligned"), (dict(idx=0), "idx"),
                    (dict(rows=0), "rows"), (dict(rows=70000), "rows"), (dict(n=0), "n must"),
                    (dict(n=1 << 31), "n must"), (dict(stride=999), "score_row_stride"),
                    (dict(n=1001, stride=1002), "score_row_stride"), (dict(keep=-1), ">= 0"),
                    (dict(istride=399), "idx_row_stride"), (dict(keep=0, istride=319), "idx_row_stride")]:
        assert call(**kw) == vc.VC_ERR_INVALID, kw
        assert msg in _err(L), (kw, _err(L))
    assert L.vc_select_keep(P, 1000, 4, 1000, 64, 256, 400, P, 400, None, None) == vc.VC_ERR_INVALID


def test_generic_workspace_query_matches_the_per_op_queries(L):
    """vc_workspace_bytes forwards to the per-operation sizes for every op, and rejects unknown ops
    and wrong dim counts."""
    one = ctypes.c_size_t()
    k = _kivi(B=8, Hkv=8, tok_cap=32768)
    assert L.vc_draft_quant_workspace(ctypes.byref(k), 32640, 128, 32, ctypes.byref(one)) == vc.VC_OK
    assert vc.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, [8, 8, 32, 32640]) == one.value
    # 4-bit caches split the context more coarsely: the generic size (2-bit) still covers them
    for B, Hkv, Hq, n_q in ((8, 8, 32, 32640), (1, 8, 32, 499872), (1, 8, 32, 2016)):
        k4 = _kivi(bits=4, B=B, Hkv=Hkv, tok_cap=n_q + 128)
        assert L.vc_draft_quant_workspace(ctypes.byref(k4), n_q, 128, Hq, ctypes.byref(one)) == vc.VC_OK
        assert vc.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, [B, Hkv, Hq, n_q]) >= one.value
    assert L.vc_draft_drop_workspace(4, 8, 64, 25000, ctypes.byref(one)) == vc.VC_OK
    assert vc.vc_workspace_bytes(vc.VC_OP_DRAFT_DROP, [4, 8, 64, 25000]) == one.value
    for dims in ([8, 32, 8, 31, 32768, 0, 0, vc.VC_BF16], [1, 32, 8, 31, 500000, 1, 65536, vc.VC_BF16],
                 [1, 32, 8, 9, 2048, 0, 0, vc.VC_F32]):
        assert L.vc_verify_workspace(*dims, ctypes.byref(one)) == vc.VC_OK
        assert vc.vc_workspace_bytes(vc.VC_OP_VERIFY, dims) == one.value
    assert L.vc_project_workspace(8, 31, 2048, ctypes.byref(one)) == vc.VC_OK
    assert vc.vc_workspace_bytes(vc.VC_OP_PROJECT, [8, 31, 2048]) == one.value
    arr = (ctypes.c_int64 * 8)(8, 8, 32, 32640, 0, 0, 0, 0)
    assert L.vc_workspace_bytes(99, arr, 4, ctypes.byref(one)) == vc.VC_ERR_INVALID and "unknown op" in _err(L)
    assert L.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, arr, 3, ctypes.byref(one)) == vc.VC_ERR_INVALID
    assert L.vc_workspace_bytes(vc.VC_OP_VERIFY, arr, 4, ctypes.byref(one)) == vc.VC_ERR_INVALID
    assert L.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, arr, 4, None) == vc.VC_ERR_INVALID
    bad = (ctypes.c_int64 * 4)(8, 8, 33, 32640)                    # Hq not a multiple of Hkv
    assert L.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, bad, 4, ctypes.byref(one)) == vc.VC_ERR_INVALID
    bad = (ctypes.c_int64 * 4)(8, 8, 32, 100)                      # n_q not a multiple of 32
    assert L.vc_workspace_bytes(vc.VC_OP_DRAFT_QUANT, bad, 4, ctypes.byref(one)) == vc.VC_ERR_INVALID


def test_decoder_workspace_query(L):
    """The matrix-core form's workspace: none where it does not apply (fp32 weights, K not a multiple
    of 32, gate/up halves not in blocks of 64), tickets only when K is not cut (K < 256), tickets
    plus one 128 x 16 tile (+ 16 sums of squares) per slice otherwise; the generic query agrees."""
    q = lambda *d: vc.vc_decoder_gemv_workspace(*d)
    assert q(vc.VC_DEC_STORE, vc.VC_F32, 32000, 2048, 16) == 0
    assert q(vc.VC_DEC_STORE, vc.VC_BF16, 32000, 2044, 16) == 0
    assert q(vc.VC_DEC_SWIGLU, vc.VC_BF16, 2 * 1000, 2048, 16) == 0
    T = 4096 * 4  # the tickets: a fixed region, so that differently shaped products can share
    assert q(vc.VC_DEC_STORE, vc.VC_BF16, 200, 160, 16) == T
    # q/k/v of 16 + 2 x 4 heads, K 2048, 16 rows: 24 column groups, 8 slices of 256
    assert q(vc.VC_DEC_ROPE, vc.VC_BF16, 3072, 2048, 16) == T + 24 * 8 * (128 * 16 + 16) * 4
    # three row tiles: tickets and tiles per row tile
    assert q(vc.VC_DEC_ADD, vc.VC_BF16, 512, 512, 33) == T + 3 * 4 * 2 * (128 * 16 + 16) * 4
    # more than 4096 column groups x row tiles: the vector form only
    assert q(vc.VC_DEC_STORE, vc.VC_BF16, 128 * 4097, 256, 16) == 0
    for d in ([vc.VC_DEC_ROPE, vc.VC_BF16, 3072, 2048, 16], [vc.VC_DEC_SWIGLU, vc.VC_BF16, 11264, 2048, 16],
              [vc.VC_DEC_STORE, vc.VC_F32, 77, 2560, 5]):
        assert vc.vc_workspace_bytes(vc.VC_OP_DECODER, d) == q(*d)
    one = ctypes.c_size_t()
    assert L.vc_decoder_gemv_workspace(9, vc.VC_BF16, 64, 64, 1, ctypes.byref(one)) == vc.VC_ERR_INVALID
    assert L.vc_decoder_gemv_workspace(0, vc.VC_BF16, 64, 66, 1, ctypes.byref(one)) == vc.VC_ERR_INVALID
    assert L.vc_decoder_gemv_workspace(0, vc.VC_BF16, 64, 64, 0, ctypes.byref(one)) == vc.VC_ERR_INVALID


def test_prefill_rejects_and_sizes(L):
    """Argument checks of the prefill call (all before any HIP call) and its workspace: one split
    partial (128 + 2 floats) per row and tile range; the generic query agrees."""
    one = ctypes.c_size_t()
    call = lambda **a: L.vc_prefill_attn(a.get("q", P), P, P, a.get("stride", 4096), a.get("n", 4000),
                                         a.get("B", 1), a.get("Hq", 32), a.get("Hkv", 8), ctypes.c_float(0.1),
                                         a.get("out", P), None, a.get("ws", P), a.get("wsb", 1 << 34), None)
    assert call(n=0) == vc.VC_ERR_INVALID and "n must" in _err(L)
    assert call(stride=3999) == vc.VC_ERR_INVALID and "kv_stride" in _err(L)
    assert call(Hq=30) == vc.VC_ERR_INVALID
    assert call(q=0) == vc.VC_ERR_INVALID
    assert call(out=BAD) == vc.VC_ERR_INVALID
    assert call(Hq=72) == vc.VC_ERR_UNSUPPORTED
    assert call(n=8388608, stride=8388608) == vc.VC_ERR_UNSUPPORTED
    assert call(wsb=16) == vc.VC_ERR_WORKSPACE
    assert call(ws=0) == vc.VC_ERR_WORKSPACE
    for d in ([1, 16, 4, 16384], [2, 8, 2, 33], [1, 64, 8, 1]):
        assert L.vc_prefill_workspace(*d, ctypes.byref(one)) == vc.VC_OK
        assert vc.vc_workspace_bytes(vc.VC_OP_PREFILL, d) == one.value
        B, Hq, Hkv, n = d
        splits = one.value // (B * Hq * n * 130 * 4)
        assert splits >= 1 and one.value >= B * Hq * n * splits * 130 * 4
    assert L.vc_prefill_workspace(1, 16, 4, 0, ctypes.byref(one)) == vc.VC_ERR_INVALID


def test_read_stream_rejects(L):
    assert L.vc_hbm_read_stream(P, 0, P, 4, None) == vc.VC_ERR_INVALID
    assert L.vc_hbm_read_stream(P, 24, P, 4, None) == vc.VC_ERR_INVALID
    assert L.vc_hbm_read_stream(P, 32, P, 0, None) == vc.VC_ERR_INVALID
    assert L.vc_hbm_read_stream(BAD, 32, P, 4, None) == vc.VC_ERR_INVALID
    assert L.vc_hbm_read_stream(P, 32, None, 4, None) == vc.VC_ERR_INVALID


def test_logit_margins_rejects(L):
    assert L.vc_logit_margins(P, 0, 10, P, None) == vc.VC_ERR_INVALID
    assert L.vc_logit_margins(P, 4, 0, P, None) == vc.VC_ERR_INVALID
    assert L.vc_logit_margins(None, 4, 10, P, None) == vc.VC_ERR_INVALID
    assert L.vc_logit_margins(P, 4, 10, None, None) == vc.VC_ERR_INVALID


def test_stream_copies_rejects(L):
    """Argument checks of the copy-only transfer (all before any HIP call)."""
    call = lambda **a: L.vc_verify_stream_copies(
        a.get("kp", P), P, a.get("stride", 4096), a.get("n", 4000), a.get("chunk", 1024), 2,
        a.get("Hq", 8), 2, a.get("L", 31), P, 1 << 34, None)
    assert call(L=0) == vc.VC_ERR_INVALID
    assert call(n=0) == vc.VC_ERR_INVALID and "n >= 1" in _err(L)
    assert call(stride=100) == vc.VC_ERR_INVALID
    assert call(kp=0) == vc.VC_ERR_INVALID
    assert call(kp=BAD) == vc.VC_ERR_INVALID
    assert call(chunk=16) == vc.VC_ERR_INVALID
    assert call(Hq=5) == vc.VC_ERR_INVALID
