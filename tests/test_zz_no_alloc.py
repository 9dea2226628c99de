"""The no-allocation draft call (vc_draft_attn_quant_noalloc) against the workspace call
(vc_draft_attn_quant) through the C ABI: identical outputs on two calls in a row, the second with a
smaller input (fewer batch rows, a shorter context, fewer splits), with and without the step's own
key/value stored in the same launch; a shape whose workspace exceeds the scratch is rejected with
nothing enqueued. The workspace call's outputs are checked against the oracle in the parity tests;
here they are the reference, since both calls run the same kernel and its merge is deterministic.
"""
import ctypes

import numpy as np
import pytest
import torch

from kv_cache_compressed_amd import harness, synth, vc
from oracle import attention as oatt
from oracle import quant as oq

pytestmark = pytest.mark.gpu


def _case(w, seed):
    nq = oq.quantised_prefix(w.n, w.R, w.group)
    K, V = synth.kv_past(w, seed)
    Kn, Vn = synth.kv_new(w, seed)
    Q = synth.q_new(w, seed)
    c = vc.KiviCache(w.B, w.Hkv, max(nq, 32), w.bits, vc.VC_F16, vc.VC_F16, w.res_cap, "cuda")
    Kd = torch.from_numpy(K).to("cuda", torch.bfloat16)
    Vd = torch.from_numpy(V).to("cuda", torch.bfloat16)
    vc.vc_quantize_kv(c, Kd, Vd, 0, nq)
    vc.vc_kivi_append(c, Kd[:, :, nq:], Vd[:, :, nq:], nq, w.n - nq, src_bh_stride=w.n * 128)
    q = torch.from_numpy(Q[:, :, 0]).to("cuda", torch.bfloat16).contiguous()
    kn = torch.from_numpy(Kn[:, :, 0]).to("cuda", torch.bfloat16).contiguous()
    vn = torch.from_numpy(Vn[:, :, 0]).to("cuda", torch.bfloat16).contiguous()
    return c, nq, q, kn, vn, (K, V, Kn, Vn, Q)


def test_noalloc_draft_equals_workspace_draft(gpu_lib):
    big = synth.WORKLOADS["c2"].with_(B=2, n=1500)
    small = synth.WORKLOADS["c2"].with_(B=1, n=700)
    for w, seed in ((big, 0), (small, 1)):
        c, nq, q, kn, vn, host = _case(w, seed)
        for fused in (False, True):
            r = (w.n - nq) + (1 if fused else 0)
            kw = dict(k_new=kn, v_new=vn) if fused else {}
            ws = torch.zeros(vc.vc_draft_quant_workspace(c, nq, r, w.Hq), dtype=torch.uint8, device="cuda")
            ref_o = torch.full((w.B, w.Hq, 128), float("nan"), device="cuda")
            ref_l = torch.full((w.B, w.Hq), float("nan"), device="cuda")
            vc.vc_draft_attn_quant(c, nq, r, q, ref_o, ref_l, ws, harness.SM_SCALE, **kw)
            out = torch.full_like(ref_o, float("nan"))
            lse = torch.full_like(ref_l, float("nan"))
            vc.vc_draft_attn_quant_noalloc(c, nq, r, q, out, lse, harness.SM_SCALE, **kw)
            torch.cuda.synchronize()
            print(f"[noalloc B={w.B} n={w.n} n_q={nq} r={r}] max|diff| out "
                  f"{float((out - ref_o).abs().max()):.3e} lse {float((lse - ref_l).abs().max()):.3e}",
                  flush=True)
            assert torch.isfinite(out).all() and torch.isfinite(lse).all()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), (w.B, w.n, fused)
        # and the oracle's bar on a few heads of the last (fused) call
        K, V, Kn, Vn, Q = host
        for h in range(0, w.Hq, 7):
            g = h // w.G
            lay = oq.KiviLayer(K[0, g], V[0, g], nq, w.bits, w.meta_dtype, w.res_dtype)
            lay.append(Kn[0, g, 0], Vn[0, g, 0])
            o, l = oatt.decode(Q[0, h, 0], lay.keys(r), lay.values(r))
            assert np.abs(out[0, h].cpu().numpy() - o).max() <= 2e-2
            assert abs(float(lse[0, h]) - l) < 2e-3


def test_noalloc_draft_rejects_oversized_shapes(gpu_lib):
    """64 batch rows x 8 kv heads x 8 query heads each need 3 splits of 4096 rows (6.4 MB of
    partials): more than the 4 MiB scratch, so the call fails with VC_ERR_WORKSPACE."""
    w = synth.WORKLOADS["c2"].with_(B=64, Hq=64, Hkv=8, n=512, R=0)
    c = vc.KiviCache(w.B, w.Hkv, 512, 2, vc.VC_F16, vc.VC_F16, 256, "cuda")
    need = vc.vc_draft_quant_workspace(c, 512, 1, w.Hq)
    assert need > (4 << 20)
    q = torch.zeros((w.B, w.Hq, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((w.B, w.Hq, 128), device="cuda")
    d = c.desc()
    st = vc.lib().vc_draft_attn_quant_noalloc(ctypes.byref(d), 512, 1, None, None, 0, 0, q.data_ptr(),
                                              vc.VC_BF16, w.Hq, harness.SM_SCALE, out.data_ptr(), None,
                                              None)
    assert st == vc.VC_ERR_WORKSPACE
    assert b"scratch" in vc.lib().vc_last_error()
