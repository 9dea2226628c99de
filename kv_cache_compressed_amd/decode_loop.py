"""Token-level VeriCache decoding of one request on a one-layer decoder, on the GPU.

"VeriCache: making lossy KV compression exact", The Core Idea (the round, the accept rule, the
guarantee that the output equals full-cache greedy decoding) and "VeriCache: Turning Lossy KV Cache
into Lossless LLM Inference", Methodology (the drafter and the verifier are the same weights and
differ only in the cache they read).

The model: token + position embeddings x, grouped-query attention (head dim 128) with keys and
values projected from x, a residual connection and an untied output head:
    q, k, v = Wq x, Wk x, Wv x;   o = attention(q; keys and values of positions 0..p);
    logits = Wlm (x + Wo o) = [Wlm Wo | Wlm] [o ; x].
The second form is what runs: x rides along as extra "heads" of the attention output, so one
projection call (with the greedy argmax fused in for draft steps) gives the logits.

Round layout (the kernels' convention: row i of a round sits at position n + i): the cached past is
every committed token but the last; block entry 0 is the last committed token and entries 1..x the
draft tokens. Draft step j embeds entry j's token (read on the device, so no host round trip),
projects q, k, v, runs draft attention over the compressed cache (which stores k, v into the
residual ring) and writes its greedy token into entry j + 1. The verifier scores all x + 1 entries
over the full cache, the accept step compares, and the commit keeps entries 0..a in the full cache
and the residual, flushing whole groups into the codes.

Every attention, quantisation, residual append, logits and accept step is a libvc call; the
embeddings and the q/k/v projections are plain fp32 GEMMs through PyTorch. The cache holds fp32 or
bf16 keys/values (q, k, v rounded to bf16 with ties to even), in HBM or, for bf16, in pinned host
memory that every verify streams in chunks (the pages' long-context setting).
"""
from __future__ import annotations

import numpy as np
import torch

from . import vc

SM_SCALE = float(np.float32(1.0 / np.sqrt(128.0)))
D = 128


def _dev(a, device) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.float32).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def _head(weights, device) -> torch.Tensor:
    """[Wlm Wo | Wlm] in fp32 (the product formed in float64 for host arrays, fp32 on the device
    for device tensors)."""
    Wo, Wlm = weights["Wo"], weights["Wlm"]
    if isinstance(Wlm, torch.Tensor):
        Wlm, Wo = _dev(Wlm, device), _dev(Wo, device)
        return torch.cat([Wlm @ Wo, Wlm], dim=1).contiguous()
    Wo, Wlm = np.asarray(Wo, np.float64), np.asarray(Wlm, np.float64)
    return _dev(np.concatenate([Wlm @ Wo, Wlm], axis=1), device)


class _Model:
    """Weights on the device and the per-position computations both decoders share."""

    def __init__(self, weights, Hq: int, Hkv: int, kv_dtype: str, device: str):
        self.E, self.P = _dev(weights["E"], device), _dev(weights["P"], device)
        self.Wq, self.Wk = _dev(weights["Wq"], device), _dev(weights["Wk"], device)
        self.Wv = _dev(weights["Wv"], device)
        self.Wqkv = torch.cat([self.Wq, self.Wk, self.Wv]).contiguous()  # [(Hq + 2 Hkv) 128, dm]
        self.Wp = _head(weights, device)  # [V, Hq*128 + dm]
        self.V, self.dm = self.E.shape
        assert self.dm % D == 0 and Hq % Hkv == 0
        self.Hq, self.Hkv, self.Hx = Hq, Hkv, Hq + self.dm // D
        assert kv_dtype in ("f32", "bf16")
        self.tdt = torch.float32 if kv_dtype == "f32" else torch.bfloat16
        self.vdt = vc.VC_F32 if kv_dtype == "f32" else vc.VC_BF16
        self.device = device

    def embed(self, tok1, pos: int):
        """x of the token in the 1-element device tensor `tok1` at position `pos` (fp32)."""
        return self.E[tok1.long()][0] + self.P[pos]

    def prefill(self, prompt, n: int, chunk: int, sink):
        """Keys/values of positions 0..n-1 in chunks: sink(t0, t1, K, V) with K, V [1, Hkv, m, 128]
        in the cache dtype (device tensors)."""
        ids = torch.tensor(prompt[:n], device=self.device)
        for t0 in range(0, n, chunk):
            t1 = min(n, t0 + chunk)
            X = self.E[ids[t0:t1]] + self.P[t0:t1]
            m = t1 - t0
            K = (X @ self.Wk.T).view(m, self.Hkv, D).transpose(0, 1).unsqueeze(0).to(self.tdt).contiguous()
            V = (X @ self.Wv.T).view(m, self.Hkv, D).transpose(0, 1).unsqueeze(0).to(self.tdt).contiguous()
            sink(t0, t1, K, V)


def _causal_attention(Q, K, V, n: int, Hq: int, Hkv: int, vdt: int, ws: "vc.Workspace", device) -> torch.Tensor:
    """Causal self-attention of a prompt's n rows for the prefill: Q [1, Hq, n, 128], K, V
    [1, Hkv, n, 128] in the cache dtype -> O [n, Hq * 128] fp32. bf16: one vc_prefill_attn launch;
    fp32 caches: the verify call block by block (32 rows over the keys before the block)."""
    if vdt == vc.VC_BF16:
        o = torch.empty((1, Hq, n, D), dtype=torch.float32, device=device)
        vc.vc_prefill_attn(Q, K, V, n, o, None, ws.get(vc.vc_prefill_workspace(1, Hq, Hkv, n)), SM_SCALE)
        return o[0].transpose(0, 1).reshape(n, -1)
    O = torch.zeros((n, Hq * D), dtype=torch.float32, device=device)
    for b0 in range(0, n, 32):
        b1 = min(n, b0 + 32)
        m = b1 - b0
        o = torch.zeros((1, Hq, m, D), dtype=torch.float32, device=device)
        nb = vc.vc_verify_workspace(1, Hq, Hkv, m, b0, False, 0, vdt)
        vc.vc_verify_attn(Q[:, :, b0:b1].contiguous(), K[:, :, b0:b1].contiguous(), V[:, :, b0:b1].contiguous(),
                          K, V, b0, o, None, ws.get(nb), SM_SCALE, past_stride=n)
        O[b0:b1] = o[0].transpose(0, 1).reshape(m, -1)
    return O


class _Store:
    """The full cache [1, Hkv, cap, 128] in the cache dtype, in HBM or in pinned host memory."""

    def __init__(self, Hkv: int, cap: int, dtype, host: bool, device: str):
        self.host, self.cap, self.device = host, cap, device
        if host:
            self.k = torch.empty((1, Hkv, cap, D), dtype=dtype, pin_memory=True)
            self.v = torch.empty_like(self.k, pin_memory=True)
            # CPU views of the same memory (16-bit rows as int16), for host-side row copies
            raw = (lambda t: t.view(torch.int16)) if dtype.itemsize == 2 else (lambda t: t)
            self.k_np, self.v_np = raw(self.k).numpy(), raw(self.v).numpy()
        else:
            self.k = torch.zeros((1, Hkv, cap, D), dtype=dtype, device=device)
            self.v = torch.zeros_like(self.k)

    def write(self, t0: int, K, V):
        """Rows t0 .. t0+m-1 from device tensors [1, Hkv, m, 128]."""
        m = K.shape[2]
        self.k[:, :, t0:t0 + m].copy_(K)
        self.v[:, :, t0:t0 + m].copy_(V)

    def device_rows(self, t0: int, t1: int):
        """(K, V, source stride) of rows t0..t1-1 on the device, for the quantiser (staged when
        the cache is in host memory)."""
        if self.host:
            return (self.k[:, :, t0:t1].to(self.device), self.v[:, :, t0:t1].to(self.device),
                    (t1 - t0) * D)
        return self.k[:, :, t0:], self.v[:, :, t0:], self.cap * D


class TokenDecoder:
    """weights: dict of fp32 arrays or device tensors E [V, dm], P [max_pos, dm], Wq [Hq*128, dm],
    Wk/Wv [Hkv*128, dm], Wo [dm, Hq*128], Wlm [V, dm]; dm a multiple of 128. kv_dtype "f32" or
    "bf16"; host_past (bf16 only): the full cache in pinned host memory, streamed by every verify in
    chunks of chunk_tokens on copy_stream; prefetch_verify: each round's draft phase first issues
    the copies of the verify's first two chunks (vc_verify_prefetch)."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, x: int, bits: int = 4, R: int = 32,
                 max_new: int = 256, kv_dtype: str = "f32", host_past: bool = False,
                 chunk_tokens: int = 65536, copy_stream=None, prefetch_verify: bool = True,
                 device: str = "cuda"):
        mdl = self.m = _Model(weights, Hq, Hkv, kv_dtype, device)
        assert not host_past or kv_dtype == "bf16", "a host-streamed cache is bf16"
        f32 = dict(dtype=torch.float32, device=device)
        tdt = mdl.tdt
        self.Hq, self.Hkv, self.x, self.L, self.R = Hq, Hkv, x, x + 1, R
        self.host, self.chunk = host_past, chunk_tokens
        self.copy_stream = (copy_stream or torch.cuda.Stream()) if host_past else None
        self.prefetch_verify, self._prefetched = prefetch_verify, None
        prompt = [int(t) for t in prompt]
        assert len(prompt) >= 2
        self.n = len(prompt) - 1  # cached positions: every prompt token but the last
        L = self.L
        self.cap = (self.n + max_new + 2 * L + 63) // 32 * 32
        assert self.cap <= mdl.P.shape[0], "position table too short"
        self.store = _Store(Hkv, self.cap, tdt, host_past, device)
        self.k_blk = torch.zeros((1, Hkv, L, D), dtype=tdt, device=device)
        self.v_blk = torch.zeros_like(self.k_blk)
        self.q_verify = torch.zeros((1, Hq, L, D), dtype=tdt, device=device)
        # per block entry: [o ; x] of its draft step (x written by the embedding, o by the draft
        # attention, both read by the projection in place) and q, k, v side by side (fp32 from
        # one GEMV, then in the cache dtype)
        self.odx = torch.zeros((L, mdl.Hx, D), **f32)
        nqkv = (Hq + 2 * Hkv) * D
        self.y32 = torch.zeros((L, nqkv), **f32)
        self.yc = self.y32 if tdt == torch.float32 else torch.zeros((L, nqkv), dtype=tdt, device=device)
        self.lse_d = torch.zeros((1, Hq), **f32)
        self.ov = torch.zeros((1, mdl.Hx, L, D), **f32)    # verify rows [o ; x]
        self.lse_v = torch.zeros((1, Hq, L), **f32)
        self.logits_v = torch.zeros((1, L, mdl.V), **f32)
        i32 = dict(dtype=torch.int32, device=device)
        self.tok = torch.zeros((L + 1,), **i32)             # block tokens (entry L: spare)
        self.accept_len = torch.zeros((1,), **i32)
        self.next_tok = torch.zeros((1,), **i32)
        self.argmax_v = torch.zeros((1, L), **i32)
        self.ws_draft = vc.Workspace(device)
        self.ws_verify = vc.Workspace(device)
        self.ws_proj = torch.zeros((vc.vc_project_workspace(1, 1, mdl.V) + 3) // 4, **i32)
        # prefill: keys/values of positions 0..n-1 into the full cache, the quantised prefix into
        # the codes (chunk by chunk), the rest into the residual
        n = self.n
        self.n_q = 32 * (max(0, n - R) // 32)
        res_cap = (R + 32 + L + 31) // 32 * 32
        meta = vc.VC_F32 if kv_dtype == "f32" else vc.VC_F16
        self.cache = vc.KiviCache(1, Hkv, self.cap, bits, meta, meta, res_cap, device)

        def sink(t0, t1, K, V):
            self.store.write(t0, K, V)
            q1 = min(t1, self.n_q)
            if t0 < q1:
                vc.vc_quantize_kv(self.cache, K, V, t0, q1 - t0, src_bh_stride=(t1 - t0) * D)

        mdl.prefill(prompt, n, max(32, chunk_tokens // 32 * 32), sink)
        if n > self.n_q:
            Kr, Vr, stride = self.store.device_rows(self.n_q, n)
            vc.vc_kivi_append(self.cache, Kr, Vr, self.n_q, n - self.n_q, src_bh_stride=stride)
        self.tok[0] = prompt[-1]
        self.rounds = []  # accepted count per round

    def warm(self):
        """Size every workspace for the largest context this decoder can reach, so that no
        allocation falls inside a timed decode."""
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.cap, self.host, self.chunk,
                                    self.m.vdt)
        self.ws_verify.get(nb)
        r = self.R + 32 + self.L
        self.ws_draft.get(vc.vc_draft_quant_workspace(self.cache, (self.cap - r) // 32 * 32, r, self.Hq))
        torch.cuda.synchronize()

    # ---- one block entry: embedding and projections -----------------------------------------
    def _entry(self, j: int):
        """x of entry j (its token read on the device) into odx[j]'s x rows; q, k, v into yc[j]."""
        mdl = self.m
        x = self.odx[j, self.Hq:].view(1, mdl.dm)
        torch.index_select(mdl.E, 0, self.tok[j:j + 1], out=x)
        x.add_(mdl.P[self.n + j])
        torch.mv(mdl.Wqkv, x[0], out=self.y32[j])
        if self.yc is not self.y32:
            self.yc[j].copy_(self.y32[j])

    def _qkv(self, j: int):
        """Views of entry j's q [1, Hq, 128], k and v [1, Hkv, 128] in the cache dtype."""
        Hq, Hkv, y = self.Hq, self.Hkv, self.yc[j]
        return (y[:Hq * D].view(1, Hq, D), y[Hq * D:(Hq + Hkv) * D].view(1, Hkv, D),
                y[(Hq + Hkv) * D:].view(1, Hkv, D))

    def draft_step(self, j: int):
        """Draft step j: attention over the compressed cache (storing entry j's key/value into the
        residual), logits of [o ; x] and the greedy token into block entry j + 1."""
        self._entry(j)
        q, k, v = self._qkv(j)
        r = (self.n - self.n_q) + j + 1
        nb = vc.vc_draft_quant_workspace(self.cache, self.n_q, r, self.Hq)
        vc.vc_draft_attn_quant(self.cache, self.n_q, r, q, self.odx[j, :self.Hq].view(1, self.Hq, D),
                               self.lse_d, self.ws_draft.get(nb), SM_SCALE, k_new=k, v_new=v)
        vc.vc_project_logits(self.m.Wp, self.odx[j].view(1, self.m.Hx, D),
                             argmax=self.tok[j + 1:j + 2], argmax_b_stride=1, ws=self.ws_proj)

    def verify_step(self):
        """Entry x's projections, verify attention over the full cache, logits of every row and
        the greedy accept."""
        self._entry(self.x)
        Hq, Hkv = self.Hq, self.Hkv
        y = self.yc.view(self.L, Hq + 2 * Hkv, D)
        self.q_verify[0].copy_(y[:, :Hq].transpose(0, 1))
        self.k_blk[0].copy_(y[:, Hq:Hq + Hkv].transpose(0, 1))
        self.v_blk[0].copy_(y[:, Hq + Hkv:].transpose(0, 1))
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.n, self.host, self.chunk,
                                    self.m.vdt)
        mode = int(self.host)
        if self.host and self._prefetched == self.n:
            mode = vc.VC_PAST_HOST_PREFETCHED
        self._prefetched = None
        vc.vc_verify_attn(self.q_verify, self.k_blk, self.v_blk, self.store.k, self.store.v, self.n,
                          self.ov, self.lse_v, self.ws_verify.get(nb), SM_SCALE,
                          past_stride=self.cap, past_on_host=mode, chunk_tokens=self.chunk,
                          copy_stream=self.copy_stream)
        self.ov[0, self.Hq:] = self.odx[:, self.Hq:].transpose(0, 1)
        vc.vc_project_logits(self.m.Wp, self.ov, logits=self.logits_v)
        vc.vc_accept(self.logits_v, self.tok[1:self.L].view(1, self.x), self.accept_len,
                     self.next_tok, self.argmax_v)

    def commit(self):
        """Keep entries 0..a (positions n..n+a) in the full cache and the residual (entry x, never
        drafted, is appended when every draft stands), flush whole residual groups into the codes,
        and start the next round from the emitted token. Returns the emitted tokens."""
        a = int(self.accept_len[0].item())
        emitted = [int(t) for t in self.tok[1:a + 1].tolist()] + [int(self.next_tok[0].item())]
        n0, n1 = self.n, self.n + a + 1
        assert n1 + self.L <= self.cap, "cache capacity exhausted (raise max_new)"
        self.store.write(n0, self.k_blk[:, :, :a + 1], self.v_blk[:, :, :a + 1])
        if a == self.x:
            vc.vc_kivi_append(self.cache, self.k_blk[:, :, self.x], self.v_blk[:, :, self.x],
                              n0 + self.x, 1, src_bh_stride=self.L * D)
        self.n = n1
        while self.n - self.n_q >= self.R + 32:
            Kg, Vg, stride = self.store.device_rows(self.n_q, self.n_q + 32)
            vc.vc_quantize_kv(self.cache, Kg, Vg, self.n_q, 32, src_bh_stride=stride)
            self.n_q += 32
        self.tok[0:1] = self.next_tok
        self.rounds.append(a)
        return emitted

    def stage_remote(self):
        """Remote prefix caching (simulated): move the compressed cache's current contents (codes
        and metadata of the n_q quantised tokens, both residual rings) to pinned host memory, as
        the far side's copy, and clear the device copy, which must then arrive before the next
        draft step (harness.remote_prefix_decode sends self.remote_pieces over a ThrottledLink).
        Returns the compressed bytes."""
        c, nq = self.cache, self.n_q
        dev = []
        for h in range(self.Hkv):
            dev += [c.k_codes[0, h, :nq], c.v_codes[0, h, :nq], c.k_meta[0, h, :nq // 32],
                    c.v_meta[0, h, :nq]]
        dev += [c.k_res, c.v_res]
        dev = [t for t in dev if t.numel()]
        host = [torch.empty(t.shape, dtype=t.dtype, pin_memory=True) for t in dev]
        for d, h in zip(dev, host):
            h.copy_(d)
        torch.cuda.synchronize()
        for d in dev:
            d.zero_()
        self.remote_pieces = list(zip(dev, host))
        return sum(t.numel() * t.element_size() for t in dev)

    def prefetch(self):
        """Host-streamed cache: issue the copies of this round's first two verify chunks now (the
        committed past is fixed for the round), so they cross the link while the draft steps run;
        the round's verify_step then skips them."""
        if not self.host:
            return
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.n, True, self.chunk, self.m.vdt)
        vc.vc_verify_prefetch(self.store.k, self.store.v, self.n, self.ws_verify.get(nb), 1, self.Hq,
                              self.Hkv, self.L, self.chunk, past_stride=self.cap,
                              copy_stream=self.copy_stream)
        self._prefetched = self.n

    def draft_phase(self):
        if self.prefetch_verify:
            self.prefetch()
        for j in range(self.x):
            self.draft_step(j)

    def set_round_inputs(self):
        """Nothing to load: the next round starts from the committed token (for the schedules in
        harness, which pass each group its next round's inputs)."""

    def generate(self, steps: int):
        """Rounds until `steps` tokens are emitted; returns them."""
        out = []
        while len(out) < steps:
            self.draft_phase()
            self.verify_step()
            out += self.commit()
        return out[:steps]


class GreedyDecoder:
    """The baseline without a drafter: greedy decoding over the full cache, one token per step
    (the entry's projections, attention of one query row over the full cache, logits with the
    greedy argmax, the entry's key/value appended to the full cache). Same model, cache placement
    and calls as TokenDecoder."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, max_new: int = 256, kv_dtype: str = "f32",
                 host_past: bool = False, chunk_tokens: int = 65536, copy_stream=None,
                 device: str = "cuda"):
        mdl = self.m = _Model(weights, Hq, Hkv, kv_dtype, device)
        assert not host_past or kv_dtype == "bf16", "a host-streamed cache is bf16"
        f32 = dict(dtype=torch.float32, device=device)
        tdt = mdl.tdt
        self.Hq, self.Hkv = Hq, Hkv
        self.host, self.chunk = host_past, chunk_tokens
        self.copy_stream = (copy_stream or torch.cuda.Stream()) if host_past else None
        prompt = [int(t) for t in prompt]
        self.n = len(prompt) - 1
        self.cap = (self.n + max_new + 63) // 32 * 32
        self.store = _Store(Hkv, self.cap, tdt, host_past, device)
        mdl.prefill(prompt, self.n, max(32, chunk_tokens // 32 * 32),
                    lambda t0, t1, K, V: self.store.write(t0, K, V))
        self.q = torch.zeros((1, Hq, 1, D), dtype=tdt, device=device)
        self.k1 = torch.zeros((1, Hkv, 1, D), dtype=tdt, device=device)
        self.v1 = torch.zeros_like(self.k1)
        self.o = torch.zeros((1, mdl.Hx, 1, D), **f32)
        self.lse = torch.zeros((1, Hq, 1), **f32)
        i32 = dict(dtype=torch.int32, device=device)
        self.toks = torch.zeros((max_new + 1,), **i32)
        self.toks[0] = prompt[-1]
        self.i = 0  # tokens generated so far (generate() continues from there)
        self.ws = vc.Workspace(device)
        self.ws_proj = torch.zeros((vc.vc_project_workspace(1, 1, mdl.V) + 3) // 4, **i32)

    def stage_remote(self):
        """Remote prefix caching (simulated), the full-cache baseline: move the device-resident
        full cache's rows 0..n-1 to pinned host memory as the far side's copy and clear them; they
        must arrive (self.remote_pieces over a harness.ThrottledLink) before the next step.
        Returns the bytes."""
        assert not self.host, "the baseline ships the full cache into HBM"
        dev = []
        for h in range(self.Hkv):
            dev += [self.store.k[0, h, :self.n], self.store.v[0, h, :self.n]]
        host = [torch.empty(t.shape, dtype=t.dtype, pin_memory=True) for t in dev]
        for d, h in zip(dev, host):
            h.copy_(d)
        torch.cuda.synchronize()
        for d in dev:
            d.zero_()
        self.remote_pieces = list(zip(dev, host))
        return sum(t.numel() * t.element_size() for t in dev)

    def warm(self):
        """Size the workspace for the largest context this decoder can reach."""
        self.ws.get(vc.vc_verify_workspace(1, self.Hq, self.Hkv, 1, self.cap, self.host, self.chunk,
                                           self.m.vdt))
        torch.cuda.synchronize()

    def generate(self, steps: int):
        """The next `steps` tokens."""
        mdl = self.m
        i0 = self.i
        assert i0 + steps < self.toks.numel(), "max_new exhausted"
        for i in range(i0, i0 + steps):
            x = mdl.embed(self.toks[i:i + 1], self.n)
            self.q[0, :, 0] = (mdl.Wq @ x).view(self.Hq, D)
            self.k1[0, :, 0] = (mdl.Wk @ x).view(self.Hkv, D)
            self.v1[0, :, 0] = (mdl.Wv @ x).view(self.Hkv, D)
            nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, 1, self.n, self.host, self.chunk, mdl.vdt)
            vc.vc_verify_attn(self.q, self.k1, self.v1, self.store.k, self.store.v, self.n, self.o,
                              self.lse, self.ws.get(nb), SM_SCALE, past_stride=self.cap,
                              past_on_host=self.host, chunk_tokens=self.chunk,
                              copy_stream=self.copy_stream)
            self.o[0, self.Hq:, 0] = x.view(-1, D)
            vc.vc_project_logits(mdl.Wp, self.o, argmax=self.toks[i + 1:i + 2], argmax_b_stride=1,
                                 ws=self.ws_proj)
            self.store.write(self.n, self.k1, self.v1)
            self.n += 1
        self.i = i0 + steps
        return [int(t) for t in self.toks[i0 + 1:i0 + steps + 1].tolist()]


class LayeredDecoder:
    """VeriCache decoding of one request on a stack of layers on the residual stream. Two layer
    forms: attention only (x_{l+1} = x_l + Wo_l attention_l(x_l), logits = Wlm x_L; weights E, P,
    Wlm as for TokenDecoder and per-layer lists Wq, Wk, Wv, Wo), or the Llama form when the
    weights hold per-layer gains g_att, g_mlp, MLP matrices W1, W3 [F, dm], W2 [dm, F] and a final
    gain g_f (pre-norm RMSNorm, rotary positions on q and k with theta `rope_theta`, channel i
    paired with i + 64, SwiGLU MLP, final RMSNorm; no position table). Every layer has its own
    full cache (HBM or pinned host memory) and KIVI cache; keys are cached after the rotation.
    Draft steps thread the residual stream through every layer's draft attention over the
    compressed caches; the verify runs every layer over the full caches for all x + 1 entries.
    Above the first layer the drafter's keys/values of its own positions differ from the
    verifier's (their inputs went through compressed attention), so the commit writes the
    verifier's keys/values of the kept positions into the full caches and over the draft-time
    entries of the residual rings. Norms, rotations, MLPs and the q/k/v/o GEMMs are fp32 PyTorch
    ops; attention, quantisation, appends, logits and accept are libvc calls."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, x: int, bits: int = 4, R: int = 32,
                 max_new: int = 256, kv_dtype: str = "f32", host_past: bool = False,
                 chunk_tokens: int = 65536, rope_theta: float = 500000.0, graphs: bool = True,
                 device: str = "cuda"):
        self.llama = "g_att" in weights
        self.E = _dev(weights["E"], device)
        self.P = None if self.llama else _dev(weights["P"], device)
        self.Wlm = _dev(weights["Wlm"], device)
        self.Wo = [_dev(w, device) for w in weights["Wo"]]
        # q, k, v from one GEMM per layer
        self.Wqkv = [torch.cat([_dev(q, device), _dev(k, device), _dev(v, device)]).contiguous()
                     for q, k, v in zip(weights["Wq"], weights["Wk"], weights["Wv"])]
        if self.llama:
            lst = lambda k: [_dev(w, device) for w in weights[k]]
            self.g_att, self.g_mlp = lst("g_att"), lst("g_mlp")
            self.W2 = lst("W2")
            self.W13 = [torch.cat([_dev(a, device), _dev(b, device)]).contiguous()  # gate and up
                        for a, b in zip(weights["W1"], weights["W3"])]
            self.g_f = _dev(weights["g_f"], device)
        self.nl = len(self.Wqkv)
        self.V, self.dm = self.E.shape
        assert self.dm % D == 0 and Hq % Hkv == 0
        assert not host_past or kv_dtype == "bf16", "a host-streamed cache is bf16"
        self.tdt = torch.float32 if kv_dtype == "f32" else torch.bfloat16
        self.vdt = vc.VC_F32 if kv_dtype == "f32" else vc.VC_BF16
        self.Hq, self.Hkv, self.x, self.L, self.R = Hq, Hkv, x, x + 1, R
        self.host, self.chunk, self.device = host_past, chunk_tokens, device
        self.copy_stream = torch.cuda.Stream() if host_past else None
        prompt = [int(t) for t in prompt]
        n = self.n = len(prompt) - 1
        L = self.L
        self.cap = (n + max_new + 2 * L + 63) // 32 * 32
        if self.llama:
            # rotation angles in float64 on the host, cos/sin rounded once to fp32
            ang = np.arange(self.cap)[:, None] * rope_theta ** (-2.0 * np.arange(D // 2) / D)
            self.cos = torch.from_numpy(np.cos(ang).astype(np.float32)).to(device)
            self.sin = torch.from_numpy(np.sin(ang).astype(np.float32)).to(device)
        else:
            assert self.cap <= self.P.shape[0], "position table too short"
        f32 = dict(dtype=torch.float32, device=device)
        tk = dict(dtype=self.tdt, device=device)
        nl = self.nl
        self.stores = [_Store(Hkv, self.cap, self.tdt, host_past, device) for _ in range(nl)]
        self.kd = [torch.zeros((1, Hkv, L, D), **tk) for _ in range(nl)]   # draft-time k, v
        self.vd = [torch.zeros((1, Hkv, L, D), **tk) for _ in range(nl)]
        self.kv_ = [torch.zeros((1, Hkv, L, D), **tk) for _ in range(nl)]  # verifier's k, v
        self.vv_ = [torch.zeros((1, Hkv, L, D), **tk) for _ in range(nl)]
        self.qd = torch.zeros((1, Hq, D), **tk)
        self.qv = torch.zeros((1, Hq, L, D), **tk)
        self.od = torch.zeros((1, Hq, D), **f32)
        self.lse_d = torch.zeros((1, Hq), **f32)
        self.ov = torch.zeros((1, Hq, L, D), **f32)
        self.lse_v = torch.zeros((1, Hq, L), **f32)
        self.logits_v = torch.zeros((1, L, self.V), **f32)
        i32 = dict(dtype=torch.int32, device=device)
        self.tok = torch.zeros((L + 1,), **i32)
        self.accept_len = torch.zeros((1,), **i32)
        self.next_tok = torch.zeros((1,), **i32)
        self.argmax_v = torch.zeros((1, L), **i32)
        self.ws_draft = vc.Workspace(device)
        self.ws_verify = vc.Workspace(device)
        self.ws_proj = torch.zeros((vc.vc_project_workspace(1, 1, self.V) + 3) // 4, **i32)
        self.n_q = 32 * (max(0, n - R) // 32)
        res_cap = (R + 32 + L + 31) // 32 * 32
        meta = vc.VC_F32 if kv_dtype == "f32" else vc.VC_F16
        self.caches = [vc.KiviCache(1, Hkv, self.cap, bits, meta, meta, res_cap, device)
                       for _ in range(nl)]
        # one-row steps of the Llama form replay the layer's glue from HIP graphs (captured on
        # first use): the row's residual stream, position and q/k/v live in fixed buffers, the
        # position is read on the device
        self.use_graphs = graphs and self.llama
        if self.use_graphs:
            # the one-row GEMVs read bf16 copies of weights whose values are all bf16 (widened
            # exactly in the kernel, so the results are the fp32 weights' bit for bit)
            def gemv_w(w):
                wb = w.to(torch.bfloat16)
                return wb if torch.equal(wb.float(), w) else w
            self.gWqkv = [gemv_w(w) for w in self.Wqkv]
            self.gWo = [gemv_w(w) for w in self.Wo]
            self.gW13 = [gemv_w(w) for w in self.W13]
            self.gW2 = [gemv_w(w) for w in self.W2]
            self.gWlm = gemv_w(self.Wlm)
        self.xb = torch.zeros((1, self.dm), **f32)
        self.hb = torch.zeros((1, self.dm), **f32)
        self.posb = torch.zeros((1,), dtype=torch.int64, device=device)
        # the row's q, k, v in the cache dtype, one buffer (each layer's attention reads them
        # before the next layer's glue rewrites them)
        self.qkvc = torch.zeros((1, Hq + 2 * Hkv, D), **tk)
        self.ks1, self.vs1 = self.qkvc[:, Hq:Hq + Hkv], self.qkvc[:, Hq + Hkv:]
        if self.llama:  # per position: [cos | cos] and [-sin | sin] over the 128 channels
            self.cs = torch.stack([torch.cat([self.cos, self.cos], 1),
                                   torch.cat([-self.sin, self.sin], 1)], 1).contiguous()
        self.gA = self.gB = self.gH = None
        self._prefill(prompt)
        self.tok[0] = prompt[-1]
        self.rounds = []

    # ---- graph-replayed glue of one-row steps ------------------------------------------------
    @staticmethod
    def _gemv(W, x):
        """W [N, K] fp32 times the row x [1, K] (K a multiple of 128) -> [1, N], through the
        projection kernel (one row: weight-bound, coalesced 16-byte loads of every W row)."""
        out = torch.empty((1, 1, W.shape[0]), dtype=torch.float32, device=x.device)
        vc.vc_project_logits(W, x.contiguous().view(1, -1, D), logits=out)
        return out.view(1, -1)

    def _glue_a(self, l: int):
        """Layer l's norm, q/k/v GEMV and rotation of the row in xb at position posb, then q, k, v
        into qkvc (cache dtype): the pair (a, b) = (channel i, channel i + 64) becomes
        (a c - b s, b c + a s), i.e. y c2 + roll(y, 64) s2 with c2 = [c | c], s2 = [-s | s]."""
        Hq, Hkv = self.Hq, self.Hkv
        Y = self._gemv(self.gWqkv[l], self._rms(self.xb, self.g_att[l])).view(1, Hq + 2 * Hkv, D)
        cs = self.cs.index_select(0, self.posb)  # [1, 2, 128]
        qk = Y[:, :Hq + Hkv]
        r = torch.roll(qk, D // 2, dims=-1)
        qk.mul_(cs[:, 0:1])
        qk.addcmul_(r, cs[:, 1:2])
        self.qkvc.copy_(Y)

    def _glue_b(self, l: int):
        """Layer l's output projection, residual and MLP on xb, from the attention output od."""
        X = self.xb + self._gemv(self.gWo[l], self.od.view(1, -1))
        Z = self._gemv(self.gW13[l], self._rms(X, self.g_mlp[l]))
        F = Z.shape[-1] // 2
        torch.add(X, self._gemv(self.gW2[l], torch.nn.functional.silu(Z[:, :F]) * Z[:, F:]), out=self.xb)

    def _glue_h(self):
        self.hb.copy_(self._head_in(self.xb))

    def _capture(self):
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        pool = torch.cuda.graph_pool_handle()
        with torch.cuda.stream(side):
            for l in range(self.nl):  # one eager pass first (library set-up outside capture)
                self._glue_a(l)
                self._glue_b(l)
            self._glue_h()
            side.synchronize()
            gA, gB = [], []
            for l in range(self.nl):  # captured in the order the steps replay them
                for lst, fn in ((gA, self._glue_a), (gB, self._glue_b)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side, pool=pool):
                        fn(l)
                    lst.append(g)
            gH = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gH, stream=side, pool=pool):
                self._glue_h()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.gA, self.gB, self.gH = gA, gB, gH

    def _begin_row(self, tok1, pos: int):
        """xb = embedding of the device token tok1 (1 element), posb = pos."""
        if self.gH is None:
            self._capture()
        torch.index_select(self.E, 0, tok1, out=self.xb)
        self.posb.fill_(pos)

    # ---- the layer's parts outside attention (fp32) ------------------------------------------
    def _embed(self, tok, pos0: int):
        """Residual stream rows [m, dm] of the device int32 tokens `tok` at positions pos0.."""
        X = self.E[tok.long()]
        return X if self.llama else X + self.P[pos0:pos0 + X.shape[0]]

    def _rms(self, X, g):
        return torch.nn.functional.rms_norm(X, (self.dm,), g, 1e-5)

    def _rope(self, Y, pos0: int):
        """Rows Y [m, heads, 128] at positions pos0.. rotated (pair i, i + 64)."""
        c = self.cos[pos0:pos0 + Y.shape[0]].unsqueeze(1)
        s = self.sin[pos0:pos0 + Y.shape[0]].unsqueeze(1)
        a, b = Y[..., :D // 2], Y[..., D // 2:]
        return torch.cat([a * c - b * s, b * c + a * s], dim=-1)

    def _qkv(self, l: int, X, pos0: int):
        """q [m, Hq, 128], k and v [m, Hkv, 128] (fp32) of rows X [m, dm] at positions pos0.."""
        m, Hq, Hkv = X.shape[0], self.Hq, self.Hkv
        H = self._rms(X, self.g_att[l]) if self.llama else X
        Y = (H @ self.Wqkv[l].T).view(m, Hq + 2 * Hkv, D)
        if self.llama:  # q and k rotated together
            Y = torch.cat([self._rope(Y[:, :Hq + Hkv], pos0), Y[:, Hq + Hkv:]], dim=1)
        return Y[:, :Hq], Y[:, Hq:Hq + Hkv], Y[:, Hq + Hkv:]

    def _block_out(self, l: int, X, O):
        """The residual stream after layer l's attention output O [m, Hq*128] (and MLP)."""
        X = X + O @ self.Wo[l].T
        if self.llama:
            Z = self._rms(X, self.g_mlp[l]) @ self.W13[l].T
            F = Z.shape[-1] // 2
            X = X + (torch.nn.functional.silu(Z[..., :F]) * Z[..., F:]) @ self.W2[l].T
        return X

    def _head_in(self, X):
        return self._rms(X, self.g_f) if self.llama else X

    def _verify(self, l: int, q, k, v, n: int, out, lse):
        host = self.host and n > 0  # no past yet: nothing to stream (the block alone)
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, q.shape[2], n, host, self.chunk, self.vdt)
        st = self.stores[l]
        kp, vp, stride = (st.k, st.v, self.cap) if n > 0 else (k, v, q.shape[2])
        vc.vc_verify_attn(q, k, v, kp, vp, n, out, lse, self.ws_verify.get(nb), SM_SCALE,
                          past_stride=stride, past_on_host=host, chunk_tokens=self.chunk,
                          copy_stream=self.copy_stream)

    def _prefill(self, prompt):
        """Layer by layer over positions 0..n-1: keys/values into the full cache and the KIVI
        cache, causal attention over the layer's device-resident keys/values (whatever the cache
        placement; see _causal_attention), the residual stream updated."""
        n, Hq, Hkv = self.n, self.Hq, self.Hkv
        X = self._embed(torch.tensor(prompt[:n], device=self.device), 0)
        cache_layout = lambda Y: Y.transpose(0, 1).unsqueeze(0).to(self.tdt).contiguous()
        for l in range(self.nl):
            Q, K, V = self._qkv(l, X, 0)
            K, V = cache_layout(K), cache_layout(V)
            self.stores[l].write(0, K, V)
            c = self.caches[l]
            if self.n_q:
                vc.vc_quantize_kv(c, K, V, 0, self.n_q, src_bh_stride=n * D)
            if n > self.n_q:
                vc.vc_kivi_append(c, K[:, :, self.n_q:], V[:, :, self.n_q:], self.n_q, n - self.n_q,
                                  src_bh_stride=n * D)
            O = _causal_attention(cache_layout(Q), K, V, n, Hq, Hkv, self.vdt, self.ws_verify, self.device)
            X = self._block_out(l, X, O)

    def draft_step(self, j: int):
        r = (self.n - self.n_q) + j + 1
        if self.use_graphs:
            self._begin_row(self.tok[j:j + 1], self.n + j)
            for l in range(self.nl):
                self.gA[l].replay()
                c = self.caches[l]
                nb = vc.vc_draft_quant_workspace(c, self.n_q, r, self.Hq)
                vc.vc_draft_attn_quant(c, self.n_q, r, self.qkvc[:, :self.Hq], self.od, self.lse_d,
                                       self.ws_draft.get(nb), SM_SCALE, k_new=self.ks1,
                                       v_new=self.vs1)
                self.gB[l].replay()
            self.gH.replay()
            vc.vc_project_logits(self.gWlm, self.hb.view(1, -1, D), argmax=self.tok[j + 1:j + 2],
                                 argmax_b_stride=1, ws=self.ws_proj)
            return
        x = self._embed(self.tok[j:j + 1], self.n + j)
        for l in range(self.nl):
            q, k, v = self._qkv(l, x, self.n + j)
            self.qd.copy_(q)
            self.kd[l][0, :, j] = k[0]
            self.vd[l][0, :, j] = v[0]
            c = self.caches[l]
            nb = vc.vc_draft_quant_workspace(c, self.n_q, r, self.Hq)
            vc.vc_draft_attn_quant(c, self.n_q, r, self.qd, self.od, self.lse_d, self.ws_draft.get(nb),
                                   SM_SCALE, k_new=self.kd[l][:, :, j], v_new=self.vd[l][:, :, j])
            x = self._block_out(l, x, self.od.view(1, -1))
        vc.vc_project_logits(self.Wlm, self._head_in(x).view(1, -1, D), argmax=self.tok[j + 1:j + 2],
                             argmax_b_stride=1, ws=self.ws_proj)

    def verify_step(self):
        L, n = self.L, self.n
        X = self._embed(self.tok[:L], n)
        for l in range(self.nl):
            q, k, v = self._qkv(l, X, n)
            self.qv.copy_(q.transpose(0, 1).unsqueeze(0))
            self.kv_[l].copy_(k.transpose(0, 1).unsqueeze(0))
            self.vv_[l].copy_(v.transpose(0, 1).unsqueeze(0))
            self._verify(l, self.qv, self.kv_[l], self.vv_[l], n, self.ov, self.lse_v)
            X = self._block_out(l, X, self.ov[0].transpose(0, 1).reshape(L, -1))
        xl = self._head_in(X).view(L, -1, D).transpose(0, 1).unsqueeze(0).contiguous()
        vc.vc_project_logits(self.Wlm, xl, logits=self.logits_v)
        vc.vc_accept(self.logits_v, self.tok[1:L].view(1, self.x), self.accept_len, self.next_tok,
                     self.argmax_v)

    def commit(self):
        a = int(self.accept_len[0].item())
        emitted = [int(t) for t in self.tok[1:a + 1].tolist()] + [int(self.next_tok[0].item())]
        n0, n1 = self.n, self.n + a + 1
        assert n1 + self.L <= self.cap, "cache capacity exhausted (raise max_new)"
        for l in range(self.nl):
            k, v = self.kv_[l][:, :, :a + 1], self.vv_[l][:, :, :a + 1]
            self.stores[l].write(n0, k, v)
            vc.vc_kivi_append(self.caches[l], k, v, n0, a + 1, src_bh_stride=self.L * D)
        self.n = n1
        while self.n - self.n_q >= self.R + 32:
            for l in range(self.nl):
                Kg, Vg, stride = self.stores[l].device_rows(self.n_q, self.n_q + 32)
                vc.vc_quantize_kv(self.caches[l], Kg, Vg, self.n_q, 32, src_bh_stride=stride)
            self.n_q += 32
        self.tok[0:1] = self.next_tok
        self.rounds.append(a)
        return emitted

    def warm(self):
        """Size the workspaces for the largest context this decoder can reach, so that no
        allocation falls inside a timed decode."""
        self.ws_verify.get(vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.cap, self.host,
                                                  self.chunk, self.vdt))
        r = self.R + 32 + self.L
        self.ws_draft.get(vc.vc_draft_quant_workspace(self.caches[0], (self.cap - r) // 32 * 32, r,
                                                      self.Hq))
        torch.cuda.synchronize()

    def generate(self, steps: int):
        """Rounds until `steps` tokens are emitted; returns them (later calls continue)."""
        out = []
        while len(out) < steps:
            for j in range(self.x):
                self.draft_step(j)
            self.verify_step()
            out += self.commit()
        return out[:steps]


class LayeredGreedyDecoder(LayeredDecoder):
    """Greedy decoding over the full caches of the same layer stack, one token per step (no
    drafter; the KIVI caches are built by the shared prefill and not read)."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, max_new: int = 256, **kw):
        super().__init__(weights, Hq, Hkv, prompt, x=1, max_new=max_new, **kw)
        self.q1 = torch.zeros((1, Hq, 1, D), dtype=self.tdt, device=self.device)
        self.k1 = torch.zeros((1, Hkv, 1, D), dtype=self.tdt, device=self.device)
        self.v1 = torch.zeros_like(self.k1)
        self.o1 = torch.zeros((1, Hq, 1, D), dtype=torch.float32, device=self.device)
        self.lse1 = torch.zeros((1, Hq, 1), dtype=torch.float32, device=self.device)
        self.toks = torch.zeros((max_new + 1,), dtype=torch.int32, device=self.device)
        self.toks[0] = self.tok[0]
        self.i = 0  # tokens generated so far (generate() continues from there)

    def generate(self, steps: int):
        """The next `steps` tokens."""
        i0 = self.i
        assert i0 + steps < self.toks.numel(), "max_new exhausted"
        for i in range(i0, i0 + steps):
            if self.use_graphs:
                self._begin_row(self.toks[i:i + 1], self.n)
                for l in range(self.nl):
                    self.gA[l].replay()
                    q = self.qkvc[:, :self.Hq].view(1, self.Hq, 1, D)
                    k, v = self.ks1.view(1, self.Hkv, 1, D), self.vs1.view(1, self.Hkv, 1, D)
                    self._verify(l, q, k, v, self.n, self.od.view(1, self.Hq, 1, D), self.lse1)
                    self.stores[l].write(self.n, k, v)
                    self.gB[l].replay()
                self.gH.replay()
                vc.vc_project_logits(self.gWlm, self.hb.view(1, -1, D), argmax=self.toks[i + 1:i + 2],
                                     argmax_b_stride=1, ws=self.ws_proj)
                self.n += 1
                continue
            x = self._embed(self.toks[i:i + 1], self.n)
            for l in range(self.nl):
                q, k, v = self._qkv(l, x, self.n)
                self.q1[0, :, 0] = q[0]
                self.k1[0, :, 0] = k[0]
                self.v1[0, :, 0] = v[0]
                self._verify(l, self.q1, self.k1, self.v1, self.n, self.o1, self.lse1)
                self.stores[l].write(self.n, self.k1, self.v1)
                x = self._block_out(l, x, self.o1.view(1, -1))
            vc.vc_project_logits(self.Wlm, self._head_in(x).view(1, -1, D),
                                 argmax=self.toks[i + 1:i + 2], argmax_b_stride=1, ws=self.ws_proj)
            self.n += 1
        self.i = i0 + steps
        return [int(t) for t in self.toks[i0 + 1:i0 + steps + 1].tolist()]


class BatchedLlamaDecoder:
    """VeriCache decoding of B requests at once on Llama-form layers (weights as for
    LayeredDecoder's Llama form). Every request keeps its own full caches (HBM or pinned host
    memory), KIVI caches, context length and accepted counts, so requests that accept different
    numbers of drafts drift apart and each still emits exactly its own full-KV greedy tokens. The
    layer's norms, GEMMs, rotations and MLP run once over all requests' rows (rotation angles from
    each row's own position). A layer's KIVI caches are one batched cache (a row per request; a
    request's own appends and flushes go through its row). fused=True (default): a draft step is
    libvc calls only, per layer the fused norm + q/k/v product + rotation (vc_decoder_gemv ROPE), one
    draft attention launch for the whole batch with each row's own lengths
    (vc_draft_attn_quant_rows), the output product into the residual, the fused norm + gate/up
    product + SwiGLU and the down product into the residual, then the head (final norm fused into
    its product) and the greedy argmax: 24 launches for 4 layers (weights read as bf16 when they are
    bf16 values, the same numbers in half the bytes); graphs=True replays the whole draft phase from
    one captured graph (its kernels read lengths and positions from device memory). fused=False: the same step from PyTorch ops with one attention call per request. The
    verify step's layer work (B x (x + 1) rows) runs on PyTorch GEMMs either way; its attention is one
    call per request (each request's full cache is its own store). With the full caches in host
    memory the verify's calls stream through a ring of VRING workspaces: each call's copies are
    issued VRING - 1 calls ahead (vc_verify_prefetch), and the first VRING calls' copies at the start
    of the round, under the draft steps (a round's committed past is known before its drafts), so
    the host link does not wait for any call's compute. x = 0 gives plain greedy decoding of the
    batch (a verify of one row per request over the full caches)."""

    VRING = 4

    def __init__(self, weights, Hq: int, Hkv: int, prompts, x: int, bits: int = 4, R: int = 32,
                 max_new: int = 256, kv_dtype: str = "f32", host_past: bool = False,
                 chunk_tokens: int = 65536, rope_theta: float = 500000.0, copy_stream=None,
                 fused: bool = True, graphs: bool = False, margins: bool = False, device: str = "cuda"):
        assert "g_att" in weights, "Llama-form weights"
        self.E, self.Wlm = _dev(weights["E"], device), _dev(weights["Wlm"], device)
        self.g_f = _dev(weights["g_f"], device)
        lst = lambda k: [_dev(w, device) for w in weights[k]]
        self.g_att, self.g_mlp, self.Wo, self.W2 = lst("g_att"), lst("g_mlp"), lst("Wo"), lst("W2")
        self.Wqkv = [torch.cat([_dev(q, device), _dev(k, device), _dev(v, device)]).contiguous()
                     for q, k, v in zip(weights["Wq"], weights["Wk"], weights["Wv"])]
        self.W13 = [torch.cat([_dev(a, device), _dev(b, device)]).contiguous()
                    for a, b in zip(weights["W1"], weights["W3"])]
        self.nl, (self.V, self.dm) = len(self.Wqkv), self.E.shape
        assert self.dm % D == 0 and Hq % Hkv == 0
        assert not host_past or kv_dtype == "bf16", "a host-streamed cache is bf16"
        self.tdt = torch.float32 if kv_dtype == "f32" else torch.bfloat16
        self.vdt = vc.VC_F32 if kv_dtype == "f32" else vc.VC_BF16
        self.Hq, self.Hkv, self.x, self.R = Hq, Hkv, x, R
        self.L = L = x + 1
        self.host, self.chunk, self.device = host_past, chunk_tokens, device
        self.copy_stream = (copy_stream or torch.cuda.Stream()) if host_past else None
        prompts = [[int(t) for t in p] for p in prompts]
        self.B = B = len(prompts)
        self.n = [len(p) - 1 for p in prompts]
        self.cap = (max(self.n) + max_new + 2 * L + 63) // 32 * 32
        ang = np.arange(self.cap)[:, None] * rope_theta ** (-2.0 * np.arange(D // 2) / D)
        cos = torch.from_numpy(np.cos(ang).astype(np.float32)).to(device)
        sin = torch.from_numpy(np.sin(ang).astype(np.float32)).to(device)
        self.cs = torch.stack([torch.cat([cos, cos], 1), torch.cat([-sin, sin], 1)], 1).contiguous()
        self.cos, self.sin = cos.contiguous(), sin.contiguous()
        self.fused, self.graphs = fused, graphs
        self.capture_stream = torch.cuda.Stream(device=device) if fused and graphs else None
        if fused:  # the fused one-row products read bf16 copies of bf16-valued weights (the same
            # values, half the bytes), else the fp32 weights themselves
            ws_ = self.Wqkv + self.Wo + self.W13 + self.W2 + [self.Wlm]
            exact = all(torch.equal(w.to(torch.bfloat16).float(), w) for w in ws_)
            bf = (lambda w: w.to(torch.bfloat16).contiguous()) if exact else (lambda w: w)
            self.Wqkv_b, self.Wo_b = [bf(w) for w in self.Wqkv], [bf(w) for w in self.Wo]
            self.W13_b, self.W2_b, self.Wlm_b = [bf(w) for w in self.W13], [bf(w) for w in self.W2], bf(self.Wlm)
            # one workspace for the step's products (they run in order on one stream): the
            # matrix-core form where the weights are bf16, zero-filled once
            need = [vc.vc_decoder_gemv_workspace(e, vc.dtype_code(w), w.shape[0], w.shape[1], B)
                    for e, w in ((vc.VC_DEC_ROPE, self.Wqkv_b[0]), (vc.VC_DEC_ADD, self.Wo_b[0]),
                                 (vc.VC_DEC_SWIGLU, self.W13_b[0]), (vc.VC_DEC_ADD, self.W2_b[0]),
                                 (vc.VC_DEC_STORE, self.Wlm_b))]
            self.ws_dec = torch.zeros(max(need), dtype=torch.uint8, device=device) if max(need) else None
        f32 = dict(dtype=torch.float32, device=device)
        tk = dict(dtype=self.tdt, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        nl = self.nl
        self.stores = [[_Store(Hkv, self.cap, self.tdt, host_past, device) for _ in range(nl)]
                       for _ in range(B)]
        meta = vc.VC_F32 if kv_dtype == "f32" else vc.VC_F16
        res_cap = (R + 32 + L + 31) // 32 * 32
        # per layer one batched KIVI cache; request b's row is self.caches[l].row(b)
        self.caches = [vc.KiviCache(B, Hkv, self.cap, bits, meta, meta, res_cap, device) for _ in range(nl)]
        self.n_q = [32 * (max(0, n - R) // 32) for n in self.n]
        self.qkvc = torch.zeros((B, Hq + 2 * Hkv, D), **tk)       # draft rows' q, k, v
        self.qd = torch.zeros((B, Hq, D), **tk)                   # fused step: q, k, v apart
        self.kd = torch.zeros((B, Hkv, D), **tk)
        self.vd = torch.zeros((B, Hkv, D), **tk)
        self.Xd = torch.zeros((B, self.dm), **f32)                 # fused step: residual stream
        self.Hd = torch.zeros((B, self.W13[0].shape[0] // 2), **f32)
        self.logits_d = torch.zeros((B, self.V), **f32)            # fused step: head logits
        self.acc_d = torch.zeros((B,), **i32)
        self.next_d = torch.zeros((B,), **i32)
        self.pos_d = torch.zeros((B,), **i32)                      # n_b (row positions = n_b + j)
        self.nq_d = torch.zeros((B,), dtype=torch.int64, device=device)  # n_q_b
        self.r0_d = torch.zeros((B,), **i32)                       # n_b - n_q_b (step j: + j + 1)
        self.graph, self.graph_key = None, None                    # captured fused draft phase
        self.od = torch.zeros((B, Hq, D), **f32)
        self.lse_d = torch.zeros((B, Hq), **f32)
        self.qv = torch.zeros((B, Hq, L, D), **tk)
        self.kv_ = [torch.zeros((B, Hkv, L, D), **tk) for _ in range(nl)]  # verifier's k, v
        self.vv_ = [torch.zeros((B, Hkv, L, D), **tk) for _ in range(nl)]
        # host stores: the round's block rows reach pinned staging in one copy per layer and
        # tensor, then the kept rows go to each request's store by CPU slice copies (int16 views of
        # the bf16 rows), instead of two synchronous device-to-host copies per (request, layer)
        if host_past:
            pin = lambda: torch.empty((B, Hkv, L, D), dtype=self.tdt, pin_memory=True)
            self.stage_k, self.stage_v = [pin() for _ in range(nl)], [pin() for _ in range(nl)]
            i16 = lambda t: t.view(torch.int16).numpy()
            self.stage_np = [(i16(k), i16(v)) for k, v in zip(self.stage_k, self.stage_v)]
        self.ov = torch.zeros((B, Hq, L, D), **f32)
        self.lse_v = torch.zeros((B, Hq, L), **f32)
        self.logits_v = torch.zeros((B, L, self.V), **f32)
        self.tok = torch.zeros((B, L + 1), **i32)   # per request: block entries 0..x (+ spare)
        self.accept_len = torch.zeros((B,), **i32)
        self.next_tok = torch.zeros((B,), **i32)
        self.argmax_v = torch.zeros((B, L), **i32)
        # margins=True: the top-2 logit gap of the row each emitted token was chosen from, per
        # request (self.margin_log), for token-by-token comparisons with near-ties set apart
        self.margins = margins
        self.gap_v = torch.zeros((B, L), **f32)
        self.margin_log = [[] for _ in range(B)]
        self.ws_draft = vc.Workspace(device)
        self.ws_verify = vc.Workspace(device)
        self.vring = [vc.Workspace(device) for _ in range(self.VRING)] if host_past else []
        self._pf, self._pf_open = 0, False  # verify calls whose copies are issued this round
        self.ws_proj = torch.zeros((vc.vc_project_workspace(B, 1, self.V) + 3) // 4, **i32)
        for b, p in enumerate(prompts):
            self._prefill(b, p)
        self.tok[:, 0] = torch.tensor([p[-1] for p in prompts], **i32)
        self._upload_lengths()
        self.rounds = [[] for _ in range(B)]

    # ---- the layer outside attention, over all rows ------------------------------------------
    def _rms(self, X, g):
        return torch.nn.functional.rms_norm(X, (self.dm,), g, 1e-5)

    def _qkv(self, l: int, X, pos):
        """Rows X [m, dm] at positions pos (device int64 [m]) -> [m, Hq + 2 Hkv, 128] fp32 with q
        and k rotated."""
        Y = (self._rms(X, self.g_att[l]) @ self.Wqkv[l].T).view(X.shape[0], -1, D)
        cs = self.cs.index_select(0, pos)
        qk = Y[:, :self.Hq + self.Hkv]
        r = torch.roll(qk, D // 2, dims=-1)
        qk.mul_(cs[:, 0:1])
        qk.addcmul_(r, cs[:, 1:2])
        return Y

    def _block_out(self, l: int, X, O):
        X = X + O @ self.Wo[l].T
        Z = self._rms(X, self.g_mlp[l]) @ self.W13[l].T
        F = Z.shape[-1] // 2
        return X + (torch.nn.functional.silu(Z[:, :F]) * Z[:, F:]) @ self.W2[l].T

    def _prefetch(self, upto: int):
        """Issue the copies of this round's verify calls self._pf .. upto - 1 (call l B + b: layer
        l, request b), each into its ring workspace, after the compute work enqueued so far (which
        holds the last call that used that workspace)."""
        while self._pf < min(upto, self.nl * self.B):
            i = self._pf
            l, b = divmod(i, self.B)
            n, st = self.n[b], self.stores[b][l]
            nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, n, True, self.chunk, self.vdt)
            vc.vc_verify_prefetch(st.k, st.v, n, self.vring[i % self.VRING].get(nb), 1, self.Hq, self.Hkv,
                                  self.L, self.chunk, past_stride=self.cap, copy_stream=self.copy_stream)
            self._pf += 1

    def _verify(self, b: int, l: int, q, k, v, n: int, out, lse):
        host = self.host and n > 0
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, q.shape[2], n, host, self.chunk, self.vdt)
        st = self.stores[b][l]
        kp, vp, stride = (st.k, st.v, self.cap) if n > 0 else (k, v, q.shape[2])
        if host and q.shape[2] == self.L:  # a round's verify: through the prefetch ring
            i = l * self.B + b
            self._prefetch(i + self.VRING)
            vc.vc_verify_attn(q, k, v, kp, vp, n, out, lse, self.vring[i % self.VRING].get(nb), SM_SCALE,
                              past_stride=stride, past_on_host=vc.VC_PAST_HOST_PREFETCHED,
                              chunk_tokens=self.chunk, copy_stream=self.copy_stream)
            return
        vc.vc_verify_attn(q, k, v, kp, vp, n, out, lse, self.ws_verify.get(nb), SM_SCALE,
                          past_stride=stride, past_on_host=host, chunk_tokens=self.chunk,
                          copy_stream=self.copy_stream)

    def _prefill(self, b: int, prompt):
        """Request b's positions 0..n-1, layer by layer: caches, then causal attention over the
        layer's device-resident keys/values (_causal_attention)."""
        n, Hq, Hkv = self.n[b], self.Hq, self.Hkv
        X = self.E[torch.tensor(prompt[:n], device=self.device)]
        pos = torch.arange(n, device=self.device)
        lay = lambda Y: Y.transpose(0, 1).unsqueeze(0).to(self.tdt).contiguous()
        for l in range(self.nl):
            Y = self._qkv(l, X, pos)
            Q, K, V = Y[:, :Hq], lay(Y[:, Hq:Hq + Hkv]), lay(Y[:, Hq + Hkv:])
            self.stores[b][l].write(0, K, V)
            c, nq = self.caches[l].row(b), self.n_q[b]
            if nq:
                vc.vc_quantize_kv(c, K, V, 0, nq, src_bh_stride=n * D)
            if n > nq:
                vc.vc_kivi_append(c, K[:, :, nq:], V[:, :, nq:], nq, n - nq, src_bh_stride=n * D)
            O = _causal_attention(lay(Q), K, V, n, Hq, Hkv, self.vdt, self.ws_verify, self.device)
            X = self._block_out(l, X, O)

    # ---- one round ------------------------------------------------------------------------
    def draft_step(self, j: int):
        if self.fused:
            return self._draft_step_fused(j, *self._phase_bounds())
        Hq, Hkv, B = self.Hq, self.Hkv, self.B
        pos = torch.tensor([n + j for n in self.n], device=self.device)
        X = self.E[self.tok[:, j].long()]
        for l in range(self.nl):
            self.qkvc.copy_(self._qkv(l, X, pos))
            for b in range(B):
                c, nq = self.caches[l].row(b), self.n_q[b]
                r = self.n[b] - nq + j + 1
                nb = vc.vc_draft_quant_workspace(c, nq, r, Hq)
                vc.vc_draft_attn_quant(c, nq, r, self.qkvc[b:b + 1, :Hq], self.od[b:b + 1],
                                       self.lse_d[b:b + 1], self.ws_draft.get(nb), SM_SCALE,
                                       k_new=self.qkvc[b:b + 1, Hq:Hq + Hkv],
                                       v_new=self.qkvc[b:b + 1, Hq + Hkv:])
            X = self._block_out(l, X, self.od.view(B, -1))
        h = self._rms(X, self.g_f)
        vc.vc_project_logits(self.Wlm, h.view(B, -1, D), argmax=self.tok.view(-1)[j + 1:],
                             argmax_b_stride=self.L + 1, ws=self.ws_proj)

    def _draft_step_fused(self, j: int, nq_max: int, r_max: int):
        """Draft step j of every request as libvc launches: the embedding gather, then per layer
        norm + q/k/v + rotation, the batch's draft attention (each row its own lengths from the
        device arrays, the step's key/value stored into each row's residual), output product into
        the residual, norm + gate/up + SwiGLU, down product into the residual; final norm and the
        head's greedy argmax into block entry j + 1. Host work is fixed per step (no lengths read),
        so the whole draft phase can be captured once and replayed."""
        Hq, Hkv, B = self.Hq, self.Hkv, self.B
        X = self.Xd
        vc.vc_embed_rows(self.E, self.tok[:, j], X)
        ws = self.ws_draft.get(vc.vc_draft_quant_workspace(self.caches[0], nq_max, r_max, Hq))
        for l in range(self.nl):
            vc.vc_decoder_gemv(vc.VC_DEC_ROPE, self.Wqkv_b[l], X, norm_gain=self.g_att[l], q_out=self.qd,
                               k_out=self.kd, v_out=self.vd, Hq=Hq, Hkv=Hkv, cos_t=self.cos,
                               sin_t=self.sin, pos=self.pos_d, pos_add=j, ws=self.ws_dec)
            vc.vc_draft_attn_quant_rows(self.caches[l], self.nq_d, self.r0_d, j + 1, nq_max, r_max, self.qd,
                                        self.od, self.lse_d, ws, SM_SCALE, k_new=self.kd, v_new=self.vd)
            vc.vc_decoder_gemv(vc.VC_DEC_ADD, self.Wo_b[l], self.od.view(B, -1), out=X, ws=self.ws_dec)
            vc.vc_decoder_gemv(vc.VC_DEC_SWIGLU, self.W13_b[l], X, norm_gain=self.g_mlp[l], out=self.Hd,
                               ws=self.ws_dec)
            vc.vc_decoder_gemv(vc.VC_DEC_ADD, self.W2_b[l], self.Hd, out=X, ws=self.ws_dec)
        # head: final norm fused into the logits product, then each row's greedy argmax
        vc.vc_decoder_gemv(vc.VC_DEC_STORE, self.Wlm_b, X, norm_gain=self.g_f, out=self.logits_d,
                           ws=self.ws_dec)
        vc.vc_accept(self.logits_d.view(B, 1, -1), None, self.acc_d, self.next_d)
        self.tok[:, j + 1].copy_(self.next_d)

    def _phase_bounds(self):
        """(n_q_max, r_max) the fused draft phase is launched with: the largest quantised prefix
        rounded up to 128 tokens and the residual ring's capacity, so that the launch shape (and a
        captured phase) stays the same over many rounds."""
        nq_max = min(self.caches[0].tok_cap, (max(self.n_q) + 127) // 128 * 128)
        return nq_max, self.caches[0].res_cap

    def verify_step(self):
        Hq, Hkv, B, L = self.Hq, self.Hkv, self.B, self.L
        if not self._pf_open:  # no draft phase issued this round's first copies
            self._pf = 0
        self._pf_open = False
        pos = (torch.tensor(self.n, device=self.device)[:, None]
               + torch.arange(L, device=self.device)).view(-1)
        X = self.E[self.tok[:, :L].reshape(-1).long()]
        for l in range(self.nl):
            Y = self._qkv(l, X, pos).view(B, L, -1, D)
            self.qv.copy_(Y[:, :, :Hq].transpose(1, 2))
            self.kv_[l].copy_(Y[:, :, Hq:Hq + Hkv].transpose(1, 2))
            self.vv_[l].copy_(Y[:, :, Hq + Hkv:].transpose(1, 2))
            for b in range(B):
                self._verify(b, l, self.qv[b:b + 1], self.kv_[l][b:b + 1], self.vv_[l][b:b + 1],
                             self.n[b], self.ov[b:b + 1], self.lse_v[b:b + 1])
            X = self._block_out(l, X, self.ov.transpose(1, 2).reshape(B * L, -1))
        h = self._rms(X, self.g_f).view(B, L, -1, D).permute(0, 2, 1, 3).contiguous()
        vc.vc_project_logits(self.Wlm, h, logits=self.logits_v)
        drafts = self.tok[:, 1:L].contiguous() if L > 1 else None
        vc.vc_accept(self.logits_v, drafts, self.accept_len, self.next_tok, self.argmax_v)
        if self.margins:
            vc.vc_logit_margins(self.logits_v, self.gap_v)

    def commit(self):
        """Per request: keep entries 0..a_b (the verifier's keys/values) in the full caches and the
        residual rings, flush whole groups, start the next round from the emitted token. Returns
        each request's emitted tokens."""
        if self.host:  # every layer's block rows to pinned staging (complete at the sync below)
            for l in range(self.nl):
                self.stage_k[l].copy_(self.kv_[l], non_blocking=True)
                self.stage_v[l].copy_(self.vv_[l], non_blocking=True)
        acc = self.accept_len.tolist()
        nxt = self.next_tok.tolist()
        toks = self.tok.tolist()
        gaps = self.gap_v.tolist() if self.margins else None
        L, out = self.L, []
        for b in range(self.B):
            a = acc[b]
            out.append(toks[b][1:a + 1] + [nxt[b]])
            if gaps is not None:
                self.margin_log[b] += gaps[b][:a + 1]
            n0 = self.n[b]
            assert n0 + a + 1 + L <= self.cap, "cache capacity exhausted (raise max_new)"
            for l in range(self.nl):
                k, v = self.kv_[l][b:b + 1, :, :a + 1], self.vv_[l][b:b + 1, :, :a + 1]
                if self.host:
                    st, (sk, sv) = self.stores[b][l], self.stage_np[l]
                    st.k_np[0, :, n0:n0 + a + 1] = sk[b, :, :a + 1]
                    st.v_np[0, :, n0:n0 + a + 1] = sv[b, :, :a + 1]
                else:
                    self.stores[b][l].write(n0, k, v)
                vc.vc_kivi_append(self.caches[l].row(b), k, v, n0, a + 1, src_bh_stride=L * D)
            self.n[b] = n0 + a + 1
            while self.n[b] - self.n_q[b] >= self.R + 32:
                g0 = self.n_q[b]
                for l in range(self.nl):
                    Kg, Vg, stride = self.stores[b][l].device_rows(g0, g0 + 32)
                    vc.vc_quantize_kv(self.caches[l].row(b), Kg, Vg, g0, 32, src_bh_stride=stride)
                self.n_q[b] = g0 + 32
            self.rounds[b].append(a)
        self.tok[:, 0] = self.next_tok
        self._upload_lengths()
        return out

    def _upload_lengths(self):
        """Each request's position and KIVI split (device copies read by the fused draft step)."""
        self.pos_d.copy_(torch.tensor(self.n, dtype=torch.int32))
        self.nq_d.copy_(torch.tensor(self.n_q, dtype=torch.int64))
        self.r0_d.copy_(torch.tensor([n - q for n, q in zip(self.n, self.n_q)], dtype=torch.int32))

    def warm(self):
        """Size the workspaces for the largest context this decoder can reach."""
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.cap, self.host, self.chunk, self.vdt)
        self.ws_verify.get(nb)
        for w in self.vring:
            w.get(nb)
        r = self.R + 32 + self.L
        self.ws_draft.get(vc.vc_draft_quant_workspace(self.caches[0], (self.cap - r) // 32 * 32, r,
                                                      self.Hq))
        torch.cuda.synchronize()

    def draft_phase(self):
        """The x draft steps. Fused: replayed from a HIP graph of the whole phase, captured on first
        use and again whenever the launch bounds change (every kernel of the phase reads the
        requests' lengths and positions from device memory, so one capture serves many rounds).
        With host-resident full caches the round's first verify copies are issued first."""
        if self.host:
            self._pf, self._pf_open = 0, True
            self._prefetch(self.VRING)
        if not (self.fused and self.graphs) or self.x == 0:
            for j in range(self.x):
                self.draft_step(j)
            return
        key = self._phase_bounds()
        if self.graph is None or self.graph_key != key:
            for j in range(self.x):  # eager once (sizes the workspace, loads the kernels)
                self._draft_step_fused(j, *key)
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph, stream=self.capture_stream):
                for j in range(self.x):
                    self._draft_step_fused(j, *key)
            self.graph_key = key
            return
        self.graph.replay()

    def set_round_inputs(self):
        """Nothing to load: each request's next round starts from its committed token (for the
        schedules in harness)."""

    def generate(self, steps: int):
        """Rounds until every request has `steps` more tokens; returns each request's tokens."""
        out = [[] for _ in range(self.B)]
        while min(len(o) for o in out) < steps:
            self.draft_phase()
            self.verify_step()
            for o, em in zip(out, self.commit()):
                o += em
        return [o[:steps] for o in out]
