"""One synthetic single-layer draft/verify round on the GPU, driven through libvc.

Device memory and streams come from PyTorch; every attention, quantisation, cache-append, logits,
argmax and accept step is a libvc call. The stand-in logits projection (z = W o, an fp32 product in
place of the model's LM head) is libvc's projection kernel: fused with the greedy argmax for the
draft steps, followed by the accept kernel for the B*L verify rows. Inputs come from the seeded
generator (kv_cache_compressed_amd.synth).

Round ("VeriCache: making lossy KV compression exact", The Core Idea): x draft steps over the
compressed cache (each: draft attention with the step's key/value appended by the same launch,
logits with the greedy argmax), one verify pass of x+1 rows over the full cache, logits, accept.
"""
from __future__ import annotations

import queue
import threading
import time

import numpy as np
import torch

from . import synth, vc

SM_SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


def kivi_split(n: int, R: int, group: int = 32) -> int:
    """Quantised prefix of a KIVI cache holding n tokens: whole groups, leaving at least R tokens in
    the full-precision residual (group * floor(max(0, n - R) / group)). Commits keep this true by
    flushing a group whenever the residual reaches R + group tokens."""
    return group * (max(0, n - R) // group)


def _dev(x: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


class RoundState:
    """Device state of one workload: caches, inputs, outputs and workspaces."""

    def __init__(self, w: synth.Workload, seed: int = 0, device: str = "cuda", inputs=None,
                 idx_lists=None, replicas: int = 1, copy_stream=None, extra_tokens: int = 0):
        self.w, self.seed, self.device = w, seed, device
        if inputs is None:
            K, V = synth.kv_past(w, seed)
            Kn, Vn = synth.kv_new(w, seed)
            inputs = (K, V, Kn, Vn, synth.q_new(w, seed), synth.projection(w, seed))
        K, V, Kn, Vn, Q, W = inputs
        tdt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
        self.tdt = tdt
        B, Hkv, Hq, L, n, x = w.B, w.Hkv, w.Hq, w.L, w.n, w.x
        # round block (positions n .. n+x): keys/values and queries
        self.k_blk = _dev(Kn, tdt, device)
        self.v_blk = _dev(Vn, tdt, device)
        self.q_verify = _dev(Q, tdt, device)                                   # [B, Hq, L, 128]
        self.q_draft = self.q_verify.permute(2, 0, 1, 3).contiguous()          # [L, B, Hq, 128]
        self.W = _dev(W, torch.float32, device)                                # [V, Hq*128]
        # full cache: device store [B, Hkv, tok_cap, 128] (past + block), or pinned host past
        # (extra_tokens: room for a multi-round decode to grow the context past n + L)
        cap = (w.tok_cap + extra_tokens + 31) // 32 * 32
        self.cap = cap
        self.n = n                                   # cached (committed) tokens
        self.n_q = kivi_split(n, w.R, w.group) if w.drafter == "kivi" else 0  # of which quantised
        if w.past_on_host:
            self.host_cap = n + extra_tokens
            self.k_host = torch.empty((B, Hkv, self.host_cap, 128), dtype=tdt, pin_memory=True)
            self.v_host = torch.empty_like(self.k_host, pin_memory=True)
            self.k_host[:, :, :n].copy_(torch.from_numpy(K).to(tdt))
            self.v_host[:, :, :n].copy_(torch.from_numpy(V).to(tdt))
            self.k_store = self.v_store = None
        else:
            self.k_store = torch.zeros((B, Hkv, cap, 128), dtype=tdt, device=device)
            self.v_store = torch.zeros_like(self.k_store)
            self.k_store[:, :, :n] = _dev(K, tdt, device)
            self.v_store[:, :, :n] = _dev(V, tdt, device)
            self.k_store[:, :, n:n + L] = self.k_blk
            self.v_store[:, :, n:n + L] = self.v_blk
        # drafter caches
        self.ws_draft = vc.Workspace(device)
        self._ws_sizes = {}
        self.ws_verify = vc.Workspace(device)
        self.replicas = []
        if w.drafter == "kivi":
            if w.past_on_host:  # prefill: quantise from a temporary device copy of the past
                kt = _dev(K, tdt, device)
                vt = _dev(V, tdt, device)
                src = (kt, vt, n * 128)
            else:
                src = (self.k_store, self.v_store, cap * 128)
            # Replicas hold identical copies of the quantised codes/metadata (so consecutive draft
            # steps can read different copies, as the layers of a real model would); they share one
            # residual ring, to which each draft-round entry is appended once.
            for k in range(max(1, replicas)):
                c = vc.KiviCache(B, Hkv, (max(self.n_q, 32) + extra_tokens + 31) // 32 * 32, w.bits,
                                 vc.VC_F16 if w.meta_dtype == "f16" else vc.VC_F32,
                                 vc.VC_F16 if w.res_dtype == "f16" else vc.VC_F32, w.res_cap, device)
                nq = self.n_q
                vc.vc_quantize_kv(c, src[0], src[1], 0, nq, src_bh_stride=src[2])
                if k == 0:
                    if n > nq:
                        vc.vc_kivi_append(c, src[0][:, :, nq:], src[1][:, :, nq:], nq, n - nq,
                                          src_bh_stride=src[2])
                else:
                    c.k_res, c.v_res = self.replicas[0].k_res, self.replicas[0].v_res
                self.replicas.append(c)
            if w.past_on_host:
                torch.cuda.synchronize()
                del kt, vt
        else:
            # kept positions of every (b, kv head): selected on the GPU from the seeded scores
            # (vc_select_keep), or taken from `idx_lists` when the caller gives them; the round's
            # own positions n .. n+x-1 follow, appended as the draft steps reach them
            if idx_lists is None:
                kept = self.keep_count(w)
                self.scores = torch.zeros((B, Hkv, (n + 3) // 4 * 4), dtype=torch.float32, device=device)
                self.scores[:, :, :n] = torch.from_numpy(
                    np.stack([np.stack([synth.scores(w, seed, b, h) for h in range(Hkv)]) for b in range(B)]))
                self.idx = torch.empty((B, Hkv, kept + x), dtype=torch.int32, device=device)
                got = self.select_keep()
                assert got == kept, (got, kept)
            else:
                kept = len(idx_lists[0][0])
                idx = np.zeros((B, Hkv, kept + x), np.int32)
                for b in range(B):
                    for h in range(Hkv):
                        idx[b, h, :kept] = idx_lists[b][h]
                self.idx = torch.from_numpy(idx).to(device)
            self.idx[:, :, kept:] = torch.arange(n, n + x, dtype=torch.int32, device=device)
            self.kept = kept
        # outputs
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.out_d = torch.zeros((x, B, Hq, 128), **f32)
        self.lse_d = torch.zeros((x, B, Hq), **f32)
        self.logits_d = torch.zeros((x, B, w.vocab), **f32)
        self.drafts = torch.zeros((B, x), **i32)
        self.out_v = torch.zeros((B, Hq, L, 128), **f32)
        self.lse_v = torch.zeros((B, Hq, L), **f32)
        self.logits_v = torch.zeros((B, L, w.vocab), **f32)
        self.accept_len = torch.zeros((B,), **i32)
        self.next_tok = torch.zeros((B,), **i32)
        self.argmax_v = torch.zeros((B, L), **i32)
        # host-streamed verify: the stream its chunk copies go on (may be shared between groups)
        self.copy_stream = None
        if w.past_on_host:
            self.copy_stream = copy_stream or torch.cuda.Stream(device=device)
        # host-streamed rounds: issue the verify's first two chunk copies when the round starts
        self.prefetch_verify, self._prefetched = bool(w.past_on_host), None
        # projection workspace (draft argmax tickets); zero-filled once, calls leave it zero
        self.ws_proj = torch.zeros((vc.vc_project_workspace(B, 1, w.vocab) + 3) // 4, **i32)
        self._rep = 0
        self.verify_ws_bytes = vc.vc_verify_workspace(B, Hq, Hkv, L, n, w.past_on_host,
                                                      w.chunk_tokens, self._vdt())

    @staticmethod
    def keep_count(w: synth.Workload) -> int:
        """Kept positions per (b, kv head) of the token-dropping workload: sinks + recent + the
        selected middle (the count vc_select_keep returns)."""
        lo = min(w.sinks, w.n)
        hi = max(lo, w.n - w.recent)
        fixed = lo + (w.n - hi)
        return fixed + min(max(0, w.keep - fixed), hi - lo)

    def select_keep(self) -> int:
        """Select the kept positions from the scores into idx[:, :, :kept] (vc_select_keep)."""
        w = self.w
        return vc.vc_select_keep(self.scores, w.n, w.sinks, w.recent, w.keep, self.idx)

    def _vdt(self):
        return vc.VC_BF16 if self.w.kv_dtype == "bf16" else vc.VC_F32

    # ---- steps ---------------------------------------------------------------------------
    def draft_attention(self, j: int, cache=None, append: bool = True):
        """Draft attention of step j (position n+j) into out_d[j], lse_d[j]. With the KIVI drafter
        the step's own key/value is first stored into the residual ring by the same launch
        (append=False leaves the ring as it is, e.g. after append_draft_entry)."""
        w = self.w
        if w.drafter == "kivi":
            c = cache or self.replicas[0]
            r = (self.n - self.n_q) + j + 1
            key = (id(c), self.n_q, r)
            nb = self._ws_sizes.get(key)
            if nb is None:
                nb = self._ws_sizes[key] = vc.vc_draft_quant_workspace(c, self.n_q, r, w.Hq)
            kn = vn = None
            if append:  # the step's own key/value goes into the (shared) residual ring in-kernel
                kn, vn = self.k_blk[:, :, j], self.v_blk[:, :, j]
            vc.vc_draft_attn_quant(c, self.n_q, r, self.q_draft[j], self.out_d[j], self.lse_d[j],
                                   self.ws_draft.get(nb), SM_SCALE, k_new=kn, v_new=vn)
        else:
            n_keep = self.kept + j + 1
            nb = vc.vc_draft_drop_workspace(w.B, w.Hkv, w.Hq, n_keep)
            vc.vc_draft_attn_drop(self.k_store, self.v_store, self.idx, n_keep, self.q_draft[j],
                                  self.out_d[j], self.lse_d[j], self.ws_draft.get(nb), SM_SCALE)

    def append_draft_entry(self, j: int):
        """Append the key/value of position n+j to the (shared) residual ring."""
        w = self.w
        if w.drafter == "kivi":
            vc.vc_kivi_append(self.replicas[0], self.k_blk[:, :, j], self.v_blk[:, :, j], self.n + j, 1,
                              src_bh_stride=w.L * 128)

    def draft_step(self, j: int):
        c = None
        if self.replicas:
            c = self.replicas[self._rep % len(self.replicas)]
            self._rep += 1
        self.draft_attention(j, c)
        self.draft_tokens(j)

    def _verify_ws(self):
        w = self.w
        if self.n != w.n:  # a multi-round decode has grown the context
            self.verify_ws_bytes = vc.vc_verify_workspace(w.B, w.Hq, w.Hkv, w.L, self.n, w.past_on_host,
                                                          w.chunk_tokens, self._vdt())
        return self.ws_verify.get(self.verify_ws_bytes)

    def prefetch(self):
        """Host-streamed past: the copies of this round's first two verify chunks, issued now (the
        committed past is fixed before the drafts exist) so they cross the link under the draft
        steps; the round's verify skips them."""
        w = self.w
        vc.vc_verify_prefetch(self.k_host, self.v_host, self.n, self._verify_ws(), w.B, w.Hq, w.Hkv,
                              w.L, w.chunk_tokens, past_stride=self.host_cap,
                              copy_stream=self.copy_stream)
        self._prefetched = self.n

    def verify_attention(self):
        w = self.w
        ws = self._verify_ws()
        if w.past_on_host:
            mode = vc.VC_PAST_HOST_PREFETCHED if self._prefetched == self.n else vc.VC_PAST_HOST
            self._prefetched = None
            vc.vc_verify_attn(self.q_verify, self.k_blk, self.v_blk, self.k_host, self.v_host, self.n,
                              self.out_v, self.lse_v, ws, SM_SCALE, past_stride=self.host_cap,
                              past_on_host=mode, chunk_tokens=w.chunk_tokens,
                              copy_stream=self.copy_stream)
        else:
            vc.vc_verify_attn(self.q_verify, self.k_blk, self.v_blk, self.k_store, self.v_store, self.n,
                              self.out_v, self.lse_v, ws, SM_SCALE, past_stride=self.cap)

    def draft_tokens(self, j: int):
        """Logits of draft step j and its greedy token, written straight into drafts[:, j]."""
        vc.vc_project_logits(self.W, self.out_d[j], logits=self.logits_d[j], argmax=self.drafts[:, j],
                             argmax_b_stride=self.w.x, ws=self.ws_proj)

    def verify_tokens(self):
        """Logits of the B*L verify rows (the projection kernel, reading the outputs in their
        [B, Hq, L, 128] layout), then the greedy accept against the drafts."""
        vc.vc_project_logits(self.W, self.out_v, logits=self.logits_v)
        vc.vc_accept(self.logits_v, self.drafts, self.accept_len, self.next_tok, self.argmax_v)

    def verify_step(self):
        w = self.w
        self.verify_attention()
        self.verify_tokens()

    # ---- multi-round decode of one request ------------------------------------------------
    def set_round_inputs(self, K_new, V_new, Q):
        """Load the next round's block keys/values [B, Hkv, L, d] and queries [B, Hq, L, d] (host
        arrays) into the round's device tensors, in place."""
        self.k_blk.copy_(torch.from_numpy(np.ascontiguousarray(K_new)).to(self.tdt))
        self.v_blk.copy_(torch.from_numpy(np.ascontiguousarray(V_new)).to(self.tdt))
        q = torch.from_numpy(np.ascontiguousarray(Q)).to(self.tdt)
        self.q_verify.copy_(q)
        self.q_draft.copy_(q.permute(2, 0, 1, 3))

    def commit(self) -> int:
        """After a round of a single request (B = 1, KIVI drafter): commit the
        accepted drafts and the verifier's token, i.e. positions n .. n+a, whose keys/values the
        round's block holds, to the full store (in HBM, or in pinned host memory when the verify
        streams it; the draft steps already stored positions n .. n+x-1
        in the residual ring; when all x drafts stand, position n+x is appended here); then flush whole 32-token groups of the oldest residual tokens into the codes of
        every replica while the residual holds R + 32 or more tokens ("VeriCache: Turning Lossy KV
        Cache into Lossless LLM Inference", Key Contributions: the compressor interface; the
        quantised groups are taken from the full-precision store). Returns a. The entry points take
        one length for the whole batch, so rows that accept different counts would need per-row
        lengths; this loop runs one request."""
        w = self.w
        assert w.B == 1 and w.drafter == "kivi"
        a = int(self.accept_len[0].item())
        n0, n1 = self.n, self.n + a + 1
        if w.past_on_host:  # the full cache lives in pinned host memory
            assert n1 <= self.host_cap, "host store capacity exhausted (raise extra_tokens)"
            self.k_host[:, :, n0:n1].copy_(self.k_blk[:, :, :a + 1])
            self.v_host[:, :, n0:n1].copy_(self.v_blk[:, :, :a + 1])
        else:
            assert n1 + w.L <= self.cap, "store capacity exhausted (raise extra_tokens)"
            self.k_store[:, :, n0:n1] = self.k_blk[:, :, :a + 1]
            self.v_store[:, :, n0:n1] = self.v_blk[:, :, :a + 1]
        if a == w.x:  # every draft stood: the bonus position n + x was never drafted, so its
            # key/value is not in the residual ring yet (the draft steps wrote n .. n+x-1)
            vc.vc_kivi_append(self.replicas[0], self.k_blk[:, :, w.x], self.v_blk[:, :, w.x], n0 + w.x, 1,
                              src_bh_stride=w.L * 128)
        self.n = n1
        while self.n - self.n_q >= w.R + w.group:
            g0, g1 = self.n_q, self.n_q + w.group
            if w.past_on_host:  # the group's exact keys/values, staged on the device
                ks = self.k_host[:, :, g0:g1].to(self.k_blk.device)
                vs = self.v_host[:, :, g0:g1].to(self.k_blk.device)
                src = (ks, vs, w.group * 128)
            else:
                src = (self.k_store[:, :, g0:], self.v_store[:, :, g0:], self.cap * 128)
            for c in self.replicas:
                vc.vc_quantize_kv(c, src[0], src[1], g0, w.group, src_bh_stride=src[2])
            self.n_q = g1
        return a

    def draft_phase(self):
        """The x draft steps of one round (attention with the step's append fused in, then the
        logits and greedy token), rotating over the compressed-cache replicas."""
        if self.prefetch_verify:
            self.prefetch()
        for j in range(self.w.x):
            self.draft_step(j)

    def run_round(self, timer=None):
        """One round. `timer`, if given, is called as timer(kind, start) with kind in
        {"draft", "verify"} right before (start=True) and after (start=False) each attention
        launch, on the host thread that enqueues them (for event timing on the current stream)."""
        w = self.w
        if self.prefetch_verify:
            self.prefetch()
        for j in range(w.x):
            c = None
            if self.replicas:
                c = self.replicas[self._rep % len(self.replicas)]
                self._rep += 1
            if timer:
                timer("draft", True)
            self.draft_attention(j, c)
            if timer:
                timer("draft", False)
            self.draft_tokens(j)
        if timer:
            timer("verify", True)
        self.verify_attention()
        if timer:
            timer("verify", False)
        self.verify_tokens()

    # ---- algorithmic work (what the method must move / compute) -------------------------
    def draft_bytes(self, j: int) -> int:
        """Bytes one draft-attention launch of step j must move: codes + metadata of n_q quantised
        tokens, the r full-precision residual tokens, the queries in and the outputs out."""
        w = self.w
        if w.drafter == "kivi":
            meta_b = 2 if w.meta_dtype == "f16" else 4
            res_b = 2 if w.res_dtype == "f16" else 4
            per_tok = 2 * 128 * w.bits // 8 + (128 * 2 * meta_b) // 32 + 4 * 2 * meta_b
            nq = kivi_split(w.n, w.R, w.group)
            r = (w.n - nq) + j + 1
            kv = w.B * w.Hkv * (nq * per_tok + r * 2 * 128 * res_b)
        else:
            kv_b = 2 if w.kv_dtype == "bf16" else 4
            kv = w.B * w.Hkv * (self.kept + j + 1) * (2 * 128 * kv_b + 4)
        q_b = 2 if w.kv_dtype == "bf16" else 4
        return kv + w.B * w.Hq * (128 * q_b + 129 * 4)

    def draft_flops(self, j: int) -> int:
        w = self.w
        keys = (w.n + j + 1) if w.drafter == "kivi" else (self.kept + j + 1)
        return 4 * 128 * w.B * w.Hq * keys

    def verify_bytes(self) -> int:
        w = self.w
        kv_b = 2 if w.kv_dtype == "bf16" else 4
        return (w.B * w.Hkv * (w.n + w.L) * 2 * 128 * kv_b + w.B * w.Hq * w.L * 128 * kv_b
                + w.B * w.Hq * w.L * 129 * 4)

    def verify_flops(self) -> int:
        w = self.w
        keys = sum(w.n + i + 1 for i in range(w.L))
        return 4 * 128 * w.B * w.Hq * keys

    def capture_round(self):
        """Capture one whole round (every launch of run_round, in order) into a HIP graph, after an
        eager round that sizes every workspace. Each replay redoes the round on the same inputs:
        the residual appends rewrite the same ring slots, so replays are idempotent. Not for the
        host-streamed verify (its copy-stream events are not captured)."""
        assert not self.w.past_on_host, "graph capture covers HBM-resident rounds only"
        self.run_round()
        torch.cuda.synchronize()
        rep0 = self._rep
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.run_round()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self._rep = rep0
        self.graph = g
        return g

    def replay_round(self):
        self.graph.replay()

    def results(self) -> dict:
        torch.cuda.synchronize()
        return dict(drafts=self.drafts.cpu().numpy(), draft_logits=self.logits_d.cpu().numpy(),
                    verified=self.argmax_v.cpu().numpy(), verify_logits=self.logits_v.cpu().numpy(),
                    a=self.accept_len.cpu().numpy(), next=self.next_tok.cpu().numpy(),
                    out_d=self.out_d.cpu().numpy(), lse_d=self.lse_d.cpu().numpy(),
                    out_v=self.out_v.cpu().numpy(), lse_v=self.lse_v.cpu().numpy())


# ---- schedules over several request groups ------------------------------------------------
# "VeriCache: making lossy KV compression exact", Verifying Without Giving Back the Speedup and
# Figure 2; "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference", Key Contributions
# (cross-resource staggering). Drafting reads each group's compressed cache from HBM; verifying
# streams its full cache from host memory over PCIe. A lock-step schedule runs every group's
# draft phase and then every group's verify, so PCIe idles while the groups draft and HBM idles
# while they verify. The staggered schedule runs each group on a stream of its own and starts
# group g once group g-1 has finished its first draft phase, so one group's verify transfer
# overlaps the next group's drafting. The groups are independent requests: both schedules
# produce the same results, bit for bit.
#
# Streams and hardware queues: a process on this GPU gets 4 hardware queues, and streams beyond
# that share them; two streams on one queue run in submission order, which takes the overlap
# away (a draft phase queued behind another group's verify waits for its whole transfer). So the
# groups' compute streams must be few and distinct: group 0 on the current stream, one more
# stream per further group, and one copy stream shared by all groups (pass group 0's
# `copy_stream` to the other groups' constructors; their verifies take turns on the link anyway).
def lockstep(groups, rounds: int = 1):
    """`rounds` lock-step rounds on the current stream: all groups draft, then all verify."""
    for _ in range(rounds):
        for st in groups:
            st.draft_phase()
        for st in groups:
            st.verify_step()


def staggered(groups, streams, rounds: int = 1):
    """`rounds` rounds per group, group g on streams[g] (default priority), each round its draft
    phase then its verify. The verifies take turns on the host link: verify k (group k % G, round
    k // G) starts once verify k-1 has finished, and each group drafts its next round as soon as
    its own verify is done, i.e. while the next group's verify streams. Group g > 0 drafts its
    first round after group g-1's first draft phase. Work is enqueued in timeline order (the
    next group's draft phase before this group's verify). The current stream waits for every
    group stream at the end."""
    ng = len(groups)
    assert len(streams) == ng and ng >= 1
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    first_done = [torch.cuda.Event() for _ in range(ng)]
    verify_done = None

    def draft(k):  # draft phase of slot k = (group k % ng, round k // ng)
        g = k % ng
        if k < ng and g > 0:
            streams[g].wait_event(first_done[g - 1])
        with torch.cuda.stream(streams[g]):
            groups[g].draft_phase()
            if k < ng:
                first_done[g].record(streams[g])

    total = rounds * ng
    draft(0)
    for k in range(total):
        # the next slot's draft phase goes in first when it belongs to another group (with one
        # group it is this group's next round, which follows its verify)
        early = k + 1 < total and (k + 1) % ng != k % ng
        if early:
            draft(k + 1)
        s = streams[k % ng]
        if verify_done is not None:
            s.wait_event(verify_done)
        with torch.cuda.stream(s):
            groups[k % ng].verify_step()
        verify_done = torch.cuda.Event()
        verify_done.record(s)
        if k + 1 < total and not early:
            draft(k + 1)
    for s in streams:
        cur.wait_stream(s)


def lockstep_decode(groups, rounds: int, next_inputs):
    """`rounds` chained decode rounds of single-request groups on the current stream, lock-step:
    all groups draft, all verify, then each commits and loads its next round's inputs
    (next_inputs(g, r) -> (K_new, V_new, Q) for round r >= 1). Returns the accepted counts per
    group."""
    acc = [[] for _ in groups]
    for r in range(rounds):
        for st in groups:
            st.draft_phase()
        for st in groups:
            st.verify_step()
        for g, st in enumerate(groups):
            acc[g].append(st.commit())
            if r + 1 < rounds:
                st.set_round_inputs(*next_inputs(g, r + 1))
    return acc


def staggered_decode(groups, streams, rounds: int, next_inputs):
    """The staggered schedule of `staggered` over chained decode rounds. Slot k is (group k % G,
    round k // G). Every group's first draft phase goes in first (group g after group g-1's), then
    for each slot: the previous slot's commit (the host waits on that group's stream only; the
    group loads its next round's inputs), this slot's verify (its drafts are already enqueued; it
    takes its turn on the host link after the previous verify), and the next draft phase of the
    group that just committed, which runs while this verify streams. Verifies never wait for a
    draft phase to be enqueued, so the schedule holds whether drafting is bound by the GPU or by
    the host that enqueues it. Returns what each group's commits returned, per group (the same as
    `lockstep_decode`)."""
    ng = len(groups)
    assert len(streams) == ng and ng >= 1
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    first_done = [torch.cuda.Event() for _ in range(ng)]
    acc = [[] for _ in groups]
    total = rounds * ng
    enq = set()
    verify_done = None

    def draft(k):
        if k >= total or k in enq:
            return
        enq.add(k)
        g = k % ng
        if k < ng and g > 0:
            streams[g].wait_event(first_done[g - 1])
        with torch.cuda.stream(streams[g]):
            groups[g].draft_phase()
            if k < ng:
                first_done[g].record(streams[g])

    def commit(k):
        g, r = k % ng, k // ng
        with torch.cuda.stream(streams[g]):
            acc[g].append(groups[g].commit())  # waits for this group's stream only
            if r + 1 < rounds:
                groups[g].set_round_inputs(*next_inputs(g, r + 1))

    for k in range(min(ng, total)):
        draft(k)
    for k in range(total):
        if k >= 1:
            commit(k - 1)
        draft(k)  # one group: its next round follows its commit
        s = streams[k % ng]
        if verify_done is not None:
            s.wait_event(verify_done)
        with torch.cuda.stream(s):
            groups[k % ng].verify_step()
            verify_done = torch.cuda.Event()
            verify_done.record(s)
        if ng > 1:
            draft(k + ng - 1)  # the group that just committed drafts its next round
    commit(total - 1)
    for s in streams:
        cur.wait_stream(s)
    return acc


# ------------------------------------------------------------------------------------------
# remote prefix caching, simulated: the compressed cache crosses a slow network link, the full
# cache stays behind the local host link ("VeriCache: Turning Lossy KV Cache into Lossless LLM
# Inference", Key Contributions: the second deployment pipeline; Methodology: 40 GB/s local
# against 1.2 GB/s remote; "VeriCache: making lossy KV compression exact", The Tradeoff VeriCache
# Is Trying to Escape: a prefix's cache held remotely is slow to bring in)
# ------------------------------------------------------------------------------------------
class Transfer:
    """One transfer on a ThrottledLink: (device destination, pinned host source) pieces of equal
    shape. `done` is set once every chunk's copy has been issued (the link time of the last one
    included); `event` is recorded on the link's stream after the last copy."""

    def __init__(self, pieces):
        self.pieces = list(pieces)
        self.nbytes = sum(d.numel() * d.element_size() for d, _ in self.pieces)
        self.event = torch.cuda.Event()
        self.done = threading.Event()
        self.t_start = self.t_end = None

    def wait(self, stream=None):
        """The host waits until the transfer's copies are all issued; `stream` (default: the
        current one) then waits for them to land."""
        self.done.wait()
        (stream or torch.cuda.current_stream()).wait_event(self.event)


class ThrottledLink:
    """A simulated link of `rate` bytes per second into GPU memory, for data that would come from
    another machine. Transfers go out in the order they are sent, one at a time, each split into
    chunks; chunk k of a transfer that starts at t0 is copied (pinned host -> device, on the link's
    own stream) only once t0 + (bytes up to and including chunk k) / rate has passed, so a transfer
    of B bytes lands no earlier than B / rate after it starts and the link is busy meanwhile. The
    real host link is faster than the simulated one, so the pacing sets the arrival time. A host
    thread does the pacing; nothing on the GPU waits or spins."""

    def __init__(self, rate: float, chunk_bytes: int = 1 << 21, device: str = "cuda"):
        assert rate > 0 and chunk_bytes > 0
        self.rate, self.chunk = float(rate), int(chunk_bytes)
        self.device = device
        self.stream = torch.cuda.Stream(device=device)
        self._q = queue.Queue()
        self._free = 0.0  # host time at which the link finishes its last transfer
        self._th = threading.Thread(target=self._run, daemon=True)
        self._th.start()

    def send(self, pieces) -> Transfer:
        tr = Transfer(pieces)
        for d, h in tr.pieces:
            assert d.shape == h.shape and d.dtype == h.dtype and d.is_contiguous() and h.is_contiguous()
            assert h.device.type == "cpu" and h.is_pinned(), "the far side's copy is pinned host memory"
        self._q.put(tr)
        return tr

    def _run(self):
        with torch.cuda.device(self.stream.device):
            self._serve()

    def _serve(self):
        while True:
            tr = self._q.get()
            if tr is None:
                return
            t0 = max(time.perf_counter(), self._free)
            sent = 0
            with torch.cuda.stream(self.stream):
                for d, h in tr.pieces:
                    db, hb = d.reshape(-1).view(torch.uint8), h.reshape(-1).view(torch.uint8)
                    for a in range(0, db.numel(), self.chunk):
                        b = min(db.numel(), a + self.chunk)
                        sent += b - a
                        wait = t0 + sent / self.rate - time.perf_counter()
                        if wait > 0:
                            time.sleep(wait)
                        db[a:b].copy_(hb[a:b], non_blocking=True)
                tr.event.record(self.stream)
            self._free = t0 + sent / self.rate
            tr.t_start, tr.t_end = t0, self._free
            tr.done.set()

    def close(self):
        self._q.put(None)
        self._th.join()


def remote_prefix_decode(groups, link: ThrottledLink, streams, rounds: int, staggered: bool = True,
                         max_solo: int | None = None):
    """Decode request groups whose compressed caches arrive over `link` (every group's compressed
    cache is sent at once, as if the requests arrived together; each group's `remote_pieces` are
    its compressed cache's destination/source pairs) while their full caches stay behind the local
    host link and are streamed by every verify.

    Lock-step (staggered=False): every compressed cache lands, then `rounds` lock-step rounds.
    Staggered: group 0 decodes on its own as soon as its compressed cache has landed, round after
    round (at most `max_solo` rounds, default `rounds`), while the other groups' caches are still
    crossing the link; once all have landed,
    `rounds` rounds of every group follow in the staggered schedule (`staggered_decode`). So the
    slow link's time for the later groups is spent decoding the first one.

    Returns (per group, the tokens each round emitted; {"solo_rounds": rounds group 0 ran alone,
    "transfers": [(start, end) host times of each group's transfer]})."""
    ng = len(groups)
    cur = torch.cuda.current_stream()
    transfers = [link.send(g.remote_pieces) for g in groups]
    solo = []
    if staggered:
        transfers[0].wait(cur)
        g0 = groups[0]
        limit = rounds if max_solo is None else max_solo
        while len(solo) < limit and not all(tr.done.is_set() for tr in transfers[1:]):
            g0.draft_phase()
            g0.verify_step()
            solo.append(g0.commit())
    for tr in transfers:
        tr.wait(cur)
    if staggered and ng > 1:
        acc = staggered_decode(groups, streams, rounds, lambda g, r: ())
    else:
        acc = lockstep_decode(groups, rounds, lambda g, r: ())
    acc[0] = solo + acc[0]
    return acc, {"solo_rounds": len(solo), "transfers": [(tr.t_start, tr.t_end) for tr in transfers]}
