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
embeddings and the q/k/v projections are plain fp32 GEMMs through PyTorch.
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


class TokenDecoder:
    """weights: dict of float32 arrays E [V, dm], P [max_pos, dm], Wq [Hq*128, dm],
    Wk/Wv [Hkv*128, dm], Wo [dm, Hq*128], Wlm [V, dm]; dm a multiple of 128."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, x: int, bits: int = 4, R: int = 32,
                 max_new: int = 256, device: str = "cuda"):
        f32 = dict(dtype=torch.float32, device=device)
        self.E, self.P = _dev(weights["E"], device), _dev(weights["P"], device)
        self.Wq, self.Wk = _dev(weights["Wq"], device), _dev(weights["Wk"], device)
        self.Wv = _dev(weights["Wv"], device)
        self.Wp = _head(weights, device)  # [V, Hq*128 + dm]
        self.V, self.dm = self.E.shape
        assert self.dm % D == 0 and Hq % Hkv == 0
        self.Hq, self.Hkv, self.x, self.L, self.R = Hq, Hkv, x, x + 1, R
        self.Hx = Hq + self.dm // D  # heads of the projected input [o ; x]
        prompt = [int(t) for t in prompt]
        assert len(prompt) >= 2
        self.n = len(prompt) - 1  # cached positions: every prompt token but the last
        self.cap = (self.n + max_new + 2 * self.L + 63) // 32 * 32
        assert self.cap <= self.P.shape[0], "position table too short"
        L = self.L
        # full cache, round block, outputs
        self.k_store = torch.zeros((1, Hkv, self.cap, D), **f32)
        self.v_store = torch.zeros_like(self.k_store)
        self.k_blk = torch.zeros((1, Hkv, L, D), **f32)
        self.v_blk = torch.zeros_like(self.k_blk)
        self.q_verify = torch.zeros((1, Hq, L, D), **f32)
        self.q_draft = torch.zeros((L, 1, Hq, D), **f32)
        self.xs = torch.zeros((L, self.dm), **f32)
        self.od = torch.zeros((1, self.Hx, D), **f32)       # draft step [o ; x]
        self.lse_d = torch.zeros((1, Hq), **f32)
        self.ov = torch.zeros((1, self.Hx, L, D), **f32)    # verify rows [o ; x]
        self.lse_v = torch.zeros((1, Hq, L), **f32)
        self.logits_v = torch.zeros((1, L, self.V), **f32)
        i32 = dict(dtype=torch.int32, device=device)
        self.tok = torch.zeros((L + 1,), **i32)             # block tokens (entry L: spare)
        self.accept_len = torch.zeros((1,), **i32)
        self.next_tok = torch.zeros((1,), **i32)
        self.argmax_v = torch.zeros((1, L), **i32)
        self.ws_draft = vc.Workspace(device)
        self.ws_verify = vc.Workspace(device)
        self.ws_proj = torch.zeros((vc.vc_project_workspace(1, 1, self.V) + 3) // 4, **i32)
        # prefill: keys/values of positions 0..n-1, the quantised prefix and the residual
        n = self.n
        X = self.E[torch.tensor(prompt[:n], device=device)] + self.P[:n]
        self.k_store[0, :, :n] = (X @ self.Wk.T).view(n, Hkv, D).transpose(0, 1)
        self.v_store[0, :, :n] = (X @ self.Wv.T).view(n, Hkv, D).transpose(0, 1)
        self.n_q = 32 * (max(0, n - R) // 32)
        res_cap = (R + 32 + L + 31) // 32 * 32
        self.cache = vc.KiviCache(1, Hkv, (self.cap + 31) // 32 * 32, bits, vc.VC_F32, vc.VC_F32,
                                  res_cap, device)
        if self.n_q:
            vc.vc_quantize_kv(self.cache, self.k_store, self.v_store, 0, self.n_q,
                              src_bh_stride=self.cap * D)
        if n > self.n_q:
            vc.vc_kivi_append(self.cache, self.k_store[:, :, self.n_q:], self.v_store[:, :, self.n_q:],
                              self.n_q, n - self.n_q, src_bh_stride=self.cap * D)
        self.tok[0] = prompt[-1]
        self.rounds = []  # accepted count per round

    # ---- one block entry: embedding and projections -----------------------------------------
    def _entry(self, j: int):
        x = self.E[self.tok[j:j + 1].long()][0] + self.P[self.n + j]
        self.xs[j] = x
        q = self.Wq @ x
        self.q_verify[0, :, j] = q.view(self.Hq, D)
        self.q_draft[j, 0] = q.view(self.Hq, D)
        self.k_blk[0, :, j] = (self.Wk @ x).view(self.Hkv, D)
        self.v_blk[0, :, j] = (self.Wv @ x).view(self.Hkv, D)

    def draft_step(self, j: int):
        """Draft step j: attention over the compressed cache (storing entry j's key/value into the
        residual), logits of [o ; x] and the greedy token into block entry j + 1."""
        self._entry(j)
        r = (self.n - self.n_q) + j + 1
        nb = vc.vc_draft_quant_workspace(self.cache, self.n_q, r, self.Hq)
        vc.vc_draft_attn_quant(self.cache, self.n_q, r, self.q_draft[j], self.od, self.lse_d,
                               self.ws_draft.get(nb), SM_SCALE, k_new=self.k_blk[:, :, j],
                               v_new=self.v_blk[:, :, j])
        self.od[0, self.Hq:] = self.xs[j].view(-1, D)
        vc.vc_project_logits(self.Wp, self.od, argmax=self.tok[j + 1:j + 2], argmax_b_stride=1,
                             ws=self.ws_proj)

    def verify_step(self):
        """Entry x's projections, verify attention over the full cache, logits of every row and
        the greedy accept."""
        self._entry(self.x)
        nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, self.L, self.n, False, 0, vc.VC_F32)
        vc.vc_verify_attn(self.q_verify, self.k_blk, self.v_blk, self.k_store, self.v_store, self.n,
                          self.ov, self.lse_v, self.ws_verify.get(nb), SM_SCALE, past_stride=self.cap)
        self.ov[0, self.Hq:] = self.xs.view(self.L, -1, D).transpose(0, 1)
        vc.vc_project_logits(self.Wp, self.ov, logits=self.logits_v)
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
        self.k_store[:, :, n0:n1] = self.k_blk[:, :, :a + 1]
        self.v_store[:, :, n0:n1] = self.v_blk[:, :, :a + 1]
        if a == self.x:
            vc.vc_kivi_append(self.cache, self.k_blk[:, :, self.x], self.v_blk[:, :, self.x],
                              n0 + self.x, 1, src_bh_stride=self.L * D)
        self.n = n1
        while self.n - self.n_q >= self.R + 32:
            vc.vc_quantize_kv(self.cache, self.k_store[:, :, self.n_q:], self.v_store[:, :, self.n_q:],
                              self.n_q, 32, src_bh_stride=self.cap * D)
            self.n_q += 32
        self.tok[0:1] = self.next_tok
        self.rounds.append(a)
        return emitted

    def generate(self, steps: int):
        """Rounds until `steps` tokens are emitted; returns them."""
        out = []
        while len(out) < steps:
            for j in range(self.x):
                self.draft_step(j)
            self.verify_step()
            out += self.commit()
        return out[:steps]


class GreedyDecoder:
    """The baseline without a drafter: greedy decoding over the full cache, one token per step
    (the entry's projections, attention of one query row over the full cache, logits with the
    greedy argmax, the entry's key/value appended to the full cache). Same model and calls as
    TokenDecoder."""

    def __init__(self, weights, Hq: int, Hkv: int, prompt, max_new: int = 256, device: str = "cuda"):
        f32 = dict(dtype=torch.float32, device=device)
        self.E, self.P = _dev(weights["E"], device), _dev(weights["P"], device)
        self.Wq, self.Wk = _dev(weights["Wq"], device), _dev(weights["Wk"], device)
        self.Wv = _dev(weights["Wv"], device)
        self.Wp = _head(weights, device)
        self.V, self.dm = self.E.shape
        self.Hq, self.Hkv, self.Hx = Hq, Hkv, Hq + self.dm // D
        prompt = [int(t) for t in prompt]
        self.n = len(prompt) - 1
        self.cap = (self.n + max_new + 63) // 32 * 32
        n = self.n
        self.k_store = torch.zeros((1, Hkv, self.cap, D), **f32)
        self.v_store = torch.zeros_like(self.k_store)
        X = self.E[torch.tensor(prompt[:n], device=device)] + self.P[:n]
        self.k_store[0, :, :n] = (X @ self.Wk.T).view(n, Hkv, D).transpose(0, 1)
        self.v_store[0, :, :n] = (X @ self.Wv.T).view(n, Hkv, D).transpose(0, 1)
        self.q = torch.zeros((1, Hq, 1, D), **f32)
        self.k1 = torch.zeros((1, Hkv, 1, D), **f32)
        self.v1 = torch.zeros_like(self.k1)
        self.o = torch.zeros((1, self.Hx, 1, D), **f32)
        self.lse = torch.zeros((1, Hq, 1), **f32)
        i32 = dict(dtype=torch.int32, device=device)
        self.toks = torch.zeros((max_new + 1,), **i32)
        self.toks[0] = prompt[-1]
        self.ws = vc.Workspace(device)
        self.ws_proj = torch.zeros((vc.vc_project_workspace(1, 1, self.V) + 3) // 4, **i32)

    def generate(self, steps: int):
        for i in range(steps):
            x = self.E[self.toks[i:i + 1].long()][0] + self.P[self.n]
            self.q[0, :, 0] = (self.Wq @ x).view(self.Hq, D)
            self.k1[0, :, 0] = (self.Wk @ x).view(self.Hkv, D)
            self.v1[0, :, 0] = (self.Wv @ x).view(self.Hkv, D)
            nb = vc.vc_verify_workspace(1, self.Hq, self.Hkv, 1, self.n, False, 0, vc.VC_F32)
            vc.vc_verify_attn(self.q, self.k1, self.v1, self.k_store, self.v_store, self.n, self.o,
                              self.lse, self.ws.get(nb), SM_SCALE, past_stride=self.cap)
            self.o[0, self.Hq:, 0] = x.view(-1, D)
            vc.vc_project_logits(self.Wp, self.o, argmax=self.toks[i + 1:i + 2], argmax_b_stride=1,
                                 ws=self.ws_proj)
            self.k_store[:, :, self.n] = self.k1[:, :, 0]
            self.v_store[:, :, self.n] = self.v1[:, :, 0]
            self.n += 1
        return [int(t) for t in self.toks[1:steps + 1].tolist()]

