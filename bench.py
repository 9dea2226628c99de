#!/usr/bin/env python3
"""Benchmark of the VeriCache draft/verify hot path on one MI355X.

One step = one whole draft/verify round of the 32K-context Llama-3.1-8B-shaped attention layer
(batch 8, 32 query / 8 kv heads, d 128, bf16 KV with 1% outlier channels, KIVI 2-bit drafter
with an fp16 residual of 128 tokens, draft length 30, a 31-row causal verify over the full KV held
in HBM): 30 x (draft attention with the step's residual append fused in + stand-in logits
projection with its greedy argmax fused in), then verify attention + logits projection + accept. Inputs are seeded and synthetic and resident in
HBM before the timed region starts.

Reported (one JSON line):
  value        verified tokens per second = sum_b (accepted_b + 1) / round time
  roofline     the draft attention kernel (the round's dominant kernel): algorithmic bytes per
               launch / mean launch time measured with HIP events on the launch stream, against
               8 TB/s HBM; `traffic` is the counter-measured HBM traffic per launch when a
               committed counter summary for the current kernel source exists, else null
  cpu_baseline the CPU oracle timed on one whole request of the same round (see `sample`)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")

METRIC = "draft/verify attention GB/s (% of 8 TB/s HBM) + verified tokens/s at 32K ctx"

DRAFT_NAME = {("kivi", 2): "draft attention over the 2-bit KIVI cache",
              ("kivi", 4): "draft attention over the 4-bit KIVI cache",
              ("drop", 0): "draft attention over the kept positions (token dropping)"}
WORKLOAD_TEXT = {
    "c1": "one attention layer, batch 1, 32/8 heads, d 128, context 2048, fp32 Q/K/V, KIVI 4-bit "
          "(group 32, fp32 residual 32, fp32 metadata), draft length 8, 9-row causal verify",
    "c2": "Llama-3.1-8B-shaped layer, batch 8, context 32768, 32/8 heads, d 128, KIVI 2-bit (group 32, "
          "fp16 residual 128, fp16 metadata), draft length 30, 31-row causal verify over HBM-resident "
          "bf16 KV",
    "c3": "Llama-70B-shaped layer, batch 4, context 100000, 64/8 heads, d 128, token-dropping drafter "
          "(25% kept: 64 sinks + 256 recent + top-scoring), draft length 30, 31-row causal verify over "
          "HBM-resident bf16 KV",
    "c4": "Llama-3.1-8B-shaped layer, batch 1, context 500000, 32/8 heads, d 128, full bf16 KV in pinned "
          "host memory streamed in 65536-token chunks, KIVI 4-bit drafter (fp16 residual 128, fp16 "
          "metadata) in HBM, draft length 30, 31-row causal verify"}
DATA_TEXT = {
    "c1": "synthetic (seeded N(0,1) fp32 Q/K/V, random fp32 logits projection)",
    "c2": "synthetic (seeded N(0,1) bf16 KV with 1% x8 outlier channels, random fp32 logits projection)",
    "c3": "synthetic (seeded N(0,1) bf16 KV, seeded keep-list scores, random fp32 logits projection)",
    "c4": "synthetic (seeded N(0,1) bf16 KV, random fp32 logits projection)"}


def _src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic_per_launch(name: str):
    """HBM bytes per launch from the committed counter summary profiles/<name>_traffic.json, if it
    was measured on the kernel source as it is now (else None)."""
    try:
        rec = json.load(open(os.path.join(PROFILES, f"{name}_traffic.json")))
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, rec.get("kernel_source", ""))
    if not os.path.isfile(src) or rec.get("kernel_source_sha256_16") != _src_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inputs, row: int = 0):
    """The oracle (as written, untuned) on one whole request of the same round, timed: its 30 draft
    steps over every query head, the draft logits and argmax, the 31-row verify of every head, the
    verify logits and the accept step for batch row `row`. value = the tokens that request's round
    emits (a + 1, the oracle's own accept result) per second of that wall time. The sample is one
    of the B requests, measured whole; nothing is scaled."""
    from threadpoolctl import threadpool_info

    from oracle.round import Round

    rnd = Round(w, *inputs)
    if w.drafter == "kivi":  # the compressed cache is built before the timed region, as on the GPU
        for h in range(w.Hkv):
            rnd.kivi(row, h)
    t0 = time.perf_counter()
    res = rnd.run(row)
    el = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    affinity = len(os.sched_getaffinity(0))
    threads = max(blas) if blas else 1
    return {"value": (res["a"] + 1) / el, "unit": "tok/s", "cores": int(min(threads, affinity)),
            "kind": "oracle",
            "sample": (f"oracle on batch row {row} of the same round, whole: {w.x} draft steps of all "
                       f"{w.Hq} query heads with their logits and argmax, the {w.L}-row verify of all "
                       f"heads, its logits and the accept step (1 of {w.B} requests; measured, not "
                       f"scaled); emitted {res['a'] + 1} token(s) in {el:.1f} s"),
            "seconds": round(el, 2), "emitted": int(res["a"] + 1),
            "host_cores_available": affinity, "blas_threads": int(threads)}


def _h2d_rate(torch, vc, st, passes: int = 10) -> dict:
    """Achieved pinned host -> HBM rate of the streamed verify's own transfer: vc_verify_stream_copies
    issues exactly the verify's chunk copies (one 2-D copy per chunk per tensor into the two
    stages) with nothing else; median of `passes` passes."""
    w = st.w
    ws = st._verify_ws()
    nbytes = 2 * w.B * w.Hkv * st.n * 128 * st.k_host.element_size()
    copy = st.copy_stream
    times = []
    for _ in range(passes):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        vc.vc_verify_stream_copies(st.k_host, st.v_host, st.n, ws, w.B, w.Hq, w.Hkv, w.L, w.chunk_tokens,
                                   past_stride=st.host_cap, copy_stream=copy)
        copy.synchronize()
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"bytes": nbytes, "seconds": t, "GB_s": nbytes / t / 1e9, "passes": passes}


def _read_stream(torch, vc, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """HBM read ceiling: vc_hbm_read_stream over a 1 GiB buffer (4x the 256 MB last-level cache),
    timed with HIP events on the launch stream, median of `reps` launches, at 384, 512 and 768
    workgroups (the plain read is fastest at about two workgroups per CU and falls to ~5.1 TB/s
    from 1024 up); the best of the three."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    sink = torch.empty(768 * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    best = None
    for blocks in (384, 512, 768):
        for _ in range(2):
            vc.vc_hbm_read_stream(buf, sink, blocks)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            vc.vc_hbm_read_stream(buf, sink, blocks)
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(times))
        if best is None or t < best[0]:
            best = (t, blocks)
    del buf
    t, blocks = best
    return {"GB_s": round(nbytes / t / 1e9, 1), "bytes": nbytes, "us": round(t * 1e6, 1), "reps": reps,
            "workgroups": blocks, "kernel": "vc_hbm_read_stream (16-byte loads, XOR-folded)"}


def _staggering(torch, harness, synth, st0, seed: int, rounds: int) -> dict:
    """Two request groups of the host-streamed workload (the second drawn with seed + 1): round
    time of the lock-step schedule (all groups draft, then all verify) against the staggered one
    (each group on its own stream, one group's verify transfer overlapping the other's drafting)."""
    w = st0.w
    K, V = synth.kv_past(w, seed + 1)
    Kn, Vn = synth.kv_new(w, seed + 1)
    st1 = harness.RoundState(w, seed=seed + 1, inputs=(K, V, Kn, Vn, synth.q_new(w, seed + 1),
                                                       synth.projection(w, seed + 1)),
                             copy_stream=st0.copy_stream)
    del K, V
    groups = [st0, st1]
    # group 0 on the current stream, group 1 on one more; one shared copy stream (4 hardware
    # queues per process: more streams would share queues and serialise the groups)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def measure(prefetch: bool) -> dict:
        for g in groups:
            g.prefetch_verify = prefetch
        timed(lambda: harness.lockstep(groups, 1))          # warm-up (workspaces sized)
        timed(lambda: harness.staggered(groups, streams, 1))
        out = {}
        if not prefetch:  # the phases on their own
            out["draft_phase_ms"] = round(np.median([timed(st0.draft_phase) for _ in range(3)]) * 1e3, 3)
            out["verify_ms"] = round(np.median([timed(st0.verify_step) for _ in range(3)]) * 1e3, 3)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            st0.verify_attention()  # host time to enqueue one host-streamed verify
            out["verify_enqueue_host_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
            torch.cuda.synchronize()
        t_lock = timed(lambda: harness.lockstep(groups, rounds)) / rounds
        t_stag = timed(lambda: harness.staggered(groups, streams, rounds)) / rounds
        res = [g.results() for g in groups]
        emitted = int(sum((r["a"] + 1).sum() for r in res))
        out.update({"lockstep_ms_per_round": round(t_lock * 1e3, 3),
                    "staggered_ms_per_round": round(t_stag * 1e3, 3),
                    "speedup": round(t_lock / t_stag, 4),
                    "tok_s_lockstep": round(emitted / t_lock, 3),
                    "tok_s_staggered": round(emitted / t_stag, 3)})
        return out

    # staggering on its own (every verify streams all its chunks), then with each round's first
    # two verify chunks prefetched under its own draft phase
    out = {"groups": 2, "requests_per_group": w.B, "rounds": rounds}
    out.update(measure(False))
    out["link_bound_ms_per_round"] = round(out["draft_phase_ms"] / rounds + 2 * out["verify_ms"], 3)
    out["draft_time_hidden_frac"] = round((out["lockstep_ms_per_round"] - out["staggered_ms_per_round"])
                                          / (2 * out["draft_phase_ms"]), 4)
    out["with_prefetch"] = measure(True)
    out["note"] = ("per round both groups draft 30 steps and verify 31 rows over their 500K-token "
                   "pinned-host KV; times from host clocks around synchronised schedules; "
                   "link_bound = the first draft phase plus back-to-back verifies (the host link "
                   "never idle afterwards); with_prefetch: every round's draft phase first issues "
                   "its verify's first two chunk copies")
    for g in groups:
        g.prefetch_verify = True
    return out


def _decode_loop(torch, harness, synth, w, seed: int, rounds: int) -> dict:
    """Multi-round decode of one request: each round drafts x tokens, verifies, accepts, commits
    the accepted positions and flushes whole residual groups into the codes; the next round's
    queries/keys/values are drawn beforehand and uploaded between rounds."""
    st = harness.RoundState(w, seed=seed, extra_tokens=rounds * w.L + 64)
    blocks = [(synth.kv_new(w, seed, t), synth.q_new(w, seed, t)) for t in range(1, rounds + 1)]
    st.run_round()  # warm-up (sizes every workspace); not committed, so the first timed round repeats it
    torch.cuda.synchronize()
    n0, nq0, acc = st.n, st.n_q, []
    t0 = time.perf_counter()
    for t in range(rounds):
        st.run_round()
        acc.append(st.commit())
        (Kn, Vn), Q = blocks[t]
        st.set_round_inputs(Kn, Vn, Q)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    emitted = sum(a + 1 for a in acc)
    return {"rounds": rounds, "accepted_per_round": acc, "emitted": emitted,
            "ms_per_round": round(el / rounds * 1e3, 3), "tok_s": round(emitted / el, 2),
            "context": [n0, st.n], "quantised": [nq0, st.n_q], "flushes": (st.n_q - nq0) // w.group,
            "note": "one request; per round: x draft steps, verify, accept, commit of the accepted "
                    "positions (plus the bonus one), flush of whole residual groups; next round's "
                    "inputs uploaded between rounds (host clock around the rounds)"}


def _decode_pair(torch, harness, synth, w, seed: int, rounds: int) -> dict:
    """Two requests of the host-streamed workload (seeds seed, seed + 1) decoded over `rounds`
    chained rounds each, lock-step against staggered (each from fresh caches on the same inputs)."""
    seeds = (seed, seed + 1)
    nxt = {(g, r): (*synth.kv_new(w, seeds[g], r), synth.q_new(w, seeds[g], r))
           for g in range(2) for r in range(1, rounds)}

    def build():
        g0 = harness.RoundState(w, seed=seeds[0], extra_tokens=rounds * w.L + 64)
        g1 = harness.RoundState(w, seed=seeds[1], extra_tokens=rounds * w.L + 64,
                                copy_stream=g0.copy_stream)
        for g in (g0, g1):  # warm-up round (sizes workspaces), not committed
            g.run_round()
        torch.cuda.synchronize()
        return [g0, g1]

    out = {}
    for name in ("lockstep", "staggered"):
        groups = build()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if name == "lockstep":
            acc = harness.lockstep_decode(groups, rounds, lambda g, r: nxt[(g, r)])
        else:
            acc = harness.staggered_decode(groups, [torch.cuda.current_stream(), torch.cuda.Stream()],
                                           rounds, lambda g, r: nxt[(g, r)])
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(a + 1 for ag in acc for a in ag)
        out[name] = {"ms_per_round": round(el / rounds * 1e3, 3), "tok_s": round(emitted / el, 2),
                     "accepted": acc}
        del groups
    out["speedup"] = round(out["lockstep"]["ms_per_round"] / out["staggered"]["ms_per_round"], 4)
    out["note"] = ("two requests, each round both draft 30 steps and verify 31 rows over their "
                   "500K-token pinned-host KV, then commit and flush; same inputs for both schedules")
    return out


def _e2e_decode(torch, seed: int, context: int, tokens: int) -> dict:
    """Token-level decoding of one request on a one-layer decoder (Llama-3.1-8B-shaped attention:
    32 query / 8 kv heads, d 128; d_model 256, vocab 2048, seeded random fp32 weights at the scales
    of the oracle's model) with a `context`-token prompt whose bf16 cache sits in pinned host
    memory and is streamed by every verify, in 64K-token chunks: VeriCache (4-bit KIVI drafter in
    HBM, draft length 30) against greedy decoding over the full cache (one streamed pass per
    token)."""
    from kv_cache_compressed_amd.decode_loop import GreedyDecoder, TokenDecoder

    dev, V, dm, Hq, Hkv = "cuda", 2048, 256, 32, 8
    g = torch.Generator(device=dev).manual_seed(seed)
    rn = lambda *shape: torch.randn(*shape, generator=g, device=dev)
    pair_rounds = max(12, tokens // 31)  # the two-request schedules below
    W = {"E": rn(V, dm), "P": 0.5 * rn(context + max(tokens, 31 * pair_rounds) + 256, dm),
         "Wq": rn(Hq * 128, dm) / dm ** 0.5, "Wk": rn(Hkv * 128, dm) / dm ** 0.5,
         "Wv": rn(Hkv * 128, dm) / dm ** 0.5, "Wo": rn(dm, Hq * 128) / (Hq * 128) ** 0.5,
         "Wlm": 3.0 * rn(V, dm) / dm ** 0.5}
    prompt = torch.randint(0, V, (context,), generator=g, device=dev).tolist()
    # One copy stream and one second compute stream for every decoder of this run: HIP maps streams
    # onto a few hardware queues (4 per process by default) and streams that share a queue run one
    # after the other; with a fresh copy stream per decoder the two-request pair's copy stream came
    # to share a queue with a group stream (staggered 78.8 ms per round against 73.4).
    copy, second = torch.cuda.Stream(), torch.cuda.Stream()
    opts = dict(kv_dtype="bf16", host_past=True, chunk_tokens=65536, copy_stream=copy)
    out = {"context": context, "tokens": tokens, "model": "one layer, d_model 256, 32/8 heads, d 128, "
           "vocab 2048, bf16 cache in pinned host memory, 64K-token chunks"}
    seqs = {}
    # VeriCache with the verify's first two chunks prefetched under the draft phase, and without
    for name in ("vericache", "vericache_no_prefetch", "greedy"):
        t0 = time.perf_counter()
        if name != "greedy":
            dec = TokenDecoder(W, Hq, Hkv, prompt, x=30, bits=4, R=128, max_new=tokens + 96,
                               prefetch_verify=name == "vericache", **opts)
        else:
            dec = GreedyDecoder(W, Hq, Hkv, prompt, max_new=tokens + 8, **opts)
        torch.cuda.synchronize()
        t_prefill = time.perf_counter() - t0
        dec.warm()  # workspaces sized for the whole decode before the timed region
        # one untimed warm-up round (VeriCache) or token (greedy): the first launches pay one-time
        # costs (code-object loading, the GEMV library's set-up) of ~0.1 s
        warm = dec.generate(1) if name == "greedy" else (dec.draft_phase(), dec.verify_step(), dec.commit())[2]
        torch.cuda.synchronize()
        rounds0 = len(dec.rounds) if name != "greedy" else 0
        t0 = time.perf_counter()
        seqs[name] = warm + dec.generate(tokens)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        # every token the timed rounds produced (the last round may run past `tokens`)
        emitted = sum(a + 1 for a in dec.rounds[rounds0:]) if name != "greedy" else tokens
        out[name] = {"tok_s": round(emitted / el, 2), "emitted": emitted,
                     "ms_per_token": round(el / emitted * 1e3, 3), "prefill_s": round(t_prefill, 2),
                     "warmup_tokens": len(warm)}
        if name != "greedy":
            out[name]["accepted_per_round"] = dec.rounds[rounds0:]
        del dec
    out["speedup"] = round(out["vericache"]["tok_s"] / out["greedy"]["tok_s"], 3)
    out["prefetch_speedup"] = round(out["vericache"]["tok_s"] / out["vericache_no_prefetch"]["tok_s"], 3)
    b = seqs["greedy"]
    for name in ("vericache", "vericache_no_prefetch"):
        a = seqs[name]
        m = min(len(a), len(b))  # the greedy run's warm-up token and timed tokens
        out[name]["first_divergence"] = next((i for i in range(m) if a[i] != b[i]), None)

    # two requests (the second prompt drawn after the first), lock-step against staggered
    # (harness.staggered_decode: one request's verify streams while the other drafts)
    from kv_cache_compressed_amd import harness

    prompt2 = torch.randint(0, V, (context,), generator=g, device=dev).tolist()
    # at least 12 rounds: with fewer, the start (both requests' first draft phases before any
    # verify) weighs on the per-round time as much as the schedule does
    rounds = pair_rounds

    def pair():
        d0 = TokenDecoder(W, Hq, Hkv, prompt, x=30, bits=4, R=128, max_new=rounds * 31 + 64, **opts)
        d1 = TokenDecoder(W, Hq, Hkv, prompt2, x=30, bits=4, R=128, max_new=rounds * 31 + 64, **opts)
        d0.warm()
        d1.warm()
        return [d0, d1]

    two = {"rounds_per_request": rounds}
    for name in ("lockstep", "staggered"):
        ds = pair()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if name == "lockstep":
            acc = harness.lockstep_decode(ds, rounds, lambda gi, r: ())
        else:
            acc = harness.staggered_decode(ds, [torch.cuda.current_stream(), second], rounds,
                                           lambda gi, r: ())
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(len(em) for ga in acc for em in ga)
        two[name] = {"tok_s": round(emitted / el, 2), "emitted": emitted,
                     "ms_per_round": round(el / rounds * 1e3, 2)}
        del ds
    two["speedup"] = round(two["staggered"]["tok_s"] / two["lockstep"]["tok_s"], 3)
    out["two_requests"] = two
    return out


def _e2e_llama_batch(torch, W, prompts, tokens: int, bits: int, x: int, opts: dict) -> dict:
    """The batched form: every request drafts and verifies in the same rounds (the layer's GEMMs
    over all rows, attention per request), accepts its own counts and keeps its own context
    length; greedy decoding of the same batch is the baseline."""
    from kv_cache_compressed_amd.decode_loop import BatchedLlamaDecoder

    out, seqs, margins = {}, {}, {}
    for name, xx in (("vericache", x), ("greedy", 0)):
        t0 = time.perf_counter()
        dec = BatchedLlamaDecoder(W, 16, 4, prompts, x=xx, bits=bits, R=128, max_new=tokens + 96,
                                  margins=True, **opts)
        torch.cuda.synchronize()
        t_prefill = time.perf_counter() - t0
        dec.warm()
        dec.draft_phase()  # one untimed round (captures the fused draft phase)
        dec.verify_step()
        warm = dec.commit()
        torch.cuda.synchronize()
        r0 = len(dec.rounds[0])
        t0 = time.perf_counter()
        gen = dec.generate(tokens)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(sum(a + 1 for a in r[r0:]) for r in dec.rounds)
        out[name] = {"tok_s": round(emitted / el, 2), "emitted": emitted,
                     "rounds": len(dec.rounds[0]) - r0, "prefill_s": round(t_prefill, 2)}
        print(f"# e2e_llama batch {name}: {out[name]}", file=sys.stderr, flush=True)
        if xx:
            out[name]["mean_accepted"] = round(float(np.mean([a for r in dec.rounds for a in r[r0:]])), 2)
        seqs[name] = [w + g for w, g in zip(warm, gen)]
        margins[name] = dec.margin_log
        del dec
    out["speedup"] = round(out["vericache"]["tok_s"] / out["greedy"]["tok_s"], 3)
    # two groups of half the batch each, lock-step against staggered on two streams
    # (harness.staggered_decode: one group's verify streams while the other drafts)
    from kv_cache_compressed_amd import harness

    h = len(prompts) // 2
    rounds = max(1, out["vericache"]["rounds"] // 2)
    two = {"groups": 2, "requests_per_group": h, "rounds": rounds}
    for name in ("lockstep", "staggered"):
        g0 = BatchedLlamaDecoder(W, 16, 4, prompts[:h], x=x, bits=bits, R=128,
                                 max_new=rounds * (x + 1) + 96, **opts)
        g1 = BatchedLlamaDecoder(W, 16, 4, prompts[h:2 * h], x=x, bits=bits, R=128,
                                 max_new=rounds * (x + 1) + 96, copy_stream=g0.copy_stream, **opts)
        groups = [g0, g1]
        for g in groups:
            g.warm()
        # one untimed round each (first launches), then the timed schedule
        harness.lockstep_decode(groups, 1, lambda gi, r: ())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if name == "lockstep":
            acc = harness.lockstep_decode(groups, rounds, lambda gi, r: ())
        else:
            acc = harness.staggered_decode(groups, [torch.cuda.current_stream(), torch.cuda.Stream()],
                                           rounds, lambda gi, r: ())
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(len(em) for ga in acc for ems in ga for em in ems)
        two[name] = {"tok_s": round(emitted / el, 2), "emitted": emitted,
                     "ms_per_round": round(el / rounds * 1e3, 2)}
        print(f"# e2e_llama two groups {name}: {two[name]}", file=sys.stderr, flush=True)
        del groups, g0, g1
    two["speedup"] = round(two["staggered"]["tok_s"] / two["lockstep"]["tok_s"], 3)
    out["two_groups"] = two
    # Token comparison with the greedy decoding of the batch: the first position where a request's
    # tokens differ (after it the two continue from different contexts), with the top-2 logit gap
    # of the rows both decoders chose that token from; a gap below 1e-3 is a near-tie, where two
    # correct computations in different orders may pick different tokens.
    div = []
    for r, (a, b) in enumerate(zip(seqs["vericache"], seqs["greedy"])):
        m = min(len(a), len(b))
        i = next((i for i in range(m) if a[i] != b[i]), None)
        if i is not None:
            gap = min(margins["vericache"][r][i], margins["greedy"][r][i])
            div.append({"request": r, "position": i, "margin": gap, "near_tie": gap < 1e-3})
    out["first_divergence"] = [d for d in div if not d["near_tie"]] or None
    out["near_tie_divergences"] = [d for d in div if d["near_tie"]]
    return out


def _e2e_llama(torch, seed: int, context: int, tokens: int, bits: int = 2, x: int = 30,
               batch: int = 1) -> dict:
    """Token-level decoding of one request on a random-init 4-layer Llama-form decoder (d_model 2048,
    16 query / 4 kv heads, d 128, SwiGLU width 5632, vocab 32000, weights ~N(0, 0.02) rounded to
    bf16 values, gains 1; fp32 arithmetic outside the attention calls) with a `context`-token
    random prompt whose bf16 caches (one per layer) sit in pinned host memory and are streamed by
    every verify: VeriCache (`bits`-bit KIVI drafter in HBM, fp16 residual of 128, draft length x)
    against greedy decoding over the full caches."""
    from kv_cache_compressed_amd.decode_loop import LayeredDecoder, LayeredGreedyDecoder

    dev, V, dm, Hq, Hkv, F, nl = "cuda", 32000, 2048, 16, 4, 5632, 4
    g = torch.Generator(device=dev).manual_seed(seed)
    rn = lambda *shape: (0.02 * torch.randn(*shape, generator=g, device=dev)).to(torch.bfloat16).float()
    one = lambda: torch.ones(dm, device=dev)
    W = {"E": rn(V, dm), "Wlm": rn(V, dm), "g_f": one(),
         "g_att": [one() for _ in range(nl)], "g_mlp": [one() for _ in range(nl)],
         "Wq": [rn(Hq * 128, dm) for _ in range(nl)], "Wk": [rn(Hkv * 128, dm) for _ in range(nl)],
         "Wv": [rn(Hkv * 128, dm) for _ in range(nl)], "Wo": [rn(dm, Hq * 128) for _ in range(nl)],
         "W1": [rn(F, dm) for _ in range(nl)], "W3": [rn(F, dm) for _ in range(nl)],
         "W2": [rn(dm, F) for _ in range(nl)]}
    prompt = torch.randint(0, V, (context,), generator=g, device=dev).tolist()
    opts = dict(kv_dtype="bf16", host_past=True, chunk_tokens=65536)
    out = {"context": context, "tokens": tokens, "drafter": f"KIVI {bits}-bit, x = {x}",
           "batch": batch,
           "model": "4 Llama-form layers, d_model 2048, 16/4 heads, d 128, SwiGLU 5632, vocab 32000, "
                    "bf16 caches in pinned host memory"}
    if batch > 1:
        prompts = [prompt] + [torch.randint(0, V, (context,), generator=g, device=dev).tolist()
                              for _ in range(batch - 1)]
        out.update(_e2e_llama_batch(torch, W, prompts, tokens, bits, x, opts))
        return out
    seqs = {}
    for name in ("vericache", "greedy"):
        t0 = time.perf_counter()
        if name == "vericache":
            dec = LayeredDecoder(W, Hq, Hkv, prompt, x=x, bits=bits, R=128, max_new=tokens + 96, **opts)
        else:
            dec = LayeredGreedyDecoder(W, Hq, Hkv, prompt, max_new=tokens + 8, **opts)
        torch.cuda.synchronize()
        t_prefill = time.perf_counter() - t0
        dec.warm()
        # one untimed round (greedy: token) pays the first launches' one-time costs
        if name == "greedy":
            warm = dec.generate(1)
        else:
            for j in range(dec.x):
                dec.draft_step(j)
            dec.verify_step()
            warm = dec.commit()
        torch.cuda.synchronize()
        r0 = len(dec.rounds) if name == "vericache" else 0
        t0 = time.perf_counter()
        seqs[name] = dec.generate(tokens)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        emitted = sum(a + 1 for a in dec.rounds[r0:]) if name == "vericache" else tokens
        out[name] = {"tok_s": round(emitted / el, 2), "emitted": emitted,
                     "ms_per_token": round(el / emitted * 1e3, 3), "prefill_s": round(t_prefill, 2)}
        if name == "vericache":
            acc = dec.rounds[r0:]
            out[name]["rounds"] = len(acc)
            out[name]["mean_accepted"] = round(float(np.mean(acc)), 2)
        seqs[name] = warm + seqs[name]
        del dec
    out["speedup"] = round(out["vericache"]["tok_s"] / out["greedy"]["tok_s"], 3)
    a, b = seqs["vericache"], seqs["greedy"]
    m = min(len(a), len(b))  # the greedy run's warm-up token and timed tokens
    out["first_divergence"] = next((i for i in range(m) if a[i] != b[i]), None)
    return out


def _remote_prefix(torch, seed: int, context: int, rounds: int, rate: float = 1.2e9) -> dict:
    """Remote prefix caching, simulated: two requests on the one-layer decoder of `_e2e_decode`
    (32/8 heads, d 128, d_model 256, vocab 2048), each with a `context`-token prefix whose compressed
    cache (KIVI 4-bit, fp16 residual 128) crosses a link throttled to `rate` bytes/s
    (harness.ThrottledLink) while its bf16 full cache stays in pinned host memory and is streamed
    over the local host link by every verify (x = 30). VeriCache lock-step (both compressed caches
    land, then both decode) and staggered (the first request decodes while the second's cache is
    on the link); against greedy full-KV decoding of the same requests with the full cache behind
    the local link (one streamed pass per token), and with the full cache shipped over the
    throttled link into HBM first. Times from the requests' arrival to the last token."""
    from kv_cache_compressed_amd import harness
    from kv_cache_compressed_amd.decode_loop import GreedyDecoder, TokenDecoder

    dev, V, dm, Hq, Hkv = "cuda", 2048, 256, 32, 8
    g = torch.Generator(device=dev).manual_seed(seed)
    rn = lambda *shape: torch.randn(*shape, generator=g, device=dev)
    W = {"E": rn(V, dm), "P": 0.5 * rn(context + 4096, dm),
         "Wq": rn(Hq * 128, dm) / dm ** 0.5, "Wk": rn(Hkv * 128, dm) / dm ** 0.5,
         "Wv": rn(Hkv * 128, dm) / dm ** 0.5, "Wo": rn(dm, Hq * 128) / (Hq * 128) ** 0.5,
         "Wlm": 3.0 * rn(V, dm) / dm ** 0.5}
    prompts = [torch.randint(0, V, (context,), generator=g, device=dev).tolist() for _ in range(2)]
    opts = dict(kv_dtype="bf16", host_past=True, chunk_tokens=65536)
    kw = dict(x=30, bits=4, R=128, max_new=2 * rounds * 31 + 3000)
    # warm-up: the first launches of every kernel pay one-time costs
    w = TokenDecoder(W, Hq, Hkv, prompts[0][:4096], **kw, **opts)
    w.warm()
    w.generate(31)
    del w
    out = {"context": context, "link_GB_s": rate / 1e9, "rounds": rounds,
           "model": "one layer, d_model 256, 32/8 heads, d 128, vocab 2048; KIVI 4-bit drafter, x = 30; "
                    "full bf16 caches in pinned host memory (local host link)"}
    seqs = {}
    for sched in ("lockstep", "staggered"):
        d0 = TokenDecoder(W, Hq, Hkv, prompts[0], **kw, **opts)
        d1 = TokenDecoder(W, Hq, Hkv, prompts[1], copy_stream=d0.copy_stream, **kw, **opts)
        for d in (d0, d1):
            d.warm()
        nb = [d.stage_remote() for d in (d0, d1)]
        link = harness.ThrottledLink(rate)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        acc, inf = harness.remote_prefix_decode([d0, d1], link, [torch.cuda.current_stream(),
                                                                 torch.cuda.Stream()], rounds,
                                                staggered=sched == "staggered")
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        link.close()
        emitted = sum(len(em) for ga in acc for em in ga)
        seqs[sched] = [[t for em in ga for t in em] for ga in acc]
        out[sched] = {"tok_s": round(emitted / el, 2), "emitted": emitted, "seconds": round(el, 4),
                      "solo_rounds": inf["solo_rounds"],
                      "transfer_ms": [round((e - s) * 1e3, 2) for s, e in inf["transfers"]],
                      "accepted": [list(d0.rounds), list(d1.rounds)]}
        out["compressed_bytes_per_request"] = nb
        del d0, d1
    out["staggered_speedup"] = round(out["staggered"]["tok_s"] / out["lockstep"]["tok_s"], 3)
    per_req = min(len(s) for s in seqs["lockstep"])
    # greedy full-KV decoding, the full cache behind the local host link (one streamed pass/token)
    gd = [GreedyDecoder(W, Hq, Hkv, p, max_new=per_req + 8, **opts) for p in prompts]
    for d in gd:
        d.warm()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    greedy = [d.generate(per_req) for d in gd]
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    out["greedy_local"] = {"tok_s": round(2 * per_req / el, 2), "tokens_per_request": per_req,
                           "seconds": round(el, 3)}
    del gd
    # greedy full-KV decoding with the full cache shipped over the throttled link into HBM first
    gd = [GreedyDecoder(W, Hq, Hkv, p, max_new=per_req + 8, kv_dtype="bf16", host_past=False)
          for p in prompts]
    for d in gd:
        d.warm()
    nbf = [d.stage_remote() for d in gd]
    link = harness.ThrottledLink(rate)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    trs = [link.send(d.remote_pieces) for d in gd]
    remote_greedy = []
    for d, tr in zip(gd, trs):
        tr.wait()
        remote_greedy.append(d.generate(per_req))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    link.close()
    out["greedy_remote_full"] = {"tok_s": round(2 * per_req / el, 2), "seconds": round(el, 3),
                                 "full_bytes_per_request": nbf}
    out["speedup_vs_greedy_local"] = round(out["staggered"]["tok_s"] / out["greedy_local"]["tok_s"], 3)
    out["speedup_vs_greedy_remote_full"] = round(out["staggered"]["tok_s"] / out["greedy_remote_full"]["tok_s"], 3)
    out["first_divergence"] = [
        next((i for i in range(per_req) if seqs[s][r][i] != ref[r][i]), None)
        for s in ("lockstep", "staggered") for ref in (greedy, remote_greedy) for r in range(2)]
    return out


def _back_to_back_us(torch, launch, n: int) -> float:
    """Mean duration of n launches enqueued back to back between two events (microseconds)."""
    for i in range(3):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=4,
                    help="copies of the compressed cache rotated over the draft steps (keeps the "
                         "205 MB working set from being re-served by the 256 MB last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the rounds, run a plain device-to-device copy of this many MB three "
                         "times (reference kernel of known traffic for HBM counter runs)")
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4"],
                    help="c2 (default, the headline line): 8 x 32K, KIVI 2-bit. c1: 1 x 2048 fp32, "
                         "KIVI 4-bit. c3: 4 x 100K, Llama-70B-shaped, token-dropping drafter (25%% "
                         "kept). c4: 1 x 500K, full KV in pinned host memory streamed in 64K-token "
                         "chunks, KIVI 4-bit drafter")
    ap.add_argument("--stagger-rounds", type=int, default=3,
                    help="host-streamed workload only: rounds per schedule for the lock-step vs "
                         "staggered comparison over two request groups (0 skips it)")
    ap.add_argument("--decode-rounds", type=int, default=0,
                    help="single-request KIVI workloads (c1, c4): also run this many chained decode "
                         "rounds (commit + residual flush between rounds) and report them")
    ap.add_argument("--llama-context", type=int, default=0,
                    help="also decode one request on a random 4-layer Llama-form decoder (d_model 2048, "
                         "16/4 heads, SwiGLU 5632, vocab 32000) with a prompt of this many tokens, "
                         "caches in pinned host memory: VeriCache (2-bit KIVI, x = 30) vs greedy")
    ap.add_argument("--llama-tokens", type=int, default=512)
    ap.add_argument("--llama-bits", type=int, default=2, choices=[2, 4])
    ap.add_argument("--llama-x", type=int, default=30, help="draft length of the Llama-form run")
    ap.add_argument("--llama-batch", type=int, default=1,
                    help="requests decoded together in the Llama-form run (config 5: 16)")
    ap.add_argument("--e2e-context", type=int, default=0,
                    help="also decode one request token by token on a one-layer decoder with a "
                         "host-streamed bf16 cache of this many tokens: VeriCache vs greedy")
    ap.add_argument("--e2e-tokens", type=int, default=64)
    ap.add_argument("--remote-prefix", type=int, default=0,
                    help="also decode two requests whose compressed caches (KIVI 4-bit) of a prefix of "
                         "this many tokens cross a simulated 1.2 GB/s link, full caches in pinned host "
                         "memory: VeriCache lock-step vs staggered vs greedy full-KV decoding")
    ap.add_argument("--remote-rounds", type=int, default=8)
    ap.add_argument("--eager", action="store_true",
                    help="enqueue every launch of a round from Python instead of replaying the "
                         "round captured as a HIP graph")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_compressed_amd import harness, synth, vc

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)

    w = synth.WORKLOADS[args.workload]
    t_setup = time.perf_counter()
    K, V = synth.kv_past(w, args.seed)
    Kn, Vn = synth.kv_new(w, args.seed)
    inputs = (K, V, Kn, Vn, synth.q_new(w, args.seed), synth.projection(w, args.seed))
    st = harness.RoundState(w, seed=args.seed, inputs=inputs,
                            replicas=args.replicas if w.drafter == "kivi" else 1)
    if w.past_on_host:
        args.eager = True  # the host-streamed verify's copy-stream events are not captured
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    if args.copy_mb:
        src = torch.empty(args.copy_mb << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # One round = 30 x (append + draft attention, logits projection + argmax) + verify attention,
    # projection and accept: ~65 launches, replayed from a HIP graph so the host enqueue cost
    # (~10 us per launch from Python) does not pace the GPU.
    if not args.eager:
        st.capture_round()
    step = st.run_round if args.eager else st.replay_round
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps
    res = st.results()
    # Kernel durations for the roofline: the same launches (draft steps 0..29 over the rotating
    # replicas, the round's verify) enqueued back to back between two events on the launch stream,
    # so host enqueue time cannot show up as kernel time.
    reps = st.replicas or [None]
    d_kernel_us = _back_to_back_us(torch, lambda i: st.draft_attention(i % w.x, reps[i % len(reps)]),
                                   3 * w.x)
    v_kernel_us = _back_to_back_us(torch, lambda i: st.verify_attention(), 3 if w.past_on_host else 10)
    h2d = _h2d_rate(torch, vc, st) if w.past_on_host else None
    a_plus_1 = int((res["a"] + 1).sum())
    tok_s = a_plus_1 / (elapsed / args.steps)

    d_bytes = np.mean([st.draft_bytes(j) for j in range(w.x)])
    d_flops = np.mean([st.draft_flops(j) for j in range(w.x)])
    d_mean_s = d_kernel_us * 1e-6
    achieved = d_bytes / d_mean_s / 1e9
    traffic = _traffic_per_launch({"c2": "draft_quant_c2", "c3": "draft_drop_c3"}.get(args.workload, ""))
    v_traffic = _traffic_per_launch({"c2": "verify_c2", "c3": "verify_c3"}.get(args.workload, ""))
    v_mean_s = v_kernel_us * 1e-6
    v_gbs = st.verify_bytes() / v_mean_s / 1e9
    v_tflops = st.verify_flops() / v_mean_s / 1e12

    line = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.kv_dtype == "f32" else "bf16",
        "data": DATA_TEXT[args.workload],
        "config": {"workload": WORKLOAD_TEXT[args.workload],
                   "global_batch": w.B, "seq_len": w.n, "parallelism": "single GPU",
                   "compressed_cache_replicas": args.replicas,
                   "round_launch": "eager" if args.eager else "hip graph replay"},
        "roofline": {"bound": "hbm", "kernel": DRAFT_NAME[w.drafter, w.bits],
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": int(d_bytes), "launch_us": round(d_kernel_us, 2),
                     "timing": f"HIP events around {3 * w.x} back-to-back launches of the round's draft "
                               "calls on the launch stream, after the timed replays (mean per launch)"},
        "draft_attention": {"launch_us": round(d_kernel_us, 2), "GB_s": round(achieved, 1),
                            "TFLOP_s": round(d_flops / d_mean_s / 1e12, 2)},
        "verify_attention": {"launch_us": round(v_kernel_us, 2), "traffic": v_traffic,
                             "bytes_per_launch": int(st.verify_bytes()),
                             "GB_s": round(v_gbs, 1), "frac_hbm": round(v_gbs / HBM_PEAK_GBS, 4),
                             "TFLOP_s": round(v_tflops, 2),
                             "frac_bf16_mfma": round(v_tflops / 2500.0, 4)},
        "round": {"accepted": [int(a) for a in res["a"]], "emitted_per_round": a_plus_1,
                  "positions_verified_per_s": round(w.B * w.L / (elapsed / args.steps), 1)},
    }
    rs = _read_stream(torch, vc)
    line["roofline"]["read_stream"] = dict(rs, frac=round(achieved / rs["GB_s"], 4))
    if h2d is not None:
        v_gbs_pcie = st.verify_bytes() / v_mean_s / 1e9
        line["verify_attention"]["pcie"] = {
            "bound": "pcie", "achieved": round(v_gbs_pcie, 2), "peak": round(h2d["GB_s"], 2),
            "unit": "GB/s", "frac": round(v_gbs_pcie / h2d["GB_s"], 4),
            "peak_is": "achieved pinned host->device rate of the verify's own transfer alone "
                       "(vc_verify_stream_copies: the same 2-D copies of the same 64K-token chunks, "
                       "no compute; median of 10)",
            "frac_of_64GBs": round(v_gbs_pcie / 64.0, 4)}
    if w.drafter == "drop":
        sel_us = _back_to_back_us(torch, lambda i: st.select_keep(), 20)
        sel_bytes = w.B * w.Hkv * (w.n * 4 + st.kept * 4)
        line["keep_selection"] = {
            "launch_us": round(sel_us, 2), "rows": w.B * w.Hkv, "n": w.n, "kept": st.kept,
            "GB_s": round(sel_bytes / (sel_us * 1e-6) / 1e9, 1),
            "note": "vc_select_keep: scores read once (4 B per position) and kept positions written "
                    "(4 B each) per (b, kv head); one workgroup per row reads its row three times "
                    "(first-digit histogram, gathering that digit's candidates, writing the kept "
                    "positions)"}
    if w.past_on_host and args.stagger_rounds > 0:
        line["staggering"] = _staggering(torch, harness, synth, st, args.seed, args.stagger_rounds)
    if args.decode_rounds > 0 and w.B == 1 and w.drafter == "kivi":
        dl = _decode_loop(torch, harness, synth, w, args.seed, args.decode_rounds)
        if w.past_on_host:
            # full-KV greedy decode without a drafter streams the whole past once per token: its
            # rate is bounded by one host-streamed pass (the verify call measured above)
            dl["full_kv_decode_tok_s_bound"] = round(1e6 / v_kernel_us, 2)
            dl["full_kv_bound_is"] = ("1 / (one host-streamed pass over the full KV, the measured "
                                      "verify call): no run of a drafter-less decode")
        line["decode_loop"] = dl
        if w.past_on_host and args.stagger_rounds > 0:
            line["decode_two_requests"] = _decode_pair(torch, harness, synth, w, args.seed,
                                                       args.decode_rounds)
    if args.e2e_context > 0:
        line["e2e_decode"] = _e2e_decode(torch, args.seed, args.e2e_context, args.e2e_tokens)
    if args.remote_prefix > 0:
        line["remote_prefix"] = _remote_prefix(torch, args.seed, args.remote_prefix, args.remote_rounds)
    if args.llama_context > 0:
        line["e2e_llama"] = _e2e_llama(torch, args.seed, args.llama_context, args.llama_tokens,
                                       args.llama_bits, args.llama_x, args.llama_batch)
    if not args.no_cpu_baseline and args.workload == "c2":
        line["cpu_baseline"] = cpu_baseline(w, inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
