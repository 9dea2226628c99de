"""Host logic of the request-group schedules (no GPU): the order in which the staggered schedule
enqueues work and the stream dependencies it sets, checked with recording stand-ins for the
groups, streams and events.

The staggered schedule ("VeriCache: making lossy KV compression exact", Verifying Without Giving
Back the Speedup and Figure 2) must (1) keep each group's own order (draft phase, verify, draft
phase, ...), (2) let verifies take turns on the host link (verify k waits for verify k-1),
(3) start group g's first draft phase after group g-1's, and (4) enqueue the next group's draft
phase before this group's verify (with one group: after it).
"""
import contextlib
import types

import pytest

from kv_cache_compressed_amd import harness


class _Group:
    def __init__(self, i, log):
        self.i, self.log = i, log

    def draft_phase(self):
        self.log.append(("D", self.i))

    def verify_step(self):
        self.log.append(("V", self.i))


class _Stream:
    def __init__(self, name, log):
        self.name, self.log = name, log

    def wait_stream(self, other):
        self.log.append(("wait_stream", self.name, other.name))

    def wait_event(self, ev):
        self.log.append(("wait", self.name, ev.id))


def _fake_torch(log, cur):
    count = [0]
    current = [cur]

    class _Event:
        def __init__(self):
            count[0] += 1
            self.id = count[0]

        def record(self, stream):
            log.append(("rec", stream.name, self.id))

    @contextlib.contextmanager
    def stream(s):
        prev = current[0]
        current[0] = s
        try:
            yield
        finally:
            current[0] = prev

    cuda = types.SimpleNamespace(current_stream=lambda: current[0], Event=_Event, stream=stream)
    return types.SimpleNamespace(cuda=cuda), current


@pytest.mark.parametrize("ng,rounds", [(1, 3), (2, 1), (2, 4), (3, 3)])
def test_staggered_order_and_dependencies(monkeypatch, ng, rounds):
    log = []
    cur = _Stream("cur", log)
    fake, current = _fake_torch(log, cur)
    monkeypatch.setattr(harness, "torch", fake)
    streams = [_Stream(g, log) for g in range(ng)]
    # record which stream each phase is enqueued on
    groups = []
    for g in range(ng):
        grp = _Group(g, log)
        grp.draft_phase = (lambda g=g: log.append(("D", g, current[0].name)))
        grp.verify_step = (lambda g=g: log.append(("V", g, current[0].name)))
        groups.append(grp)
    harness.staggered(groups, streams, rounds)

    phases = [e for e in log if e[0] in ("D", "V")]
    # every phase on its group's stream; per group: D V D V ... (rounds times)
    for kind, g, s in phases:
        assert s == g
    for g in range(ng):
        assert [k for k, gg, _ in phases if gg == g] == ["D", "V"] * rounds
    # timeline order: D(0), then for each slot k: D(k+1) before V(k)
    total = ng * rounds
    expect = [("D", 0)]
    for k in range(total):
        if k + 1 < total and ng > 1:
            expect.append(("D", (k + 1) % ng))
        expect.append(("V", k % ng))
        if k + 1 < total and ng == 1:
            expect.append(("D", 0))
    assert [(k, g) for k, g, _ in phases] == expect

    # verify k (k >= 1) is preceded on its stream by a wait for the event recorded after verify k-1
    pos = {id(e): i for i, e in enumerate(log)}
    vidx = [i for i, e in enumerate(log) if e[0] == "V"]
    for k in range(1, total):
        prev_rec = next(e for e in log[vidx[k - 1] + 1:] if e[0] == "rec")
        assert prev_rec[1] == (k - 1) % ng
        waits = [e for e in log[vidx[k - 1]:vidx[k]] if e[0] == "wait" and e[1] == k % ng]
        assert any(w[2] == prev_rec[2] for w in waits), f"verify {k} does not wait for verify {k - 1}"
    # group g > 0 waits for the event recorded after group g-1's first draft phase, before drafting
    for g in range(1, ng):
        d_prev = next(i for i, e in enumerate(log) if e[0] == "D" and e[1] == g - 1)
        rec = next(e for e in log[d_prev + 1:] if e[0] == "rec" and e[1] == g - 1)
        d_g = next(i for i, e in enumerate(log) if e[0] == "D" and e[1] == g)
        assert ("wait", g, rec[2]) in log[:d_g]
    # the current stream waits for every group stream at the end
    tail = log[-ng:]
    assert tail == [("wait_stream", "cur", g) for g in range(ng)]


def test_lockstep_order(monkeypatch):
    log = []
    groups = [_Group(g, log) for g in range(3)]
    harness.lockstep(groups, rounds=2)
    assert log == [("D", 0), ("D", 1), ("D", 2), ("V", 0), ("V", 1), ("V", 2)] * 2


@pytest.mark.parametrize("ng,rounds", [(1, 3), (2, 3), (3, 2)])
def test_staggered_decode_order(monkeypatch, ng, rounds):
    """Chained decode rounds: per group D, V, C(ommit), I(nputs) in order on the group's own
    stream; every verify after the previous slot's commit and before the draft phase of the group
    that just committed, which is enqueued while that verify is in flight (before the next commit);
    verifies take turns on the host link."""
    log = []
    cur = _Stream("cur", log)
    fake, current = _fake_torch(log, cur)
    monkeypatch.setattr(harness, "torch", fake)

    class G:
        def __init__(self, i):
            self.i = i

        def draft_phase(self):
            log.append(("D", self.i, current[0].name))

        def verify_step(self):
            log.append(("V", self.i, current[0].name))

        def commit(self):
            log.append(("C", self.i, current[0].name))
            return 0

        def set_round_inputs(self, *a):
            log.append(("I", self.i, current[0].name))

    acc = harness.staggered_decode([G(g) for g in range(ng)], [_Stream(g, log) for g in range(ng)],
                                   rounds, lambda g, r: ())
    assert acc == [[0] * rounds for _ in range(ng)]
    ph = [e for e in log if e[0] in "DVCI"]
    for kind, g, s in ph:
        assert s == g
    for g in range(ng):
        seq = [k for k, gg, _ in ph if gg == g]
        assert seq == ["D", "V", "C", "I"] * (rounds - 1) + ["D", "V", "C"]
    order = [(k, g) for k, g, _ in ph]
    total = ng * rounds
    vs = [i for i, e in enumerate(order) if e[0] == "V"]
    cs = [i for i, e in enumerate(order) if e[0] == "C"]
    ds = [i for i, e in enumerate(order) if e[0] == "D"]
    assert [order[i][1] for i in vs] == [k % ng for k in range(total)]  # slot order
    for k in range(1, total):
        assert cs[k - 1] < vs[k]          # the previous commit precedes this verify
    if ng > 1:
        for k in range(total):
            if k + ng - 1 < total:        # the committed group's next draft phase under verify k
                assert vs[k] < ds[k + ng - 1] or k + ng - 1 < ng
                if k + 1 < total:
                    assert ds[k + ng - 1] < cs[k]
        assert all(ds[g] < vs[0] for g in range(ng))  # every group's first draft phase up front
    # verify k waits for the event recorded after verify k-1 on the previous slot's stream
    vlog = [i for i, e in enumerate(log) if e[0] == "V"]
    for k in range(1, total):
        rec = next(e for e in log[vlog[k - 1] + 1:] if e[0] == "rec")
        assert ("wait", k % ng, rec[2]) in log[vlog[k - 1]:vlog[k]]
