"""Pins of the transfer state-machine model (oracle/xfer_model.py): each test
is a scenario the pages describe, with the outcome their rules fix, worked out
by hand.  A planted-mistake check at the end shows the scenarios catch the
plausible slips.

[PUSH] "Implementierungsdetails" steps 1-3; [MORI] §3.1, §3.2, §6.
"""
import importlib.util
import os
import sys

import pytest

from oracle import xfer_model as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sc_register_first(M):
    """Registration before prefill: each saved layer is written at once."""
    m = M()
    assert m.register(1, 0, [7, 8], now=0.0)
    assert m.prefill(1, 0, 20, [3, 4], now=0.5)
    for l in range(3):
        assert m.save_layer(1, 0, l, now=1.0 + l)
    assert m.issued == [(1, 0, 0), (1, 0, 1), (1, 0, 2)]
    assert m.seal(1, 0)
    assert m.status(1) == (0, X.PENDING)
    for l in range(3):
        m.complete(1, 0, l)
    assert m.status(1) == (0, X.DONE)
    assert m.pop_finished() == [(1, 0, X.DONE)]
    assert m.pop_finished() == []
    assert m.recompute_blocks(1) == []


def sc_prefill_first(M):
    """Prefill finished before registration: writes wait, and the registration
    (arriving second) triggers them, in layer order."""
    m = M()
    assert m.prefill(2, 0, 20, [3, 4], now=0.0)
    for l in (1, 0, 2):
        assert m.save_layer(2, 0, l, now=1.0)
    assert m.issued == []
    assert m.seal(2, 0)
    assert m.register(2, 0, [9, 10], now=5.0)
    assert m.issued == [(2, 0, 0), (2, 0, 1), (2, 0, 2)]
    for l in range(3):
        m.complete(2, 0, l)
    assert m.status(2) == (0, X.DONE)


def sc_defer_timeout(M):
    """No registration within the defer timeout: the request is given up and
    its blocks freed; a late registration is ignored."""
    m = M(defer_timeout=60.0)
    m.prefill(3, 0, 20, [3, 4], now=0.0)
    m.save_layer(3, 0, 0, now=10.0)
    m.tick(69.9)
    assert m.status(3) == (0, X.PENDING)
    m.tick(70.0)
    assert m.status(3) == (0, X.EXPIRED)
    assert not m.register(3, 0, [5, 6], now=71.0)
    assert m.issued == []
    assert m.pop_finished() == [(3, 0, X.EXPIRED)]


def sc_expired_recompute(M):
    """Registered consumer blocks of a request that never got its KV are
    reported for recompute."""
    m = M(defer_timeout=60.0)
    m.register(4, 0, [11, 12, 13], now=0.0)
    m.save_layer(4, 0, 0, now=1.0)          # saved before the producer's block list: deferred
    assert m.issued == []
    m.prefill(4, 0, 40, [1, 2, 3], now=2.0)  # second of the two: the deferred write goes out
    assert m.issued == [(4, 0, 0)]
    assert m.save_layer(4, 0, 0, now=3.0)    # saving the same layer again changes nothing
    assert m.issued == [(4, 0, 0)]
    m.fail(4, 0, 0)
    assert m.status(4) == (0, X.FAILED)
    assert m.recompute_blocks(4) == [11, 12, 13]


def sc_seal_counts_queued_writes(M):
    """A hybrid model saves fewer layers than it has: the expected count is
    the number of writes actually queued when sealed."""
    m = M()
    m.register(5, 0, [1], now=0.0)
    m.prefill(5, 0, 8, [2], now=0.0)
    for l in (0, 2, 4):
        m.save_layer(5, 0, l, now=1.0)
    m.save_layer(5, 0, 2, now=1.5)           # a repeated save counts once
    assert m.seal(5, 0)
    assert not m.save_layer(5, 0, 6, now=2.0)  # nothing is queued after seal
    m.complete(5, 0, 0)
    m.complete(5, 0, 2)
    assert m.status(5) == (0, X.PENDING)
    m.complete(5, 0, 4)
    assert m.status(5) == (0, X.DONE)


def sc_middle_layer_failure(M):
    """The outcome is judged over every layer batch: a failed middle layer
    fails the transfer although later layers finished."""
    m = M()
    m.register(6, 0, [1], now=0.0)
    m.prefill(6, 0, 8, [2], now=0.0)
    for l in range(4):
        m.save_layer(6, 0, l, now=1.0)
    m.seal(6, 0)
    m.complete(6, 0, 0)
    m.fail(6, 0, 1)
    m.complete(6, 0, 2)
    m.complete(6, 0, 3)
    assert m.status(6) == (0, X.FAILED)


def sc_retry(M):
    """A re-sent request (new attempt) replaces the old attempt's state; old
    attempt messages are ignored afterwards."""
    m = M()
    m.prefill(7, 0, 20, [3, 4], now=0.0)
    m.save_layer(7, 0, 0, now=1.0)           # deferred under attempt 0
    assert m.prefill(7, 1, 20, [5, 6], now=2.0)
    assert not m.register(7, 0, [8, 9], now=3.0)   # stale attempt
    assert not m.save_layer(7, 0, 1, now=3.0)
    assert m.register(7, 1, [10, 11], now=4.0)
    assert m.issued == []                    # attempt 0's deferred write is gone
    m.save_layer(7, 1, 0, now=5.0)
    assert m.issued == [(7, 1, 0)]
    m.seal(7, 1)
    m.complete(7, 1, 0)
    assert m.status(7) == (1, X.DONE)
    assert m.pop_finished() == [(7, 1, X.DONE)]


def sc_transfer_timeout(M):
    """A write that does not finish within the transfer timeout fails the
    request."""
    m = M(transfer_timeout=30.0)
    m.register(8, 0, [1], now=0.0)
    m.prefill(8, 0, 8, [2], now=0.0)
    m.save_layer(8, 0, 0, now=10.0)
    m.save_layer(8, 0, 1, now=20.0)
    m.complete(8, 0, 0)
    m.tick(49.9)
    assert m.status(8) == (0, X.PENDING)
    m.tick(50.0)
    assert m.status(8) == (0, X.FAILED)


def sc_many_requests_order(M):
    """pop_finished reports by request ID, each once."""
    m = M()
    for rid in (30, 10, 20):
        m.register(rid, 0, [rid], now=0.0)
        m.prefill(rid, 0, 4, [rid + 1], now=0.0)
        m.save_layer(rid, 0, 0, now=0.0)
        m.seal(rid, 0)
    m.complete(20, 0, 0)
    m.complete(30, 0, 0)
    assert m.pop_finished() == [(20, 0, X.DONE), (30, 0, X.DONE)]
    m.complete(10, 0, 0)
    assert m.pop_finished() == [(10, 0, X.DONE)]


def sc_forget(M):
    """A request's record is dropped only once the request has finished
    ([MORI] §3.2: a finished request frees what it holds; a pending one still
    has writes in flight).  After that the ID is unknown: no status, no
    recompute list, and a second forget finds nothing."""
    m = M(defer_timeout=60.0, transfer_timeout=30.0)
    # 40: DONE; 41: FAILED (its only write failed); 42: EXPIRED (never registered); 43: PENDING
    for rid in (40, 41):
        m.register(rid, 0, [rid, rid + 100], now=0.0)
        m.prefill(rid, 0, 20, [1, 2], now=0.0)
        m.save_layer(rid, 0, 0, now=0.0)
        m.seal(rid, 0)
    m.complete(40, 0, 0)
    m.fail(41, 0, 0)
    m.prefill(42, 0, 20, [5, 6], now=0.0)
    m.save_layer(42, 0, 0, now=0.0)
    m.register(43, 0, [7], now=0.0)
    m.prefill(43, 0, 8, [8], now=0.0)
    m.save_layer(43, 0, 0, now=0.0)
    m.tick(60.0)                              # 42's deferral runs out; 43's write is 60 s old too
    assert [m.status(r) for r in (40, 41, 42)] == [(0, X.DONE), (0, X.FAILED), (0, X.EXPIRED)]
    assert m.status(43) == (0, X.FAILED)      # 43's write passed the 30 s transfer timeout
    m2 = M()
    m2.register(44, 0, [9], now=0.0)
    m2.prefill(44, 0, 8, [9], now=0.0)
    m2.save_layer(44, 0, 0, now=0.0)
    assert not m2.forget(44)                  # still pending: refused, record kept
    assert m2.status(44) == (0, X.PENDING)
    m2.seal(44, 0)
    m2.complete(44, 0, 0)
    assert m2.forget(44)
    assert m2.status(44) is None
    assert not m2.forget(44)
    assert m.recompute_blocks(41) == [41, 141]
    assert m.forget(41) and m.forget(42) and m.forget(40)
    assert [m.status(r) for r in (40, 41, 42)] == [None, None, None]
    assert m.recompute_blocks(41) == []       # the failed request's list left with its record
    assert m.pop_finished() == [(43, 0, X.FAILED)]   # forgotten requests are not reported
    assert not m.forget(99)                   # never seen
    # a forgotten ID starts over: a new registration is a new request
    assert m.register(40, 0, [50], now=61.0)
    assert m.status(40) == (0, X.PENDING)


def sc_save_layer_many(M):
    """One layer saved for a batch of requests ([MORI] §3.2, writes queued
    per layer right after its compute): a request whose blocks are known on
    both sides is written at once, one that still misses its registration is
    deferred until it arrives, and a stale attempt, an unknown request or a
    sealed request is refused.  The writes go out in batch order."""
    m = M()
    m.register(50, 0, [1], now=0.0)
    m.prefill(50, 0, 8, [2], now=0.0)         # ready
    m.prefill(51, 0, 8, [3], now=0.0)         # consumer not registered yet
    m.register(52, 1, [4], now=0.0)
    m.prefill(52, 1, 8, [5], now=0.0)         # attempt 1 is current
    m.register(53, 0, [6], now=0.0)
    m.prefill(53, 0, 8, [7], now=0.0)
    m.save_layer(53, 0, 0, now=0.0)
    m.seal(53, 0)                             # sealed: no more saves
    m.register(54, 0, [8], now=0.0)
    m.prefill(54, 0, 8, [9], now=0.0)         # ready, listed after 50
    acc = m.save_layer_many(3, [54, 51, 52, 77, 53, 50], [0, 0, 0, 0, 0, 0], now=1.0)
    assert acc == [True, True, False, False, False, True]
    assert m.issued == [(53, 0, 0), (54, 0, 3), (50, 0, 3)]
    m.register(51, 0, [10], now=2.0)          # the deferred write goes out now
    assert m.issued[-1] == (51, 0, 3)
    assert m.save_layer_many(3, [50, 51], [0, 0], now=3.0) == [True, True]   # repeats count once
    assert len(m.issued) == 4
    assert m.save_layer_many(4, [], [], now=3.0) == []


SCENARIOS = [sc_register_first, sc_prefill_first, sc_defer_timeout, sc_expired_recompute,
             sc_seal_counts_queued_writes, sc_middle_layer_failure, sc_retry, sc_transfer_timeout,
             sc_many_requests_order, sc_forget, sc_save_layer_many]


@pytest.mark.parametrize("scenario", SCENARIOS, ids=lambda f: f.__name__)
def test_scenario(scenario):
    scenario(X.XferModel)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def fresh_model():
    name = f"xfer_model_mut_{len(sys.modules)}"
    spec = importlib.util.spec_from_file_location(name, os.path.join(ROOT, "oracle", "xfer_model.py"))
    m = importlib.util.module_from_spec(spec)
    sys.modules[name] = m
    spec.loader.exec_module(m)
    return m


def mut_latest_layer_only(mod):
    def _settle(self, r):
        if r.state != mod.PENDING:
            return
        last = max(r.layers) if r.layers else None
        if last is not None and r.layers[last] == mod.L_FAILED:
            r.state = mod.FAILED
        elif r.sealed and sum(s == mod.L_DONE for s in r.layers.values()) == r.expected:
            r.state = mod.DONE
    mod.XferModel._settle = _settle


def mut_no_flush_on_register(mod):
    orig = mod.XferModel.register

    def register(self, rid, attempt, dst_ids, now):
        r = self._get(rid, attempt, create=True)
        if r is None or r.state != mod.PENDING or r.dst_ids is not None:
            return False
        r.dst_ids = tuple(dst_ids)
        return True
    mod.XferModel.register = register


def mut_strict_defer(mod):
    orig = mod.XferModel.tick

    def tick(self, now):
        return orig(self, now - 1e-9)
    mod.XferModel.tick = tick


def mut_expected_all_layers(mod):
    def seal(self, rid, attempt):
        r = self._get(rid, attempt, create=False)
        if r is None or r.state != mod.PENDING or r.sealed:
            return False
        r.sealed = True
        r.expected = max(r.layers) + 1 if r.layers else 0
        self._settle(r)
        return True
    mod.XferModel.seal = seal


def mut_stale_attempt_accepted(mod):
    def _get(self, rid, attempt, create):
        r = self.reqs.get(rid)
        if r is None:
            if not create:
                return None
            r = mod._Req(attempt)
            self.reqs[rid] = r
        return r
    mod.XferModel._get = _get


def mut_deferred_reverse_order(mod):
    def _flush_deferred(self, rid, r, now):
        if r.state != mod.PENDING or not self._ready(r):
            return
        for layer in sorted((l for l, s in r.layers.items() if s == mod.L_DEFERRED), reverse=True):
            self._issue(rid, r, layer, now)
        r.deferred_since = None
    mod.XferModel._flush_deferred = _flush_deferred


def mut_forget_pending(mod):
    def forget(self, rid):
        if rid not in self.reqs:
            return False
        del self.reqs[rid]
        return True
    mod.XferModel.forget = forget


def mut_forget_keeps_record(mod):
    def forget(self, rid):
        r = self.reqs.get(rid)
        return r is not None and r.state != mod.PENDING
    mod.XferModel.forget = forget


def mut_many_ready_only(mod):
    def save_layer_many(self, layer, rids, attempts, now):
        out = []
        for rid, a in zip(rids, attempts):
            r = self._get(rid, a, create=False)
            out.append(self.save_layer(rid, a, layer, now) if r is not None and self._ready(r) else False)
        return out
    mod.XferModel.save_layer_many = save_layer_many


def mut_many_reverse_order(mod):
    def save_layer_many(self, layer, rids, attempts, now):
        pairs = list(zip(rids, attempts))
        acc = [self.save_layer(r, a, layer, now) for r, a in reversed(pairs)]
        return acc[::-1]
    mod.XferModel.save_layer_many = save_layer_many


MUTATIONS = [mut_latest_layer_only, mut_no_flush_on_register, mut_strict_defer, mut_expected_all_layers,
             mut_stale_attempt_accepted, mut_deferred_reverse_order, mut_forget_pending,
             mut_forget_keeps_record, mut_many_ready_only, mut_many_reverse_order]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_caught(mutation):
    mod = fresh_model()
    mutation(mod)
    caught = 0
    for sc in SCENARIOS:
        try:
            sc(mod.XferModel)
        except Exception:
            caught += 1
    assert caught, mutation.__name__
