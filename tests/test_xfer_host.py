"""The native transfer state machine (kvx_xfer_*, host-only mode) against the
oracle model on random event sequences: same issued writes in the same order,
same request states, finished reports and recompute lists after every event."""
import numpy as np
import pytest

from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import workloads as W
from oracle import xfer_model as X
from test_abi_host import fake_pool

STATE = {kvx.KVX_REQ_PENDING: X.PENDING, kvx.KVX_REQ_DONE: X.DONE, kvx.KVX_REQ_FAILED: X.FAILED,
         kvx.KVX_REQ_EXPIRED: X.EXPIRED}
SPEC = W.PoolSpec(4, 64, 4, 1, 16, W.U8)


def run_sequence(seed, steps=300, ids=(1, 2, 3, 4, 5)):
    rng = np.random.Generator(np.random.PCG64(seed))
    prod, cons = fake_pool(SPEC, 0), fake_pool(SPEC, 1)
    defer_t, xfer_t = float(rng.choice([5.0, 20.0])), float(rng.choice([3.0, 10.0]))
    nat = kvx.Xfer(prod, defer_timeout=defer_t, transfer_timeout=xfer_t, host_only=True, log=True)
    mod = X.XferModel(defer_timeout=defer_t, transfer_timeout=xfer_t)
    now = 0.0
    seen = set()
    attempts = {i: 0 for i in ids}
    for step in range(steps):
        rid = int(rng.choice(ids))
        att = attempts[rid] + int(rng.choice([0, 0, 0, 0, 0, 1, -1])) if attempts[rid] > 0 else \
            attempts[rid] + int(rng.choice([0, 0, 0, 0, 1]))
        att = max(att, 0)
        attempts[rid] = max(attempts[rid], att)
        op = rng.choice(["register", "prefill", "save", "save", "save", "save_many", "seal", "complete",
                         "complete", "fail", "tick", "pop", "forget"])
        if op == "register":
            ids_d = (rng.permutation(64)[:3]).astype(np.int32)
            a = nat.register(rid, att, cons, ids_d, now)
            b = mod.register(rid, att, ids_d, now)
        elif op == "prefill":
            ids_s = (rng.permutation(64)[:3]).astype(np.int32)
            n = int(rng.integers(0, 13))
            a = nat.prefill(rid, att, n, ids_s, now)
            b = mod.prefill(rid, att, n, ids_s, now)
        elif op == "save":
            layer = int(rng.integers(0, 4))
            a = nat.save_layer(rid, att, layer, now)
            b = mod.save_layer(rid, att, layer, now)
        elif op == "save_many":
            layer = int(rng.integers(0, 4))
            k = int(rng.integers(0, 4))
            rs = [int(v) for v in rng.choice(ids, size=k)]
            ats = [attempts[v] + int(rng.choice([0, 0, -1])) for v in rs]
            ats = [max(v, 0) for v in ats]
            a = nat.save_layer_many(layer, rs, ats, now)
            b = mod.save_layer_many(layer, rs, ats, now)
        elif op == "seal":
            a, b = nat.seal(rid, att), mod.seal(rid, att)
        elif op in ("complete", "fail"):
            issued = [e for e in mod.issued if e[0] == rid]
            if not issued:
                continue
            _, at2, layer = issued[int(rng.integers(0, len(issued)))]
            nat.complete(rid, at2, layer, ok=(op == "complete"))
            (mod.complete if op == "complete" else mod.fail)(rid, at2, layer)
            a = b = None
        elif op == "tick":
            now += float(rng.choice([0.5, 1.0, 4.0, 8.0]))
            nat.poll(now)
            mod.tick(now)
            a = b = None
        elif op == "pop":
            a = [(r, at2, STATE[s]) for r, at2, s in nat.pop_finished()]
            b = mod.pop_finished()
            seen |= {s for _, _, s in b}
        else:
            st = mod.status(rid)
            if st is None or st[1] == X.PENDING:
                continue
            nat.forget(rid)
            mod.forget(rid)
            a = b = None
        assert a == b, (seed, step, op, rid, att, a, b)
        assert nat.issued() == mod.issued, (seed, step, op)
        for i in ids:
            s_nat, s_mod = nat.status(i), mod.status(i)
            assert (None if s_nat is None else (s_nat[0], STATE[s_nat[1]])) == s_mod, (seed, step, i)
            r_nat = nat.recompute_blocks(i)
            assert (r_nat or []) == mod.recompute_blocks(i), (seed, step, i)
    nat.close()
    return len(mod.issued), {r.state for r in mod.reqs.values()} | seen


@pytest.mark.parametrize("seed", range(40))
def test_native_matches_model(seed):
    run_sequence(seed)


def test_sequences_exercise_every_outcome():
    """The random sequences issue writes and reach DONE, FAILED and EXPIRED."""
    outcomes, issued = set(), 0
    for seed in range(40):
        n, seen = run_sequence(seed, steps=300)
        issued += n
        outcomes |= seen
    assert {X.DONE, X.FAILED, X.EXPIRED} <= outcomes
    assert issued > 100


def test_native_errors():
    prod = fake_pool(SPEC, 0)
    x = kvx.Xfer(prod, host_only=True)
    with pytest.raises(kvx.KvxError) as e:
        x.save_layer(1, 0, 4, 0.0)           # layer out of range
    assert e.value.code == kvx.KVX_E_RANGE
    assert not x.save_layer(1, 0, 0, 0.0)    # unknown request: ignored
    assert x.status(9) is None
    x.register(1, 0, fake_pool(SPEC, 1), [70, 71], 0.0)   # IDs outside the consumer pool
    with pytest.raises(kvx.KvxError) as e:
        x.prefill(1, 0, 4, [1], 0.0)         # rendezvous builds the plan: range error, request failed
    assert e.value.code == kvx.KVX_E_RANGE
    assert x.status(1) == (0, kvx.KVX_REQ_FAILED)
    with pytest.raises(kvx.KvxError):
        x.forget(2)
    with pytest.raises(kvx.KvxError) as e:   # no issue log without KVX_XFER_LOG
        x.issued()
    assert e.value.code == kvx.KVX_E_INVAL
    x.close()
    import ctypes
    cfg = kvx.kvx_xfer_config(60.0, 30.0, kvx.KVX_XFER_HOST_ONLY | 4)
    h = ctypes.c_void_p()
    assert kvx.lib().kvx_xfer_create(prod.handle, ctypes.byref(cfg), None, ctypes.byref(h)) == kvx.KVX_E_INVAL
    assert b"unknown flags 0x5" in kvx.lib().kvx_last_error()


def test_threads_share_one_instance():
    """Calls on one kvx_xfer are serialized internally: eight threads drive
    disjoint requests through registration, prefill, layer saves (half of
    them deferred), seal and completion at once (ctypes releases the GIL
    around each foreign call).  Every request ends DONE, every write is logged
    exactly once, and each request's writes keep layer order in the log."""
    import threading
    prod, cons = fake_pool(SPEC, 0), fake_pool(SPEC, 1)
    x = kvx.Xfer(prod, host_only=True, log=True)
    T, PER, L = 8, 40, SPEC.num_layers
    errors = []

    def worker(t):
        try:
            for k in range(PER):
                rid = t * 1000 + k
                first = (lambda: x.register(rid, 0, cons, [3, 4], 0.0)) if k % 2 else \
                        (lambda: x.prefill(rid, 0, 8, [1, 2], 0.0))
                second = (lambda: x.prefill(rid, 0, 8, [1, 2], 0.0)) if k % 2 else \
                         (lambda: x.register(rid, 0, cons, [3, 4], 0.0))
                assert first()
                for l in range(L // 2):
                    assert x.save_layer(rid, 0, l, 0.0)         # deferred: one side unknown
                assert second()                                 # both sides known: deferred writes go out
                for l in range(L // 2, L):
                    assert x.save_layer(rid, 0, l, 0.0)
                assert x.seal(rid, 0)
                for l in range(L):
                    x.complete(rid, 0, l, True)
                assert x.status(rid) == (0, kvx.KVX_REQ_DONE), rid
        except Exception as e:   # reported by the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(T)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    log = x.issued()
    assert len(log) == T * PER * L
    assert len(set(log)) == len(log)
    for t in range(T):
        for k in range(PER):
            rid = t * 1000 + k
            assert [e[2] for e in log if e[0] == rid] == list(range(L)), rid
    done = []
    while True:
        got = x.pop_finished()
        if not got:
            break
        done += got
    assert len(done) == T * PER and all(s == kvx.KVX_REQ_DONE for _, _, s in done)
    x.close()


class NativeAsModel:
    """The native state machine (host-only) behind the oracle model's
    interface, so the hand-worked page scenarios pin it directly."""

    # one 64-slot block holds every scenario's prompt; IDs up to 255, layers up to 7
    SPEC = W.PoolSpec(8, 256, 64, 1, 16, W.U8)

    def __init__(self, defer_timeout: float = 60.0, transfer_timeout: float = 30.0):
        self._prod, self._cons = fake_pool(self.SPEC, 0), fake_pool(self.SPEC, 1)
        self._x = kvx.Xfer(self._prod, defer_timeout=defer_timeout, transfer_timeout=transfer_timeout,
                           host_only=True, log=True)

    @property
    def issued(self):
        return [tuple(int(v) for v in e) for e in self._x.issued()]

    def register(self, rid, attempt, dst_ids, now):
        return self._x.register(rid, attempt, self._cons, dst_ids, now)

    def prefill(self, rid, attempt, num_tokens, src_ids, now):
        return self._x.prefill(rid, attempt, num_tokens, src_ids, now)

    def save_layer(self, rid, attempt, layer, now):
        return self._x.save_layer(rid, attempt, layer, now)

    def save_layer_many(self, layer, rids, attempts, now):
        return self._x.save_layer_many(layer, rids, attempts, now)

    def seal(self, rid, attempt):
        return self._x.seal(rid, attempt)

    def complete(self, rid, attempt, layer):
        self._x.complete(rid, attempt, layer, ok=True)

    def fail(self, rid, attempt, layer):
        self._x.complete(rid, attempt, layer, ok=False)

    def tick(self, now):
        self._x.poll(now)

    def status(self, rid):
        s = self._x.status(rid)
        return None if s is None else (s[0], STATE[s[1]])

    def pop_finished(self):
        return [(int(r), int(a), STATE[s]) for r, a, s in self._x.pop_finished()]

    def forget(self, rid):
        try:
            self._x.forget(rid)
            return True
        except kvx.KvxError:
            return False

    def recompute_blocks(self, rid):
        return self._x.recompute_blocks(rid) or []


def page_scenarios():
    import test_xfer_oracle as T
    return T.SCENARIOS


@pytest.mark.parametrize("scenario", page_scenarios(), ids=lambda f: f.__name__)
def test_native_follows_page_scenarios(scenario):
    """Every hand-worked scenario that pins the model also holds for the
    native state machine, forget and batched saves included."""
    scenario(NativeAsModel)
