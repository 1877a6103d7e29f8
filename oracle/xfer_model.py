"""Oracle model of the producer-side transfer state machine -- TEST
INFRASTRUCTURE ONLY (see oracle/__init__.py for who may use it).

It follows the pages' description of when KV writes happen and when a
request counts as transferred, independently of the native implementation
(``kvx_xfer_*`` in libkvx):

* [PUSH] "Implementierungsdetails" steps 1-3: the consumer registers the block
  positions it reserved; registration and the producer's prefill may arrive
  in either order and whichever comes second triggers the transfer; requests
  are matched by ID, and re-sent, preempted or retried requests are mapped to
  the right state.
* [MORI] §3.2: each layer's write is queued right after that layer's compute
  and runs once the layer's event has fired; a write whose destination blocks
  are not known yet waits in a deferred list and is given up after a defer
  timeout (default 60 s), finishing the request so its blocks are freed; at
  the end of the forward pass the count of writes actually queued is sealed
  as the expected count (hybrid models save fewer layers than they register),
  and the request is done when the completed writes reach it.
* [MORI] §6: the transfer outcome is judged over the state of every layer
  batch (DONE / FAILED / PENDING), not the most recent one, because a middle
  layer can fail while later ones succeed; timeouts bound a stuck transfer
  (30 s by default).
* [MORI] §3.1: blocks whose KV failed to arrive are reported so the consumer
  recomputes them.

Readings where the pages leave a step open (listed in the design notes):
* An attempt number orders re-sends of one request ID: a message for an
  older attempt is ignored, one for a newer attempt discards everything held
  for the older one.
* The recompute list of a failed or expired request is every destination
  block the request registered (a failed layer batch leaves every block
  without that layer's KV); a done request has none.
* A layer saved twice in one attempt counts once.
* The deferral clock starts at the request's first deferred write; the
  transfer clock at each layer's issue.
* Seal before every queued write has completed is allowed (the request stays
  PENDING); a save after seal is rejected.

The model does not move bytes: an issued write completes when the driver says
so (``complete``) or fails (``fail``); the native state machine is compared
with this model on the same event sequences, and its real pushes are checked
against the copy oracle separately.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

PENDING, DONE, FAILED, EXPIRED = "PENDING", "DONE", "FAILED", "EXPIRED"
L_DEFERRED, L_ISSUED, L_DONE, L_FAILED = "DEFERRED", "ISSUED", "DONE", "FAILED"


@dataclass
class _Req:
    attempt: int
    num_tokens: Optional[int] = None
    src_ids: Optional[Tuple[int, ...]] = None
    dst_ids: Optional[Tuple[int, ...]] = None
    layers: Dict[int, str] = field(default_factory=dict)      # layer -> state
    issued_at: Dict[int, float] = field(default_factory=dict)
    deferred_since: Optional[float] = None
    sealed: bool = False
    expected: int = 0
    state: str = PENDING
    reported: bool = False


class XferModel:
    def __init__(self, defer_timeout: float = 60.0, transfer_timeout: float = 30.0):
        self.defer_timeout = defer_timeout
        self.transfer_timeout = transfer_timeout
        self.reqs: Dict[int, _Req] = {}
        self.issued: List[Tuple[int, int, int]] = []   # (request, attempt, layer) in issue order

    # -- matching by ID and attempt ([PUSH] step 2) ------------------------
    def _get(self, rid: int, attempt: int, create: bool) -> Optional[_Req]:
        r = self.reqs.get(rid)
        if r is not None and attempt < r.attempt:
            return None                       # stale message of an older attempt
        if r is None or attempt > r.attempt:
            if not create:
                return None
            r = _Req(attempt)
            self.reqs[rid] = r
        return r

    def _ready(self, r: _Req) -> bool:
        return r.dst_ids is not None and r.src_ids is not None

    def _issue(self, rid: int, r: _Req, layer: int, now: float) -> None:
        r.layers[layer] = L_ISSUED
        r.issued_at[layer] = now
        self.issued.append((rid, r.attempt, layer))

    def _flush_deferred(self, rid: int, r: _Req, now: float) -> None:
        if r.state != PENDING or not self._ready(r):
            return
        for layer in sorted(l for l, s in r.layers.items() if s == L_DEFERRED):
            self._issue(rid, r, layer, now)
        r.deferred_since = None

    # -- events -------------------------------------------------------------
    def register(self, rid: int, attempt: int, dst_ids: Sequence[int], now: float) -> bool:
        """Consumer registration: its reserved block positions ([PUSH] step 1)."""
        r = self._get(rid, attempt, create=True)
        if r is None or r.state != PENDING or r.dst_ids is not None:
            return False
        r.dst_ids = tuple(int(x) for x in dst_ids)
        self._flush_deferred(rid, r, now)
        return True

    def prefill(self, rid: int, attempt: int, num_tokens: int, src_ids: Sequence[int], now: float) -> bool:
        """Producer side: the request's token count and source blocks."""
        r = self._get(rid, attempt, create=True)
        if r is None or r.state != PENDING or r.src_ids is not None:
            return False
        r.num_tokens = int(num_tokens)
        r.src_ids = tuple(int(x) for x in src_ids)
        self._flush_deferred(rid, r, now)
        return True

    def save_layer(self, rid: int, attempt: int, layer: int, now: float) -> bool:
        """Layer computed: write now, or defer until both sides are known."""
        r = self._get(rid, attempt, create=False)
        if r is None or r.state != PENDING or r.sealed:
            return False
        if layer in r.layers:
            return True
        if self._ready(r):
            self._issue(rid, r, layer, now)
        else:
            r.layers[layer] = L_DEFERRED
            if r.deferred_since is None:
                r.deferred_since = now
        return True

    def save_layer_many(self, layer: int, rids: Sequence[int], attempts: Sequence[int], now: float) -> List[bool]:
        """One layer saved for a batch of requests: the same as saving it for
        each in order."""
        return [self.save_layer(r, a, layer, now) for r, a in zip(rids, attempts)]

    def seal(self, rid: int, attempt: int) -> bool:
        """End of the forward pass: the writes queued so far are the expected ones."""
        r = self._get(rid, attempt, create=False)
        if r is None or r.state != PENDING or r.sealed:
            return False
        r.sealed = True
        r.expected = len(r.layers)
        self._settle(r)
        return True

    def complete(self, rid: int, attempt: int, layer: int) -> None:
        """An issued write finished."""
        r = self._get(rid, attempt, create=False)
        if r is not None and r.layers.get(layer) == L_ISSUED:
            r.layers[layer] = L_DONE
            self._settle(r)

    def fail(self, rid: int, attempt: int, layer: int) -> None:
        """An issued write failed ([MORI] §6: one failed batch fails the transfer)."""
        r = self._get(rid, attempt, create=False)
        if r is not None and r.layers.get(layer) == L_ISSUED:
            r.layers[layer] = L_FAILED
            self._settle(r)

    def tick(self, now: float) -> None:
        """Timeouts: deferral ([MORI] §3.2) and stuck transfers ([MORI] §6)."""
        for r in self.reqs.values():
            if r.state != PENDING:
                continue
            if r.deferred_since is not None and now - r.deferred_since >= self.defer_timeout:
                r.state = EXPIRED
                continue
            for layer, s in r.layers.items():
                if s == L_ISSUED and now - r.issued_at[layer] >= self.transfer_timeout:
                    r.layers[layer] = L_FAILED
            self._settle(r)

    def _settle(self, r: _Req) -> None:
        if r.state != PENDING:
            return
        if any(s == L_FAILED for s in r.layers.values()):
            r.state = FAILED
        elif r.sealed and sum(s == L_DONE for s in r.layers.values()) == r.expected:
            r.state = DONE

    # -- queries -------------------------------------------------------------
    def status(self, rid: int) -> Optional[Tuple[int, str]]:
        r = self.reqs.get(rid)
        return None if r is None else (r.attempt, r.state)

    def pop_finished(self) -> List[Tuple[int, int, str]]:
        """Requests that reached DONE, FAILED or EXPIRED since the last call, by ID."""
        out = []
        for rid in sorted(self.reqs):
            r = self.reqs[rid]
            if r.state != PENDING and not r.reported:
                r.reported = True
                out.append((rid, r.attempt, r.state))
        return out

    def forget(self, rid: int) -> bool:
        """Drop a finished request's record."""
        r = self.reqs.get(rid)
        if r is None or r.state == PENDING:
            return False
        del self.reqs[rid]
        return True

    def recompute_blocks(self, rid: int) -> List[int]:
        """Destination blocks the consumer has to recompute ([MORI] §3.1)."""
        r = self.reqs.get(rid)
        if r is None or r.state not in (FAILED, EXPIRED) or r.dst_ids is None:
            return []
        return list(r.dst_ids)
