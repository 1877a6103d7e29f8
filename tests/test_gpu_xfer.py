"""The transfer state machine driving real pushes on the GPU.

A synthetic compute kernel stands in for each layer's forward pass and
writes a canary into that layer's source blocks as its last act; each layer
is saved with the compute stream's event.  Half of the requests register
before their prefill (writes go out as layers are saved), half after (writes
are deferred and go out at registration, [PUSH] "Implementierungsdetails"
step 2).  Every request must finish DONE, and every destination byte must
equal the oracle's push of the final source bytes.  A write reported failed
turns its request FAILED with all its registered blocks to recompute."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import bench_support as B
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_xfer_drives_pushes():
    spec = W.PoolSpec(8, 1024, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(77))
    R = 6
    plen = [int(x) for x in rng.integers(100, 1500, size=R)]
    need = [W.alloc_blocks(p, 16) for p in plen]
    st = W.split_tables(W.geometric_run_table(rng, 1024, 3.0), need)
    dt = W.split_tables(W.geometric_run_table(rng, 1024, 3.0), need)
    gs = S.device_side(spec, 5, 1)
    gd = S.device_side(spec, 5, 2)
    dst0 = gd.kv.cpu().numpy().copy()
    side = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    x = kvx.Xfer(gs.pool, log=True, stream=side)
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in plen]
    bb = 16 * 8 * 128 * 2
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    now = 0.0
    for r in range(R):
        if r % 2 == 0:
            assert x.register(r, 0, gd.pool, dt[r], now)
        assert x.prefill(r, 0, toks[r], st[r], now)
    for l in range(spec.num_layers):
        if l % 2 == 0:    # one save per request
            for r in range(R):
                blocks = torch.from_numpy(st[r][:-(-toks[r] // 16)].astype(np.int32)).cuda()
                B.layer_compute(sink, 3000, 64, gs.region(l, 0), gs.region(l, 1), blocks, bb,
                                0xAB00 + 16 * r + l, stream=compute)
                ev = torch.cuda.Event()
                ev.record(compute)
                assert x.save_layer(r, 0, l, now, ready=ev)
        else:             # one save of the layer for the whole batch
            for r in range(R):
                blocks = torch.from_numpy(st[r][:-(-toks[r] // 16)].astype(np.int32)).cuda()
                B.layer_compute(sink, 3000, 64, gs.region(l, 0), gs.region(l, 1), blocks, bb,
                                0xAB00 + 16 * r + l, stream=compute)
            ev = torch.cuda.Event()
            ev.record(compute)
            assert all(x.save_layer_many(l, range(R), [0] * R, now, ready=ev))
    for r in range(R):
        assert x.seal(r, 0)
    now = 1.0
    for r in range(1, R, 2):
        assert x.register(r, 0, gd.pool, dt[r], now)   # deferred writes go out now
    done = {}
    for _ in range(2000):
        x.poll(now)
        for rid, att, stt in x.pop_finished():
            done[rid] = stt
        if len(done) == R:
            break
        torch.cuda.synchronize()
    assert done == {r: kvx.KVX_REQ_DONE for r in range(R)}
    issued = x.issued()
    assert len(issued) == R * spec.num_layers
    torch.cuda.synchronize()
    g = P.geom(O, spec)
    src = O.Pool(g, gs.kv.cpu().numpy(), None)
    exp = O.Pool(g, dst0, None)
    O.push(src, exp, O.make_plan(g, g, [O.Request(n, s, d) for n, s, d in zip(toks, st, dt)]))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    x.close()


def test_xfer_reported_failure():
    spec = W.PoolSpec(2, 64, 16, 2, 64, W.BF16)
    gs = S.device_side(spec, 6, 1)
    gd = S.device_side(spec, 6, 2)
    side = torch.cuda.Stream()
    x = kvx.Xfer(gs.pool, stream=side)
    x.register(7, 0, gd.pool, [3, 4, 5], 0.0)
    x.prefill(7, 0, 40, [10, 11, 12], 0.0)
    x.save_layer(7, 0, 0, 0.0)
    x.save_layer(7, 0, 1, 0.0)
    x.seal(7, 0)
    x.complete(7, 0, 1, ok=False)
    assert x.status(7) == (0, kvx.KVX_REQ_FAILED)
    assert x.recompute_blocks(7) == [3, 4, 5]
    with pytest.raises(kvx.KvxError):
        x.complete(7, 0, 0, ok=True)     # device mode: completion comes from the stream
    x.poll(100.0)
    assert x.pop_finished() == [(7, 0, kvx.KVX_REQ_FAILED)]
    x.forget(7)
    assert x.status(7) is None
    x.close()


def test_poll_frees_plans_without_waiting_for_the_device():
    """A finished request's plan is released inside kvx_xfer_poll once the
    work enqueued with it is done.  Releasing it must not wait for unrelated
    device work: a long compute kernel is still running on another stream
    when that poll returns (hipFree would have waited for it)."""
    spec = W.PoolSpec(2, 256, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(78))
    need = [W.alloc_blocks(900, 16)]
    st = W.split_tables(W.geometric_run_table(rng, 256, 3.0), need)
    dt = W.split_tables(W.geometric_run_table(rng, 256, 3.0), need)
    gs = S.device_side(spec, 6, 1)
    gd = S.device_side(spec, 6, 2)
    side = torch.cuda.Stream()
    compute = torch.cuda.Stream()
    x = kvx.Xfer(gs.pool, stream=side)
    n = kvx.kvx_tokens_to_move(900, 0)
    assert x.register(7, 0, gd.pool, dt[0], 0.0)
    assert x.prefill(7, 0, n, st[0], 0.0)
    for l in range(spec.num_layers):
        assert x.save_layer(7, 0, l, 0.0)
    assert x.seal(7, 0)
    torch.cuda.synchronize()
    x.poll(0.0)                  # a mark behind the writes
    torch.cuda.synchronize()
    x.poll(0.0)                  # the writes are seen done: DONE, its plan retired behind a new mark
    assert x.status(7) == (0, kvx.KVX_REQ_DONE)
    torch.cuda.synchronize()     # that mark has fired: the next poll releases the plan
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    B.layer_compute(sink, 100_000_000, 256, stream=compute)   # bounded: a fixed loop, tens of ms at least
    busy = torch.cuda.Event()
    busy.record(compute)
    print("long compute kernel enqueued", flush=True)
    x.poll(0.0)
    assert not busy.query(), "kvx_xfer_poll waited for unrelated device work"
    torch.cuda.synchronize()
    assert x.pop_finished() == [(7, 0, kvx.KVX_REQ_DONE)]
    x.close()


@pytest.mark.parametrize("seed", range(6))
def test_xfer_random_device_sequences(seed):
    """Seeded random schedules in device mode: each request registers before
    a random layer or only after the forward pass (deferred writes, gated on
    events captured at their save); each layer's compute writes a canary into
    every request's source blocks and records the layer's event; layers are
    saved for the whole batch at once or request by request in random
    order; polls interleave with the work.  Every request ends DONE and the
    consumer pool equals the oracle's push of the final source bytes."""
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    spec = W.PoolSpec(4, 1024, 16, 8, 128, W.BF16) if seed % 2 else W.PoolSpec(5, 900, 16, 4, 64, W.BF16)
    R, L = 8, spec.num_layers
    plen = [int(x) for x in rng.integers(60, 1500, size=R)]
    need = [W.alloc_blocks(p, 16) for p in plen]
    st = W.split_tables(W.geometric_run_table(rng, spec.num_blocks, float(rng.choice([1.5, 6.0]))), need)
    dt = W.split_tables(W.geometric_run_table(rng, spec.num_blocks, float(rng.choice([1.5, 6.0]))), need)
    gs = S.device_side(spec, 8 + seed, 1)
    gd = S.device_side(spec, 8 + seed, 2)
    dst0 = gd.kv.cpu().numpy().copy()
    side = torch.cuda.Stream()
    compute = torch.cuda.Stream()
    x = kvx.Xfer(gs.pool, stream=side)
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in plen]
    bb = spec.block_size * spec.num_heads * spec.head_dim * spec.elem_bytes
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    blocks = torch.from_numpy(np.concatenate([st[r][:-(-toks[r] // 16)] for r in range(R)]).astype(np.int32)).cuda()
    reg_at = [int(rng.integers(0, L + 1)) for _ in range(R)]     # L: after the forward pass
    now = 0.0
    for r in range(R):
        assert x.prefill(r, 0, toks[r], st[r], now)
    print(f"seed {seed}: registration layers {reg_at}", flush=True)
    for l in range(L):
        for r in range(R):
            if reg_at[r] == l:
                assert x.register(r, 0, gd.pool, dt[r], now)
        B.layer_compute(sink, 2000, 64, gs.region(l, 0), gs.region(l, 1), blocks, bb, 0xC000 + 64 * seed + l,
                        stream=compute)
        ev = torch.cuda.Event()
        ev.record(compute)
        if rng.integers(0, 2):
            assert all(x.save_layer_many(l, range(R), [0] * R, now, ready=ev))
        else:
            for r in rng.permutation(R):
                assert x.save_layer(int(r), 0, l, now, ready=ev)
        if rng.integers(0, 3) == 0:
            x.poll(now)
    for r in range(R):
        assert x.seal(r, 0)
    for r in range(R):
        if reg_at[r] == L:
            assert x.register(r, 0, gd.pool, dt[r], now)
    done = {}
    for _ in range(2000):
        x.poll(now)
        for rid, att, stt in x.pop_finished():
            done[rid] = stt
        if len(done) == R:
            break
        torch.cuda.synchronize()
    assert done == {r: kvx.KVX_REQ_DONE for r in range(R)}, done
    torch.cuda.synchronize()
    g = P.geom(O, spec)
    src = O.Pool(g, gs.kv.cpu().numpy(), None)
    exp = O.Pool(g, dst0, None)
    O.push(src, exp, O.make_plan(g, g, [O.Request(n, s, d) for n, s, d in zip(toks, st, dt)]))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    x.close()
