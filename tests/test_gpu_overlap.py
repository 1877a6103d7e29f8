"""Ordering and overlap on the GPU.

A synthetic compute kernel stands in for layer l's forward pass: it spins,
then writes a canary into the first 16 bytes of each of layer l's planned
source blocks, and the compute stream records ev[l].  kvx_push_layer(l,
ready=ev[l]) on a side stream must deliver the canary: the write waits for the
layer's event ([MORI] 3.2).  Also: two plans with disjoint destinations pushed
concurrently on two streams give the same bytes as one after the other."""

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


def test_event_gating_canary():
    spec = W.PoolSpec(8, 1024, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(11))
    st = [W.geometric_run_table(rng, 1024, 3.0)[:200]]
    dt = [W.geometric_run_table(rng, 1024, 3.0)[:200]]
    gs = S.device_side(spec, 3, 1)
    gd = S.device_side(spec, 3, 2)
    plan = kvx.kvx_plan(gs.pool, gd.pool, [200 * 16 - 1], st, dt)
    blocks = torch.from_numpy(st[0].astype(np.int32)).cuda()
    dblocks = torch.from_numpy(dt[0].astype(np.int64)).cuda()
    bb = 16 * 8 * 128 * 2
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for rep in range(100):
        if rep % 10 == 0:
            print("rep", rep, flush=True)
        canary = 0x1000 + rep
        evs = []
        for l in range(spec.num_layers):
            B.layer_compute(sink, 20000, 256, gs.region(l, 0), gs.region(l, 1), blocks, bb, canary + l,
                            stream=compute)
            e = torch.cuda.Event()
            e.record(compute)
            evs.append(e)
            kvx.kvx_push_layer(plan, l, ready=e, stream=side)
        side.synchronize()
        torch.cuda.synchronize()
        for l in range(spec.num_layers):
            for kv in (0, 1):
                reg = gd.region(l, kv).view(-1, bb)[dblocks][:, :16].cpu().numpy().view(np.uint32)
                c = (canary + l) & 0xFFFFFFFF
                exp = np.array([c, c ^ 0x5A5A5A5A, (c + 1) & 0xFFFFFFFF, ~c & 0xFFFFFFFF], np.uint32)
                assert (reg == exp[None, :]).all(), (rep, l, kv)
    plan.close()


def test_concurrent_streams_disjoint():
    spec = W.PoolSpec(4, 2048, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(12))
    dperm = rng.permutation(2048).astype(np.int32)
    s1 = [W.geometric_run_table(rng, 2048, 4.0)[:300]]
    s2 = [W.geometric_run_table(rng, 2048, 4.0)[:300]]
    d1, d2 = [dperm[:300]], [dperm[300:600]]
    hs, hd = W.host_values(spec, 4, 1), W.host_values(spec, 4, 2)
    gs = S.device_side(spec, 4, 1, values=hs)
    gd = S.device_side(spec, 4, 2, values=hd)
    p1 = kvx.kvx_plan(gs.pool, gd.pool, [300 * 16 - 3], s1, d1)
    p2 = kvx.kvx_plan(gs.pool, gd.pool, [300 * 16 - 9], s2, d2)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        for l in range(4):
            kvx.kvx_push_layer(p1, l, stream=a)
            kvx.kvx_push_layer(p2, l, stream=b)
    torch.cuda.synchronize()
    g = P.geom(O, spec)
    exp = O.Pool(g, hd[0].copy(), None)
    src = O.Pool(g, hs[0], None)
    O.push(src, exp, O.make_plan(g, g, [O.Request(300 * 16 - 3, s1[0], d1[0])]))
    O.push(src, exp, O.make_plan(g, g, [O.Request(300 * 16 - 9, s2[0], d2[0])]))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    p1.close()
    p2.close()


def test_plan_destroy_waits():
    """Destroying a plan right after enqueueing work on it is safe: the
    destroy waits for that work before freeing the descriptors."""
    spec = W.PoolSpec(16, 1024, 16, 8, 128, W.BF16)
    hs, hd = W.host_values(spec, 6, 1), W.host_values(spec, 6, 2)
    gs = S.device_side(spec, 6, 1, values=hs)
    gd = S.device_side(spec, 6, 2, values=hd)
    rng = np.random.Generator(np.random.PCG64(13))
    st, dt = [rng.permutation(1024)[:500].astype(np.int32)], [rng.permutation(1024)[:500].astype(np.int32)]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, [500 * 16], st, dt, stream=side)
    for l in range(16):
        kvx.kvx_push_layer(plan, l, stream=side)
    plan.close()
    side.synchronize()
    g = P.geom(O, spec)
    exp = O.Pool(g, hd[0].copy(), None)
    O.push(O.Pool(g, hs[0], None), exp, O.make_plan(g, g, [O.Request(500 * 16, st[0], dt[0])]))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)



def test_plan_released_after_its_stream():
    """kvx_plan_destroy_after: a plan released right after its pushes were
    enqueued stays intact until they ran, while plans built meanwhile get
    work lists of their own (both destinations match the oracle).
    Reclaiming a released plan does not wait for unrelated device work: a
    long compute kernel on another stream is still running when it returns."""
    from decode_kv_cache_amd import bench_support as B
    torch.cuda.synchronize()
    kvx.kvx_plan_reclaim(True)     # the release list is process-wide: start it empty
    spec = W.PoolSpec(8, 1024, 16, 8, 128, W.BF16)
    hs, hd = W.host_values(spec, 7, 1), W.host_values(spec, 7, 2)
    gs = S.device_side(spec, 7, 1, values=hs)
    gd = S.device_side(spec, 7, 2, values=hd)
    gd2 = S.device_side(spec, 7, 2, values=hd)
    rng = np.random.Generator(np.random.PCG64(14))
    st = [rng.permutation(1024)[:400].astype(np.int32)]
    dt = [rng.permutation(1024)[:400].astype(np.int32)]
    dt2 = [rng.permutation(1024)[:300].astype(np.int32)]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, [400 * 16], st, dt, stream=side)
    for l in range(8):
        kvx.kvx_push_layer(plan, l, stream=side)
    plan.close_after(side)                          # the pushes may still be queued
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, [300 * 16], [st[0][:300]], dt2, stream=side)
    for l in range(8):
        kvx.kvx_push_layer(plan2, l, stream=side)
    side.synchronize()
    g = P.geom(O, spec)
    exp = O.Pool(g, hd[0].copy(), None)
    O.push(O.Pool(g, hs[0], None), exp, O.make_plan(g, g, [O.Request(400 * 16, st[0], dt[0])]))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    exp2 = O.Pool(g, hd[0].copy(), None)
    O.push(O.Pool(g, hs[0], None), exp2, O.make_plan(g, g, [O.Request(300 * 16, st[0][:300], dt2[0])]))
    assert np.array_equal(gd2.kv.cpu().numpy(), exp2.kv)
    plan2.close_after(side)
    side.synchronize()                              # plan2's work is done
    compute = torch.cuda.Stream()
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    B.layer_compute(sink, 100_000_000, 256, stream=compute)   # bounded: a fixed loop, tens of ms at least
    busy = torch.cuda.Event()
    busy.record(compute)
    print("long compute kernel enqueued", flush=True)
    assert kvx.kvx_plan_reclaim(False) == 0          # both released plans freed
    assert not busy.query(), "kvx_plan_reclaim waited for unrelated device work"
    torch.cuda.synchronize()
    assert kvx.kvx_plan_reclaim(True) == 0

def test_overlap_plan_two_streams():
    """A plan built with KVX_PLAN_OVERLAP (whole 32 KiB blocks, 4 KiB pieces)
    pushed with its layers alternating over two side streams, each layer
    after its own fired event: byte-exact against the oracle, and the same
    bytes as the plan without the flag."""
    spec = W.PoolSpec(6, 1200, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(9600))
    need = [W.alloc_blocks(9000, 16)]
    wl = W.Workload("overlap_two_streams", 9600, spec, spec, [9000],
                    W.split_tables(W.geometric_run_table(rng, 1200, 4.0), need),
                    W.split_tables(W.geometric_run_table(rng, 1200, 4.0), need))
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    sides = [torch.cuda.Stream(), torch.cuda.Stream()]
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=True, stream=sides[0])
    base = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, host_only=True)
    assert plan.launch_shape()["piece_bytes"] == 4096 and base.launch_shape()["piece_bytes"] == 32768
    assert np.array_equal(plan.triples(), base.triples())
    ready = [torch.cuda.Event() for _ in range(spec.num_layers)]
    for e in ready:
        e.record()
    torch.cuda.synchronize()
    for l in range(spec.num_layers):
        kvx.kvx_push_layer(plan, l, ready=ready[l], stream=sides[l % 2])
    torch.cuda.synchronize()
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    exp = dst.copy()
    O.push(src, exp, op)
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    assert np.array_equal(gs.kv.cpu().numpy(), src.kv)
    plan.close()
