"""Ordering and overlap on the GPU.

A synthetic compute kernel stands in for layer l's forward pass: it spins,
then writes a canary into the first 16 bytes of each of layer l's planned
source blocks, and the compute stream records ev[l].  kvx_push_layer(l,
ready=ev[l]) on a side stream must deliver the canary: the write waits for the
layer's event ([MORI] 3.2).  Also: two plans with disjoint destinations pushed
concurrently on two streams give the same bytes as one after the other."""
import sys

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
    for rep in range(25):
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
