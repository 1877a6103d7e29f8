"""The layer write queue (kvx_queue_*) on the GPU, against the oracle.

- The Qwen3-32B-shaped push at full size through the queue, events already
  fired (writes back up and leave in merged launch groups): sampled layers
  byte for byte against the oracle, fewer launch groups than writes.
- Event gating: a synthetic compute kernel writes a canary into each layer's
  planned source blocks before its event; every queued write must carry it,
  and the whole consumer pool must equal the oracle's push of the source as
  the compute left it ([MORI] §3.2, the event sync before each layer write).
- Random small cases: several plans with disjoint destinations, layers in
  random order, a mix of fired, pending and absent events, flushes in
  between; pool bytes and scales against the oracle.
- Head-slice writes (kvx_queue_push_heads) in random layouts and slices,
  mixed in one queue with pushes of the same source into a pool of its own
  geometry, under the same mix of events: both consumer pools and their
  scales against the oracle's head transform and push.
- Argument errors, and refusal under graph capture."""
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
from test_gpu_parity import check_layers, dev_scales, host_sides, oracle_requests, snapshot, tokens

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_queue_qwen32b_full():
    wl = W.qwen32b_push()
    say("workload qwen32b_push through the queue")
    gs = S.device_side(wl.src, wl.seed, 1)
    gd = S.device_side(wl.dst, wl.seed, 2)
    torch.cuda.synchronize()
    layers = [0, 1, 37, 63]
    src_snap, dst_snap = snapshot(gs, layers), snapshot(gd, layers)
    toks = tokens(wl)
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    evs = []
    for l in range(wl.src.num_layers):
        e = torch.cuda.Event()
        e.record()
        evs.append(e)
    torch.cuda.synchronize()
    q = kvx.Queue(side)
    for l in range(wl.src.num_layers):
        q.push(plan, l, ready=evs[l])
    q.flush()
    done = torch.cuda.Event()
    done.record(side)
    done.synchronize()
    writes, groups = q.stats()
    say("writes", writes, "launch groups", groups)
    assert writes == wl.src.num_layers and 1 <= groups < writes
    op = O.make_plan(P.geom(O, wl.src), P.geom(O, wl.dst), oracle_requests(wl, toks))
    check_layers(wl, gs, gd, src_snap, dst_snap, op, layers, "qwen32b_push via kvx_queue")
    q.close()
    plan.close()
    del gs, gd
    torch.cuda.empty_cache()


def test_queue_event_gating_canary():
    """Writes of layers whose compute is still running wait for it; the
    consumer pool equals the oracle's push of the source after the canaries."""
    spec = W.PoolSpec(8, 1024, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(21))
    st = [W.geometric_run_table(rng, 1024, 3.0)[:200]]
    dt = [W.geometric_run_table(rng, 1024, 3.0)[:200]]
    hs, hd = W.host_values(spec, 5, 1), W.host_values(spec, 5, 2)
    gs = S.device_side(spec, 5, 1, values=hs)
    gd = S.device_side(spec, 5, 2, values=hd)
    n = 200 * 16 - 1
    plan = kvx.kvx_plan(gs.pool, gd.pool, [n], st, dt)
    blocks = torch.from_numpy(st[0].astype(np.int32)).cuda()
    bb = 16 * 8 * 128 * 2
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    q = kvx.Queue(side)
    for rep in range(40):
        if rep % 10 == 0:
            say("rep", rep)
        canary = 0x2000 + 16 * rep
        iters = int(rng.choice([0, 2000, 20000]))
        for l in range(spec.num_layers):
            B.layer_compute(sink, iters, 256, gs.region(l, 0), gs.region(l, 1), blocks, bb, canary + l,
                            stream=compute)
            e = torch.cuda.Event()
            e.record(compute)
            q.push(plan, l, ready=e)
        q.flush()
        side.synchronize()
        torch.cuda.synchronize()
        if rep % 8 == 7 or rep == 0:
            g = P.geom(O, spec)
            src = O.Pool(g, gs.kv.cpu().numpy(), None)
            exp = O.Pool(g, hd[0].copy(), None)
            O.push(src, exp, O.make_plan(g, g, [O.Request(n, st[0], dt[0])]))
            assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), rep
        else:
            dblocks = torch.from_numpy(dt[0].astype(np.int64)).cuda()
            for l in range(spec.num_layers):
                for kv in (0, 1):
                    reg = gd.region(l, kv).view(-1, bb)[dblocks][:, :16].cpu().numpy().view(np.uint32)
                    c = (canary + l) & 0xFFFFFFFF
                    want = np.array([c, c ^ 0x5A5A5A5A, (c + 1) & 0xFFFFFFFF, ~c & 0xFFFFFFFF], np.uint32)
                    assert (reg == want[None, :]).all(), (rep, l, kv)
    w, g = q.stats()
    say("writes", w, "groups", g)
    assert w == 40 * spec.num_layers
    q.close()
    plan.close()


def test_queue_random_small():
    rng = np.random.Generator(np.random.PCG64(22))
    sink = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
    compute = torch.cuda.Stream()
    for case in range(24):
        L = int(rng.integers(1, 5))
        spec = W.PoolSpec(L, 300, int(rng.choice([1, 4, 16])), int(rng.integers(1, 4)),
                          int(rng.choice([16, 64, 128])), [W.U8, W.BF16][case % 2], ["NHD", "HND"][(case // 2) % 2],
                          has_scales=bool(case % 3 == 0))
        hs, hd = W.host_values(spec, 900 + case, 1), W.host_values(spec, 900 + case, 2)
        gs = S.device_side(spec, 900 + case, 1, values=hs)
        gd = S.device_side(spec, 900 + case, 2, values=hd)
        dperm = rng.permutation(300).astype(np.int32)
        nplans = int(rng.integers(1, 4))
        plans, reqs = [], []
        used = 0
        for k in range(nplans):
            ntok = int(rng.integers(0, 20 * spec.block_size))
            nb = -(-ntok // spec.block_size)
            sids = rng.permutation(300).astype(np.int32)[:nb + 1]
            dids = dperm[used:used + nb + 1]
            used += nb + 1
            plans.append(kvx.kvx_plan(gs.pool, gd.pool, [ntok], [sids], [dids]))
            reqs.append(O.Request(ntok, sids, dids))
        say("case", case, spec, [r.num_tokens for r in reqs])
        side = torch.cuda.Stream()
        q = kvx.Queue(side)
        writes = [(k, l) for k in range(nplans) for l in range(L)]
        rng.shuffle(writes)
        for i, (k, l) in enumerate(writes):
            kind = int(rng.integers(0, 3))
            ev = None
            if kind == 1:      # fired
                ev = torch.cuda.Event()
                ev.record(compute)
                compute.synchronize()
            elif kind == 2:    # likely still pending when queued
                B.layer_compute(sink, 5000, 64, stream=compute)
                ev = torch.cuda.Event()
                ev.record(compute)
            q.push(plans[k], l, ready=ev)
            if rng.random() < 0.2:
                q.flush()
        q.close()
        torch.cuda.synchronize()
        g = P.geom(O, spec)
        src = O.Pool(g, hs[0], hs[1])
        exp = O.Pool(g, hd[0].copy(), None if hd[1] is None else hd[1].copy())
        for k in range(nplans):
            O.push(src, exp, O.make_plan(g, g, [reqs[k]]))
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), case
        if exp.scales is not None:
            assert np.array_equal(S.scale_bits(gd.sc), exp.scales), case
        for p in plans:
            p.close()


def test_queue_heads_random_small():
    rng = np.random.Generator(np.random.PCG64(23))
    sink = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
    compute = torch.cuda.Stream()
    for i, (sl, dl) in enumerate([("NHD", "HND"), ("HND", "NHD"), ("NHD", "NHD"), ("HND", "HND")] * 3):
        hs = int(rng.integers(1, 9))
        hd = int(rng.integers(1, 9))
        L = int(rng.integers(1, 6))
        wl = W.random_case(8300 + i, layout=sl, dst_layout=dl, elem_bytes=int(rng.choice([1, 2])),
                           num_layers=L, num_blocks=120, block_size=int(rng.choice([1, 4, 16])),
                           num_heads=hs, dst_heads=hd, head_dim=int(rng.choice([16, 64, 128])),
                           has_scales=bool(i % 2), num_requests=3, max_tokens=40, run_mean=2.0)
        src, dst, gs, gd = host_sides(wl)
        toks = tokens(wl)
        reqs = oracle_requests(wl, toks)
        nh = int(rng.integers(0, min(hs, hd) + 1))
        s0 = int(rng.integers(0, hs - nh + 1))
        d0 = int(rng.integers(0, hd - nh + 1))
        say("case", wl.name, sl, dl, hs, hd, L, (s0, d0, nh))
        hplan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
        # a second consumer with the source's geometry, pushed in the same queue
        h2 = W.host_values(wl.src, wl.seed, 3)
        g2 = S.device_side(wl.src, wl.seed, 3, values=h2)
        pplan = kvx.kvx_plan(gs.pool, g2.pool, toks, wl.src_tables, wl.dst_tables)
        side = torch.cuda.Stream()
        q = kvx.Queue(side)
        writes = [(kind, l) for kind in ("heads", "push") for l in range(L)]
        rng.shuffle(writes)
        for kind, l in writes:
            ev_kind = int(rng.integers(0, 3))
            ev = None
            if ev_kind == 1:      # fired
                ev = torch.cuda.Event()
                ev.record(compute)
                compute.synchronize()
            elif ev_kind == 2:    # likely still pending when queued
                B.layer_compute(sink, 5000, 64, stream=compute)
                ev = torch.cuda.Event()
                ev.record(compute)
            if kind == "heads":
                q.push_heads(hplan, l, s0, d0, nh, ready=ev)
            else:
                q.push(pplan, l, ready=ev)
            if rng.random() < 0.2:
                q.flush()
        q.close()
        torch.cuda.synchronize()
        exp = dst.copy()
        if nh:
            op = O.make_plan(src.geom, dst.geom, reqs)
            for l in range(L):
                O.copy_heads(src, exp, op, reqs, l, s0, d0, nh)
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), wl.name
        if exp.scales is not None:
            assert np.array_equal(dev_scales(gd), exp.scales), wl.name
        exp2 = O.Pool(src.geom, h2[0].copy(), None if h2[1] is None else h2[1].copy())
        O.push(src, exp2, O.make_plan(src.geom, src.geom, reqs))
        assert np.array_equal(g2.kv.cpu().numpy(), exp2.kv), wl.name
        if exp2.scales is not None:
            assert np.array_equal(dev_scales(g2), exp2.scales), wl.name
        hplan.close()
        pplan.close()


def test_queue_heads_errors():
    """kvx_queue_push_heads validates as kvx_copy_heads does, and a state
    pool has no heads."""
    src_spec = W.PoolSpec(2, 64, 4, 4, 16, W.BF16, "NHD")
    dst_spec = W.PoolSpec(2, 64, 4, 2, 16, W.BF16, "HND")
    gs, gd = S.device_side(src_spec, 5, 1), S.device_side(dst_spec, 5, 2)
    plan = kvx.kvx_plan(gs.pool, gd.pool, [8], [[1, 2]], [[3, 4]])
    q = kvx.Queue()
    for args, code in (((2, 0, 0, 1), kvx.KVX_E_RANGE), ((0, 3, 0, 2), kvx.KVX_E_RANGE),
                       ((0, 0, 1, 2), kvx.KVX_E_RANGE), ((0, -1, 0, 1), kvx.KVX_E_INVAL)):
        with pytest.raises(kvx.KvxError) as e:
            q.push_heads(plan, *args)
        assert e.value.code == code, args
    # a plan between pools of different head counts admits no push
    with pytest.raises(kvx.KvxError) as e:
        q.push(plan, 0)
    assert e.value.code == kvx.KVX_E_MISMATCH
    st = W.StateSpec(2, 8, (64, 128))
    ss, sd = S.state_device_side(st, 5, 1), S.state_device_side(st, 5, 2)
    splan = kvx.kvx_plan(ss.pool, sd.pool, [4], [[1]], [[2]])
    with pytest.raises(kvx.KvxError) as e:
        q.push_heads(splan, 0, 0, 0, 1)
    assert e.value.code == kvx.KVX_E_MISMATCH
    L = kvx.lib()
    assert L.kvx_queue_push_heads(None, plan.handle, 0, 0, 0, 1, None) == kvx.KVX_E_INVAL
    assert L.kvx_queue_push_heads(q.handle, None, 0, 0, 0, 1, None) == kvx.KVX_E_INVAL
    q.push_heads(plan, 1, 0, 0, 0)   # an empty slice is a write that moves nothing
    q.flush()
    torch.cuda.synchronize()
    assert q.stats()[0] == 1
    q.close()
    plan.close()
    splan.close()


def test_queue_errors():
    spec = W.PoolSpec(2, 64, 4, 1, 16, W.U8)
    gs = S.device_side(spec, 1, 1)
    gd = S.device_side(spec, 1, 2)
    plan = kvx.kvx_plan(gs.pool, gd.pool, [8], [[1, 2]], [[3, 4]])
    host = kvx.kvx_plan(gs.pool, gd.pool, [8], [[1, 2]], [[3, 4]], host_only=True)
    q = kvx.Queue()
    with pytest.raises(kvx.KvxError) as e:
        q.push(plan, 2)
    assert e.value.code == kvx.KVX_E_RANGE
    with pytest.raises(kvx.KvxError) as e:
        q.push(host, 0)
    assert e.value.code == kvx.KVX_E_INVAL
    L = kvx.lib()
    assert L.kvx_queue_push(None, plan.handle, 0, None) == kvx.KVX_E_INVAL
    assert L.kvx_queue_push(q.handle, None, 0, None) == kvx.KVX_E_INVAL
    assert L.kvx_queue_flush(None) == kvx.KVX_E_INVAL
    assert L.kvx_queue_destroy(None) == kvx.KVX_OK
    q.push(plan, 1)
    q.flush()
    torch.cuda.synchronize()
    assert q.stats() == (1, 1)
    # under capture the queue refuses and the capture stays valid
    s = torch.cuda.Stream()
    cq = kvx.Queue(s)
    kvx.kvx_plan_wait(plan)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        with pytest.raises(kvx.KvxError) as e:
            cq.push(plan, 0)
        assert e.value.code == kvx.KVX_E_INVAL
        kvx.kvx_push_layer(plan, 0, stream=torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    cq.close()
    q.close()
    plan.close()
    host.close()
