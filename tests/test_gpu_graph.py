"""The layerwise push captured in a HIP graph (torch.cuda.CUDAGraph on ROCm)
and replayed: once the plan's upload has been observed (kvx_plan_wait), kvx_push_layer
without a ready event enqueues nothing but its kernel (a captured step
orders the push after the captured compute by stream order), so a serving
loop can capture a step once and replay it.  The source is rewritten between replays
by ordinary eager work; every replay must equal the oracle's push of the
source as it stood, and the layers that no push touches stay unchanged."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_push_replayed_from_graph():
    wl = W.random_case(9500, num_layers=4, num_blocks=300, block_size=16, num_heads=4, head_dim=64,
                       num_requests=3, max_tokens=700, run_mean=3.0)
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    ready = [torch.cuda.Event() for _ in range(4)]
    for e in ready:
        e.record()
    kvx.kvx_push_layer(plan, 0, ready=ready[0], stream=side)   # events fired
    kvx.kvx_plan_wait(plan)                                   # upload observed before capturing
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for l in (0, 1, 3):
            kvx.kvx_push_layer(plan, l, stream=torch.cuda.current_stream())
    exp = dst.copy()
    rng = np.random.Generator(np.random.PCG64(3))
    for rep in range(3):
        new = rng.integers(0, 256, size=src.kv.shape, dtype=np.uint8)
        gs.kv.copy_(torch.from_numpy(new).cuda())        # eager work between replays
        src.kv[...] = new
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        O.push(src, exp, op, layers=[0, 1, 3])
        got = gd.kv.cpu().numpy()
        assert np.array_equal(got, exp.kv), rep
        assert np.array_equal(got[2], dst.kv[2]), rep          # layer 2 is not in the graph
    plan.close()


def test_fresh_plan_captured_after_plan_wait():
    """A plan whose upload has not been observed on the host: inside a
    capture its device call is an argument error and the capture stays
    valid; after kvx_plan_wait its calls capture, and a ready event recorded
    on a forked stream inside the capture becomes a graph edge (the forked
    stream writes the source before the push reads it)."""
    wl = W.random_case(9501, num_layers=3, num_blocks=200, block_size=16, num_heads=2, head_dim=64,
                       num_requests=2, max_tokens=500, run_mean=2.0)
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    other = torch.cuda.Stream()
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    stage = torch.empty_like(gs.kv)
    torch.cuda.synchronize()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g0, stream=side):
        stage.zero_()
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_push_layer(plan, 0, stream=torch.cuda.current_stream())
        assert e.value.code == kvx.KVX_E_INVAL
    del g0
    kvx.kvx_plan_wait(plan)
    ready = torch.cuda.Event()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        cap = torch.cuda.current_stream()
        other.wait_stream(cap)                      # fork
        with torch.cuda.stream(other):
            gs.kv.copy_(stage)                      # "compute" that produces the source
            ready.record(other)
        for l in range(3):
            kvx.kvx_push_layer(plan, l, ready=ready if l == 0 else None, stream=cap)   # join at layer 0
    exp = dst.copy()
    rng = np.random.Generator(np.random.PCG64(4))
    for rep in range(3):
        new = rng.integers(0, 256, size=src.kv.shape, dtype=np.uint8)
        stage.copy_(torch.from_numpy(new).cuda())
        src.kv[...] = new
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        O.push(src, exp, op)
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), rep
        assert np.array_equal(gs.kv.cpu().numpy(), new), rep
    plan.close()


def test_plan_on_capturing_stream_is_rejected():
    """kvx_plan's upload would only run at replay, so a capturing upload
    stream is an argument error; the capture itself stays valid."""
    wl = W.random_case(9502, num_layers=2, num_blocks=64, block_size=16, num_heads=2, head_dim=64,
                       num_requests=1, max_tokens=100)
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    kvx.kvx_push_layer(plan, 0, stream=side)
    kvx.kvx_plan_wait(plan)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=torch.cuda.current_stream())
        assert e.value.code == kvx.KVX_E_INVAL
        kvx.kvx_push_layer(plan, 1, stream=torch.cuda.current_stream())
    gd.kv.copy_(torch.from_numpy(dst.kv).cuda())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    exp = dst.copy()
    O.push(src, exp, op, layers=[1])
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    plan.close()


def test_push_many_and_staging_replayed_from_graph():
    """kvx_push_many over every layer and kvx_pack + kvx_unpack over every
    layer, captured once and replayed with the source rewritten eagerly
    between replays.  The plan takes the 16 KiB one-wave shape, and four
    layers of it exceed one round, so the batched launches stream its
    pieces as 4 KiB chunks from the destination-ordered copy."""
    spec = W.PoolSpec(4, 400, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(9502))
    need = [W.alloc_blocks(3000, 16)]
    wl = W.Workload("graph_many", 9502, spec, spec, [3000],
                    W.split_tables(W.geometric_run_table(rng, 400, 12.0), need),
                    W.split_tables(W.geometric_run_table(rng, 400, 12.0), need))
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    gd2 = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, toks, wl.src_tables, wl.dst_tables, stream=side)
    shape = plan.launch_shape()
    L = spec.num_layers
    assert (shape["lanes"], shape["vectors"]) == (64, 16), shape
    # 32 KiB units over all four layers beyond one round (1312): the batched launches stream
    assert L * shape["pieces"] * shape["piece_bytes"] // 32768 > 1312, shape
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    stg = torch.empty(kvx.kvx_staging_bytes(plan2, 0, L), dtype=torch.uint8, device="cuda")
    kvx.kvx_plan_wait(plan)
    kvx.kvx_plan_wait(plan2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        cur = torch.cuda.current_stream()
        kvx.kvx_push_many([plan] * L, list(range(L)), stream=cur)
        kvx.kvx_pack(plan2, 0, L, stg, stream=cur)
        kvx.kvx_unpack(plan2, 0, L, stg, stream=cur)
    exp = dst.copy()
    rng = np.random.Generator(np.random.PCG64(4))
    for rep in range(3):
        new = rng.integers(0, 256, size=src.kv.shape, dtype=np.uint8)
        gs.kv.copy_(torch.from_numpy(new).cuda())        # eager work between replays
        src.kv[...] = new
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        O.push(src, exp, op)
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), ("push_many", rep)
        assert np.array_equal(stg.cpu().numpy(), O.pack(src, op, 0, L)), ("pack", rep)
        assert np.array_equal(gd2.kv.cpu().numpy(), exp.kv), ("unpack", rep)
    plan.close()
    plan2.close()
