"""Run-table plans (KVX_PLAN_RUNS) on the GPU against the oracle: the
kernel finds each 16-byte unit's run itself from a table of one record per
merged run ([MORI] §6: one (offset, offset, size) list per layer, adjacent
blocks merged), so push, pack and unpack must move exactly the bytes the
pages' procedure defines.

- random small cases in both layouts, 1- and 2-byte elements, scales, ragged
  tails and empty requests: push, and pack + unpack over every layer;
- runs shorter than a wave's 64 units (16-byte rows, one-slot blocks,
  scattered), so that a wave walks several windows of run records;
- batched_push at full size (2 GiB regions) and the last multi-turn turn
  (fp8 with scales) on sampled layers."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W
from test_gpu_parity import check_layers, oracle_requests, snapshot, tokens

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_case(wl):
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = tokens(wl)
    op = O.make_plan(src.geom, dst.geom, oracle_requests(wl, toks))
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, runs=True)
    L = wl.src.num_layers
    for l in range(L):
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    exp = dst.copy()
    O.push(src, exp, op)
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), (wl.name, "push")
    if exp.scales is not None:
        assert np.array_equal(S.scale_bits(gd.sc), exp.scales), (wl.name, "push scales")
    # pack + unpack into a fresh consumer
    gd2 = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, toks, wl.src_tables, wl.dst_tables, runs=True)
    nbytes = kvx.kvx_staging_bytes(plan2, 0, L)
    stg = torch.full((max(nbytes, 16),), 0x77, dtype=torch.uint8, device="cuda")
    kvx.kvx_pack(plan2, 0, L, stg)
    kvx.kvx_unpack(plan2, 0, L, stg)
    torch.cuda.synchronize()
    packed = O.pack(src, op, 0, L)
    assert np.array_equal(stg[:nbytes].cpu().numpy(), packed), (wl.name, "pack")
    exp2 = dst.copy()
    O.unpack(packed, exp2, op, 0, L)
    assert np.array_equal(gd2.kv.cpu().numpy(), exp2.kv), (wl.name, "unpack")
    if exp2.scales is not None:
        assert np.array_equal(S.scale_bits(gd2.sc), exp2.scales), (wl.name, "unpack scales")
    assert np.array_equal(gs.kv.cpu().numpy(), src.kv), (wl.name, "source changed")
    shape = plan.launch_shape()
    plan.close()
    plan2.close()
    return shape


def test_runs_random_small():
    rng = np.random.Generator(np.random.PCG64(31))
    taken = 0
    for i in range(36):
        bs = int(rng.choice([1, 3, 4, 16]))
        try:
            wl = W.random_case(31000 + i, layout=["NHD", "HND"][i % 2], elem_bytes=int(rng.choice([1, 2])),
                               num_layers=int(rng.integers(1, 4)), num_blocks=int(rng.integers(200, 320)),
                               block_size=bs, num_heads=int(rng.integers(1, 5)),
                               head_dim=int(rng.choice([16, 32, 64, 128])), has_scales=bool(i % 3 == 0),
                               num_requests=int(rng.integers(0, 6)),
                               max_tokens=40 if bs == 1 else int(rng.choice([20, 60, 300])),
                               run_mean=float(rng.choice([1.2, 2.0, 8.0])), extra_ids=int(rng.integers(0, 3)))
        except ValueError:
            continue
        say("case", i, wl.name, wl.src)
        shape = one_case(wl)
        taken += shape["run_table"]
    assert taken >= 20, taken   # most of these plans stream, so the run table is taken


def test_runs_short_runs_several_windows():
    """16-byte rows in one-slot blocks, every other block: runs of one row, so
    a wave's 64 units span 64 runs and a 4 KiB chunk 256 of them."""
    for seed in (1, 2, 3):
        wl = W.random_case(32000 + seed, layout="NHD", elem_bytes=1, num_layers=2, num_blocks=9000, block_size=1,
                           num_heads=1, head_dim=16, has_scales=seed == 2, num_requests=3, max_tokens=1400,
                           run_mean=1.0, extra_ids=0)
        say("short runs", wl.name, wl.src)
        shape = one_case(wl)
        assert shape["run_table"]


def test_runs_batched_full():
    wl = W.batched_push()
    say("workload batched_push, run-table plan")
    gs = S.device_side(wl.src, wl.seed, 1)
    gd = S.device_side(wl.dst, wl.seed, 2)
    torch.cuda.synchronize()
    slabs = [0, wl.src.n_phys - 1]
    src_snap, dst_snap = snapshot(gs, slabs), snapshot(gd, slabs)
    toks = tokens(wl)
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, runs=True)
    assert plan.launch_shape()["run_table"]
    side = torch.cuda.Stream()
    for l in range(wl.src.num_layers):
        kvx.kvx_push_layer(plan, l, stream=side)
    side.synchronize()
    op = O.make_plan(P.geom(O, wl.src), P.geom(O, wl.dst), oracle_requests(wl, toks))
    check_layers(wl, gs, gd, src_snap, dst_snap, op, slabs, "batched_push with run tables")
    plan.close()
    del gs, gd
    torch.cuda.empty_cache()


def test_runs_multiturn_last_turn():
    wl = W.multiturn_fp8()
    ex = wl.extra
    say("workload multiturn_fp8 turn 8, run-table plan")
    dec = S.device_side(wl.src, wl.seed, 1)
    pre = S.device_side(wl.dst, wl.seed, 2)
    torch.cuda.synchronize()
    layers = [0, wl.src.num_layers - 1]
    dsnap, psnap = snapshot(dec, layers), snapshot(pre, layers)
    t = ex["turns"]
    reusable = ex["growth"] * (t - 1)
    plan = kvx.kvx_plan(dec.pool, pre.pool, [reusable] * ex["sessions"], ex["decode_tables"],
                        ex["prefill_tables"][t], runs=True)
    assert plan.launch_shape()["run_table"]
    for l in layers:
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    g = P.geom(O, wl.src)
    reqs = [O.reuse_request(t, ex["growth"], ex["threshold"], ex["decode_tables"][s], ex["prefill_tables"][t][s])
            for s in range(ex["sessions"])]
    op = O.make_plan(g, g, reqs)
    for l in layers:
        for kv in (0, 1):
            exp = psnap[l][0][kv].copy()
            O.push_region(dsnap[l][0][kv], exp, op.triples)
            assert np.array_equal(pre.kv[l, kv].cpu().numpy(), exp), (l, kv)
            es = psnap[l][1][kv].copy()
            O.push_scales(dsnap[l][1][kv], es, op.pairs)
            assert np.array_equal(S.scale_bits(pre.sc[l, kv]), es), (l, kv)
    plan.close()
    del dec, pre
    torch.cuda.empty_cache()
