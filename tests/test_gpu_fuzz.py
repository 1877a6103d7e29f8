"""Seeded random sweep of every device call against the oracle.  Each case
draws a geometry of one of three kinds:
  - whole 32 KiB blocks in long runs, so that plans take the one-wave launch
    shapes and batched launches read their destination-ordered piece copy;
  - small random geometries (either layout, 1- or 2-byte elements, ragged
    tails, scales), whose plans take the 4 KiB shape;
  - different block sizes and head counts per side (head transform only).
Each case is built with or without KVX_PLAN_OVERLAP and with or without
KVX_PLAN_RUNS (streaming plans then read run tables; a head transform
reads its block pairs either way). Where both pools have
the same head count and layout, its requests are pushed layer by layer.
They are also split into two plans with disjoint destinations, whose layers
go out in one kvx_push_many call, and packed and unpacked over a random
layer range.  Otherwise a random head slice is transformed, the first
layers one launch each and the rest in one kvx_copy_heads_layers call.
Either way every layer's write also goes through a write queue once, in a
random layer order (kvx_queue_push, kvx_queue_push_heads).  Every
destination byte, staging byte and scale must equal the oracle's."""
import os

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

# KVX_FUZZ_CASES / KVX_FUZZ_SEED widen or redraw the sweep for a longer run
CASES = int(os.environ.get("KVX_FUZZ_CASES", "160"))
SEED = int(os.environ.get("KVX_FUZZ_SEED", "2024"))


def say(*a):
    print(*a, flush=True)


def draw(i, rng):
    kind = ("big", "small", "small", "heads")[i % 4]
    if kind == "big":
        return kind, W.random_case(20000 + i + 100000 * (SEED - 2024), layout="NHD", elem_bytes=2, num_layers=int(rng.integers(1, 4)),
                                   num_blocks=1200, block_size=16, num_heads=8, head_dim=128,
                                   has_scales=bool(rng.integers(0, 2)), num_requests=int(rng.integers(1, 5)),
                                   max_tokens=int(rng.choice([1000, 4000, 6000])), run_mean=float(rng.choice([4.0, 12.0])),
                                   extra_ids=int(rng.integers(0, 2)))
    if kind == "small":
        bs = int(rng.choice([1, 3, 4, 16]))
        return kind, W.random_case(20000 + i + 100000 * (SEED - 2024), layout=["NHD", "HND"][int(rng.integers(0, 2))],
                                   elem_bytes=int(rng.choice([1, 2])), num_layers=int(rng.integers(1, 5)),
                                   num_blocks=int(rng.integers(200, 320)), block_size=bs,
                                   num_heads=int(rng.integers(1, 5)), head_dim=int(rng.choice([16, 32, 64, 128])),
                                   has_scales=bool(rng.integers(0, 2)), num_requests=int(rng.integers(0, 6)),
                                   max_tokens=40 if bs == 1 else int(rng.choice([20, 60, 300])),
                                   run_mean=float(rng.choice([1.2, 2.0, 8.0])), extra_ids=int(rng.integers(0, 3)))
    bs, bsd = [int(x) for x in rng.choice([2, 4, 8, 16], size=2, replace=False)]
    return kind, W.random_case(20000 + i + 100000 * (SEED - 2024), layout=["NHD", "HND"][int(rng.integers(0, 2))],
                               dst_layout=["NHD", "HND"][int(rng.integers(0, 2))], elem_bytes=int(rng.choice([1, 2])),
                               num_layers=int(rng.integers(1, 4)), num_blocks=300, block_size=bs, dst_block_size=bsd,
                               num_heads=int(rng.integers(2, 9)), dst_heads=int(rng.integers(1, 5)),
                               head_dim=int(rng.choice([16, 64])), num_requests=int(rng.integers(1, 5)),
                               max_tokens=200, run_mean=float(rng.choice([1.5, 4.0])), extra_ids=1)


def check_pool(side, exp, what):
    assert np.array_equal(side.kv.cpu().numpy(), exp.kv), what
    if exp.scales is not None:
        assert np.array_equal(S.scale_bits(side.sc), exp.scales), what


def fresh(wl, dst):
    return S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))


def test_random_sweep():
    rng = np.random.Generator(np.random.PCG64(SEED))
    shapes = set()
    done = 0
    for i in range(CASES):
        try:
            kind, wl = draw(i, rng)
        except ValueError:         # pools too small for the drawn requests
            continue
        overlap = bool(rng.integers(0, 2))
        runs = bool(rng.integers(0, 2))
        src, dst = P.pools(O, wl)
        toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
        reqs = [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)]
        op = O.make_plan(src.geom, dst.geom, reqs)
        gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
        L = wl.src.num_layers
        push_ok = wl.src.num_heads == wl.dst.num_heads and wl.src.layout == wl.dst.layout
        say("case", i, kind, wl.name, "overlap" if overlap else "", "runs" if runs else "", wl.src, wl.dst)
        if push_ok:
            # layer by layer
            gd = fresh(wl, dst)
            plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=overlap, runs=runs)
            sh = plan.launch_shape()
            shapes.add((sh["lanes"], sh["vectors"]) + (("runs",) if sh["run_table"] else ()))
            for l in rng.permutation(L):
                kvx.kvx_push_layer(plan, int(l))
            torch.cuda.synchronize()
            exp = dst.copy()
            O.push(src, exp, op)
            check_pool(gd, exp, (wl.name, "push"))
            plan.close()
            # the same writes through a write queue, layers in a random order
            gd = fresh(wl, dst)
            plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=overlap, runs=runs)
            q = kvx.Queue()
            for l in rng.permutation(L):
                q.push(plan, int(l))
            q.close()
            torch.cuda.synchronize()
            check_pool(gd, exp, (wl.name, "queue"))
            plan.close()
            # two plans over disjoint request groups, every layer in one kvx_push_many call
            gd = fresh(wl, dst)
            cut = int(rng.integers(0, len(toks) + 1))
            groups = [(toks[:cut], wl.src_tables[:cut], wl.dst_tables[:cut]),
                      (toks[cut:], wl.src_tables[cut:], wl.dst_tables[cut:])]
            plans = [kvx.kvx_plan(gs.pool, gd.pool, t, s, d, overlap=bool(rng.integers(0, 2)),
                                  runs=bool(rng.integers(0, 2))) for t, s, d in groups]
            pairs = [(p, l) for l in range(L) for p in plans]
            order = rng.permutation(len(pairs))
            kvx.kvx_push_many([pairs[k][0] for k in order], [pairs[k][1] for k in order])
            torch.cuda.synchronize()
            check_pool(gd, exp, (wl.name, "push_many"))
            for p in plans:
                p.close()
            # pack and unpack over a random layer range
            gd = fresh(wl, dst)
            plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=overlap, runs=runs)
            l0 = int(rng.integers(0, L))
            l1 = int(rng.integers(l0, L + 1))
            nbytes = kvx.kvx_staging_bytes(plan, l0, l1)
            assert nbytes == O.staging_bytes(op, l0, l1)
            stg = torch.full((max(nbytes, 16),), 0x5C, dtype=torch.uint8, device="cuda")
            kvx.kvx_pack(plan, l0, l1, stg)
            kvx.kvx_unpack(plan, l0, l1, stg)
            torch.cuda.synchronize()
            packed = O.pack(src, op, l0, l1)
            assert np.array_equal(stg[:nbytes].cpu().numpy(), packed), (wl.name, "pack", l0, l1)
            exp = dst.copy()
            O.unpack(packed, exp, op, l0, l1)
            check_pool(gd, exp, (wl.name, "unpack", l0, l1))
            plan.close()
        else:
            gd = fresh(wl, dst)
            plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=overlap, runs=runs)
            nh = int(rng.integers(1, min(wl.src.num_heads, wl.dst.num_heads) + 1))
            s0 = int(rng.integers(0, wl.src.num_heads - nh + 1))
            d0 = int(rng.integers(0, wl.dst.num_heads - nh + 1))
            exp = dst.copy()
            l0 = int(rng.integers(0, L + 1))   # [0, l0) one launch per layer, [l0, L) in batched launches
            for l in range(l0):
                kvx.kvx_copy_heads(plan, l, s0, d0, nh)
            kvx.kvx_copy_heads_layers(plan, l0, L, s0, d0, nh)
            for l in range(L):
                O.copy_heads(src, exp, op, reqs, l, s0, d0, nh)
            torch.cuda.synchronize()
            check_pool(gd, exp, (wl.name, "copy_heads", s0, d0, nh, l0))
            plan.close()
            # the same slice through a write queue, layers in a random order
            gd = fresh(wl, dst)
            plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables, overlap=overlap, runs=runs)
            q = kvx.Queue()
            for l in rng.permutation(L):
                q.push_heads(plan, int(l), s0, d0, nh)
            q.close()
            torch.cuda.synchronize()
            check_pool(gd, exp, (wl.name, "queue_heads", s0, d0, nh))
            plan.close()
        assert np.array_equal(gs.kv.cpu().numpy(), src.kv), (wl.name, "source changed")
        done += 1
    say("cases run", done, "launch shapes seen", sorted(shapes))
    assert done >= CASES * 3 // 4
    assert {(64, 32), (64, 16), (256, 1), (256, 1, "runs")} <= shapes, shapes   # every launch shape exercised
