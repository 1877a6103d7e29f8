"""GPU parity for every launch shape of the copy kernels.  The library picks
a shape per plan from how fully its runs fill 32 KiB pieces and how many
pieces a launch has; the cases here are built to span those ranges (long
runs of whole 32 KiB blocks in large and small launches, runs of a few
16 KiB blocks with ragged ends, fp8 blocks with scales, short runs of small
blocks with scales).  Each case runs the push of every layer, pack/unpack of every
layer and kvx_push_many over all layers, byte for byte against the
oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def make(name, seed, spec, prompts, run_mean):
    rng = np.random.Generator(np.random.PCG64(seed))
    need = [W.alloc_blocks(p, spec.block_size) for p in prompts]
    return W.Workload(name, seed, spec, spec, prompts,
                      W.split_tables(W.geometric_run_table(rng, spec.num_blocks, run_mean), need),
                      W.split_tables(W.geometric_run_table(rng, spec.num_blocks, run_mean), need))


CASES = [
    # whole 32 KiB blocks, long runs, about one round of one-wave workgroups (1126 pieces per launch)
    make("long_round", 31, W.PoolSpec(2, 1400, 16, 8, 128, W.BF16), [9000], 12.0),
    # whole 32 KiB blocks, long runs, more pieces than one round (2390 per launch): 4 KiB pieces
    make("long_large", 36, W.PoolSpec(2, 1400, 16, 8, 128, W.BF16), [9000, 2100, 8000], 12.0),
    # whole 32 KiB blocks, long runs, a few hundred pieces per launch
    make("long_small", 32, W.PoolSpec(2, 400, 16, 8, 128, W.BF16), [3000], 12.0),
    # 16 KiB blocks in runs of about 2.5 with ragged request ends
    make("medium", 33, W.PoolSpec(2, 900, 16, 8, 64, W.BF16), [1500, 1700, 900, 2300], 2.5),
    # fp8 16 KiB blocks with one scale each, runs of about 2.5
    make("medium_fp8_scales", 34, W.PoolSpec(2, 900, 16, 8, 128, W.FP8, has_scales=True), [2000, 1800, 2500], 2.5),
    # 2 KiB blocks with scales, short runs
    make("short_scales", 35, W.PoolSpec(2, 2000, 16, 1, 64, W.BF16, has_scales=True), [3000, 1200, 4100], 1.5),
]


# (lanes, vectors per lane) the library picks for each case
EXPECT = {"long_round": (64, 32), "long_large": (256, 1), "long_small": (64, 16), "medium": (256, 1),
          "medium_fp8_scales": (256, 1), "short_scales": (256, 1)}


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_shape_parity(wl):
    src, dst = P.pools(O, wl)
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    n32 = 2 * sum(-(-t[2] // 32768) for t in op.triples)
    print(wl.name, "32 KiB pieces per launch", n32, "fill", round(2 * op.payload_bytes / (n32 * 32768), 3),
          flush=True)
    sys.stdout.flush()
    L = wl.src.num_layers
    exp = dst.copy()
    O.push(src, exp, op)

    def side():
        return S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))

    def check(gd, what):
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), (wl.name, what)
        if exp.scales is not None:
            assert np.array_equal(S.scale_bits(gd.sc), exp.scales), (wl.name, what)

    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    # push, layer by layer
    gd = side()
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
    shape = plan.launch_shape()
    assert (shape["lanes"], shape["vectors"]) == EXPECT[wl.name], shape
    for l in range(L):
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    check(gd, "push")
    # staging
    gd2 = side()
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, toks, wl.src_tables, wl.dst_tables)
    nbytes = kvx.kvx_staging_bytes(plan2, 0, L)
    stg = torch.full((nbytes,), 0x77, dtype=torch.uint8, device="cuda")
    kvx.kvx_pack(plan2, 0, L, stg)
    torch.cuda.synchronize()
    assert np.array_equal(stg.cpu().numpy(), O.pack(src, op, 0, L)), wl.name
    kvx.kvx_unpack(plan2, 0, L, stg)
    torch.cuda.synchronize()
    check(gd2, "unpack")
    # every layer in one kvx_push_many call
    gd3 = side()
    plan3 = kvx.kvx_plan(gs.pool, gd3.pool, toks, wl.src_tables, wl.dst_tables)
    kvx.kvx_push_many([plan3] * L, list(range(L)))
    torch.cuda.synchronize()
    check(gd3, "push_many")
    for p in (plan, plan2, plan3):
        p.close()
