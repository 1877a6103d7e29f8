"""kvx_pack / kvx_unpack over more layers than one launch takes (a plan
without scales copies up to 32 layers per launch): 40-layer K/V plans in
both layouts, a latent plan and a state-slot plan, packed over [0, 40),
[3, 38) and [5, 6) and unpacked over the first two ranges, byte for byte
against the oracle's staging layout and its unpack.  A plan with scales
(one launch per layer) runs the same ranges for contrast."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

L = 40
RANGES = ((0, L), (3, 38), (5, 6))


def kv_cases():
    return [W.random_case(9700, num_layers=L, num_blocks=160, block_size=16, num_heads=2, head_dim=64,
                          num_requests=3, max_tokens=600, run_mean=3.0),
            W.random_case(9701, num_layers=L, num_blocks=160, block_size=16, num_heads=2, head_dim=64,
                          num_requests=3, max_tokens=600, run_mean=3.0, layout="HND"),
            W.random_case(9702, num_layers=L, num_blocks=800, block_size=1, num_heads=1, head_dim=576,
                          num_requests=2, max_tokens=300, run_mean=8.0, regions=1),
            W.random_case(9703, num_layers=L, num_blocks=160, block_size=16, num_heads=2, head_dim=64,
                          elem_bytes=1, has_scales=True, num_requests=3, max_tokens=600)]


@pytest.mark.parametrize("idx", range(4))
def test_kv_pack_unpack_past_one_launch(idx):
    wl = kv_cases()[idx]
    print("case", wl.name, wl.src, flush=True)
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    for l0, l1 in RANGES:
        gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
        plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
        nbytes = kvx.kvx_staging_bytes(plan, l0, l1)
        assert nbytes == O.staging_bytes(op, l0, l1)
        stg = torch.full((max(nbytes, 16),), 0x5C, dtype=torch.uint8, device="cuda")
        kvx.kvx_pack(plan, l0, l1, stg)
        torch.cuda.synchronize()
        packed = O.pack(src, op, l0, l1)
        assert np.array_equal(stg[:nbytes].cpu().numpy(), packed), (wl.name, l0, l1)
        if l1 - l0 > 1:
            kvx.kvx_unpack(plan, l0, l1, stg)
            torch.cuda.synchronize()
            exp = dst.copy()
            O.unpack(packed, exp, op, l0, l1)
            assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), (wl.name, l0, l1)
            if exp.scales is not None:
                assert np.array_equal(S.scale_bits(gd.sc), exp.scales), (wl.name, l0, l1)
        plan.close()


def test_state_pack_unpack_past_one_launch():
    wl = W.random_state_case(9704, num_layers=L, num_slots=20, slot_bytes=(4096, 65552), num_requests=5,
                             max_tokens=3)
    hs = O.StatePool(P.state_geom(O, wl.src), W.state_host_values(wl.src, wl.seed, 1))
    hd = O.StatePool(P.state_geom(O, wl.dst), W.state_host_values(wl.dst, wl.seed, 2))
    gs = S.state_device_side(wl.src, wl.seed, 1, values=hs.regions)
    toks = list(wl.prompt_lens)
    op = O.make_state_plan(hs.geom, hd.geom, [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    for l0, l1 in RANGES:
        gd = S.state_device_side(wl.dst, wl.seed, 2, values=hd.regions)
        plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
        nbytes = kvx.kvx_staging_bytes(plan, l0, l1)
        stg = torch.full((max(nbytes, 16),), 0x5C, dtype=torch.uint8, device="cuda")
        kvx.kvx_pack(plan, l0, l1, stg)
        torch.cuda.synchronize()
        packed = O.pack_state(hs, op, l0, l1)
        assert nbytes == packed.size
        assert np.array_equal(stg[:nbytes].cpu().numpy(), packed), (l0, l1)
        if l1 - l0 > 1:
            kvx.kvx_unpack(plan, l0, l1, stg)
            torch.cuda.synchronize()
            exp = hd.copy()
            O.unpack_state(packed, exp, op, l0, l1)
            for r in range(2):
                assert np.array_equal(gd.regions[r].cpu().numpy(), exp.regions[r]), (l0, l1, r)
        plan.close()
