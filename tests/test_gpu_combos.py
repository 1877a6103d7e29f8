"""GPU parity on random cases that combine the geometry options (one or two
regions, sliding window, block sizes per side, scales, layouts, null entries
of dropped blocks): every layer pushed, and staged through pack/unpack,
byte for byte against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from combo_cases import combo_cases
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S

pytestmark = pytest.mark.gpu


def test_combinations_push_and_staging():
    for wl in combo_cases(40, 7, max_tokens=200, head_dims=(16, 64)):
        print("combo", wl.name, wl.src, wl.dst.block_size, flush=True)
        sys.stdout.flush()
        src, dst = P.pools(O, wl)
        gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
        gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
        toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
        plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
        op = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in
                                              zip(toks, wl.src_tables, wl.dst_tables)])
        L = wl.src.num_layers
        for l in range(L):
            kvx.kvx_push_layer(plan, l)
        torch.cuda.synchronize()
        exp = dst.copy()
        O.push(src, exp, op)
        assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), wl.name
        if exp.scales is not None:
            assert np.array_equal(S.scale_bits(gd.sc), exp.scales), wl.name
        nbytes = kvx.kvx_staging_bytes(plan, 0, L)
        stg = torch.full((max(nbytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
        kvx.kvx_pack(plan, 0, L, stg)
        torch.cuda.synchronize()
        assert np.array_equal(stg[:nbytes].cpu().numpy(), O.pack(src, op, 0, L)), wl.name
        gd2 = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
        plan2 = kvx.kvx_plan(gs.pool, gd2.pool, toks, wl.src_tables, wl.dst_tables)
        kvx.kvx_unpack(plan2, 0, L, stg)
        torch.cuda.synchronize()
        assert np.array_equal(gd2.kv.cpu().numpy(), exp.kv), wl.name
        plan.close()
        plan2.close()
