"""Host-only planning against the oracle on random cases that combine the
geometry options (regions, sliding window, block sizes per side, scales,
layouts, null entries of dropped blocks)."""

import oracle as O
import oracle_pins as P
from combo_cases import combo_cases
from decode_kv_cache_amd import kvx
from test_abi_host import fake_pool


def test_host_plans_match_oracle_on_combinations():
    seen = {"mixed": 0, "window": 0, "latent": 0, "null": 0, "scales": 0}
    for wl in combo_cases(300, 1):
        toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
        plan = kvx.kvx_plan(fake_pool(wl.src, 0), fake_pool(wl.dst, 1), toks, wl.src_tables, wl.dst_tables,
                            host_only=True)
        reqs = [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)]
        op = O.make_plan(P.geom(O, wl.src), P.geom(O, wl.dst), reqs)
        for r in range(wl.src.regions):
            assert plan.triples(0, r).tolist() == [list(t) for t in op.triples], wl.name
        assert plan.bytes_per_layer() == op.bytes_per_layer(), wl.name
        L = wl.src.num_layers
        assert kvx.kvx_staging_bytes(plan, 0, L) == O.staging_bytes(op, 0, L), wl.name
        if wl.src.block_size == wl.dst.block_size:
            assert plan.runs().tolist() == [[r.src0, r.dst0, r.nblk, r.tail] for r in op.runs], wl.name
        plan.close()
        seen["mixed"] += wl.src.block_size != wl.dst.block_size
        seen["window"] += wl.src.window > 0
        seen["latent"] += wl.src.regions == 1
        seen["null"] += wl.name.endswith("_null")
        seen["scales"] += wl.src.has_scales
    assert min(seen.values()) >= 20, seen
