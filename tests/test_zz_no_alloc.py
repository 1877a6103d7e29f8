"""kvx_plan_noalloc: a plan whose device work list lives in the library's
static scratch array moves exactly the bytes a kvx_plan plan moves.  Two
calls in a row, the second with a smaller input; the first plan is refused
once the second has replaced its work list; a work list larger than the
array is refused before anything is copied."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W
from test_abi_host import fake_pool

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def both_ways(wl, runs):
    """Push every layer and pack + unpack every layer with a kvx_plan plan and
    with a kvx_plan_noalloc plan into separate consumer pools."""
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    ga = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    gb = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    ref = kvx.kvx_plan(gs.pool, ga.pool, toks, wl.src_tables, wl.dst_tables, runs=runs)
    nof = kvx.kvx_plan_noalloc(gs.pool, gb.pool, toks, wl.src_tables, wl.dst_tables, runs=runs)
    assert nof.launch_shape() == ref.launch_shape()
    L = wl.src.num_layers
    for l in range(L):
        kvx.kvx_push_layer(ref, l)
        kvx.kvx_push_layer(nof, l)
    torch.cuda.synchronize()
    assert np.array_equal(gb.kv.cpu().numpy(), ga.kv.cpu().numpy()), (wl.name, "push")
    if ga.sc is not None:
        assert np.array_equal(S.scale_bits(gb.sc), S.scale_bits(ga.sc)), (wl.name, "push scales")
    exp = dst.copy()
    O.push(src, exp, O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in
                                                      zip(toks, wl.src_tables, wl.dst_tables)]))
    assert np.array_equal(gb.kv.cpu().numpy(), exp.kv), (wl.name, "push vs oracle")
    nbytes = kvx.kvx_staging_bytes(nof, 0, L)
    sa = torch.full((max(nbytes, 16),), 0x11, dtype=torch.uint8, device="cuda")
    sb = torch.full((max(nbytes, 16),), 0x11, dtype=torch.uint8, device="cuda")
    kvx.kvx_pack(ref, 0, L, sa)
    kvx.kvx_pack(nof, 0, L, sb)
    torch.cuda.synchronize()
    assert torch.equal(sa, sb), (wl.name, "pack")
    ref.close()
    return nof, gs, gb


def test_noalloc_matches_kvx_plan_twice():
    big = W.random_case(41001, layout="NHD", elem_bytes=2, num_layers=3, num_blocks=1200, block_size=16,
                        num_heads=8, head_dim=128, has_scales=True, num_requests=4, max_tokens=4000, run_mean=4.0,
                        extra_ids=1)
    small = W.random_case(41002, layout="HND", elem_bytes=1, num_layers=2, num_blocks=300, block_size=4,
                          num_heads=3, head_dim=32, has_scales=False, num_requests=3, max_tokens=60, run_mean=2.0,
                          extra_ids=1)
    say("first call", big.name, big.src)
    first, gs1, gb1 = both_ways(big, runs=False)
    say("second call (smaller)", small.name, small.src)
    second, gs2, gb2 = both_ways(small, runs=True)
    # the first plan's work list was replaced: its device calls are refused
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_push_layer(first, 0)
    assert e.value.code == kvx.KVX_E_INVAL
    first.close()
    # the second plan still works after the first is destroyed
    kvx.kvx_push_layer(second, 0)
    torch.cuda.synchronize()
    second.close()


def test_noalloc_refuses_oversized_work_list():
    """Every block of a 2 GiB region in one request, in random order: 524,288
    pieces of 32 bytes plus 1 MiB of block pairs exceed the 16 MiB array and
    are refused on the host, nothing copied.  The same table kept as run
    tables fits.  The pools have made-up addresses: these plans are never
    launched."""
    spec = W.PoolSpec(1, 65536, 16, 8, 128, W.BF16)
    sp, dp = fake_pool(spec, 0), fake_pool(spec, 1)
    rng = np.random.Generator(np.random.PCG64(7))
    st, dt = [rng.permutation(65536).astype(np.int32)], [rng.permutation(65536).astype(np.int32)]
    toks = [65536 * 16]
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_plan_noalloc(sp, dp, toks, st, dt)
    assert e.value.code == kvx.KVX_E_NOMEM
    p = kvx.kvx_plan_noalloc(sp, dp, toks, st, dt, runs=True)
    assert p.launch_shape()["run_table"]
    p.close()
    h = kvx.C.c_void_p()
    rc = kvx.lib().kvx_plan_noalloc(sp.handle, dp.handle, 0, None, None, None, None, None, kvx.KVX_PLAN_HOST_ONLY,
                                    None, kvx.C.byref(h))
    assert rc == kvx.KVX_E_INVAL and not h.value   # a host-only plan has no work list to place
