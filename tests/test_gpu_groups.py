"""GPU parity of layer groups of other shapes against the CPU oracle, byte for
byte: pools of one latent region (MLA), sliding-window groups that skip the
blocks the next query no longer sees, and state-slot groups whose conv and
SSM regions move slot by slot.  Small random cases cover push, pack/unpack
and the head kernel; the three hybrid workloads run at full size, every
model layer pushed in model order on one side stream as the bench times
them, and sampled layers of each group are checked against the oracle."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def toks_of(wl):
    return [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]


def reqs_of(toks, st, dt):
    return [O.Request(n, s, d) for n, s, d in zip(toks, st, dt)]


def bits(sc):
    return S.scale_bits(sc) if sc is not None else None


def attention_case(wl, *, with_heads=False):
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    toks = toks_of(wl)
    reqs = reqs_of(toks, wl.src_tables, wl.dst_tables)
    op = O.make_plan(src.geom, dst.geom, reqs)
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, wl.src_tables, wl.dst_tables)
    L = wl.src.num_layers
    for l in range(L):
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    exp = dst.copy()
    O.push(src, exp, op)
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv), wl.name
    assert np.array_equal(gs.kv.cpu().numpy(), src.kv), wl.name
    if exp.scales is not None:
        assert np.array_equal(bits(gd.sc), exp.scales), wl.name
    # staging: pack into a poisoned buffer, unpack into a fresh copy of dst
    nbytes = kvx.kvx_staging_bytes(plan, 0, L)
    assert nbytes == O.staging_bytes(op, 0, L)
    stg = torch.full((max(nbytes, 16),), 0xCD, dtype=torch.uint8, device="cuda")
    kvx.kvx_pack(plan, 0, L, stg)
    torch.cuda.synchronize()
    ref = O.pack(src, op, 0, L)
    assert np.array_equal(stg[:nbytes].cpu().numpy(), ref), wl.name
    gd2 = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, toks, wl.src_tables, wl.dst_tables)
    kvx.kvx_unpack(plan2, 0, L, stg)
    torch.cuda.synchronize()
    assert np.array_equal(gd2.kv.cpu().numpy(), exp.kv), wl.name
    if with_heads:
        gd3 = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
        plan3 = kvx.kvx_plan(gs.pool, gd3.pool, toks, wl.src_tables, wl.dst_tables)
        for l in range(L):
            kvx.kvx_copy_heads(plan3, l, 0, 0, wl.src.num_heads)
        torch.cuda.synchronize()
        assert np.array_equal(gd3.kv.cpu().numpy(), exp.kv), wl.name
        plan3.close()
    plan.close()
    plan2.close()


def test_latent_random_small():
    for wl in P.latent_cases(24, seed0=101):
        say("latent case", wl.name, wl.src)
        attention_case(wl, with_heads=True)
    # several pieces per run and a ragged last piece: 576-element latent rows
    for i, bs in enumerate((1, 16, 64)):
        wl = W.random_case(8100 + i, num_layers=2, num_blocks=max(64, 2048 // bs), block_size=bs, num_heads=1,
                           head_dim=576, elem_bytes=2, num_requests=3, max_tokens=600, run_mean=12.0,
                           has_scales=bs == 64, regions=1)
        say("latent case", wl.name, wl.src)
        attention_case(wl, with_heads=True)


def test_window_random_small():
    for wl in P.window_cases(40, seed0=103):
        say("window case", wl.name, wl.src, wl.dst.block_size)
        attention_case(wl, with_heads=wl.src.block_size == wl.dst.block_size)


def test_window_null_entries():
    """Entries of skipped blocks may be anything (here -1, an engine's null
    block stands there): the kernels never touch them."""
    spec = W.PoolSpec(2, 64, 16, 4, 32, W.BF16, window=40)
    wl = W.random_case(8200, num_layers=2, num_blocks=64, block_size=16, num_heads=4, head_dim=32,
                       num_requests=3, max_tokens=300, run_mean=3.0, window=40)
    toks = toks_of(wl)
    st, dt = [], []
    for n, s, d in zip(toks, wl.src_tables, wl.dst_tables):
        j0 = O.window_start(n, 40, 16, 16) // 16
        s, d = s.copy(), d.copy()
        s[:j0] = -1
        d[:j0] = -1
        st.append(s)
        dt.append(d)
    src, dst = P.pools(O, wl)
    gs = S.device_side(wl.src, wl.seed, 1, values=(src.kv, src.scales))
    gd = S.device_side(wl.dst, wl.seed, 2, values=(dst.kv, dst.scales))
    plan = kvx.kvx_plan(gs.pool, gd.pool, toks, st, dt)
    for l in range(2):
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    exp = dst.copy()
    O.push(src, exp, O.make_plan(src.geom, dst.geom, reqs_of(toks, st, dt)))
    assert np.array_equal(gd.kv.cpu().numpy(), exp.kv)
    assert spec.window == wl.src.window
    plan.close()


def state_case(wl):
    sv = W.state_host_values(wl.src, wl.seed, 1)
    dv = W.state_host_values(wl.dst, wl.seed, 2)
    gs = S.state_device_side(wl.src, wl.seed, 1, values=sv)
    gd = S.state_device_side(wl.dst, wl.seed, 2, values=dv)
    reqs = reqs_of(wl.prompt_lens, wl.src_tables, wl.dst_tables)
    src = O.StatePool(P.state_geom(O, wl.src), [a.copy() for a in sv])
    dst = O.StatePool(P.state_geom(O, wl.dst), [a.copy() for a in dv])
    op = O.make_state_plan(src.geom, dst.geom, reqs)
    plan = kvx.kvx_plan(gs.pool, gd.pool, wl.prompt_lens, wl.src_tables, wl.dst_tables)
    L = wl.src.num_layers
    for l in range(L):
        kvx.kvx_push_layer(plan, l)
    torch.cuda.synchronize()
    exp = dst.copy()
    O.push_state(src, exp, op)
    for r in range(2):
        assert np.array_equal(gd.regions[r].cpu().numpy(), exp.regions[r]), (wl.name, r)
        assert np.array_equal(gs.regions[r].cpu().numpy(), sv[r]), (wl.name, r)
    nbytes = kvx.kvx_staging_bytes(plan, 0, L)
    assert nbytes == O.state_staging_bytes(op, 0, L)
    stg = torch.full((max(nbytes, 16),), 0xCD, dtype=torch.uint8, device="cuda")
    kvx.kvx_pack(plan, 0, L, stg)
    torch.cuda.synchronize()
    assert np.array_equal(stg[:nbytes].cpu().numpy(), O.pack_state(src, op, 0, L)), wl.name
    gd2 = S.state_device_side(wl.dst, wl.seed, 2, values=dv)
    plan2 = kvx.kvx_plan(gs.pool, gd2.pool, wl.prompt_lens, wl.src_tables, wl.dst_tables)
    kvx.kvx_unpack(plan2, 0, L, stg)
    torch.cuda.synchronize()
    for r in range(2):
        assert np.array_equal(gd2.regions[r].cpu().numpy(), exp.regions[r]), (wl.name, r)
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_copy_heads(plan, 0, 0, 0, 1)
    assert e.value.code == kvx.KVX_E_MISMATCH
    plan.close()
    plan2.close()


def test_state_random_small():
    for wl in P.state_cases(30, seed0=105):
        say("state case", wl.name, wl.src, wl.prompt_lens)
        state_case(wl)
    # slots spanning several pieces, with a ragged last piece in region 1
    wl = W.random_state_case(8300, num_layers=2, num_slots=16, slot_bytes=(49152, 98320), num_requests=7,
                             max_tokens=5)
    say("state case", wl.name, wl.src, wl.prompt_lens)
    state_case(wl)


# ---------------------------------------------------------------------------
# hybrid workloads at full size
# ---------------------------------------------------------------------------
def _snap(side, layer):
    if isinstance(side, S.StateSide):
        return [side.regions[r][layer].cpu().numpy().copy() for r in range(2)], None
    p = side.spec.phys(layer)
    return ([side.kv[p, r].cpu().numpy().copy() for r in range(side.spec.regions)],
            [S.scale_bits(side.sc[p, r]).copy() for r in range(side.spec.regions)] if side.sc is not None else None)


def _now(side, layer):
    return _snap(side, layer)


def hybrid_full(wl, sample, via="layer"):
    """Push every model layer in model order on one side stream (one
    kvx_push_layer per layer, the stream's write queue with fired events, or
    one kvx_push_many call over every layer: the last two gather one-region
    and two-region layers into launches of their own); check the sampled
    (group, layer-in-group) pairs against the oracle."""
    say("workload", wl.name, "via", via)
    sides, plans, ops = [], [], []
    toks = toks_of(wl)
    for gi, g in enumerate(wl.groups):
        gs = S.group_side(g.src, wl.seed, 1 + 10 * gi)
        gd = S.group_side(g.dst, wl.seed, 2 + 10 * gi)
        sides.append((gs, gd))
        plans.append(kvx.kvx_plan(gs.pool, gd.pool, toks, g.src_tables, g.dst_tables))
        reqs = reqs_of(toks, g.src_tables, g.dst_tables)
        if isinstance(g.src, W.StateSpec):
            ops.append(O.make_state_plan(P.state_geom(O, g.src), P.state_geom(O, g.dst), reqs))
        else:
            ops.append(O.make_plan(P.geom(O, g.src), P.geom(O, g.dst), reqs))
    torch.cuda.synchronize()
    snaps = {(gi, l): (_snap(sides[gi][0], l), _snap(sides[gi][1], l)) for gi, l in sample}
    side = torch.cuda.Stream()
    if via == "layer":
        for gi, l in wl.layer_map:
            e = torch.cuda.Event()
            e.record()
            kvx.kvx_push_layer(plans[gi], l, ready=e, stream=side)
    elif via == "queue":   # events fired before the writes are queued: the writes back up and merge
        evs = [torch.cuda.Event() for _ in wl.layer_map]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        q = kvx.Queue(side)
        for (gi, l), e in zip(wl.layer_map, evs):
            q.push(plans[gi], l, ready=e)
        q.flush()
        w, g, n = q.stats3()
        assert w == len(wl.layer_map) and n < w, (w, g, n)
        q.close()
    else:
        kvx.kvx_push_many([plans[gi] for gi, _ in wl.layer_map], [l for _, l in wl.layer_map],
                          ready=torch.cuda.current_stream().record_event(), stream=side)
    side.synchronize()
    for gi, l in sample:
        (skv, ssc), (dkv, dsc) = snaps[(gi, l)]
        op = ops[gi]
        (gkv, gsc) = _now(sides[gi][1], l)
        (s_after, _) = _now(sides[gi][0], l)
        for r in range(len(skv)):
            tr = op.triples[r] if isinstance(op, O.StatePlan) else op.triples
            exp = dkv[r].copy()
            O.push_region(skv[r], exp, tr)
            assert np.array_equal(gkv[r], exp), (wl.name, gi, l, r)
            assert np.array_equal(s_after[r], skv[r]), (wl.name, "source changed", gi, l, r)
            if ssc is not None:
                es = dsc[r].copy()
                O.push_scales(ssc[r], es, op.pairs)
                assert np.array_equal(gsc[r], es), (wl.name, gi, l, r)
        say("checked group", gi, "layer", l)
    for p in plans:
        p.close()
    del sides
    torch.cuda.empty_cache()


def test_dsr1_mla_full():
    hybrid_full(W.dsr1_mla_push(), [(0, 0), (0, 29), (0, 60)])


def test_gptoss_swa_full():
    hybrid_full(W.gptoss_swa_push(), [(0, 0), (0, 17), (1, 0), (1, 17)])


def test_qwen3next_state_full():
    hybrid_full(W.qwen3next_state_push(), [(0, 0), (0, 11), (1, 0), (1, 35)])


def test_qwen3next_state_full_queue():
    hybrid_full(W.qwen3next_state_push(), [(0, 0), (0, 11), (1, 0), (1, 35)], via="queue")


def test_gptoss_swa_full_push_many():
    hybrid_full(W.gptoss_swa_push(), [(0, 0), (0, 17), (1, 0), (1, 17)], via="many")
