"""kvx_push_many on the GPU: a list of (plan, layer) pairs, batched into few
launches, leaves every destination exactly as the oracle's push of each pair
does.  The list mixes K/V, latent, sliding-window and state-slot plans with
different pools (so grid heights differ between neighbours), more than 32
pairs (several launches), the three launch shapes (long runs of whole
blocks, long state slots in a small launch, short runs), plans with per-block
scales (K/V in both layouts and a latent pool: their scales go out in a
small launch behind each batched launch), an empty plan (skipped), and a
pair repeated in a later call.
Argument errors enqueue nothing."""
import numpy as np
import pytest
import torch

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


class Case:
    """One plan with host copies of both pools and its oracle plan."""

    def __init__(self, wl, state=False):
        self.wl, self.state = wl, state
        if state:
            self.hs = O.StatePool(P.state_geom(O, wl.src), W.state_host_values(wl.src, wl.seed, 1))
            self.hd = O.StatePool(P.state_geom(O, wl.dst), W.state_host_values(wl.dst, wl.seed, 2))
            self.gs = S.state_device_side(wl.src, wl.seed, 1, values=self.hs.regions)
            self.gd = S.state_device_side(wl.dst, wl.seed, 2, values=self.hd.regions)
            toks = list(wl.prompt_lens)
            self.op = O.make_state_plan(self.hs.geom, self.hd.geom,
                                        [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
        else:
            self.hs, self.hd = P.pools(O, wl)
            self.gs = S.device_side(wl.src, wl.seed, 1, values=(self.hs.kv, self.hs.scales))
            self.gd = S.device_side(wl.dst, wl.seed, 2, values=(self.hd.kv, self.hd.scales))
            toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
            self.op = O.make_plan(self.hs.geom, self.hd.geom,
                                  [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
        self.plan = kvx.kvx_plan(self.gs.pool, self.gd.pool, toks, wl.src_tables, wl.dst_tables)
        self.exp = self.hd.copy()

    def expect(self, layer):
        if self.state:
            O.push_state(self.hs, self.exp, self.op, [layer])
        else:
            O.push(self.hs, self.exp, self.op, [layer])

    def check(self):
        if self.state:
            for r in range(2):
                assert np.array_equal(self.gd.regions[r].cpu().numpy(), self.exp.regions[r]), self.wl.name
        else:
            assert np.array_equal(self.gd.kv.cpu().numpy(), self.exp.kv), self.wl.name
            if self.exp.scales is not None:
                assert np.array_equal(S.scale_bits(self.gd.sc), self.exp.scales), self.wl.name


def cases():
    out = []
    for i in range(6):
        out.append(Case(W.random_case(9000 + i, num_layers=4, num_blocks=[1000, 300, 200][i % 3], block_size=[1, 4, 16][i % 3],
                                      num_heads=2, head_dim=64, num_requests=3, max_tokens=300, run_mean=3.0,
                                      layout=["NHD", "HND"][i % 2])))
    out.append(Case(W.random_case(9010, num_layers=4, num_blocks=200, block_size=16, num_heads=1, head_dim=576,
                                  num_requests=2, max_tokens=400, regions=1)))
    out.append(Case(W.random_case(9011, num_layers=4, num_blocks=200, block_size=8, num_heads=2, head_dim=64,
                                  num_requests=3, max_tokens=300, window=37)))
    out.append(Case(W.random_state_case(9012, num_layers=4, num_slots=16, slot_bytes=(4096, 65552),
                                        num_requests=5, max_tokens=3), state=True))
    out.append(Case(W.random_case(9013, num_layers=4, num_blocks=200, block_size=16, num_heads=2, head_dim=64,
                                  elem_bytes=1, has_scales=True, num_requests=3, max_tokens=300)))
    out.append(Case(W.random_case(9014, num_layers=4, num_blocks=64, block_size=16, num_heads=2, head_dim=64,
                                  num_requests=1, max_tokens=0)))
    out.append(Case(W.random_case(9018, num_layers=4, num_blocks=700, block_size=4, num_heads=4, head_dim=32,
                                  elem_bytes=1, has_scales=True, num_requests=4, max_tokens=500, layout="HND")))
    out.append(Case(W.random_case(9019, num_layers=4, num_blocks=600, block_size=1, num_heads=1, head_dim=576,
                                  elem_bytes=1, has_scales=True, num_requests=3, max_tokens=200, regions=1)))
    # whole 32 KiB blocks in long runs, enough of them for the 32 KiB one-wave
    # launch shape; and state slots of 64 KiB + 128 KiB (16 KiB one-wave shape)
    spec = W.PoolSpec(4, 1200, 16, 8, 128, W.BF16)
    rng = np.random.Generator(np.random.PCG64(9016))
    need = [W.alloc_blocks(9000, 16)]
    out.append(Case(W.Workload("long_runs", 9016, spec, spec, [9000],
                               W.split_tables(W.geometric_run_table(rng, 1200, 8.0), need),
                               W.split_tables(W.geometric_run_table(rng, 1200, 8.0), need))))
    out.append(Case(W.random_state_case(9017, num_layers=4, num_slots=16, slot_bytes=(65536, 131072),
                                        num_requests=6, max_tokens=3), state=True))
    return out


def test_push_many_matches_oracle():
    cs = cases()
    rng = np.random.Generator(np.random.PCG64(5))
    # every (case, layer) pair once, shuffled: 60 pairs, destinations disjoint
    pairs = [(c, l) for c in cs for l in range(4)]
    order = rng.permutation(len(pairs))
    pairs = [pairs[i] for i in order]
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    kvx.kvx_push_many([c.plan for c, _ in pairs], [l for _, l in pairs], ready=ev, stream=side)
    side.synchronize()
    for c, l in pairs:
        c.expect(l)
    for c in cs:
        c.check()
    # a second call over a subset (pushing the same bytes again changes nothing)
    sub = pairs[::5]
    kvx.kvx_push_many([c.plan for c, _ in sub], [l for _, l in sub], stream=side)
    kvx.kvx_push_many([], [], stream=side)
    side.synchronize()
    for c in cs:
        c.check()
    for c in cs:
        c.plan.close()


def test_push_many_launch_choices():
    """Each launch choice of kvx_push_many against the oracle: one layer of a
    plan of whole 32 KiB blocks alone (its own one-wave shape, one round),
    four of its layers together (past one round: each 32 KiB piece runs as
    eight 4 KiB chunks, the ragged last piece of each run with fewer), state
    layers of one shape (kept), and a plan of 16 KiB pieces sharing a launch
    with the 32 KiB one (shapes differ: four and eight chunks per piece).
    That plan moves the first 200 blocks of the long case's own tables, so
    its bytes are a subset of the long plan's push of the same layer."""
    cs = cases()
    longc = next(c for c in cs if c.wl.name == "long_runs")
    state = cs[-1]
    assert longc.plan.launch_shape()["piece_bytes"] == 32768 and longc.plan.launch_shape()["pieces"] > 608
    assert state.plan.launch_shape()["piece_bytes"] == 16384
    wl = longc.wl
    prefix = kvx.kvx_plan(longc.gs.pool, longc.gd.pool, [200 * 16], [wl.src_tables[0][:200]],
                          [wl.dst_tables[0][:200]])
    assert prefix.launch_shape()["piece_bytes"] == 16384
    side = torch.cuda.Stream()
    for plans, layers in (([longc.plan], [2]), ([longc.plan] * 4, [0, 1, 2, 3]),
                          ([state.plan] * 4, [0, 1, 2, 3]),
                          ([prefix, longc.plan, prefix], [1, 1, 3])):
        kvx.kvx_push_many(plans, layers, stream=side)
    side.synchronize()
    for l in (0, 1, 2, 3):
        longc.expect(l)
        state.expect(l)
    longc.check()
    state.check()
    prefix.close()
    for c in cs:
        c.plan.close()


def test_push_many_errors_enqueue_nothing():
    cs = cases()[:2]
    host_plan = kvx.kvx_plan(cs[0].gs.pool, cs[0].gd.pool, [0], [[0]], [[0]], host_only=True)
    for plans, layers, code in (([cs[0].plan, host_plan], [0, 0], kvx.KVX_E_INVAL),
                                ([cs[0].plan, cs[1].plan], [0, 4], kvx.KVX_E_RANGE),
                                ([cs[0].plan, cs[1].plan], [-1, 0], kvx.KVX_E_RANGE)):
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_push_many(plans, layers)
        assert e.value.code == code
    torch.cuda.synchronize()
    for c in cs:
        c.check()   # nothing moved
    rc = kvx.lib().kvx_push_many(None, None, 1, None, None)
    assert rc == kvx.KVX_E_INVAL
    for c in cs:
        c.plan.close()
