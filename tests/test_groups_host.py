"""Host-only planning of layer groups of other shapes against the oracle:
pools of one latent region (MLA), sliding-window groups and state-slot
groups.  Run tables, per-region triples, byte counts, staging sizes and
error classes must equal the oracle's; no device memory is touched."""
import numpy as np
import pytest

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import workloads as W
from test_abi_host import compare, fake_pool, fake_state_pool


def test_latent_plans_match_oracle():
    for wl in P.latent_cases(24, seed0=91):
        compare(wl)
    wl = W.dsr1_mla_push()
    g = wl.groups[0]
    compare(W.Workload("mla", wl.seed, g.src, g.dst, wl.prompt_lens, g.src_tables, g.dst_tables))


def test_window_plans_match_oracle():
    for wl in P.window_cases(60, seed0=93):
        if wl.src.block_size == wl.dst.block_size:
            compare(wl)
        else:
            plan = kvx.kvx_plan(fake_pool(wl.src, 0), fake_pool(wl.dst, 1),
                                [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens],
                                wl.src_tables, wl.dst_tables, host_only=True)
            reqs = P.requests_for(O, wl)
            op = O.make_plan(P.geom(O, wl.src), P.geom(O, wl.dst), reqs)
            assert plan.triples(0, 0).tolist() == [list(t) for t in op.triples]
            assert plan.bytes_per_layer() == op.bytes_per_layer()
            with pytest.raises(kvx.KvxError) as e:
                plan.runs()
            assert e.value.code == kvx.KVX_E_MISMATCH
    wl = W.gptoss_swa_push()
    for g in wl.groups:
        compare(W.Workload(g.name, wl.seed, g.src, g.dst, wl.prompt_lens, g.src_tables, g.dst_tables))


def test_window_skipped_entries_are_not_validated():
    spec = W.PoolSpec(1, 64, 4, 1, 16, W.U8, window=3)
    sp, dp = fake_pool(spec, 0), fake_pool(spec, 1)
    # 21 tokens: next query at 21 sees 19..21 -> blocks 4 and 5 are kept
    src = [-1, -1, -1, -1, 10, 11]
    dst = [99999, 7, 7, 7, 20, 21]
    plan = kvx.kvx_plan(sp, dp, [21], [src], [dst], host_only=True)
    assert plan.runs().tolist() == [[10, 20, 2, 1]]
    assert plan.triples(0, 1).tolist() == [[10 * 64, 20 * 64, 5 * 16]]
    rc, _ = kvx.kvx_plan_raw(sp, dp, 1, np.array([21], np.int64), np.array([0, 6], np.int64),
                             np.array([0, 6], np.int64), np.array([-1] * 4 + [10, 64], np.int32),
                             np.array(dst, np.int32))
    assert rc == kvx.KVX_E_RANGE


def state_compare(wl):
    sp, dp = fake_state_pool(wl.src, 0), fake_state_pool(wl.dst, 1)
    plan = kvx.kvx_plan(sp, dp, wl.prompt_lens, wl.src_tables, wl.dst_tables, host_only=True)
    reqs = [O.Request(n, s, d) for n, s, d in zip(wl.prompt_lens, wl.src_tables, wl.dst_tables)]
    op = O.make_state_plan(P.state_geom(O, wl.src), P.state_geom(O, wl.dst), reqs)
    assert plan.runs().tolist() == [[r.src0, r.dst0, r.nblk, r.tail] for r in op.runs]
    for layer in (0, wl.src.num_layers - 1):
        for r in range(2):
            assert plan.triples(layer, r).tolist() == [list(t) for t in op.triples[r]]
    assert plan.bytes_per_layer() == op.bytes_per_layer()
    L = wl.src.num_layers
    assert kvx.kvx_staging_bytes(plan, 0, L) == O.state_staging_bytes(op, 0, L)
    plan.close()


def test_state_plans_match_oracle():
    for wl in P.state_cases(40, seed0=95):
        state_compare(wl)
    wl = W.qwen3next_state_push()
    g = wl.groups[1]
    state_compare(W.Workload("state", wl.seed, g.src, g.dst, [8191] * len(wl.prompt_lens),
                             g.src_tables, g.dst_tables))


def test_state_errors():
    spec = W.StateSpec(1, 32, (16, 48), W.U8)
    sp, dp = fake_state_pool(spec, 0), fake_state_pool(spec, 1)
    cases = [([1, 1], [[0], [1]], [[5], [5]], kvx.KVX_E_DUPDST),
             ([1], [[32]], [[0]], kvx.KVX_E_RANGE),
             ([1], [[0]], [[-1]], kvx.KVX_E_RANGE),
             ([1], [[]], [[0]], kvx.KVX_E_INVAL),
             ([-1], [[0]], [[0]], kvx.KVX_E_INVAL)]
    for toks, st, dt, code in cases:
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_plan(sp, dp, toks, st, dt, host_only=True)
        assert e.value.code == code, (toks, st, dt)
    # the same error classes in the oracle
    g = O.StateGeometry(1, 32, (16, 48))
    for toks, st, dt, code in cases:
        with pytest.raises(O.OracleError) as e:
            O.make_state_plan(g, g, [O.Request(n, s, d) for n, s, d in zip(toks, st, dt)])
        assert e.value.kind == KIND[code]
    assert kvx.kvx_plan(sp, dp, [0], [[]], [[]], host_only=True).triples(0, 1).tolist() == []
    other = fake_state_pool(W.StateSpec(1, 32, (16, 64), W.U8), 2)
    attn = fake_pool(W.PoolSpec(1, 32, 4, 1, 16, W.U8), 3)
    for a, b in ((sp, other), (sp, attn), (attn, sp)):
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_plan(a, b, [], [], [], host_only=True)
        assert e.value.code == kvx.KVX_E_MISMATCH
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_copy_heads(kvx.kvx_plan(sp, dp, [], [], [], host_only=True), 0, 0, 0, 1, stream=0)
    assert e.value.code == kvx.KVX_E_INVAL    # host-only plan: checked first


def test_group_pool_errors():
    spec = W.PoolSpec(1, 32, 4, 1, 16, W.U8)
    a = fake_pool(spec, 0)
    for other in (W.PoolSpec(1, 32, 4, 1, 16, W.U8, regions=1), W.PoolSpec(1, 32, 4, 1, 16, W.U8, window=8)):
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_plan(a, fake_pool(other, 1), [], [], [], host_only=True)
        assert e.value.code == kvx.KVX_E_MISMATCH
    with pytest.raises(kvx.KvxError) as e:
        fake_pool(W.PoolSpec(1, 32, 4, 1, 16, W.U8, window=-1), 2)
    assert e.value.code == kvx.KVX_E_INVAL
    for sb, code in (((8, 16), kvx.KVX_E_UNSUPPORTED), ((16, 40), kvx.KVX_E_UNSUPPORTED)):
        with pytest.raises(kvx.KvxError) as e:
            fake_state_pool(W.StateSpec(1, 8, sb, W.U8), 3)
        assert e.value.code == code
    with pytest.raises(kvx.KvxError) as e:
        kvx.Pool(num_blocks=8, block_size=4, num_heads=1, head_dim=16, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE_BASE], v_bases=None, k_scales=[FAKE_BASE // 2], v_scales=[FAKE_BASE // 4])
    assert e.value.code == kvx.KVX_E_INVAL


FAKE_BASE = 1 << 41
KIND = {kvx.KVX_E_INVAL: "INVAL", kvx.KVX_E_RANGE: "RANGE", kvx.KVX_E_DUPDST: "DUPDST"}


def test_xfer_drives_any_group_kind():
    """The transfer state machine plans through kvx_plan and is blind to the
    group's shape: a state-slot group and a sliding-window group go through
    register / prefill / save / seal / complete like a K/V group, and the
    recompute list of a failed request is its registered entries."""
    cases = [(fake_state_pool(W.StateSpec(3, 16, (16, 48), W.U8), 0),
              fake_state_pool(W.StateSpec(3, 16, (16, 48), W.U8), 1), [4], [9]),
             (fake_pool(W.PoolSpec(3, 64, 4, 1, 16, W.U8, window=5), 2),
              fake_pool(W.PoolSpec(3, 64, 4, 1, 16, W.U8, window=5), 3), list(range(10, 20)), list(range(30, 40)))]
    for prod, cons, src, dst in cases:
        x = kvx.Xfer(prod, host_only=True)
        assert x.prefill(1, 0, 37, src, 0.0)
        for l in range(3):
            assert x.save_layer(1, 0, l, 0.0)
        assert x.register(1, 0, cons, dst, 0.5)
        assert x.seal(1, 0)
        for l in range(3):
            x.complete(1, 0, l, ok=True)
        x.poll(1.0)
        assert x.pop_finished() == [(1, 0, kvx.KVX_REQ_DONE)]
        assert x.register(2, 0, cons, dst[::-1] if len(dst) > 1 else [10], 2.0)
        assert x.prefill(2, 0, 37, src, 2.0)
        assert x.save_layer(2, 0, 0, 2.0)
        x.complete(2, 0, 0, ok=False)
        assert x.status(2) == (0, kvx.KVX_REQ_FAILED)
        assert x.recompute_blocks(2) == (dst[::-1] if len(dst) > 1 else [10])
        x.close()


def test_push_many_argument_errors():
    """Argument errors of kvx_push_many need no device: they are reported
    before anything is enqueued."""
    spec = W.PoolSpec(2, 32, 4, 1, 16, W.U8)
    p = kvx.kvx_plan(fake_pool(spec, 0), fake_pool(spec, 1), [5], [[1, 2]], [[3, 4]], host_only=True)
    L = kvx.lib()
    assert L.kvx_push_many(None, None, -1, None, None) == kvx.KVX_E_INVAL
    assert L.kvx_push_many(None, None, 2, None, None) == kvx.KVX_E_INVAL
    assert L.kvx_push_many(None, None, 0, None, None) == kvx.KVX_OK
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_push_many([p], [0], stream=0)
    assert e.value.code == kvx.KVX_E_INVAL     # host-only plan
    with pytest.raises(ValueError):
        kvx.kvx_push_many([p], [0, 1], stream=0)


def test_launch_shape_rule():
    """The copy kernels' launch shape follows how fully a plan's runs fill
    32 KiB pieces and how many of those pieces one layer's launch has: runs
    of whole 32 KiB blocks take one-wave workgroups, 32 KiB pieces from 608
    to 1312 pieces per launch and 16 KiB pieces below; larger launches and
    runs that fill pieces less (blocks of 16 KiB or smaller, ragged ends)
    take 4 KiB pieces of four-wave workgroups.  The work list is cut to that
    size."""
    big = W.PoolSpec(1, 2000, 16, 8, 128, W.BF16)       # 32 KiB blocks
    mid = W.PoolSpec(1, 2000, 16, 8, 64, W.BF16)        # 16 KiB blocks
    tiny = W.PoolSpec(1, 4000, 1, 1, 576, W.BF16)       # 1152-byte blocks

    def shape(spec, tokens, ids_src, ids_dst):
        p = kvx.kvx_plan(fake_pool(spec, 0), fake_pool(spec, 1), [tokens], [ids_src], [ids_dst], host_only=True)
        s = p.launch_shape()
        t = p.triples(0, 0)
        assert s["pieces"] == 2 * sum(-(-int(x) // s["piece_bytes"]) for x in t[:, 2])   # K and V
        return s["lanes"], s["vectors"], s["piece_bytes"]
    seq = list(range(2000))
    assert shape(big, 16 * 512, seq[:512], seq[:512]) == (64, 32, 32768)        # 1024 pieces
    assert shape(big, 16 * 656, seq[:656], seq[:656]) == (64, 32, 32768)        # 1312 pieces
    assert shape(big, 16 * 657, seq[:657], seq[:657]) == (256, 1, 4096)         # 1314 pieces: streams
    assert shape(big, 16 * 304, seq[:304], seq[:304]) == (64, 32, 32768)        # 608 pieces
    assert shape(big, 16 * 303, seq[:303], seq[:303]) == (64, 16, 16384)        # 606 pieces
    pairs = [b for k in range(0, 4000, 3) for b in (k, k + 1)][:600]
    assert shape(mid, 16 * 600, pairs, pairs) == (64, 16, 16384)                # 32 KiB runs, 600 pieces
    threes = [b for k in range(0, 4000, 4) for b in (k, k + 1, k + 2)][:600]
    assert shape(mid, 16 * 600, threes, threes) == (256, 1, 4096)               # 48 KiB runs: fill 0.75
    scattered = list(range(0, 4000, 7))[:500]
    assert shape(tiny, 500, scattered, scattered) == (256, 1, 4096)             # 1152-byte runs


def test_launch_shape_fill_boundary():
    """Fill exactly 0.9 takes one-wave workgroups, one token less four-wave
    workgroups of 4 KiB pieces: runs of nine 16 KiB blocks (144 KiB) cover
    five 32 KiB pieces (160 KiB)."""
    mid = W.PoolSpec(1, 4000, 16, 8, 64, W.BF16)        # 16 KiB blocks
    sp, dp = fake_pool(mid, 0), fake_pool(mid, 1)
    nines = [10 * k + j for k in range(100) for j in range(9)]     # 100 runs of 9 blocks: 1000 pieces
    s = kvx.kvx_plan(sp, dp, [16 * 900], [nines], [nines], host_only=True).launch_shape()
    assert (s["lanes"], s["vectors"]) == (64, 32)
    s = kvx.kvx_plan(sp, dp, [16 * 900 - 1], [nines], [nines], host_only=True).launch_shape()
    assert (s["lanes"], s["vectors"]) == (256, 1)


def test_launch_shape_overlap_flag():
    """KVX_PLAN_OVERLAP: the caller keeps several launches of the plan in
    flight, so even runs of whole 32 KiB blocks in a launch of one round
    take 4 KiB pieces of four-wave workgroups; the copied bytes (triples) are
    those of the plan without the flag."""
    big = W.PoolSpec(1, 2000, 16, 8, 128, W.BF16)
    sp, dp = fake_pool(big, 0), fake_pool(big, 1)
    seq = list(range(512))
    a = kvx.kvx_plan(sp, dp, [16 * 512], [seq], [seq], host_only=True)
    b = kvx.kvx_plan(sp, dp, [16 * 512], [seq], [seq], host_only=True, overlap=True)
    assert (a.launch_shape()["lanes"], a.launch_shape()["vectors"]) == (64, 32)
    assert (b.launch_shape()["lanes"], b.launch_shape()["vectors"], b.launch_shape()["pieces"]) == (256, 1, 8192)
    assert np.array_equal(a.triples(), b.triples()) and a.bytes_per_layer() == b.bytes_per_layer()
    rc, _ = kvx.kvx_plan_raw(sp, dp, 1, np.array([16], np.int64), np.array([0, 1], np.int64),
                             np.array([0, 1], np.int64), np.array([0], np.int32), np.array([0], np.int32),
                             flags=kvx.KVX_PLAN_HOST_ONLY | kvx.KVX_PLAN_OVERLAP | 8)   # an unknown flag
    assert rc == kvx.KVX_E_INVAL


def test_run_table_plans_host():
    """KVX_PLAN_RUNS is honoured for streaming plans of K/V pools and ignored
    for one-wave plans and state pools; the chunk count covers the flat
    space of the shared list, and the triples do not depend on it."""
    big = W.PoolSpec(1, 2000, 16, 8, 128, W.BF16)       # 32 KiB blocks
    tiny = W.PoolSpec(1, 4000, 1, 1, 576, W.BF16)       # 1152-byte blocks
    seq = list(range(2000))
    one_wave = kvx.kvx_plan(fake_pool(big, 0), fake_pool(big, 1), [16 * 512], [seq[:512]], [seq[:512]],
                            host_only=True, runs=True)
    assert not one_wave.launch_shape()["run_table"]
    scattered = list(range(0, 4000, 7))[:500]
    a = kvx.kvx_plan(fake_pool(tiny, 0), fake_pool(tiny, 1), [500], [scattered], [scattered], host_only=True,
                     runs=True)
    b = kvx.kvx_plan(fake_pool(tiny, 0), fake_pool(tiny, 1), [500], [scattered], [scattered], host_only=True)
    sa, sb = a.launch_shape(), b.launch_shape()
    assert sa["run_table"] and not sb["run_table"]
    assert (sa["lanes"], sa["vectors"], sa["piece_bytes"]) == (256, 1, 4096)
    flat = int(a.triples(0, 0)[:, 2].sum())
    assert sa["pieces"] == 2 * -(-flat // 4096)
    assert np.array_equal(a.triples(0, 0), b.triples(0, 0))
    assert a.bytes_per_layer() == b.bytes_per_layer()
    assert kvx.kvx_staging_bytes(a, 0, 1) == kvx.kvx_staging_bytes(b, 0, 1)
