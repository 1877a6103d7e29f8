"""libkvx on the CPU: the library loads and exports every function kvx.h
declares, and its host-only planning (KVX_PLAN_HOST_ONLY) matches the oracle
exactly -- run tables, per-region triples, byte counts, staging sizes and
error classes.  No device memory is touched: pools are registered with
made-up 16-byte-aligned addresses that host-only plans never dereference."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(kvx_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = kvx.lib()
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(kvx.EXPORTED)
    want = int(re.search(r"#define KVX_ABI_VERSION (\d+)", open(os.path.join(ROOT, "include", "kvx.h")).read()).group(1))
    assert kvx.kvx_abi_version() == want
    assert L.kvx_status_str(kvx.KVX_E_DUPDST) == b"KVX_E_DUPDST"


FAKE = 1 << 40


def fake_pool(spec: W.PoolSpec, tag: int, scales=None):
    base = FAKE * (tag + 1)
    L = spec.num_layers
    kb = [base + (2 * spec.phys(l)) * spec.region_bytes for l in range(L)]
    vb = [base + (2 * spec.phys(l) + 1) * spec.region_bytes for l in range(L)]
    sc = spec.has_scales if scales is None else scales
    ks = [base // 2 + 8 * spec.num_blocks * l for l in range(L)] if sc else None
    vs = [base // 2 + 8 * spec.num_blocks * l + 4 * spec.num_blocks for l in range(L)] if sc else None
    two = spec.regions == 2
    return kvx.Pool(num_blocks=spec.num_blocks, block_size=spec.block_size, num_heads=spec.num_heads,
                    head_dim=spec.head_dim, elem_bytes=spec.elem_bytes, layout=spec.layout,
                    k_bases=kb, v_bases=vb if two else None, k_scales=ks, v_scales=vs if two else None,
                    sliding_window=spec.window)


def fake_state_pool(spec: W.StateSpec, tag: int):
    base = FAKE * (tag + 1)
    L = spec.num_layers
    b0 = [base + l * (spec.region_bytes(0) + spec.region_bytes(1)) for l in range(L)]
    b1 = [x + spec.region_bytes(0) for x in b0]
    return kvx.StatePool(num_slots=spec.num_slots, slot_bytes=spec.slot_bytes, bases0=b0, bases1=b1)


def host_plan(wl, tokens=None):
    sp, dp = fake_pool(wl.src, 0), fake_pool(wl.dst, 1)
    n = tokens if tokens is not None else [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    return kvx.kvx_plan(sp, dp, n, wl.src_tables, wl.dst_tables, host_only=True), n


def oracle_plan(wl, tokens):
    reqs = [O.Request(k, s, d) for k, s, d in zip(tokens, wl.src_tables, wl.dst_tables)]
    return O.make_plan(P.geom(O, wl.src), P.geom(O, wl.dst), reqs)


def gpu_sized_random_cases(count, seed0):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        yield W.random_case(
            500 + seed0 + i, layout=["NHD", "HND"][i % 2], elem_bytes=int(rng.choice([1, 2])),
            num_layers=int(rng.integers(1, 4)), num_blocks=int(rng.integers(200, 260)),
            block_size=int(rng.choice([1, 3, 4, 16])), num_heads=int(rng.integers(1, 5)),
            head_dim=int(rng.choice([16, 32, 64])), has_scales=bool(i % 2), num_requests=int(rng.integers(0, 5)),
            max_tokens=40, run_mean=float(rng.choice([1.2, 2.0, 5.0])), extra_ids=int(rng.integers(0, 3)))


def compare(wl, tokens=None):
    plan, n = host_plan(wl, tokens)
    op = oracle_plan(wl, n)
    runs = plan.runs()
    assert runs.tolist() == [[r.src0, r.dst0, r.nblk, r.tail] for r in op.runs]
    if wl.src.num_heads == wl.dst.num_heads and wl.src.layout == wl.dst.layout:
        for layer in (0, wl.src.num_layers - 1):
            for kv in range(wl.src.regions):
                assert plan.triples(layer, kv).tolist() == [list(t) for t in op.triples]
        rd, wr = plan.bytes_per_layer()
        assert (rd, wr) == op.bytes_per_layer()
        L = wl.src.num_layers
        assert kvx.kvx_staging_bytes(plan, 0, L) == O.staging_bytes(op, 0, L)
        assert kvx.kvx_staging_bytes(plan, 1, L) == O.staging_bytes(op, 1, L)
    plan.close()


def test_plan_matches_oracle_random():
    for wl in gpu_sized_random_cases(60, 0):
        compare(wl)


def test_plan_matches_oracle_workloads():
    for fn in (W.tiny_push, W.qwen32b_push, W.batched_push, W.tp4_share):
        compare(fn())


def test_plan_matches_oracle_multiturn():
    wl = W.multiturn_fp8()
    ex = wl.extra
    for t in (2, 5, 8):
        reqs = [O.reuse_request(t, ex["growth"], ex["threshold"], ex["decode_tables"][s],
                                ex["prefill_tables"][t][s]) for s in range(ex["sessions"])]
        toks = [r.num_tokens for r in reqs]
        turn = W.Workload("turn", wl.seed, wl.src, wl.dst, toks, list(ex["decode_tables"]),
                          list(ex["prefill_tables"][t]))
        compare(turn, toks)


def test_tokens_and_threshold_helpers():
    for p in range(0, 70):
        for c in range(0, 5):
            assert kvx.kvx_tokens_to_move(p, c) == O.tokens_to_move(p, c)
    for thr in (0, 1, 64, 512):
        for r in range(max(0, thr - 3), thr + 3):
            assert kvx.kvx_should_reuse(r, thr) == O.should_reuse(r, thr)


def test_error_classes_match_oracle():
    spec = W.PoolSpec(1, 8, 4, 1, 16, W.U8)
    sp, dp = fake_pool(spec, 0), fake_pool(spec, 1)
    g = P.geom(O, spec)
    cases = [
        ([-1], [[0]], [[0]]),
        ([5], [[0]], [[0]]),
        ([4], [[8]], [[0]]),
        ([4], [[0]], [[-1]]),
        ([4, 4], [[0], [1]], [[3], [3]]),
        ([4, 4], [[0], [0]], [[3], [4]]),
        ([4], [[0, 99]], [[3, 3]]),
        ([0], [[]], [[]]),
        ([], [], []),
    ]
    for toks, st, dt in cases:
        reqs = [O.Request(n, s, d) for n, s, d in zip(toks, st, dt)]
        try:
            O.make_plan(g, g, reqs)
            exp = "OK"
        except O.OracleError as e:
            exp = e.kind
        off = np.zeros(len(toks) + 1, np.int64)
        off[1:] = np.cumsum([len(x) for x in st])
        sid = np.array([x for s in st for x in s] or [0], np.int32)
        did = np.array([x for d in dt for x in d] or [0], np.int32)
        rc, plan = kvx.kvx_plan_raw(sp, dp, len(toks), np.array(toks or [0], np.int64), off, off, sid, did)
        got = "OK" if rc == 0 else kvx.lib().kvx_status_str(rc).decode().replace("KVX_E_", "")
        assert got == exp, (toks, st, dt, got, exp)
        if plan:
            plan.close()


def test_argument_errors():
    spec = W.PoolSpec(2, 8, 4, 2, 16, W.BF16)
    sp, dp = fake_pool(spec, 0), fake_pool(spec, 1)
    off = np.array([0, 1], np.int64)
    ids = np.array([0], np.int32)
    n = np.array([4], np.int64)
    assert kvx.kvx_plan_raw(sp, sp, 1, n, off, off, ids, ids)[0] == kvx.KVX_E_INVAL  # same pool
    assert kvx.kvx_plan_raw(sp, dp, -1, n, off, off, ids, ids)[0] == kvx.KVX_E_INVAL
    assert kvx.kvx_plan_raw(sp, dp, 1, n, off, off, ids, ids, flags=8)[0] == kvx.KVX_E_INVAL
    assert kvx.kvx_plan_raw(sp, dp, 1, n, np.array([1, 0], np.int64), off, ids, ids)[0] == kvx.KVX_E_INVAL
    assert kvx.kvx_plan_raw(sp, dp, 1, None, off, off, ids, ids)[0] == kvx.KVX_E_INVAL
    # geometry mismatch at plan time: head_dim differs
    other = fake_pool(W.PoolSpec(2, 8, 4, 2, 32, W.BF16), 2)
    assert kvx.kvx_plan_raw(sp, other, 1, n, off, off, ids, ids)[0] == kvx.KVX_E_MISMATCH
    # head count differs: plan is fine, push-only queries are mismatches
    fewer = fake_pool(W.PoolSpec(2, 8, 4, 1, 16, W.BF16, "HND"), 3)
    rc, plan = kvx.kvx_plan_raw(sp, fewer, 1, n, off, off, ids, ids)
    assert rc == 0
    with pytest.raises(kvx.KvxError) as e:
        plan.triples()
    assert e.value.code == kvx.KVX_E_MISMATCH
    assert plan.runs().tolist() == [[0, 0, 1, 4]]
    # device calls on a host-only plan are argument errors, and range checks hold
    rc, plan = kvx.kvx_plan_raw(sp, dp, 1, n, off, off, ids, ids)
    L = kvx.lib()
    assert L.kvx_push_layer(plan.handle, 0, None, None) == kvx.KVX_E_INVAL
    assert L.kvx_copy_heads(plan.handle, 0, 0, 0, 1, None, None) == kvx.KVX_E_INVAL
    assert L.kvx_plan_wait(plan.handle) == kvx.KVX_OK          # nothing uploaded: returns at once
    assert L.kvx_plan_wait(None) == kvx.KVX_E_INVAL
    assert L.kvx_plan_destroy_after(None, None) == kvx.KVX_OK   # NULL: no-op
    other = kvx.kvx_plan_raw(sp, dp, 1, n, off, off, ids, ids)[1]
    other.close_after(0)                                      # host-only: freed at once
    assert other.handle is None and kvx.kvx_plan_reclaim(False) == 0
    with pytest.raises(kvx.KvxError):
        plan.triples(2, 0)
    b = ctypes.c_int64()
    assert L.kvx_staging_bytes(plan.handle, 1, 0, ctypes.byref(b)) == kvx.KVX_E_RANGE
    assert L.kvx_staging_bytes(plan.handle, 0, 3, ctypes.byref(b)) == kvx.KVX_E_RANGE
    assert b"layers" in L.kvx_last_error()


def test_pool_create_errors():
    spec = W.PoolSpec(1, 8, 4, 1, 16, W.BF16)
    with pytest.raises(kvx.KvxError) as e:  # head_dim*elem_bytes = 8*1: not a multiple of 16
        kvx.Pool(num_blocks=8, block_size=4, num_heads=1, head_dim=8, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_UNSUPPORTED
    with pytest.raises(kvx.KvxError) as e:  # misaligned base
        kvx.Pool(num_blocks=8, block_size=4, num_heads=1, head_dim=16, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE + 8], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_UNSUPPORTED
    with pytest.raises(kvx.KvxError) as e:
        kvx.Pool(num_blocks=0, block_size=4, num_heads=1, head_dim=16, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_INVAL
    with pytest.raises(kvx.KvxError) as e:  # only one of the scale arrays
        kvx.Pool(num_blocks=8, block_size=4, num_heads=1, head_dim=16, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE], v_bases=[FAKE * 2], k_scales=[FAKE * 3])
    assert e.value.code == kvx.KVX_E_INVAL
    with pytest.raises(kvx.KvxError) as e:
        kvx.Pool(num_blocks=8, block_size=4, num_heads=1, head_dim=16, elem_bytes=3, layout="NHD",
                 k_bases=[FAKE], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_INVAL
    # a block of 2^31 bytes per region (32768 slots x 16 heads x 1024 x 4 B) is refused; one slot less is not
    with pytest.raises(kvx.KvxError) as e:
        kvx.Pool(num_blocks=1, block_size=32768, num_heads=16, head_dim=1024, elem_bytes=4, layout="HND",
                 k_bases=[FAKE], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_UNSUPPORTED
    assert b"2^31" in kvx.lib().kvx_last_error()
    kvx.Pool(num_blocks=1, block_size=32767, num_heads=16, head_dim=1024, elem_bytes=4, layout="HND",
             k_bases=[FAKE], v_bases=[FAKE * 2]).close()
    fake_pool(spec, 0).close()


def test_reblock_plan_matches_oracle():
    """Different block sizes per side: triples, bytes and staging sizes equal
    the oracle's token-segment procedure; runs are refused."""
    rng = np.random.Generator(np.random.PCG64(17))
    for i in range(40):
        bs, bsd = [int(x) for x in rng.choice([1, 2, 3, 4, 8, 16, 32], size=2, replace=False)]
        wl = W.random_case(9000 + i, layout=["NHD", "HND"][i % 2], elem_bytes=int(rng.choice([1, 2])),
                           num_layers=2, num_blocks=400, block_size=bs, dst_block_size=bsd,
                           num_heads=int(rng.integers(1, 4)), head_dim=int(rng.choice([16, 32])),
                           num_requests=int(rng.integers(0, 4)), max_tokens=80,
                           run_mean=float(rng.choice([1.5, 4.0])), extra_ids=int(rng.integers(0, 2)))
        plan, n = host_plan(wl)
        op = oracle_plan(wl, n)
        assert plan.triples(0, 0).tolist() == [list(t) for t in op.triples], wl.name
        assert plan.bytes_per_layer() == op.bytes_per_layer()
        assert kvx.kvx_staging_bytes(plan, 0, 2) == O.staging_bytes(op, 0, 2)
        with pytest.raises(kvx.KvxError) as e:
            plan.runs()
        assert e.value.code == kvx.KVX_E_MISMATCH
        plan.close()


def test_reblock_errors():
    a = W.PoolSpec(1, 8, 4, 1, 16, W.U8, has_scales=True)
    b = W.PoolSpec(1, 8, 8, 1, 16, W.U8, has_scales=True)
    with pytest.raises(kvx.KvxError) as e:
        kvx.kvx_plan(fake_pool(a, 0), fake_pool(b, 1), [8], [[0, 1]], [[2]], host_only=True)
    assert e.value.code == kvx.KVX_E_UNSUPPORTED
    a, b = W.PoolSpec(1, 8, 4, 1, 16, W.U8), W.PoolSpec(1, 8, 8, 1, 16, W.U8)
    pa, pb = fake_pool(a, 0), fake_pool(b, 1)
    kvx.kvx_plan(pa, pb, [8], [[0, 1]], [[2]], host_only=True).close()
    for st, dt in (([0, 1], [2, 3]), ([0, 1, 2], [2])):
        with pytest.raises(kvx.KvxError) as e:
            kvx.kvx_plan(pa, pb, [9], [st], [dt], host_only=True)
        assert e.value.code == kvx.KVX_E_INVAL
    with pytest.raises(kvx.KvxError) as e:
        kvx.Pool(num_blocks=8, block_size=65536, num_heads=1, head_dim=16, elem_bytes=1, layout="NHD",
                 k_bases=[FAKE], v_bases=[FAKE * 2])
    assert e.value.code == kvx.KVX_E_UNSUPPORTED


def test_build_entry_version_check():
    """__graft_entry__.build() ends by comparing the built library's ABI
    version with include/kvx.h; the same check without the compile."""
    import __graft_entry__ as G
    assert G.header_abi_version() == kvx.kvx_abi_version()
