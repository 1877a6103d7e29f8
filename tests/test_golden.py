"""The oracle reproduces its stored digests (tests/golden/oracle_digests.txt,
written by tests/golden/make_golden.py from the oracle alone), and the
seeded generators are deterministic."""
import hashlib
import os

import numpy as np

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import workloads as W

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_digests.txt")


def stored():
    out = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        wl, what, val = line.strip().split(" ", 2)
        out[(wl, what)] = val
    return out


def sha(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def test_tiny_push_digests():
    g = stored()
    wl = W.tiny_push()
    src, dst = P.pools(O, wl)
    reqs = P.requests_for(O, wl)
    plan = O.make_plan(src.geom, dst.geom, reqs)
    assert " ".join(f"{r.src0}:{r.dst0}:{r.nblk}:{r.tail}" for r in plan.runs) == g[("tiny_push", "runs")]
    assert sha(src.kv) == g[("tiny_push", "src_sha256")]
    assert sha(dst.kv) == g[("tiny_push", "dst_before_sha256")]
    O.push(src, dst, plan)
    assert sha(dst.kv) == g[("tiny_push", "dst_after_sha256")]
    assert sha(O.pack(src, plan, 0, 2)) == g[("tiny_push", "staging_sha256")]


def test_qwen32b_runs_digest():
    g = stored()
    wl = W.qwen32b_push()
    reqs = P.requests_for(O, wl)
    gm = P.geom(O, wl.src)
    plan = O.make_plan(gm, gm, reqs)
    assert str(len(plan.runs)) == g[("qwen32b_push", "num_runs")]
    arr = np.array([(r.src0, r.dst0, r.nblk, r.tail) for r in plan.runs], "int32")
    assert sha(arr) == g[("qwen32b_push", "runs_sha256")]


def test_generators_deterministic():
    for name, fn in W.WORKLOADS.items():
        a, b = fn(), fn()
        assert a.prompt_lens == b.prompt_lens
        for x, y in zip(a.src_tables + a.dst_tables, b.src_tables + b.dst_tables):
            assert np.array_equal(x, y)


def test_generator_shapes():
    wl = W.batched_push()
    assert len(wl.prompt_lens) == 64 and all(1024 <= p <= 16384 for p in wl.prompt_lens)
    allsrc = np.concatenate(wl.src_tables)
    alldst = np.concatenate(wl.dst_tables)
    assert len(np.unique(allsrc)) == len(allsrc) and len(np.unique(alldst)) == len(alldst)
    assert allsrc.max() < 65536
    wl = W.multiturn_fp8()
    assert all(len(t) == 896 for t in wl.extra["decode_tables"])
    assert all(len(t) == 128 * 8 for t in wl.extra["prefill_tables"][8])
    seq = W.geometric_run_table(np.random.Generator(np.random.PCG64(1)), 100000, 4.0)
    assert sorted(seq.tolist()) == list(range(100000))
    # mean segment length close to 4
    breaks = np.count_nonzero(np.diff(seq) != 1) + 1
    assert 3.6 < 100000 / breaks < 4.4
