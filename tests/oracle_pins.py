"""Pins of the CPU oracle: checks against things other than the oracle itself.

Every ``pin_*`` takes the oracle module as an argument, so that
test_oracle_mutations.py can hand in a copy with a planted mistake and check
that some pin catches it.  The pins are:

* library special cases computed with torch CPU ops (``index_select`` /
  ``index_copy_`` on whole blocks, slice copies for one contiguous run,
  ``permute`` for the NHD -> HND head-slice transform);
* brute force: the plain per-(token, head) definition against the merged-run
  procedure on many tiny random cases (both layouts, 1- and 2-byte elements,
  tails 1..BS, empty requests, prompt lengths = 1 mod BS, scales);
* closed forms of the five workloads' token, block and byte counts, worked out
  by hand from their descriptions;
* invariants: unmapped destination bytes and the source never change, the
  final prompt token's slot never reaches the consumer, the run table is the
  unique maximal decomposition, pack/unpack round-trips to push;
* the values the pages print (tests/golden/pages_values.txt).
"""
from __future__ import annotations

import os

import numpy as np
import torch

from decode_kv_cache_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pages_values():
    out = {}
    with open(os.path.join(GOLDEN, "pages_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, val = line.split("|")[0].split()
            out[name] = int(val)
    return out


# ---------------------------------------------------------------------------
# helpers (inputs only; no transfer arithmetic)
# ---------------------------------------------------------------------------
def geom(O, spec):
    return O.Geometry(spec.num_layers, spec.num_blocks, spec.block_size, spec.num_heads,
                      spec.head_dim, spec.elem_bytes, spec.layout, spec.has_scales,
                      spec.regions, spec.window)


def state_geom(O, spec):
    return O.StateGeometry(spec.num_layers, spec.num_slots, tuple(spec.slot_bytes))


def pools(O, wl):
    gs, gd = geom(O, wl.src), geom(O, wl.dst)
    skv, ssc = W.host_values(wl.src, wl.seed, 1)
    dkv, dsc = W.host_values(wl.dst, wl.seed, 2)
    return O.Pool(gs, skv, ssc), O.Pool(gd, dkv, dsc)


def requests_for(O, wl, tokens=None):
    n = tokens if tokens is not None else [O.tokens_to_move(p) for p in wl.prompt_lens]
    return [O.Request(k, s, d) for k, s, d in zip(n, wl.src_tables, wl.dst_tables)]


def random_cases(count=48, seed0=7):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        layout = ["NHD", "HND"][i % 2]
        bs = int(rng.choice([1, 2, 3, 4, 5, 16]))
        yield W.random_case(
            1000 + i, layout=layout, elem_bytes=int(rng.choice([1, 2])), num_layers=int(rng.integers(1, 3)),
            num_blocks=int(rng.integers(24, 40)), block_size=bs, num_heads=int(rng.integers(1, 4)),
            head_dim=int(rng.choice([4, 8, 16])), has_scales=bool(i % 3 == 0),
            num_requests=int(rng.integers(1, 4)), max_tokens=int(min(6 * bs, 40)),
            run_mean=float(rng.choice([1.5, 3.0])), extra_ids=int(rng.integers(0, 2)))


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
def pin_brute_vs_procedure(O):
    """Plain definition == merged-run procedure, byte for byte; source unchanged."""
    for wl in random_cases():
        src, dst = pools(O, wl)
        src0 = src.copy()
        reqs = requests_for(O, wl)
        a, b = dst.copy(), dst.copy()
        O.push_plain(src, a, reqs)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        O.push(src, b, plan)
        assert np.array_equal(a.kv, b.kv), wl.name
        if a.scales is not None:
            assert np.array_equal(a.scales, b.scales), wl.name
        assert np.array_equal(src.kv, src0.kv)


def pin_full_blocks_index_copy(O):
    """Whole-block transfers equal torch index_select -> index_copy_ on the
    block dimension, per (layer, K/V) region, in both layouts."""
    for layout in ("NHD", "HND"):
        for seed in range(4):
            wl = W.random_case(50 + seed, layout=layout, num_blocks=32, block_size=4, num_heads=2,
                               head_dim=8, num_requests=2, max_tokens=12, has_scales=True)
            bs = wl.src.block_size
            # whole blocks only: move every allocated block completely
            toks = [len(t) * bs for t in wl.src_tables]
            src, dst = pools(O, wl)
            reqs = requests_for(O, wl, toks)
            plan = O.make_plan(src.geom, dst.geom, reqs)
            got = dst.copy()
            O.push(src, got, plan)
            sid = torch.from_numpy(np.concatenate(wl.src_tables).astype(np.int64))
            did = torch.from_numpy(np.concatenate(wl.dst_tables).astype(np.int64))
            exp = torch.from_numpy(dst.kv.copy())
            es = torch.from_numpy(dst.scales.copy().view(np.int32))
            s = torch.from_numpy(src.kv)
            ss = torch.from_numpy(src.scales.view(np.int32))
            nb = wl.src.num_blocks
            for l in range(wl.src.num_layers):
                for kv in range(2):
                    e = exp[l, kv].view(nb, -1)
                    e.index_copy_(0, did, s[l, kv].view(nb, -1).index_select(0, sid))
                    es[l, kv].index_copy_(0, did, ss[l, kv].index_select(0, sid))
            assert np.array_equal(got.kv, exp.numpy())
            assert np.array_equal(got.scales.view(np.int32), es.numpy())


def pin_single_run_slice(O):
    """One request whose blocks are consecutive on both sides (NHD): the moved
    bytes are one slice of n token rows."""
    spec = W.PoolSpec(1, 20, 4, 2, 8, W.BF16)
    g = geom(O, spec)
    for n in (1, 3, 4, 5, 11, 16):
        wl = W.Workload("run", 3, spec, spec, [n + 1], [np.arange(2, 9, dtype=np.int32)],
                        [np.arange(11, 18, dtype=np.int32)])
        src, dst = pools(O, wl)
        got = dst.copy()
        reqs = requests_for(O, wl)
        O.push(src, got, O.make_plan(g, g, reqs))
        tb = 2 * 8 * 2
        bb = 4 * tb
        exp = dst.kv.copy()
        exp[0, :, 11 * bb:11 * bb + n * tb] = src.kv[0, :, 2 * bb:2 * bb + n * tb]
        assert np.array_equal(got.kv, exp), n


def pin_nhd_to_hnd_permute(O):
    """Whole blocks, head slice: NHD [blk, slot, head, dim] -> HND [blk, head,
    slot, dim] equals torch permute(0, 2, 1, 3) on the selected heads."""
    src_spec = W.PoolSpec(2, 16, 4, 4, 8, W.BF16, "NHD")
    for d_layout in ("HND", "NHD"):
        dst_spec = W.PoolSpec(2, 12, 4, 3, 8, W.BF16, d_layout)
        rng = np.random.Generator(np.random.PCG64(5))
        st = rng.permutation(16)[:5].astype(np.int32)
        dt = rng.permutation(12)[:5].astype(np.int32)
        wl = W.Workload("perm", 9, src_spec, dst_spec, [20], [st], [dt])
        src, dst = pools(O, wl)
        gs, gd = src.geom, dst.geom
        reqs = requests_for(O, wl, [20])
        plan = O.make_plan(gs, gd, reqs)
        for s0, d0, nh in ((0, 0, 2), (2, 1, 2), (1, 0, 3), (3, 2, 1)):
            got = dst.copy()
            for l in range(2):
                O.copy_heads(src, got, plan, reqs, l, s0, d0, nh)
            exp = torch.from_numpy(dst.kv.copy())
            s = torch.from_numpy(src.kv)
            for l in range(2):
                for kv in range(2):
                    blk = s[l, kv].view(16, 4, 4, 16)[torch.from_numpy(st.astype(np.int64))]
                    sl = blk[:, :, s0:s0 + nh, :]
                    if d_layout == "HND":
                        e = exp[l, kv].view(12, 3, 4, 16)
                        e[torch.from_numpy(dt.astype(np.int64)), d0:d0 + nh] = sl.permute(0, 2, 1, 3)
                    else:
                        e = exp[l, kv].view(12, 4, 3, 16)
                        e[torch.from_numpy(dt.astype(np.int64)), :, d0:d0 + nh] = sl
            assert np.array_equal(got.kv, exp.numpy()), (d_layout, s0, d0, nh)


def pin_final_token_never_sent(O):
    """A P->D push with n = tokens_to_move(prompt) delivers every prompt token
    but the last, whose slot keeps its old bytes; when prompt = 1 mod BS the
    final token's whole block is never touched."""
    assert pages_values()["decode_recomputes_final_token"] == 1
    spec = W.PoolSpec(1, 40, 4, 2, 4, W.U8, "NHD")
    for layout in ("NHD", "HND"):
        spec = W.PoolSpec(1, 40, 4, 2, 4, W.U8, layout)
        g = geom(O, spec)
        for prompt in range(1, 14):
            nb_alloc = W.alloc_blocks(prompt, 4)
            rng = np.random.Generator(np.random.PCG64(prompt))
            st = rng.permutation(40)[:nb_alloc].astype(np.int32)
            dt = rng.permutation(40)[:nb_alloc].astype(np.int32)
            wl = W.Workload("ft", prompt, spec, spec, [prompt], [st], [dt])
            src, dst = pools(O, wl)
            got = dst.copy()
            reqs = requests_for(O, wl)
            O.push(src, got, O.make_plan(g, g, reqs))
            for p in range(prompt):
                j, s = divmod(p, 4)
                for h in range(2):
                    so, do = g.row_offset(int(st[j]), s, h), g.row_offset(int(dt[j]), s, h)
                    row_s = src.kv[0, :, so:so + 4]
                    row_d = got.kv[0, :, do:do + 4]
                    if p < prompt - 1:
                        assert np.array_equal(row_d, row_s), (layout, prompt, p)
                    else:
                        assert np.array_equal(row_d, dst.kv[0, :, do:do + 4]), (layout, prompt)
            if prompt % 4 == 1:
                last = int(dt[-1])
                bb = g.block_bytes
                assert np.array_equal(got.kv[0, :, last * bb:(last + 1) * bb],
                                      dst.kv[0, :, last * bb:(last + 1) * bb])


def pin_untouched_bytes(O):
    """Bytes outside the moved (block, slot, head) rows keep their old value."""
    for wl in list(random_cases(12, seed0=11)):
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        got = dst.copy()
        O.push(src, got, plan)
        gd = dst.geom
        mask = np.zeros(gd.region_bytes, bool)
        for req in reqs:
            for p in range(req.num_tokens):
                j, s = divmod(p, gd.block_size)
                for h in range(gd.num_heads):
                    o = gd.row_offset(int(req.dst_ids[j]), s, h)
                    mask[o:o + gd.row_bytes] = True
        for l in range(gd.num_layers):
            for kv in range(2):
                assert np.array_equal(got.kv[l, kv][~mask], dst.kv[l, kv][~mask])
        if dst.scales is not None:
            used = {d for r in reqs for d in r.dst_ids[:W.alloc_blocks(r.num_tokens, gd.block_size)]}
            keep = np.array([b not in used for b in range(gd.num_blocks)])
            assert np.array_equal(got.scales[:, :, keep], dst.scales[:, :, keep])


def pin_plan_invariants(O):
    """Run table = the unique maximal decomposition: (i) runs concatenate to
    the used ID lists, (ii) each run is +1-consecutive on both sides, (iii) no
    two neighbouring runs of a request could merge, (iv) only a request's last
    run is partly filled, (v) block total, (vi) triple bytes = tokens x token
    bytes per region."""
    cases = list(random_cases(30, seed0=3)) + [W.qwen32b_push()]
    for wl in cases:
        g = geom(O, wl.src)
        reqs = requests_for(O, wl)
        runs = O.plan_runs(reqs, g.block_size, g.num_blocks, wl.dst.num_blocks)
        pos = 0
        tot_blocks = 0
        for req in reqs:
            n = req.num_tokens
            nb = -(-n // g.block_size)
            got_s, got_d, mine = [], [], []
            while len(got_s) < nb:
                r = runs[pos]
                pos += 1
                mine.append(r)
                got_s += list(range(r.src0, r.src0 + r.nblk))
                got_d += list(range(r.dst0, r.dst0 + r.nblk))
            assert got_s == [int(x) for x in req.src_ids[:nb]]
            assert got_d == [int(x) for x in req.dst_ids[:nb]]
            for a, b in zip(mine, mine[1:]):
                assert not (b.src0 == a.src0 + a.nblk and b.dst0 == a.dst0 + a.nblk)
                assert a.tail == g.block_size
            if mine:
                assert mine[-1].tail == n - (nb - 1) * g.block_size
            tot_blocks += nb
        assert pos == len(runs)
        assert sum(r.nblk for r in runs) == tot_blocks
        tr = O.triples(runs, g)
        assert sum(t[2] for t in tr) == sum(r.num_tokens for r in reqs) * g.token_bytes


def pin_closed_forms(O):
    """Token, block and byte counts of the five workloads, by hand:
    tiny_push: 200-token prompt -> 199 tokens, 13 blocks, last block 7 tokens;
      199 x 8 heads x 64 x 2 B = 203,776 B per (layer, K/V); x 4 regions x
      (read + write) = 1,630,208 B.
    qwen32b_push: 8191 tokens, 512 blocks, last block 15 tokens; 8191 x 2048 B
      x 128 regions = 2,147,221,504 B read.
    tp4_share: 32 x 4095 tokens x 2 heads x 256 B x 128 regions =
      8,587,837,440 B read.
    multiturn_fp8: turns 2..8 reuse 2048 (t-1) tokens of 32 sessions:
      32 x 2048 x 28 = 1,835,008 tokens, 114,688 block copies; x 1024 B x 96
      regions + 4 B scale x 114,688 x 96 = 180,432,666,624 B read."""
    wl = W.tiny_push()
    reqs = requests_for(O, wl)
    g = geom(O, wl.src)
    assert reqs[0].num_tokens == 199
    runs = O.plan_runs(reqs, 16, 256, 256)
    assert sum(r.nblk for r in runs) == 13 and runs[-1].tail == 7
    plan = O.make_plan(g, g, reqs)
    assert plan.payload_bytes == 203_776
    rd, wr = plan.bytes_per_layer()
    assert (rd + wr) * g.num_layers == 1_630_208

    wl = W.qwen32b_push()
    reqs = requests_for(O, wl)
    g = geom(O, wl.src)
    plan = O.make_plan(g, g, reqs)
    assert reqs[0].num_tokens == 8191 and len(plan.pairs) == 512 and plan.runs[-1].tail == 15
    assert plan.bytes_per_layer()[0] * 64 == 2_147_221_504

    wl = W.tp4_share()
    reqs = requests_for(O, wl)
    gs, gd = geom(O, wl.src), geom(O, wl.dst)
    plan = O.make_plan(gs, gd, reqs)
    sr, dr = O.head_rows(plan, 0, 0, 2, reqs)
    assert len(sr) * gs.row_bytes * 128 == 8_587_837_440

    wl = W.multiturn_fp8()
    g = geom(O, wl.src)
    ex = wl.extra
    toks = blocks = 0
    for t in range(1, ex["turns"] + 1):
        for s in range(ex["sessions"]):
            r = O.reuse_request(t, ex["growth"], ex["threshold"], ex["decode_tables"][s],
                                ex["prefill_tables"][t][s])
            if r is not None:
                toks += r.num_tokens
                blocks += len(O.block_pairs(O.plan_runs([r], 16, g.num_blocks, g.num_blocks)))
    assert toks == 1_835_008 and blocks == 114_688
    assert toks * g.token_bytes * 96 + blocks * 4 * 96 == 180_432_666_624


def pin_threshold(O):
    """Reuse at or above the threshold, recompute below: the pages' default 64
    and the multi-turn workload's 512; turn 1 has nothing to reuse; turn 2
    reuses exactly the first turn's 2048-token context."""
    thr = pages_values()["recompute_threshold_default"]
    assert thr == 64
    assert not O.should_reuse(63, thr) and O.should_reuse(64, thr) and O.should_reuse(65, thr)
    assert not O.should_reuse(511, 512) and O.should_reuse(512, 512)
    ids = list(range(200))
    assert O.reuse_request(1, 2048, 512, ids, ids) is None
    r = O.reuse_request(2, 2048, 512, ids, ids)
    assert r is not None and r.num_tokens == 2048
    assert O.reuse_request(2, 511, 512, ids, ids) is None
    assert O.reuse_request(2, 512, 512, ids, ids).num_tokens == 512
    assert O.reuse_request(3, 300, 512, ids, ids).num_tokens == 600


def pin_pack_unpack(O):
    """unpack(pack(x)) == push(x); staging size = layers x 2 x (tokens x token
    bytes + scales padded to 16 B); for NHD the payload of a region is the
    moved tokens' rows in request order."""
    for wl in list(random_cases(16, seed0=21)):
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        g = src.geom
        L = g.num_layers
        stg = O.pack(src, plan, 0, L)
        ntok = sum(r.num_tokens for r in reqs)
        nblk = sum(-(-r.num_tokens // g.block_size) for r in reqs)
        sc = ((4 * nblk + 15) // 16 * 16) if g.has_scales else 0
        assert stg.size == L * 2 * (ntok * g.token_bytes + sc)
        if g.has_scales:
            reg = ntok * g.token_bytes + sc
            for i in range(L * 2):
                assert not stg[i * reg + ntok * g.token_bytes + 4 * nblk:(i + 1) * reg].any()
        a, b = dst.copy(), dst.copy()
        O.unpack(stg, a, plan, 0, L)
        O.push(src, b, plan)
        assert np.array_equal(a.kv, b.kv)
        if a.scales is not None:
            assert np.array_equal(a.scales, b.scales)
        if g.layout == "NHD":
            rows = []
            for req in reqs:
                for p in range(req.num_tokens):
                    j, s = divmod(p, g.block_size)
                    o = int(req.src_ids[j]) * g.block_size * g.token_bytes + s * g.token_bytes
                    rows.append(src.kv[0, 0, o:o + g.token_bytes])
            exp = np.concatenate(rows) if rows else np.zeros(0, np.uint8)
            assert np.array_equal(stg[:exp.size], exp)
            if g.has_scales:
                pairs = []
                for req in reqs:
                    pairs += [int(x) for x in req.src_ids[:-(-req.num_tokens // g.block_size)]]
                got = stg[exp.size:exp.size + 4 * len(pairs)].view(np.uint32)
                assert np.array_equal(got, src.scales[0, 0, pairs])
                assert not stg[exp.size + 4 * len(pairs):exp.size + sc].any()
        # sub-range of layers
        if L > 1:
            s1 = O.pack(src, plan, 1, L)
            assert np.array_equal(s1, stg[stg.size // L:])


def pin_copy_heads(O):
    """Head-slice transform: all heads in the same layout equals push; NHD ->
    HND -> NHD is the identity on moved rows; the union of the four TP4 shares
    equals one full-head NHD -> HND copy; the per-region gather equals the
    plain per-row definition."""
    for i, wl in enumerate(random_cases(10, seed0=31)):
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        g = src.geom
        plan = O.make_plan(src.geom, dst.geom, reqs)
        a, b, c = dst.copy(), dst.copy(), dst.copy()
        for l in range(g.num_layers):
            O.copy_heads(src, a, plan, reqs, l, 0, 0, g.num_heads)
        O.push(src, b, plan)
        O.copy_heads_plain(src, c, reqs, 0, 0, g.num_heads)
        assert np.array_equal(a.kv, b.kv) and np.array_equal(a.kv, c.kv)
    # round trip and TP shares
    H = 8
    nhd = W.PoolSpec(1, 24, 4, H, 4, W.BF16, "NHD")
    hnd = W.PoolSpec(1, 24, 4, H, 4, W.BF16, "HND")
    rng = np.random.Generator(np.random.PCG64(77))
    st = rng.permutation(24)[:6].astype(np.int32)
    dt = rng.permutation(24)[:6].astype(np.int32)
    wl = W.Workload("rt", 4, nhd, hnd, [23], [st], [dt])
    src, dst = pools(O, wl)
    reqs = requests_for(O, wl)
    plan = O.make_plan(src.geom, dst.geom, reqs)
    full = dst.copy()
    O.copy_heads(src, full, plan, reqs, 0, 0, 0, H)
    shares = dst.copy()
    for r in range(4):
        O.copy_heads(src, shares, plan, reqs, 0, 2 * r, 2 * r, 2)
    assert np.array_equal(full.kv, shares.kv)
    back = O.Pool(src.geom, np.zeros_like(src.kv), None)
    rev = [O.Request(q.num_tokens, q.dst_ids, q.src_ids) for q in reqs]
    plan_b = O.make_plan(dst.geom, src.geom, rev)
    O.copy_heads(full, back, plan_b, rev, 0, 0, 0, H)
    mask = np.zeros(src.geom.region_bytes, bool)
    for p in range(22):
        j, s = divmod(p, 4)
        o = int(st[j]) * src.geom.block_bytes + s * src.geom.token_bytes
        mask[o:o + src.geom.token_bytes] = True
    for kv in range(2):
        assert np.array_equal(back.kv[0, kv][mask], src.kv[0, kv][mask])
        assert not back.kv[0, kv][~mask].any()


def pin_errors(O):
    """Error classes: negative counts and short lists are argument errors,
    IDs outside the pool are range errors, a destination used twice is an
    error, geometry differences are mismatches."""
    g = O.Geometry(1, 8, 4, 1, 4, 2, "NHD")

    def kind(reqs, gd=g):
        try:
            O.make_plan(g, gd, reqs)
        except O.OracleError as e:
            return e.kind
        return "OK"

    assert kind([O.Request(-1, [0], [0])]) == "INVAL"
    assert kind([O.Request(5, [0], [0, 1])]) == "INVAL"
    assert kind([O.Request(4, [8], [0])]) == "RANGE"
    assert kind([O.Request(4, [0], [-1])]) == "RANGE"
    assert kind([O.Request(4, [0], [3]), O.Request(4, [1], [3])]) == "DUPDST"
    assert kind([O.Request(4, [0], [3]), O.Request(4, [0], [4])]) == "OK"  # shared source
    assert kind([O.Request(4, [0, 99], [3, 3])]) == "OK"  # ids past the used blocks ignored
    assert kind([O.Request(0, [], [])]) == "OK"
    src = O.Pool.zeros(g)
    dst = O.Pool.zeros(O.Geometry(1, 8, 4, 2, 4, 2, "NHD"))
    try:
        O.push(src, dst, O.make_plan(g, dst.geom, [O.Request(4, [0], [0])]))
        raise AssertionError("mismatch accepted")
    except O.OracleError as e:
        assert e.kind == "MISMATCH"


def reblock_cases(count=30, seed0=41):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        bs, bsd = [int(x) for x in rng.choice([1, 2, 3, 4, 8, 16], size=2, replace=False)]
        yield W.random_case(
            3000 + seed0 + i, layout=["NHD", "HND"][i % 2], elem_bytes=int(rng.choice([1, 2])),
            num_layers=int(rng.integers(1, 3)), num_blocks=160, block_size=bs, dst_block_size=bsd,
            num_heads=int(rng.integers(1, 4)), head_dim=int(rng.choice([4, 8])),
            num_requests=int(rng.integers(1, 4)), max_tokens=40, run_mean=float(rng.choice([1.5, 4.0])),
            extra_ids=int(rng.integers(0, 2)))


def pin_reblock_brute_vs_procedure(O):
    """Different block sizes per side: the plain per-token definition equals
    the token-segment procedure, byte for byte; pack/unpack round-trips."""
    for wl in reblock_cases():
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        a, b, c = dst.copy(), dst.copy(), dst.copy()
        O.push_plain(src, a, reqs)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        O.push(src, b, plan)
        assert np.array_equal(a.kv, b.kv), wl.name
        L = src.geom.num_layers
        O.unpack(O.pack(src, plan, 0, L), c, plan, 0, L)
        assert np.array_equal(c.kv, b.kv), wl.name
        assert plan.payload_bytes == sum(r.num_tokens for r in reqs) * src.geom.token_bytes


def pin_reblock_equal_sizes_agree(O):
    """With equal block sizes the token-segment procedure gives exactly the
    run-based triple list."""
    for wl in random_cases(24, seed0=51):
        g = geom(O, wl.src)
        reqs = requests_for(O, wl)
        runs = O.plan_runs(reqs, g.block_size, g.num_blocks, wl.dst.num_blocks)
        segs = O.token_segments(reqs, g.block_size, g.block_size)
        assert O.triples_reblock(segs, g, g) == O.triples(runs, g), wl.name


def pin_reblock_torch_pairs(O):
    """NHD, destination blocks twice the source size, each destination block
    filled by two source blocks: equals torch index_select of source block
    pairs viewed as one destination block."""
    src_spec = W.PoolSpec(2, 40, 4, 2, 8, W.BF16)
    dst_spec = W.PoolSpec(2, 30, 8, 2, 8, W.BF16)
    rng = np.random.Generator(np.random.PCG64(9))
    st = rng.permutation(40)[:12].astype(np.int32)
    dt = rng.permutation(30)[:6].astype(np.int32)
    wl = W.Workload("pairs", 21, src_spec, dst_spec, [48], [st], [dt])
    src, dst = pools(O, wl)
    got = dst.copy()
    reqs = requests_for(O, wl, [48])
    O.push(src, got, O.make_plan(src.geom, dst.geom, reqs))
    exp = torch.from_numpy(dst.kv.copy())
    s = torch.from_numpy(src.kv)
    for l in range(2):
        for kv in range(2):
            blk = s[l, kv].view(40, -1).index_select(0, torch.from_numpy(st.astype(np.int64)))
            exp[l, kv].view(30, -1).index_copy_(0, torch.from_numpy(dt.astype(np.int64)), blk.reshape(6, -1))
    assert np.array_equal(got.kv, exp.numpy())


def pin_reblock_round_trip(O):
    """16-slot blocks -> 6-slot blocks -> 16-slot blocks restores every moved
    token row, both layouts."""
    for layout in ("NHD", "HND"):
        a_spec = W.PoolSpec(1, 20, 16, 2, 8, W.U8, layout)
        b_spec = W.PoolSpec(1, 60, 6, 2, 8, W.U8, layout)
        rng = np.random.Generator(np.random.PCG64(33))
        n = 70
        at = rng.permutation(20)[:5].astype(np.int32)
        bt = rng.permutation(60)[:12].astype(np.int32)
        wl = W.Workload("rt", 5, a_spec, b_spec, [n + 1], [at], [bt])
        a, b = pools(O, wl)
        reqs = [O.Request(n, at, bt)]
        O.push(a, b, O.make_plan(a.geom, b.geom, reqs))
        back = O.Pool(a.geom, np.zeros_like(a.kv), None)
        rev = [O.Request(n, bt, at)]
        O.push(b, back, O.make_plan(b.geom, a.geom, rev))
        g = a.geom
        for p in range(n):
            j, sl = divmod(p, 16)
            for h in range(2):
                o = g.row_offset(int(at[j]), sl, h)
                assert np.array_equal(back.kv[0, :, o:o + g.row_bytes], a.kv[0, :, o:o + g.row_bytes])


def pin_reblock_errors(O):
    """Scales need equal block sizes; each side's list must cover its own
    block count."""
    gs = O.Geometry(1, 8, 4, 1, 4, 1, "NHD", True)
    gd = O.Geometry(1, 8, 8, 1, 4, 1, "NHD", True)
    try:
        O.make_plan(gs, gd, [O.Request(8, [0, 1], [2])])
        raise AssertionError("scales with different block sizes accepted")
    except O.OracleError as e:
        assert e.kind == "UNSUPPORTED"
    gs = O.Geometry(1, 8, 4, 1, 4, 1, "NHD")
    gd = O.Geometry(1, 8, 8, 1, 4, 1, "NHD")
    assert len(O.make_plan(gs, gd, [O.Request(8, [0, 1], [2])]).triples) >= 1
    for bad in ([O.Request(9, [0, 1], [2, 3])], [O.Request(9, [0, 1, 2], [2])]):
        try:
            O.make_plan(gs, gd, bad)
            raise AssertionError("short list accepted")
        except O.OracleError as e:
            assert e.kind == "INVAL"


# ---------------------------------------------------------------------------
# layer groups of other shapes: one latent region (MLA), sliding window,
# state slots
# ---------------------------------------------------------------------------
def latent_cases(count=24, seed0=61):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        bs = int(rng.choice([1, 2, 4, 16]))
        yield W.random_case(
            4000 + i, layout=["NHD", "HND"][i % 2], elem_bytes=int(rng.choice([1, 2])),
            num_layers=int(rng.integers(1, 3)), num_blocks=int(max(48, 8 * bs)), block_size=bs, num_heads=1,
            head_dim=int(rng.choice([16, 32, 48])), has_scales=bool(i % 3 == 0),
            num_requests=int(rng.integers(1, 4)), max_tokens=int(min(5 * bs, 40)),
            run_mean=float(rng.choice([1.5, 4.0])), regions=1)


def pin_latent_region(O):
    """A pool of one latent region per layer (MLA) moves exactly what region
    0 of a K/V pool holding the same bytes would; with block size 1 every
    token is a block and the move is torch index_select -> index_copy_ of
    token rows; staging holds one region per layer."""
    for wl in latent_cases():
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        a, b = dst.copy(), dst.copy()
        O.push_plain(src, a, reqs)
        O.push(src, b, plan)
        assert np.array_equal(a.kv, b.kv), wl.name
        # the same bytes as region 0 of a two-region pool
        g2s = O.Geometry(*[getattr(src.geom, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                           "head_dim", "elem_bytes", "layout", "has_scales")])
        g2d = O.Geometry(*[getattr(dst.geom, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                           "head_dim", "elem_bytes", "layout", "has_scales")])
        rng = np.random.Generator(np.random.PCG64(wl.seed))
        s2 = O.Pool(g2s, np.concatenate([src.kv, rng.integers(0, 256, src.kv.shape, dtype=np.uint8)], 1),
                    None if src.scales is None else np.concatenate([src.scales, src.scales], 1))
        d2 = O.Pool(g2d, np.concatenate([dst.kv, dst.kv], 1),
                    None if dst.scales is None else np.concatenate([dst.scales, dst.scales], 1))
        O.push(s2, d2, O.make_plan(g2s, g2d, reqs))
        assert np.array_equal(d2.kv[:, :1], b.kv), wl.name
        if b.scales is not None:
            assert np.array_equal(d2.scales[:, :1], b.scales), wl.name
        L = src.geom.num_layers
        stg = O.pack(src, plan, 0, L)
        sc = -(-4 * len(plan.pairs) // 16) * 16 if src.scales is not None else 0
        assert stg.size == O.staging_bytes(plan, 0, L) == L * (plan.payload_bytes + sc)
        c = dst.copy()
        O.unpack(stg, c, plan, 0, L)
        assert np.array_equal(c.kv, b.kv), wl.name
        if wl.src.block_size == 1:
            nb = wl.src.num_blocks
            exp = torch.from_numpy(dst.kv.copy())
            s = torch.from_numpy(src.kv)
            sid = torch.from_numpy(np.concatenate([t[:q.num_tokens] for t, q in zip(wl.src_tables, reqs)]
                                                  ).astype(np.int64))
            did = torch.from_numpy(np.concatenate([t[:q.num_tokens] for t, q in zip(wl.dst_tables, reqs)]
                                                  ).astype(np.int64))
            for l in range(L):
                exp[l, 0].view(nb, -1).index_copy_(0, did, s[l, 0].view(nb, -1).index_select(0, sid))
            assert np.array_equal(b.kv, exp.numpy()), wl.name


def window_cases(count=40, seed0=71):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        mixed = i % 3 == 2
        bs = int(rng.choice([1, 2, 3, 4, 8]))
        bsd = int(rng.choice([x for x in (1, 2, 3, 4, 8) if x != bs])) if mixed else bs
        w = int(rng.choice([1, 2, 3, bs, bs + 1, 2 * bs + 1, 7, 64]))
        yield W.random_case(
            5000 + i, layout=["NHD", "HND"][i % 2], elem_bytes=1, num_layers=1, num_blocks=120,
            block_size=bs, dst_block_size=bsd, num_heads=int(rng.integers(1, 3)), head_dim=16,
            has_scales=bool(i % 4 == 0 and not mixed), num_requests=int(rng.integers(1, 4)), max_tokens=30,
            run_mean=float(rng.choice([1.5, 4.0])), window=w)


def _attended(n, w):
    """Positions the query at position n sees under a sliding window of w
    positions: row n of torch's banded causal mask."""
    m = torch.ones(n + 1, n + 1, dtype=torch.bool).tril().triu(-(w - 1))
    return set(int(k) for k in torch.nonzero(m[n]).flatten())


def pin_window_mask(O):
    """Sliding window, checked against the band mask: every key position the
    receiving side's next query (at position n) sees arrives; no block that
    holds none of the positions that query sees (its own included) is read or
    written; with equal block sizes each kept block moves whole; table
    entries of dropped blocks are neither read nor validated; a window of at
    least n + 1 positions moves what full attention moves."""
    for wl in window_cases():
        src, dst = pools(O, wl)
        reqs = requests_for(O, wl)
        a, b = dst.copy(), dst.copy()
        O.push_plain(src, a, reqs)
        plan = O.make_plan(src.geom, dst.geom, reqs)
        O.push(src, b, plan)
        assert np.array_equal(a.kv, b.kv), wl.name
        gs, gd = src.geom, dst.geom
        w, bss, bsd = gs.window, gs.block_size, gd.block_size
        for q in reqs:
            n = q.num_tokens
            seen = _attended(n, w)
            for p in range(n):
                for h in range(gs.num_heads):
                    so = gs.row_offset(int(q.src_ids[p // bss]), p % bss, h)
                    do = gd.row_offset(int(q.dst_ids[p // bsd]), p % bsd, h)
                    same = np.array_equal(b.kv[:, :, do:do + gs.row_bytes], src.kv[:, :, so:so + gs.row_bytes])
                    if p in seen:
                        assert same, (wl.name, "a seen position did not arrive", p)
                    kept_s = any(k // bss == p // bss for k in seen)
                    kept_d = any(k // bsd == p // bsd for k in seen)
                    if bss == bsd and kept_s:
                        assert same, (wl.name, "a kept block did not move whole", p)
                    if not kept_d:
                        changed = not np.array_equal(b.kv[:, :, do:do + gs.row_bytes],
                                                     dst.kv[:, :, do:do + gs.row_bytes])
                        assert not changed, (wl.name, "a dropped destination block was written", p)
        # dropped entries: poison them; nothing may read or validate them
        poisoned = []
        for q in reqs:
            n = q.num_tokens
            seen = _attended(n, w)
            s_ids = np.array(q.src_ids, np.int64)
            d_ids = np.array(q.dst_ids, np.int64)
            for j in range(O.blocks_in_use(n, bss)):
                if not any(k // bss == j for k in seen):
                    s_ids[j] = -1
            for j in range(O.blocks_in_use(n, bsd)):
                if not any(k // bsd == j for k in seen):
                    d_ids[j] = -1
            poisoned.append(O.Request(n, s_ids, d_ids))
        c = dst.copy()
        O.push(src, c, O.make_plan(gs, gd, poisoned))
        assert np.array_equal(c.kv, b.kv), wl.name
        if b.scales is not None:
            assert np.array_equal(c.scales, b.scales), wl.name
        # a window covering everything is full attention
        full = [O.Request(q.num_tokens, q.src_ids, q.dst_ids) for q in reqs]
        wide = max(q.num_tokens for q in reqs) + 1
        gsw = O.Geometry(*[getattr(gs, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                     "head_dim", "elem_bytes", "layout", "has_scales",
                                                     "regions")], wide)
        gdw = O.Geometry(*[getattr(gd, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                     "head_dim", "elem_bytes", "layout", "has_scales",
                                                     "regions")], wide)
        g0s = O.Geometry(*[getattr(gs, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                     "head_dim", "elem_bytes", "layout", "has_scales")])
        g0d = O.Geometry(*[getattr(gd, f) for f in ("num_layers", "num_blocks", "block_size", "num_heads",
                                                     "head_dim", "elem_bytes", "layout", "has_scales")])
        x, y = dst.copy(), dst.copy()
        O.push(O.Pool(gsw, src.kv, src.scales), O.Pool(gdw, x.kv, x.scales), O.make_plan(gsw, gdw, full))
        O.push(O.Pool(g0s, src.kv, src.scales), O.Pool(g0d, y.kv, y.scales), O.make_plan(g0s, g0d, full))
        assert np.array_equal(x.kv, y.kv), wl.name


def pin_window_closed_form(O):
    """Worked by hand: an 8192-token prompt (8191 tokens move) under a
    128-position window with 16-slot blocks keeps positions 8064..8190 of the
    moved range, i.e. blocks 504..511 (127 tokens); a window of one position
    moves only the tokens sharing position n's block."""
    g = O.Geometry(1, 600, 16, 8, 64, 2, "NHD", False, 2, 128)
    ids = list(range(512))
    plan = O.make_plan(g, g, [O.Request(8191, ids, ids)])
    assert plan.runs == [O.Run(504, 504, 8, 15)]
    assert plan.payload_bytes == 127 * 8 * 64 * 2
    assert plan.bytes_per_layer() == (2 * 127 * 1024, 2 * 127 * 1024)
    g1 = O.Geometry(1, 20, 8, 1, 16, 1, "NHD", False, 2, 1)
    assert O.make_plan(g1, g1, [O.Request(40, list(range(5)), list(range(5)))]).payload_bytes == 0
    assert O.make_plan(g1, g1, [O.Request(43, list(range(6)), list(range(6)))]).payload_bytes == 3 * 16


def state_cases(count=30, seed0=81):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        yield W.random_state_case(6000 + i, num_layers=int(rng.integers(1, 3)), num_slots=40,
                                  slot_bytes=(int(rng.choice([16, 48, 96])), int(rng.choice([32, 160, 256]))),
                                  num_requests=int(rng.integers(1, 9)), max_tokens=int(rng.choice([3, 20])),
                                  extra_ids=int(rng.integers(0, 2)))


def _state_pools(O, wl):
    gs, gd = state_geom(O, wl.src), state_geom(O, wl.dst)
    return (O.StatePool(gs, W.state_host_values(wl.src, wl.seed, 1)),
            O.StatePool(gd, W.state_host_values(wl.dst, wl.seed, 2)))


def pin_state_slots(O):
    """State slots: the procedure equals the plain slot copy and torch
    index_select -> index_copy_ on the slot dimension of each region (rows of
    that region's slot size) for the requests that move tokens; requests that
    move none leave their destination slot untouched; the triple list is the
    unique maximal merge; pack/unpack round-trips."""
    for wl in state_cases():
        src, dst = _state_pools(O, wl)
        reqs = requests_for(O, wl, wl.prompt_lens)
        plan = O.make_state_plan(src.geom, dst.geom, reqs)
        a, b = dst.copy(), dst.copy()
        O.push_state_plain(src, a, reqs)
        O.push_state(src, b, plan)
        for r in range(2):
            assert np.array_equal(a.regions[r], b.regions[r]), wl.name
        mv = [q for q in reqs if q.num_tokens > 0]
        sid = torch.tensor([int(q.src_ids[0]) for q in mv], dtype=torch.int64)
        did = torch.tensor([int(q.dst_ids[0]) for q in mv], dtype=torch.int64)
        for r in range(2):
            sb = wl.src.slot_bytes[r]
            exp = torch.from_numpy(dst.regions[r].copy())
            s = torch.from_numpy(src.regions[r])
            for l in range(wl.src.num_layers):
                exp[l].view(-1, sb).index_copy_(0, did, s[l].view(-1, sb).index_select(0, sid))
            assert np.array_equal(b.regions[r], exp.numpy()), wl.name
            tr = plan.triples[r]
            assert sum(t[2] for t in tr) == len(mv) * sb
            for x, y in zip(tr, tr[1:]):
                assert not (x[0] + x[2] == y[0] and x[1] + x[2] == y[1]), "not maximal"
        L = wl.src.num_layers
        stg = O.pack_state(src, plan, 0, L)
        assert stg.size == O.state_staging_bytes(plan, 0, L) == L * len(mv) * sum(wl.src.slot_bytes)
        c = dst.copy()
        O.unpack_state(stg, c, plan, 0, L)
        for r in range(2):
            assert np.array_equal(c.regions[r], b.regions[r]), wl.name


def pin_state_closed_form_and_errors(O):
    """Worked by hand: sixteen requests with 48 KiB + 1 MiB slots move
    16 * 1,097,728 = 17,563,648 bytes per layer; slots 3, 4, 5 -> 10, 11, 12
    merge into one range per region and 9 -> 20 stays apart.  Errors: a
    destination slot used twice, a slot outside the pool, a moving request
    without a slot, different slot sizes."""
    g = O.StateGeometry(1, 64, (49152, 1048576))
    reqs = [O.Request(8191, [i], [63 - i]) for i in range(16)]
    assert O.make_state_plan(g, g, reqs).bytes_per_layer() == (17563648, 17563648)
    g2 = O.StateGeometry(1, 32, (16, 48))
    p = O.make_state_plan(g2, g2, [O.Request(5, [3], [10]), O.Request(1, [4], [11]), O.Request(2, [5], [12]),
                                   O.Request(0, [7], [13]), O.Request(9, [9], [20])])
    assert p.triples[0] == [(48, 160, 48), (144, 320, 16)]
    assert p.triples[1] == [(144, 480, 144), (432, 960, 48)]
    for bad, kind in (([O.Request(1, [0], [5]), O.Request(1, [1], [5])], "DUPDST"),
                      ([O.Request(1, [32], [0])], "RANGE"), ([O.Request(1, [0], [-1])], "RANGE"),
                      ([O.Request(1, [], [0])], "INVAL"), ([O.Request(-1, [0], [0])], "INVAL")):
        try:
            O.make_state_plan(g2, g2, bad)
            raise AssertionError(f"accepted {kind}")
        except O.OracleError as e:
            assert e.kind == kind, (e.kind, kind)
    assert O.make_state_plan(g2, g2, [O.Request(0, [], [])]).triples == ([], [])
    try:
        O.make_state_plan(g2, O.StateGeometry(1, 32, (16, 64)), [])
        raise AssertionError("slot sizes differ")
    except O.OracleError as e:
        assert e.kind == "MISMATCH"


def pin_group_mismatch(O):
    """Pools of one transfer agree on their region count and window."""
    a = O.Geometry(1, 8, 4, 1, 16, 1, "NHD", False, 2, 0)
    for other in (O.Geometry(1, 8, 4, 1, 16, 1, "NHD", False, 1, 0),
                  O.Geometry(1, 8, 4, 1, 16, 1, "NHD", False, 2, 8)):
        try:
            O.make_plan(a, other, [])
            raise AssertionError("mismatch accepted")
        except O.OracleError as e:
            assert e.kind == "MISMATCH"


ALL_PINS = [pin_brute_vs_procedure, pin_full_blocks_index_copy, pin_single_run_slice,
            pin_nhd_to_hnd_permute, pin_final_token_never_sent, pin_untouched_bytes,
            pin_plan_invariants, pin_closed_forms, pin_threshold, pin_pack_unpack,
            pin_copy_heads, pin_errors, pin_reblock_brute_vs_procedure, pin_reblock_equal_sizes_agree,
            pin_reblock_torch_pairs, pin_reblock_round_trip, pin_reblock_errors,
            pin_latent_region, pin_window_mask, pin_window_closed_form, pin_state_slots,
            pin_state_closed_form_and_errors, pin_group_mismatch]
