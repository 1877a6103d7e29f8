"""Planted mistakes in a private copy of the CPU oracle must each fail a pin.

This shows that the pins in oracle_pins.py are strong enough to catch the
plausible mistakes one could make writing the oracle (a dropped term, a wrong
index, a swapped operand, an off-by-one).  The mistakes live only in a fresh
module object loaded for this test; the real oracle is untouched.
"""
import importlib.util
import itertools
import os
import sys

import numpy as np
import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


_COUNTER = itertools.count()


def fresh_oracle():
    name = f"kv_oracle_mut{next(_COUNTER)}"
    spec = importlib.util.spec_from_file_location(name, os.path.join(ROOT, "oracle", "kv_oracle.py"))
    m = importlib.util.module_from_spec(spec)
    sys.modules[name] = m  # dataclasses look their module up here
    spec.loader.exec_module(m)
    return m


def m_no_minus_one(O):
    O.tokens_to_move = lambda prompt_len, num_computed=0: max(0, prompt_len - num_computed)


def m_minus_two(O):
    O.tokens_to_move = lambda prompt_len, num_computed=0: max(0, prompt_len - num_computed - 2)


def m_merge_src_only(O):
    orig = O.plan_runs

    def plan_runs(requests, bs, nsrc, ndst):
        O.validate(requests, bs, nsrc, ndst)
        runs = []
        for req in requests:
            nb = O.blocks_in_use(req.num_tokens, bs)
            if not nb:
                continue
            tail = O.last_block_fill(req.num_tokens, bs)
            start = 0
            for i in range(1, nb + 1):
                if i == nb or int(req.src_ids[i]) != int(req.src_ids[i - 1]) + 1:
                    runs.append(O.Run(int(req.src_ids[start]), int(req.dst_ids[start]), i - start,
                                      tail if i == nb else bs))
                    start = i
        return runs
    O.plan_runs = plan_runs
    return orig


def m_hnd_swap(O):
    def row_offset(self, block, slot, head):
        if self.layout == O.NHD:
            return block * self.block_bytes + slot * self.token_bytes + head * self.row_bytes
        return block * self.block_bytes + slot * self.num_heads * self.row_bytes + head * self.row_bytes
    O.Geometry.row_offset = row_offset
    orig_ri = O._row_index

    def _row_index(g, b, s, h):
        if g.layout == O.NHD:
            return orig_ri(g, b, s, h)
        return (b * g.block_size + s) * g.num_heads + h
    O._row_index = _row_index


def m_tail_ignored(O):
    O.last_block_fill = lambda n, bs: bs if n else 0


def m_tail_off_by_one(O):
    O.last_block_fill = lambda n, bs: (n - (O.blocks_in_use(n, bs) - 1) * bs - 1) if n else 0


def m_coalesce_src_only(O):
    segs = O._segments

    def triples(runs, g):
        out = []
        for so, do, ln in segs(runs, g):
            if out and out[-1][0] + out[-1][2] == so:
                out[-1][2] += ln
            else:
                out.append([so, do, ln])
        return [tuple(t) for t in out]
    O.triples = triples


def m_scale_swap(O):
    def push_scales(src_sc, dst_sc, pairs):
        for sb, db in pairs:
            dst_sc[sb] = src_sc[db]
    O.push_scales = push_scales


def m_reuse_strict(O):
    O.should_reuse = lambda r, threshold=64: r > threshold


def m_reuse_turn(O):
    O.reusable_prefix = lambda turn, growth: growth * turn


def m_nhd_row_swap(O):
    orig = O._row_index

    def _row_index(g, b, s, h):
        if g.layout == O.NHD:
            return (b * g.num_heads + h) * g.block_size + s
        return orig(g, b, s, h)
    O._row_index = _row_index


def m_pack_kv_order(O):
    orig = O.pack

    def pack(src, plan, l0, l1):
        sw = O.Pool(src.geom, src.kv[:, ::-1].copy(), None if src.scales is None else src.scales[:, ::-1].copy())
        return orig(sw, plan, l0, l1)
    O.pack = pack


def m_scale_pad_garbage(O):
    orig = O.pack

    def pack(src, plan, l0, l1):
        out = orig(src, plan, l0, l1)
        if src.scales is not None:
            out[-1] ^= 0xFF if (4 * len(plan.pairs)) % 16 else 0
        return out
    O.pack = pack


def m_hnd_tail_one_segment(O):
    def _segments(runs, g):
        bb, tb = g.block_bytes, g.token_bytes
        return [(r.src0 * bb, r.dst0 * bb, (r.nblk - 1) * bb + r.tail * tb) for r in runs]
    O._segments = _segments


def m_dupdst_allowed(O):
    orig = O.validate

    def validate(requests, bs, nsrc, ndst, *args, **kw):
        try:
            orig(requests, bs, nsrc, ndst, *args, **kw)
        except O.OracleError as e:
            if e.kind != "DUPDST":
                raise
    O.validate = validate


def m_reblock_dst_uses_src_size(O):
    orig = O.token_segments
    O.token_segments = lambda requests, bs_src, bs_dst, window=0: orig(requests, bs_src, bs_src, window)


def m_reblock_no_split(O):
    O._split_in_blocks = lambda seg, bs_src, bs_dst: iter([(seg.src_block, seg.src_slot, seg.dst_block,
                                                           seg.dst_slot, seg.ntok)])


def m_window_off_by_one(O):
    def window_start(n, w, bss, bsd):
        if w <= 0:
            return 0
        first = max(0, n - w)
        return max(first // bss * bss, first // bsd * bsd)
    O.window_start = window_start


def m_window_token_granular(O):
    O.window_start = lambda n, w, bss, bsd: max(0, n - w + 1) if w > 0 else 0


def m_window_ignored(O):
    O.window_start = lambda n, w, bss, bsd: 0


def m_window_src_blocks_only(O):
    O.window_start = lambda n, w, bss, bsd: (max(0, n - w + 1) // bss * bss) if w > 0 else 0


def m_latent_staging_two_regions(O):
    O.staging_bytes = lambda plan, l0, l1: (l1 - l0) * 2 * O.staging_region_bytes(plan)


def m_state_moves_empty(O):
    orig = O.make_state_plan

    def make_state_plan(gs, gd, requests):
        return orig(gs, gd, [O.Request(max(q.num_tokens, 1) if len(q.src_ids) and len(q.dst_ids) else 0,
                                       q.src_ids, q.dst_ids) for q in requests])
    O.make_state_plan = make_state_plan


def m_state_one_slot_size(O):
    orig = O.make_state_plan

    def make_state_plan(gs, gd, requests):
        p = orig(gs, gd, requests)
        sb0, sb1 = gs.slot_bytes
        t1 = [(so // sb1 * sb0, do // sb1 * sb0, ln // sb1 * sb0) for so, do, ln in p.triples[1]]
        return O.StatePlan(gs, gd, p.runs, (p.triples[0], t1))
    O.make_state_plan = make_state_plan


def m_state_merge_src_only(O):
    orig = O.make_state_plan

    def make_state_plan(gs, gd, requests):
        p = orig(gs, gd, requests)
        lists = []
        for r in range(2):
            sb = gs.slot_bytes[r]
            out = []
            for run in p.runs:
                so, do = run.src0 * sb, run.dst0 * sb
                if out and out[-1][0] + out[-1][2] == so:
                    out[-1][2] += sb
                else:
                    out.append([so, do, sb])
            lists.append([tuple(t) for t in out])
        return O.StatePlan(gs, gd, p.runs, (lists[0], lists[1]))
    O.make_state_plan = make_state_plan


MUTATIONS = [m_no_minus_one, m_minus_two, m_merge_src_only, m_hnd_swap, m_tail_ignored,
             m_tail_off_by_one, m_coalesce_src_only, m_scale_swap, m_reuse_strict, m_reuse_turn,
             m_nhd_row_swap, m_pack_kv_order, m_scale_pad_garbage, m_hnd_tail_one_segment,
             m_dupdst_allowed, m_reblock_dst_uses_src_size, m_reblock_no_split,
             m_window_off_by_one, m_window_token_granular, m_window_ignored, m_window_src_blocks_only,
             m_latent_staging_two_regions, m_state_moves_empty, m_state_one_slot_size,
             m_state_merge_src_only]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutation):
    O = fresh_oracle()
    mutation(O)
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(O)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught {mutation.__name__}"
