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

    def validate(requests, bs, nsrc, ndst):
        try:
            orig(requests, bs, nsrc, ndst)
        except O.OracleError as e:
            if e.kind != "DUPDST":
                raise
    O.validate = validate


def m_reblock_dst_uses_src_size(O):
    orig = O.token_segments
    O.token_segments = lambda requests, bs_src, bs_dst: orig(requests, bs_src, bs_src)


def m_reblock_no_split(O):
    O._split_in_blocks = lambda seg, bs_src, bs_dst: iter([(seg.src_block, seg.src_slot, seg.dst_block,
                                                           seg.dst_slot, seg.ntok)])


MUTATIONS = [m_no_minus_one, m_minus_two, m_merge_src_only, m_hnd_swap, m_tail_ignored,
             m_tail_off_by_one, m_coalesce_src_only, m_scale_swap, m_reuse_strict, m_reuse_turn,
             m_nhd_row_swap, m_pack_kv_order, m_scale_pad_garbage, m_hnd_tail_one_segment,
             m_dupdst_allowed, m_reblock_dst_uses_src_size, m_reblock_no_split]


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
