"""CPU oracle for paged-KV block transfer between a producer pool and a consumer pool.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
oracle leg of ``bench.py`` (the verification step before timing, and the
``cpu_baseline``) use it.  It shares no code with the HIP
library (``decode_kv_cache_amd``) and imports nothing from it.

Sources (the pages this follows):
  [PUSH]  "Push-based KV transfer for vLLM prefill/decode disaggregation with
          NIXL" (AWS blog, German translation, www.spke.com/de/ai/article/3844)
  [MORI]  "vLLM MoRIIO KV Connector (single-node PD disaggregation)"
          (donggyun112.github.io knowledge-base note)
  [BIDIR] "Bidirectional KV-cache transfer for multi-turn workloads"
          (AWS blog, German translation, www.spke.com/de/ai/article/3845)

Everything here is a byte copy: no floating-point arithmetic happens, so the
oracle works on ``numpy.uint8`` views of the KV regions and ``numpy.uint32``
views of the fp32 per-block scales (bits are moved, never interpreted).

Two independent formulations are given and must agree byte for byte:
  * the plain definition (``push_plain``, ``copy_heads_plain``): every
    (token, head) row of every moved token goes from its source block/slot to
    its destination block/slot;
  * the pages' procedure (``plan_runs`` -> ``triples`` -> ``push``/``pack``/
    ``unpack``): contiguous blocks are merged into runs, runs are expanded into
    (source offset, destination offset, length) triples per layer, and the
    triples are copied.

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force on tiny inputs, library special cases in torch, closed forms and
invariants); none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

NHD = "NHD"  # block-major, then slot (token), then head, then dim
HND = "HND"  # block-major, then head, then slot (token), then dim

K, V = 0, 1


class OracleError(Exception):
    """Invalid request.  ``kind`` is one of INVAL, RANGE, DUPDST, MISMATCH, UNSUPPORTED."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


# ---------------------------------------------------------------------------
# Geometry.  [MORI] §3 (handshake metadata: base address, block size, per-layer
# strides) and §6 (per-layer KV tensors registered with the engine); [PUSH]
# "Implementierungsdetails" step 3 (each side maps block positions onto its
# own physical layout).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    num_layers: int
    num_blocks: int
    block_size: int
    num_heads: int
    head_dim: int
    elem_bytes: int
    layout: str = NHD
    has_scales: bool = False
    regions: int = 2      # 2: K and V; 1: one latent region (MLA)
    window: int = 0       # 0: full attention; W > 0: sliding window of W positions

    @property
    def row_bytes(self) -> int:
        """Bytes of one (token, head) row: head_dim elements."""
        return self.head_dim * self.elem_bytes

    @property
    def token_bytes(self) -> int:
        """Bytes of one token in one (layer, K or V) region: all heads."""
        return self.num_heads * self.row_bytes

    @property
    def block_bytes(self) -> int:
        return self.block_size * self.token_bytes

    @property
    def region_bytes(self) -> int:
        """Bytes of one (layer, K or V) region."""
        return self.num_blocks * self.block_bytes

    def row_offset(self, block: int, slot: int, head: int) -> int:
        """Byte offset of element (block, slot, head, dim=0) inside a region."""
        if self.layout == NHD:
            return block * self.block_bytes + slot * self.token_bytes + head * self.row_bytes
        if self.layout == HND:
            return (block * self.block_bytes + head * self.block_size * self.row_bytes
                    + slot * self.row_bytes)
        raise ValueError(self.layout)


@dataclass
class Pool:
    """Host copy of one KV pool: ``kv[l, r]`` is the byte region r of layer l
    (K = 0 and V = 1, or the single latent region 0 of an MLA pool);
    ``scales[l, r, block]`` the fp32 scale bits, or None."""

    geom: Geometry
    kv: np.ndarray                 # uint8 [L, regions, region_bytes]
    scales: Optional[np.ndarray]   # uint32 [L, regions, num_blocks] or None

    @staticmethod
    def zeros(geom: Geometry) -> "Pool":
        kv = np.zeros((geom.num_layers, geom.regions, geom.region_bytes), np.uint8)
        sc = (np.zeros((geom.num_layers, geom.regions, geom.num_blocks), np.uint32)
              if geom.has_scales else None)
        return Pool(geom, kv, sc)

    def copy(self) -> "Pool":
        return Pool(self.geom, self.kv.copy(), None if self.scales is None else self.scales.copy())


@dataclass(frozen=True)
class Request:
    """One request of a transfer: move ``num_tokens`` tokens whose KV sits in
    ``src_ids`` (producer block table) into ``dst_ids`` (consumer block table).
    Lists may be longer than needed; entries past the blocks in use are ignored."""

    num_tokens: int
    src_ids: Sequence[int]
    dst_ids: Sequence[int]


# ---------------------------------------------------------------------------
# a1: how many tokens move.
# ---------------------------------------------------------------------------
def tokens_to_move(prompt_len: int, num_computed: int = 0) -> int:
    """Tokens a consumer takes from the producer: the prompt minus what it has
    already computed, minus the final prompt token, which the consumer always
    recomputes itself.  [MORI] §3.1 (READ mode, the scheduler's remote-token
    count).  Never negative."""
    return max(0, prompt_len - num_computed - 1)


def should_reuse(reusable_tokens: int, threshold: int = 64) -> bool:
    """Bidirectional D->P reuse decision: take the decode side's KV when the
    reusable token count reaches the recompute threshold (at or above), else
    recompute.  Default threshold 64 tokens.  [BIDIR] "KV-Recompute-
    Schwellenwert" and step (5) of "Bidirektionaler KV-Transfer"."""
    return reusable_tokens >= threshold


def blocks_in_use(num_tokens: int, block_size: int) -> int:
    """Number of blocks holding ``num_tokens`` tokens: ceil(n / BS)."""
    return -(-num_tokens // block_size)


def last_block_fill(num_tokens: int, block_size: int) -> int:
    """Tokens in the last block in use (1..BS); 0 when nothing moves."""
    nb = blocks_in_use(num_tokens, block_size)
    return num_tokens - (nb - 1) * block_size if nb else 0


def window_start(num_tokens: int, window: int, bs_src: int, bs_dst: int) -> int:
    """First token a sliding-window layer group moves ([MORI] §6: layers of
    other shapes, sliding window among them, get their own geometry).

    The receiving side computes position n = num_tokens next, and a query
    with a window of W positions sees positions n-W+1 .. n.  Blocks holding
    none of those are not kept (their block-table entries may be null), so
    the move starts at the later of the two sides' starts of the block that
    holds position n-W+1.  Window 0 is full attention: everything moves."""
    if window <= 0:
        return 0
    first = max(0, num_tokens - window + 1)
    return max(first // bs_src * bs_src, first // bs_dst * bs_dst)


# ---------------------------------------------------------------------------
# Validation shared by both formulations.
# ---------------------------------------------------------------------------
_COMMON = ("num_layers", "head_dim", "elem_bytes", "has_scales", "regions", "window")


def _check_same_push_geometry(gs: Geometry, gd: Geometry) -> None:
    for f in _COMMON + ("num_heads", "layout"):
        if getattr(gs, f) != getattr(gd, f):
            raise OracleError("MISMATCH", f"{f} differs: {getattr(gs, f)} vs {getattr(gd, f)}")
    _check_block_sizes(gs, gd)


def _check_block_sizes(gs: Geometry, gd: Geometry) -> None:
    """Block sizes may differ per side ([PUSH] "Implementierungsdetails" step
    3: each side maps block positions onto its own layout).  A per-block scale
    then has no single source block, so scales need equal block sizes."""
    if gs.block_size != gd.block_size and (gs.has_scales or gd.has_scales):
        raise OracleError("UNSUPPORTED", "per-block scales need equal block sizes")


def validate(requests: Sequence[Request], block_size: int, src_blocks: int, dst_blocks: int,
             dst_block_size: Optional[int] = None, window: int = 0) -> None:
    """Error classes of the transfer (argument errors, IDs out of range,
    destination used twice).  Each list must hold ceil(n/BS) IDs, BS being
    that side's block size; later entries are not looked at, nor (with a
    sliding window) the entries of blocks the window no longer holds."""
    bsd = block_size if dst_block_size is None else dst_block_size
    used_dst = set()
    for r, req in enumerate(requests):
        if req.num_tokens < 0:
            raise OracleError("INVAL", f"request {r}: negative token count")
        nbs = blocks_in_use(req.num_tokens, block_size)
        nbd = blocks_in_use(req.num_tokens, bsd)
        if len(req.src_ids) < nbs or len(req.dst_ids) < nbd:
            raise OracleError("INVAL", f"request {r}: block list shorter than needed")
        t0 = window_start(req.num_tokens, window, block_size, bsd)
        for i in range(t0 // block_size, nbs):
            s = int(req.src_ids[i])
            if not 0 <= s < src_blocks:
                raise OracleError("RANGE", f"request {r}: src block {s} outside pool")
        for i in range(t0 // bsd, nbd):
            d = int(req.dst_ids[i])
            if not 0 <= d < dst_blocks:
                raise OracleError("RANGE", f"request {r}: dst block {d} outside pool")
            if d in used_dst:
                raise OracleError("DUPDST", f"dst block {d} used twice")
            used_dst.add(d)


# ---------------------------------------------------------------------------
# Plain definition (brute force).  Each moved token's rows are copied one by
# one from (src block, slot, head) to (dst block, slot, head), and each used
# block's scale is copied.  [PUSH] "Implementierungsdetails" step 3; [MORI]
# §3.1 (only the first n = prompt - computed - 1 tokens travel).
# ---------------------------------------------------------------------------
def push_plain(src: Pool, dst: Pool, requests: Sequence[Request],
               layers: Optional[Sequence[int]] = None) -> None:
    gs, gd = src.geom, dst.geom
    _check_same_push_geometry(gs, gd)
    copy_heads_plain(src, dst, requests, 0, 0, gs.num_heads, layers)


def copy_heads_plain(src: Pool, dst: Pool, requests: Sequence[Request],
                     src_head0: int, dst_head0: int, num_heads: int,
                     layers: Optional[Sequence[int]] = None) -> None:
    """Plain definition with a head slice: source heads [src_head0,
    src_head0+num_heads) land on destination heads [dst_head0, ...), each
    side addressed in its own layout and head count.  [PUSH]
    "Implementierungsdetails" step 3 (writes address each target TP rank, each
    side maps blocks onto its own layout); [MORI] §6 (rank mapping under TP)."""
    gs, gd = src.geom, dst.geom
    _check_head_slice(gs, gd, src_head0, dst_head0, num_heads)
    validate(requests, gs.block_size, gs.num_blocks, gd.num_blocks, gd.block_size, gs.window)
    bs, bsd = gs.block_size, gd.block_size
    row = gs.row_bytes
    lay = range(gs.num_layers) if layers is None else layers
    for req in requests:
        n = req.num_tokens
        t0 = window_start(n, gs.window, bs, bsd)
        for p in range(t0, n):
            j, s = divmod(p, bs)
            jd, sd = divmod(p, bsd)
            sb, db = int(req.src_ids[j]), int(req.dst_ids[jd])
            for h in range(src_head0, src_head0 + num_heads):
                so = gs.row_offset(sb, s, h)
                do = gd.row_offset(db, sd, h - src_head0 + dst_head0)
                for l in lay:
                    for kv in range(gs.regions):
                        dst.kv[l, kv, do:do + row] = src.kv[l, kv, so:so + row]
        if src.scales is not None:
            for j in range(t0 // bs, blocks_in_use(n, bs)):
                sb, db = int(req.src_ids[j]), int(req.dst_ids[j])
                for l in lay:
                    for kv in range(gs.regions):
                        dst.scales[l, kv, db] = src.scales[l, kv, sb]


def _check_head_slice(gs: Geometry, gd: Geometry, s0: int, d0: int, nh: int) -> None:
    for f in _COMMON:
        if getattr(gs, f) != getattr(gd, f):
            raise OracleError("MISMATCH", f"{f} differs")
    _check_block_sizes(gs, gd)
    if nh < 0 or s0 < 0 or d0 < 0:
        raise OracleError("INVAL", "negative head index or count")
    if s0 + nh > gs.num_heads or d0 + nh > gd.num_heads:
        raise OracleError("RANGE", "head slice outside the pool's heads")


# ---------------------------------------------------------------------------
# The pages' procedure.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Run:
    """Blocks src0..src0+nblk-1 -> dst0..dst0+nblk-1; the last block carries
    ``tail`` tokens (BS unless it is the request's last block)."""

    src0: int
    dst0: int
    nblk: int
    tail: int


def plan_runs(requests: Sequence[Request], block_size: int, src_blocks: int,
              dst_blocks: int, window: int = 0) -> List[Run]:
    """Merge each request's block pairs into maximal runs that are consecutive
    on both sides, in list order; a run never spans two requests.  The
    background transfer thread merges contiguous blocks into larger transfer
    regions ([PUSH] "Threading-Modell"); the per-layer offset computation
    merges contiguous blocks into one transfer ([MORI] §3.1) and adjacent
    blocks are merged to cut the work-request count ([MORI] §6).  With a
    sliding window the runs start at the first block the window holds."""
    validate(requests, block_size, src_blocks, dst_blocks, window=window)
    runs: List[Run] = []
    for req in requests:
        n = req.num_tokens
        nb = blocks_in_use(n, block_size)
        j0 = window_start(n, window, block_size, block_size) // block_size
        if nb - j0 <= 0:
            continue
        tail = last_block_fill(n, block_size)
        start = j0
        for i in range(j0 + 1, nb + 1):
            breaks = (i == nb
                      or int(req.src_ids[i]) != int(req.src_ids[i - 1]) + 1
                      or int(req.dst_ids[i]) != int(req.dst_ids[i - 1]) + 1)
            if breaks:
                last = i == nb
                runs.append(Run(int(req.src_ids[start]), int(req.dst_ids[start]), i - start,
                                tail if last else block_size))
                start = i
    return runs


def block_pairs(runs: Sequence[Run]) -> List[Tuple[int, int]]:
    """(src block, dst block) of every block in use, in plan order."""
    out = []
    for r in runs:
        for k in range(r.nblk):
            out.append((r.src0 + k, r.dst0 + k))
    return out


def _segments(runs: Sequence[Run], g: Geometry) -> List[Tuple[int, int, int]]:
    """Byte segments of one (layer, kv) region that a run moves, in source
    memory order.  NHD: the full blocks and the tail's token rows are one
    range.  HND: the full blocks are one range and each head of the last block
    contributes a range of ``tail`` rows."""
    bb, tb, row = g.block_bytes, g.token_bytes, g.row_bytes
    seg = []
    for r in runs:
        if g.layout == NHD:
            seg.append((r.src0 * bb, r.dst0 * bb, (r.nblk - 1) * bb + r.tail * tb))
        else:
            if r.tail == g.block_size:
                seg.append((r.src0 * bb, r.dst0 * bb, r.nblk * bb))
                continue
            if r.nblk > 1:
                seg.append((r.src0 * bb, r.dst0 * bb, (r.nblk - 1) * bb))
            sl, dl = r.src0 + r.nblk - 1, r.dst0 + r.nblk - 1
            for h in range(g.num_heads):
                seg.append((sl * bb + h * g.block_size * row, dl * bb + h * g.block_size * row,
                            r.tail * row))
    return seg


def triples(runs: Sequence[Run], g: Geometry) -> List[Tuple[int, int, int]]:
    """(source offset, destination offset, length) list of one (layer, K or V)
    region: the run segments with neighbours merged wherever both the source
    and the destination ranges continue without a gap.  Offsets are relative to
    the region's base; with uniform layers the list is the same for every
    layer and for K and V.  [MORI] §6 (memory registration and the
    (local offset, remote offset, size) lists handed to one batch call)."""
    out: List[List[int]] = []
    for so, do, ln in _segments(runs, g):
        if out and out[-1][0] + out[-1][2] == so and out[-1][1] + out[-1][2] == do:
            out[-1][2] += ln
        else:
            out.append([so, do, ln])
    return [tuple(t) for t in out]


@dataclass
class Plan:
    """Oracle-side plan: runs, the per-region triples and the block pairs."""

    src_geom: Geometry
    dst_geom: Geometry
    runs: List[Run]
    triples: List[Tuple[int, int, int]]
    pairs: List[Tuple[int, int]]

    @property
    def payload_bytes(self) -> int:
        """Bytes moved per (layer, K or V) region."""
        return sum(t[2] for t in self.triples)

    @property
    def scale_bytes(self) -> int:
        return 4 * len(self.pairs) if self.src_geom.has_scales else 0

    def bytes_per_layer(self) -> Tuple[int, int]:
        """(read, written) bytes of one layer, every region, payload and scales."""
        b = self.src_geom.regions * (self.payload_bytes + self.scale_bytes)
        return b, b


def make_plan(src_geom: Geometry, dst_geom: Geometry, requests: Sequence[Request]) -> Plan:
    for f in ("regions", "window"):
        if getattr(src_geom, f) != getattr(dst_geom, f):
            raise OracleError("MISMATCH", f"{f} differs")
    same = all(getattr(src_geom, f) == getattr(dst_geom, f) for f in _COMMON + ("num_heads", "layout"))
    w = src_geom.window
    if src_geom.block_size == dst_geom.block_size:
        runs = plan_runs(requests, src_geom.block_size, src_geom.num_blocks, dst_geom.num_blocks, w)
        tr = triples(runs, src_geom) if same else []
        return Plan(src_geom, dst_geom, runs, tr, block_pairs(runs))
    _check_block_sizes(src_geom, dst_geom)
    validate(requests, src_geom.block_size, src_geom.num_blocks, dst_geom.num_blocks, dst_geom.block_size, w)
    segs = token_segments(requests, src_geom.block_size, dst_geom.block_size, w)
    tr = triples_reblock(segs, src_geom, dst_geom) if same else []
    return Plan(src_geom, dst_geom, [], tr, [])


# ---------------------------------------------------------------------------
# Different block sizes per side ([PUSH] "Implementierungsdetails" step 3:
# each side maps the block positions onto its own physical layout, which
# allows different block sizes).  Token p of a request sits in source block
# src_ids[p // BS_src], slot p % BS_src and lands in destination block
# dst_ids[p // BS_dst], slot p % BS_dst.  The merge then works on tokens:
# a segment is a maximal token range whose source positions and destination
# positions both advance without a jump (within a block, or into the block
# with the next ID).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Segment:
    src_block: int
    src_slot: int
    dst_block: int
    dst_slot: int
    ntok: int


def token_segments(requests: Sequence[Request], bs_src: int, bs_dst: int,
                   window: int = 0) -> List[Segment]:
    out: List[Segment] = []
    for req in requests:
        n = req.num_tokens
        p = window_start(n, window, bs_src, bs_dst)
        while p < n:
            start = p
            p += 1
            while p < n:
                src_ok = p % bs_src != 0 or int(req.src_ids[p // bs_src]) == int(req.src_ids[p // bs_src - 1]) + 1
                dst_ok = p % bs_dst != 0 or int(req.dst_ids[p // bs_dst]) == int(req.dst_ids[p // bs_dst - 1]) + 1
                if not (src_ok and dst_ok):
                    break
                p += 1
            out.append(Segment(int(req.src_ids[start // bs_src]), start % bs_src,
                               int(req.dst_ids[start // bs_dst]), start % bs_dst, p - start))
    return out


def _split_in_blocks(seg: Segment, bs_src: int, bs_dst: int):
    """Pieces of a segment that stay inside one source and one destination
    block: (src block, src slot, dst block, dst slot, tokens)."""
    sb, ss, db, ds, left = seg.src_block, seg.src_slot, seg.dst_block, seg.dst_slot, seg.ntok
    while left > 0:
        k = min(left, bs_src - ss, bs_dst - ds)
        yield sb, ss, db, ds, k
        left -= k
        ss += k
        ds += k
        if ss == bs_src:
            sb, ss = sb + 1, 0
        if ds == bs_dst:
            db, ds = db + 1, 0


def triples_reblock(segs: Sequence[Segment], gs: Geometry, gd: Geometry) -> List[Tuple[int, int, int]]:
    """Per-region (src offset, dst offset, length) list for different block
    sizes, same head count and layout: each token segment's rows per block
    pair (per head in HND), neighbours merged where both sides continue."""
    out: List[List[int]] = []

    def emit(so, do, ln):
        if out and out[-1][0] + out[-1][2] == so and out[-1][1] + out[-1][2] == do:
            out[-1][2] += ln
        else:
            out.append([so, do, ln])
    for seg in segs:
        for sb, ss, db, ds, k in _split_in_blocks(seg, gs.block_size, gd.block_size):
            if gs.layout == NHD:
                emit(gs.row_offset(sb, ss, 0), gd.row_offset(db, ds, 0), k * gs.token_bytes)
            else:
                for h in range(gs.num_heads):
                    emit(gs.row_offset(sb, ss, h), gd.row_offset(db, ds, h), k * gs.row_bytes)
    return [tuple(t) for t in out]


def push_region(src_region: np.ndarray, dst_region: np.ndarray,
                trip: Sequence[Tuple[int, int, int]]) -> None:
    """Copy one (layer, kv) region's triples: the layer write of [MORI] §3.2,
    one batch per layer."""
    for so, do, ln in trip:
        dst_region[do:do + ln] = src_region[so:so + ln]


def push_scales(src_sc: np.ndarray, dst_sc: np.ndarray, pairs: Sequence[Tuple[int, int]]) -> None:
    """A block's scale travels with the block, unchanged."""
    for sb, db in pairs:
        dst_sc[db] = src_sc[sb]


def push(src: Pool, dst: Pool, plan: Plan, layers: Optional[Sequence[int]] = None) -> None:
    """Layerwise push: for each layer, K then V, copy the triples, then the
    scales.  [MORI] §3.2 (WRITE mode, one write per layer after that layer's
    compute); [PUSH] "Implementierungsdetails" step 3."""
    _check_same_push_geometry(src.geom, dst.geom)
    lay = range(src.geom.num_layers) if layers is None else layers
    for l in lay:
        for kv in range(src.geom.regions):
            push_region(src.kv[l, kv], dst.kv[l, kv], plan.triples)
            if src.scales is not None:
                push_scales(src.scales[l, kv], dst.scales[l, kv], plan.pairs)


# ---------------------------------------------------------------------------
# a6: contiguous staging buffer (what a NIC would read).  Layout, for each
# layer in [l0, l1), region by region (K then V): the source bytes of the region's triples in
# plan order, then (if the pool has scales) the used blocks' scales in plan
# order as little-endian uint32, zero-padded to a multiple of 16 bytes.
# ---------------------------------------------------------------------------
def _pad16(x: int) -> int:
    return (x + 15) // 16 * 16


def staging_region_bytes(plan: Plan) -> int:
    sc = _pad16(4 * len(plan.pairs)) if plan.src_geom.has_scales else 0
    return plan.payload_bytes + sc


def staging_bytes(plan: Plan, l0: int, l1: int) -> int:
    return (l1 - l0) * plan.src_geom.regions * staging_region_bytes(plan)


def pack(src: Pool, plan: Plan, l0: int, l1: int) -> np.ndarray:
    out = np.empty(staging_bytes(plan, l0, l1), np.uint8)
    pos = 0
    for l in range(l0, l1):
        for kv in range(src.geom.regions):
            for so, _, ln in plan.triples:
                out[pos:pos + ln] = src.kv[l, kv, so:so + ln]
                pos += ln
            if src.scales is not None:
                sc = np.zeros(_pad16(4 * len(plan.pairs)) // 4, np.uint32)
                for i, (sb, _) in enumerate(plan.pairs):
                    sc[i] = src.scales[l, kv, sb]
                b = sc.view(np.uint8)
                out[pos:pos + b.size] = b
                pos += b.size
    assert pos == out.size
    return out


def unpack(staging: np.ndarray, dst: Pool, plan: Plan, l0: int, l1: int) -> None:
    pos = 0
    for l in range(l0, l1):
        for kv in range(dst.geom.regions):
            for _, do, ln in plan.triples:
                dst.kv[l, kv, do:do + ln] = staging[pos:pos + ln]
                pos += ln
            if dst.scales is not None:
                nsc = _pad16(4 * len(plan.pairs))
                sc = staging[pos:pos + nsc].view(np.uint32)
                for i, (_, db) in enumerate(plan.pairs):
                    dst.scales[l, kv, db] = sc[i]
                pos += nsc


# ---------------------------------------------------------------------------
# a7: layout and head-slice transform, region at a time, with rows as the unit
# (one (token, head) row of head_dim elements).  Same mapping as
# copy_heads_plain, written as one gather/scatter per region over row indices.
# ---------------------------------------------------------------------------
def _row_index(g: Geometry, block: np.ndarray, slot: np.ndarray, head: np.ndarray) -> np.ndarray:
    if g.layout == NHD:
        return (block * g.block_size + slot) * g.num_heads + head
    return (block * g.num_heads + head) * g.block_size + slot


def head_rows(plan: Plan, src_head0: int, dst_head0: int, num_heads: int,
              requests: Sequence[Request]) -> Tuple[np.ndarray, np.ndarray]:
    """Row indices (source, destination) of every moved (token, head)."""
    gs, gd = plan.src_geom, plan.dst_geom
    sb, db, sl, dl = [], [], [], []
    for req in requests:
        n = req.num_tokens
        p = np.arange(window_start(n, gs.window, gs.block_size, gd.block_size), n, dtype=np.int64)
        sb.append(np.asarray(req.src_ids, np.int64)[p // gs.block_size])
        db.append(np.asarray(req.dst_ids, np.int64)[p // gd.block_size])
        sl.append(p % gs.block_size)
        dl.append(p % gd.block_size)
    if not sb:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    sb, db, sl, dl = np.concatenate(sb), np.concatenate(db), np.concatenate(sl), np.concatenate(dl)
    h = np.arange(num_heads, dtype=np.int64)
    src_rows = _row_index(gs, sb[:, None], sl[:, None], (src_head0 + h)[None, :]).ravel()
    dst_rows = _row_index(gd, db[:, None], dl[:, None], (dst_head0 + h)[None, :]).ravel()
    return src_rows, dst_rows


def copy_heads_region(src_region: np.ndarray, dst_region: np.ndarray, row_bytes: int,
                      src_rows: np.ndarray, dst_rows: np.ndarray) -> None:
    s = src_region.reshape(-1, row_bytes)
    d = dst_region.reshape(-1, row_bytes)
    d[dst_rows] = s[src_rows]


def copy_heads(src: Pool, dst: Pool, plan: Plan, requests: Sequence[Request], layer: int,
               src_head0: int, dst_head0: int, num_heads: int) -> None:
    gs, gd = src.geom, dst.geom
    _check_head_slice(gs, gd, src_head0, dst_head0, num_heads)
    if not 0 <= layer < gs.num_layers:
        raise OracleError("RANGE", "layer")
    sr, dr = head_rows(plan, src_head0, dst_head0, num_heads, requests)
    for kv in range(gs.regions):
        copy_heads_region(src.kv[layer, kv], dst.kv[layer, kv], gs.row_bytes, sr, dr)
        if src.scales is not None:
            push_scales(src.scales[layer, kv], dst.scales[layer, kv], plan.pairs)


# ---------------------------------------------------------------------------
# a9: multi-turn D->P reuse ([BIDIR] "Bidirektionaler KV-Transfer" steps 1-6,
# "KV-Recompute-Schwellenwert").  With context growing by a fixed number of
# tokens per turn, the reusable prefix at turn t is the previous turn's
# context; the prefill side pulls it when it reaches the threshold.  D->P has
# no final-token rule: the prefill side computes the new suffix anyway.
# ---------------------------------------------------------------------------
def reusable_prefix(turn: int, growth: int) -> int:
    """Tokens the decode side retains from turn ``turn-1`` (0 at turn 1)."""
    return growth * (turn - 1)


def reuse_request(turn: int, growth: int, threshold: int, decode_ids: Sequence[int],
                  prefill_ids: Sequence[int]) -> Optional[Request]:
    """The D->P request of one session at one turn, or None to recompute."""
    r = reusable_prefix(turn, growth)
    if r <= 0 or not should_reuse(r, threshold):
        return None
    return Request(r, decode_ids, prefill_ids)


# ---------------------------------------------------------------------------
# State-slot layer groups ([MORI] §6, hybrid model support): a mamba-like
# layer keeps its recurrent state in two separately registered regions, the
# convolution state and the SSM state, and the state is moved slot by slot.
# Region r of layer l holds num_slots slots of slot_bytes[r] bytes each.
#
# Readings: each request holds one state slot per side, the first entry of
# its list; a request that moves at least one token moves its whole slot in
# both regions, one that moves none moves nothing.  The bytes move as they
# are: which recurrent state the slot holds is the engine's business.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class StateGeometry:
    num_layers: int
    num_slots: int
    slot_bytes: Tuple[int, int]   # (convolution state, SSM state) bytes per slot


@dataclass
class StatePool:
    """``regions[r][l]`` is region r (0 = conv, 1 = SSM) of layer l as a
    uint8 array of num_slots * slot_bytes[r] bytes."""

    geom: StateGeometry
    regions: List[np.ndarray]     # two uint8 arrays [L, num_slots * slot_bytes[r]]

    def copy(self) -> "StatePool":
        return StatePool(self.geom, [a.copy() for a in self.regions])


def _check_state_geometry(gs: StateGeometry, gd: StateGeometry) -> None:
    if gs.num_layers != gd.num_layers or tuple(gs.slot_bytes) != tuple(gd.slot_bytes):
        raise OracleError("MISMATCH", "state pools differ in layers or slot sizes")


def validate_state(requests: Sequence[Request], src_slots: int, dst_slots: int) -> None:
    """Requests that move tokens need one slot on each side, inside the pool;
    a destination slot may be written once per plan."""
    used = set()
    for r, req in enumerate(requests):
        if req.num_tokens < 0:
            raise OracleError("INVAL", f"request {r}: negative token count")
        if req.num_tokens == 0:
            continue
        if len(req.src_ids) < 1 or len(req.dst_ids) < 1:
            raise OracleError("INVAL", f"request {r}: no state slot")
        s, d = int(req.src_ids[0]), int(req.dst_ids[0])
        if not 0 <= s < src_slots:
            raise OracleError("RANGE", f"request {r}: src slot {s} outside pool")
        if not 0 <= d < dst_slots:
            raise OracleError("RANGE", f"request {r}: dst slot {d} outside pool")
        if d in used:
            raise OracleError("DUPDST", f"dst slot {d} used twice")
        used.add(d)


def push_state_plain(src: StatePool, dst: StatePool, requests: Sequence[Request],
                     layers: Optional[Sequence[int]] = None) -> None:
    """Plain definition: every moving request's slot, in every layer and both
    regions, is copied whole from its source slot to its destination slot."""
    gs, gd = src.geom, dst.geom
    _check_state_geometry(gs, gd)
    validate_state(requests, gs.num_slots, gd.num_slots)
    lay = range(gs.num_layers) if layers is None else layers
    for req in requests:
        if req.num_tokens == 0:
            continue
        s, d = int(req.src_ids[0]), int(req.dst_ids[0])
        for r in range(2):
            sb = gs.slot_bytes[r]
            for l in lay:
                dst.regions[r][l, d * sb:(d + 1) * sb] = src.regions[r][l, s * sb:(s + 1) * sb]


@dataclass
class StatePlan:
    src_geom: StateGeometry
    dst_geom: StateGeometry
    runs: List[Run]                                   # one per moving request, tail 1
    triples: Tuple[List[Tuple[int, int, int]], List[Tuple[int, int, int]]]

    def payload_bytes(self, region: int) -> int:
        return sum(t[2] for t in self.triples[region])

    def bytes_per_layer(self) -> Tuple[int, int]:
        b = self.payload_bytes(0) + self.payload_bytes(1)
        return b, b


def make_state_plan(src_geom: StateGeometry, dst_geom: StateGeometry,
                    requests: Sequence[Request]) -> StatePlan:
    """The procedure: one run per moving request (its slot pair), then per
    region the slot byte ranges in plan order, neighbours merged wherever
    both sides continue ([MORI] §6: adjacent blocks merged into one range)."""
    _check_state_geometry(src_geom, dst_geom)
    validate_state(requests, src_geom.num_slots, dst_geom.num_slots)
    runs = [Run(int(q.src_ids[0]), int(q.dst_ids[0]), 1, 1) for q in requests if q.num_tokens > 0]
    lists = []
    for r in range(2):
        sb = src_geom.slot_bytes[r]
        out: List[List[int]] = []
        for run in runs:
            so, do = run.src0 * sb, run.dst0 * sb
            if out and out[-1][0] + out[-1][2] == so and out[-1][1] + out[-1][2] == do:
                out[-1][2] += sb
            else:
                out.append([so, do, sb])
        lists.append([tuple(t) for t in out])
    return StatePlan(src_geom, dst_geom, runs, (lists[0], lists[1]))


def push_state(src: StatePool, dst: StatePool, plan: StatePlan,
               layers: Optional[Sequence[int]] = None) -> None:
    lay = range(src.geom.num_layers) if layers is None else layers
    for l in lay:
        for r in range(2):
            push_region(src.regions[r][l], dst.regions[r][l], plan.triples[r])


def state_staging_bytes(plan: StatePlan, l0: int, l1: int) -> int:
    """Staging per layer: region 0's moved bytes in plan order, then region 1's."""
    return (l1 - l0) * (plan.payload_bytes(0) + plan.payload_bytes(1))


def pack_state(src: StatePool, plan: StatePlan, l0: int, l1: int) -> np.ndarray:
    out = np.empty(state_staging_bytes(plan, l0, l1), np.uint8)
    pos = 0
    for l in range(l0, l1):
        for r in range(2):
            for so, _, ln in plan.triples[r]:
                out[pos:pos + ln] = src.regions[r][l, so:so + ln]
                pos += ln
    assert pos == out.size
    return out


def unpack_state(staging: np.ndarray, dst: StatePool, plan: StatePlan, l0: int, l1: int) -> None:
    pos = 0
    for l in range(l0, l1):
        for r in range(2):
            for _, do, ln in plan.triples[r]:
                dst.regions[r][l, do:do + ln] = staging[pos:pos + ln]
                pos += ln
