"""Seeded synthetic workloads for paged-KV block transfer.

This module is shared by the tests, the bench and the oracle checks.  It holds
only input generation -- pool shapes, prompt lengths, block tables as an
engine's block allocator would hand them out, and KV values -- and none of
the transfer's own arithmetic (how many tokens move, which blocks are used,
run merging, offsets or the reuse decision live in the library and,
separately, in the oracle).

Block allocation: a request of ``prompt_len`` tokens holds ceil(prompt_len /
block_size) blocks on each side, listed in order.  The transfer may use fewer
of them (the consumer recomputes the final prompt token), so block lists are
often one entry longer than what moves.

Workload names (sizes as in their descriptions):
  tiny_push      2 layers, 8 KV heads, head_dim 64, block 16, bf16 NHD, pools
                 of 256 blocks, one 200-token prompt, random permutations.
  qwen32b_push   64 layers, 8 KV heads, head_dim 128, block 16, bf16 NHD, pools
                 of 4096 blocks, one 8192-token prompt, block tables made of
                 contiguous runs with geometric length (mean 4).
  batched_push   same KV shape, 64 prompts uniform in [1024, 16384], pools of
                 65536 blocks, geometric runs of mean 2; 64 logical layers on
                 16 physical layer slabs per pool.
  tp4_share      producer NHD 8 heads, consumer HND 2 heads (one TP4 rank),
                 64 layers, head_dim 128, block 16, bf16, 32 x 4096-token
                 prompts, random tables, pools of 16384 blocks.
  multiturn_fp8  fp8 e4m3 KV with one fp32 scale per (layer, K/V, block), 48
                 layers, 8 heads, head_dim 128, block 16; 32 sessions x 8
                 turns, context +2048 tokens per turn, pools of 32768 blocks.
  qwen32b_reblock  qwen32b_push's KV with 64-slot consumer blocks (1024 of
                 them) and 16-slot producer blocks.

Layer groups of other shapes (hybrid models: each group has its own pools and
block tables; ``layer_map`` lists, per model layer, its group and its layer
inside the group):
  dsr1_mla_push  DeepSeek-R1-shaped MLA: 61 layers of one latent region
                 (512 + 64 = 576 bf16 elements per token), token-granular
                 paging (block size 1), pools of 131072 blocks, 8 prompts of
                 8192 tokens, tables of geometric runs (mean 16 tokens).
  gptoss_swa_push  gpt-oss-120b-shaped attention: 36 layers alternating
                 sliding window (128 positions) and full attention, 8 KV
                 heads, head_dim 64, block 16, bf16 NHD; 8 prompts of 8192
                 tokens.  Full group: pools of 8192 blocks, geometric runs
                 (mean 4).  Sliding group: pools of 1024 blocks; block-table
                 entries the window no longer holds are the null block 0.
  qwen3next_state_push  Qwen3-Next-shaped hybrid: 48 layers, every fourth
                 full attention (2 KV heads, head_dim 256, block 16, bf16,
                 pools of 16384 blocks) and the rest gated-delta-net layers
                 whose state slots hold a 48 KiB convolution state (8192
                 channels x 3 taps, bf16) and a 1 MiB recurrent state (32
                 heads x 128 x 128, bf16); 64 slots per pool; 16 prompts of
                 8192 tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple, Union

import numpy as np

BF16, FP8, U8 = "bf16", "fp8_e4m3", "u8"
ELEM_BYTES = {BF16: 2, FP8: 1, U8: 1}


@dataclass(frozen=True)
class PoolSpec:
    num_layers: int          # logical layers
    num_blocks: int
    block_size: int
    num_heads: int
    head_dim: int
    dtype: str
    layout: str = "NHD"
    has_scales: bool = False
    phys_layers: int = 0     # physical layer slabs (0: one per logical layer)
    regions: int = 2         # 2: K and V; 1: one latent region (MLA)
    window: int = 0          # sliding window in positions (0: full attention)

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def n_phys(self) -> int:
        return self.phys_layers or self.num_layers

    @property
    def region_bytes(self) -> int:
        return self.num_blocks * self.block_size * self.num_heads * self.head_dim * self.elem_bytes

    @property
    def pool_bytes(self) -> int:
        return self.n_phys * self.regions * self.region_bytes

    def phys(self, layer: int) -> int:
        return layer % self.n_phys


@dataclass(frozen=True)
class StateSpec:
    """State-slot pool: per layer, region 0 (convolution state) and region 1
    (recurrent state) of num_slots slots of slot_bytes[r] bytes."""
    num_layers: int
    num_slots: int
    slot_bytes: Tuple[int, int]
    dtype: str = BF16

    def region_bytes(self, r: int) -> int:
        return self.num_slots * self.slot_bytes[r]

    @property
    def pool_bytes(self) -> int:
        return self.num_layers * (self.region_bytes(0) + self.region_bytes(1))


@dataclass
class Workload:
    name: str
    seed: int
    src: PoolSpec
    dst: PoolSpec
    prompt_lens: List[int]
    src_tables: List[np.ndarray]      # int32 per request (allocated blocks, in order)
    dst_tables: List[np.ndarray]
    extra: Dict = field(default_factory=dict)


@dataclass
class Group:
    """One layer group of a hybrid model: its pools' shape and its tables."""
    name: str
    src: Union[PoolSpec, StateSpec]
    dst: Union[PoolSpec, StateSpec]
    src_tables: List[np.ndarray]
    dst_tables: List[np.ndarray]


@dataclass
class HybridWorkload:
    name: str
    seed: int
    prompt_lens: List[int]
    groups: List[Group]
    layer_map: List[Tuple[int, int]]    # model layer -> (group, layer inside the group)


# ---------------------------------------------------------------------------
# block tables
# ---------------------------------------------------------------------------
def alloc_blocks(prompt_len: int, block_size: int) -> int:
    """Blocks an engine's allocator reserves for a prompt (ceil)."""
    return -(-prompt_len // block_size)


def permutation_table(rng: np.random.Generator, num_blocks: int) -> np.ndarray:
    return rng.permutation(num_blocks).astype(np.int32)


def geometric_run_table(rng: np.random.Generator, num_blocks: int, mean_run: float) -> np.ndarray:
    """All pool blocks, ordered as shuffled contiguous segments whose lengths
    are geometric on {1, 2, ...} with the given mean (the last segment cut at
    the pool end)."""
    p = 1.0 / mean_run
    lens = []
    total = 0
    while total < num_blocks:
        ln = int(rng.geometric(p))
        ln = min(ln, num_blocks - total)
        lens.append(ln)
        total += ln
    starts = np.cumsum([0] + lens[:-1])
    order = rng.permutation(len(lens))
    return np.concatenate([np.arange(starts[i], starts[i] + lens[i]) for i in order]).astype(np.int32)


def split_tables(seq: np.ndarray, counts: Sequence[int]) -> List[np.ndarray]:
    out, pos = [], 0
    for c in counts:
        out.append(seq[pos:pos + c].copy())
        pos += c
    if pos > len(seq):
        raise ValueError("pool too small for the allocation")
    return out


def _children(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------
def tiny_push(seed: int = 1001) -> Workload:
    spec = PoolSpec(2, 256, 16, 8, 64, BF16)
    r_src, r_dst = _children(seed, 2)
    plen = [200]
    a = [alloc_blocks(x, spec.block_size) for x in plen]
    return Workload("tiny_push", seed, spec, spec, plen,
                    split_tables(permutation_table(r_src, spec.num_blocks), a),
                    split_tables(permutation_table(r_dst, spec.num_blocks), a))


def qwen32b_push(seed: int = 1002) -> Workload:
    spec = PoolSpec(64, 4096, 16, 8, 128, BF16)
    r_src, r_dst = _children(seed, 2)
    plen = [8192]
    a = [alloc_blocks(x, spec.block_size) for x in plen]
    return Workload("qwen32b_push", seed, spec, spec, plen,
                    split_tables(geometric_run_table(r_src, spec.num_blocks, 4.0), a),
                    split_tables(geometric_run_table(r_dst, spec.num_blocks, 4.0), a))


def batched_push(seed: int = 1003, phys_layers: int = 16) -> Workload:
    spec = PoolSpec(64, 65536, 16, 8, 128, BF16, phys_layers=phys_layers)
    r_len, r_src, r_dst = _children(seed, 3)
    plen = [int(x) for x in r_len.integers(1024, 16384, size=64, endpoint=True)]
    a = [alloc_blocks(x, spec.block_size) for x in plen]
    return Workload("batched_push", seed, spec, spec, plen,
                    split_tables(geometric_run_table(r_src, spec.num_blocks, 2.0), a),
                    split_tables(geometric_run_table(r_dst, spec.num_blocks, 2.0), a))


def tp4_share(seed: int = 1004, tp_rank: int = 0) -> Workload:
    src = PoolSpec(64, 16384, 16, 8, 128, BF16, layout="NHD")
    dst = PoolSpec(64, 16384, 16, 2, 128, BF16, layout="HND")
    r_src, r_dst = _children(seed, 2)
    plen = [4096] * 32
    a = [alloc_blocks(x, src.block_size) for x in plen]
    return Workload("tp4_share", seed, src, dst, plen,
                    split_tables(permutation_table(r_src, src.num_blocks), a),
                    split_tables(permutation_table(r_dst, dst.num_blocks), a),
                    extra={"tp_size": 4, "tp_rank": tp_rank})


def multiturn_fp8(seed: int = 1005) -> Workload:
    """32 sessions, 8 turns, context growing 2048 tokens per turn.  The decode
    side keeps each session's blocks for its whole conversation (session s
    owns slice s of one permutation, 896 blocks = 7 turns' context); the
    prefill side allocates fresh blocks for the full context of each turn
    (128*t blocks per session at turn t, from a new permutation).  The
    ``src``/``dst`` pools of this workload are the decode and prefill pools:
    reuse copies decode -> prefill."""
    spec = PoolSpec(48, 32768, 16, 8, 128, FP8, has_scales=True)
    sessions, turns, growth = 32, 8, 2048
    rngs = _children(seed, 1 + turns)
    per_session = alloc_blocks(growth * (turns - 1), spec.block_size)
    dec = split_tables(permutation_table(rngs[0], spec.num_blocks), [per_session] * sessions)
    pre = {}
    for t in range(1, turns + 1):
        need = alloc_blocks(growth * t, spec.block_size)
        pre[t] = split_tables(permutation_table(rngs[t], spec.num_blocks), [need] * sessions)
    return Workload("multiturn_fp8", seed, spec, spec, [growth] * sessions, dec, pre[1],
                    extra={"sessions": sessions, "turns": turns, "growth": growth,
                           "threshold": 512, "decode_tables": dec, "prefill_tables": pre})


def qwen32b_reblock(seed: int = 1006) -> Workload:
    """qwen32b_push's KV, but the consumer pages KV in 64-slot blocks while
    the producer uses 16-slot blocks; both tables of geometric runs (mean 4)."""
    src = PoolSpec(64, 4096, 16, 8, 128, BF16)
    dst = PoolSpec(64, 1024, 64, 8, 128, BF16)
    r_src, r_dst = _children(seed, 2)
    plen = [8192]
    return Workload("qwen32b_reblock", seed, src, dst, plen,
                    split_tables(geometric_run_table(r_src, src.num_blocks, 4.0),
                                 [alloc_blocks(x, src.block_size) for x in plen]),
                    split_tables(geometric_run_table(r_dst, dst.num_blocks, 4.0),
                                 [alloc_blocks(x, dst.block_size) for x in plen]))


def dsr1_mla_push(seed: int = 1007) -> HybridWorkload:
    spec = PoolSpec(61, 131072, 1, 1, 576, BF16, regions=1)
    r_src, r_dst = _children(seed, 2)
    plen = [8192] * 8
    a = [alloc_blocks(x, spec.block_size) for x in plen]
    g = Group("mla", spec, spec, split_tables(geometric_run_table(r_src, spec.num_blocks, 16.0), a),
              split_tables(geometric_run_table(r_dst, spec.num_blocks, 16.0), a))
    return HybridWorkload("dsr1_mla_push", seed, plen, [g], [(0, l) for l in range(61)])


def _window_table(rng: np.random.Generator, prompt_len: int, block_size: int, window: int,
                  free: np.ndarray, pos: int):
    """A sliding-window group's table for one request: null block 0 for the
    positions whose blocks an engine has already released (every block
    before the one holding position prompt_len - window), pool blocks from
    ``free`` for the rest."""
    nb = alloc_blocks(prompt_len, block_size)
    keep0 = max(0, prompt_len - window) // block_size
    t = np.zeros(nb, np.int32)
    t[keep0:] = free[pos:pos + nb - keep0]
    return t, pos + nb - keep0


def gptoss_swa_push(seed: int = 1008) -> HybridWorkload:
    full = PoolSpec(18, 8192, 16, 8, 64, BF16)
    swa = PoolSpec(18, 1024, 16, 8, 64, BF16, window=128)
    r_fs, r_fd, r_ss, r_sd = _children(seed, 4)
    plen = [8192] * 8
    a = [alloc_blocks(x, full.block_size) for x in plen]
    gf = Group("full", full, full, split_tables(geometric_run_table(r_fs, full.num_blocks, 4.0), a),
               split_tables(geometric_run_table(r_fd, full.num_blocks, 4.0), a))
    tabs = []
    for rng in (r_ss, r_sd):
        free = 1 + rng.permutation(swa.num_blocks - 1).astype(np.int32)   # block 0 is the null block
        pos, out = 0, []
        for p in plen:
            t, pos = _window_table(rng, p, swa.block_size, swa.window, free, pos)
            out.append(t)
        tabs.append(out)
    gs = Group("sliding", swa, swa, tabs[0], tabs[1])
    lm = [(1, l // 2) if l % 2 == 0 else (0, l // 2) for l in range(36)]
    return HybridWorkload("gptoss_swa_push", seed, plen, [gf, gs], lm)


def qwen3next_state_push(seed: int = 1009) -> HybridWorkload:
    attn = PoolSpec(12, 16384, 16, 2, 256, BF16)
    state = StateSpec(36, 64, (8192 * 3 * 2, 32 * 128 * 128 * 2))
    r_as, r_ad, r_ss, r_sd = _children(seed, 4)
    plen = [8192] * 16
    a = [alloc_blocks(x, attn.block_size) for x in plen]
    ga = Group("attention", attn, attn, split_tables(geometric_run_table(r_as, attn.num_blocks, 4.0), a),
               split_tables(geometric_run_table(r_ad, attn.num_blocks, 4.0), a))
    ones = [1] * len(plen)
    gst = Group("state", state, state, split_tables(permutation_table(r_ss, state.num_slots), ones),
                split_tables(permutation_table(r_sd, state.num_slots), ones))
    lm, na, ns = [], 0, 0
    for l in range(48):
        if l % 4 == 3:
            lm.append((0, na))
            na += 1
        else:
            lm.append((1, ns))
            ns += 1
    return HybridWorkload("qwen3next_state_push", seed, plen, [ga, gst], lm)


WORKLOADS = {
    "tiny_push": tiny_push,
    "qwen32b_push": qwen32b_push,
    "batched_push": batched_push,
    "tp4_share": tp4_share,
    "multiturn_fp8": multiturn_fp8,
    "qwen32b_reblock": qwen32b_reblock,
}

HYBRID_WORKLOADS = {
    "dsr1_mla_push": dsr1_mla_push,
    "gptoss_swa_push": gptoss_swa_push,
    "qwen3next_state_push": qwen3next_state_push,
}


# ---------------------------------------------------------------------------
# values
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def region_seed(seed: int, pool_tag: int, phys_layer: int, kv: int) -> int:
    return (seed * 1_000_003 + pool_tag * 10_007 + phys_layer * 2 + kv) & 0x7FFF_FFFF_FFFF


def fill_region(out, dtype: str, seed: int, device=None) -> None:
    """Fill a uint8 tensor (one (layer, K/V) region) with seeded values:
    N(0,1) rounded to bf16 or to fp8 e4m3fn, or uniform random bytes."""
    torch = _torch()
    dev = out.device if device is None else device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    n = out.numel()
    if dtype == U8:
        out.copy_(torch.randint(0, 256, (n,), generator=g, device=dev, dtype=torch.uint8))
        return
    eb = ELEM_BYTES[dtype]
    chunk = 1 << 28
    flat = out.view(-1)
    for s in range(0, n // eb, chunk):
        e = min(n // eb, s + chunk)
        x = torch.randn(e - s, generator=g, device=dev, dtype=torch.float32)
        if dtype == BF16:
            y = x.to(torch.bfloat16).view(torch.uint8)
        else:
            y = x.to(torch.float8_e4m3fn).view(torch.uint8)
        flat[s * eb:e * eb].copy_(y)
        del x, y


def fill_scales(out, seed: int) -> None:
    """fp32 scales uniform in [0.5, 1.5), stored into a float32 tensor."""
    torch = _torch()
    g = torch.Generator(device=out.device)
    g.manual_seed(seed)
    out.copy_(torch.rand(out.shape, generator=g, device=out.device, dtype=torch.float32) + 0.5)


def alloc_pool(spec: PoolSpec, device):
    """One tensor per pool: uint8 [phys_layers, regions, region_bytes], plus
    fp32 scales [phys_layers, regions, num_blocks] when the pool has them."""
    torch = _torch()
    kv = torch.empty((spec.n_phys, spec.regions, spec.region_bytes), dtype=torch.uint8, device=device)
    sc = (torch.empty((spec.n_phys, spec.regions, spec.num_blocks), dtype=torch.float32, device=device)
          if spec.has_scales else None)
    return kv, sc


def alloc_state_pool(spec: StateSpec, device):
    """Two tensors: uint8 [layers, num_slots * slot_bytes[r]] for r = 0, 1."""
    torch = _torch()
    return [torch.empty((spec.num_layers, spec.region_bytes(r)), dtype=torch.uint8, device=device)
            for r in range(2)]


def fill_state_pool(spec: StateSpec, regions, seed: int, pool_tag: int) -> None:
    for r in range(2):
        for l in range(spec.num_layers):
            fill_region(regions[r][l], spec.dtype, region_seed(seed, pool_tag, l, r))


def fill_pool(spec: PoolSpec, kv, sc, seed: int, pool_tag: int, dtype: Optional[str] = None) -> None:
    for p in range(spec.n_phys):
        for k in range(spec.regions):
            fill_region(kv[p, k], dtype or spec.dtype, region_seed(seed, pool_tag, p, k))
            if sc is not None:
                fill_scales(sc[p, k], region_seed(seed, pool_tag + 7, p, k))


def random_case(seed: int, *, layout="NHD", dst_layout=None, elem_bytes=2, num_layers=2,
                num_blocks=24, dst_blocks=None, block_size=4, dst_block_size=None, num_heads=3,
                dst_heads=None, head_dim=8, has_scales=False, num_requests=3, max_tokens=30,
                run_mean=2.0, extra_ids=1, regions=2, window=0):
    """Small random case for brute-force checks: random prompt lengths (0 and
    exact block multiples included by chance), block tables of geometric runs
    so that merging has work to do, each list ``extra_ids`` entries longer than
    the prompt's allocation."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dtype = BF16 if elem_bytes == 2 else U8
    src = PoolSpec(num_layers, num_blocks, block_size, num_heads, head_dim, dtype, layout, has_scales,
                   regions=regions, window=window)
    dst = PoolSpec(num_layers, dst_blocks or num_blocks, dst_block_size or block_size, dst_heads or num_heads,
                   head_dim, dtype, dst_layout or layout, has_scales, regions=regions, window=window)
    plen = [int(x) for x in rng.integers(0, max_tokens + 1, size=num_requests)]
    need_s = [alloc_blocks(x, src.block_size) + extra_ids for x in plen]
    need_d = [alloc_blocks(x, dst.block_size) + extra_ids for x in plen]
    st = geometric_run_table(rng, src.num_blocks, run_mean)
    dt = geometric_run_table(rng, dst.num_blocks, run_mean)
    if sum(need_s) > len(st) or sum(need_d) > len(dt):
        raise ValueError("pools too small for this case")
    return Workload(f"random_{seed}", seed, src, dst, plen, split_tables(st, need_s), split_tables(dt, need_d))


def host_values(spec: PoolSpec, seed: int, pool_tag: int):
    """Host (numpy) pool contents for small cases: uint8 [L, regions, region]
    and uint32 scale bits [L, regions, NB] (or None); uniform random bytes so
    that every bit pattern occurs."""
    rng = np.random.Generator(np.random.PCG64([seed, pool_tag]))
    kv = rng.integers(0, 256, size=(spec.n_phys, spec.regions, spec.region_bytes), dtype=np.uint8)
    sc = (rng.integers(0, 2**32, size=(spec.n_phys, spec.regions, spec.num_blocks), dtype=np.uint32)
          if spec.has_scales else None)
    return kv, sc


def state_host_values(spec: StateSpec, seed: int, pool_tag: int):
    """Host contents of a state pool: two uint8 arrays [L, num_slots * slot_bytes[r]]."""
    rng = np.random.Generator(np.random.PCG64([seed, pool_tag, 5]))
    return [rng.integers(0, 256, size=(spec.num_layers, spec.region_bytes(r)), dtype=np.uint8)
            for r in range(2)]


def random_state_case(seed: int, *, num_layers=2, num_slots=24, dst_slots=None, slot_bytes=(48, 160),
                      num_requests=6, max_tokens=20, extra_ids=1):
    """Small random state-slot case: prompt lengths with zeros by chance, slot
    lists drawn from a table of geometric runs so that neighbouring requests
    often hold consecutive slots on both sides."""
    rng = np.random.Generator(np.random.PCG64([seed, 77]))
    src = StateSpec(num_layers, num_slots, tuple(slot_bytes), U8)
    dst = StateSpec(num_layers, dst_slots or num_slots, tuple(slot_bytes), U8)
    plen = [int(x) for x in rng.integers(0, max_tokens + 1, size=num_requests)]
    st = geometric_run_table(rng, src.num_slots, 3.0)
    dt = geometric_run_table(rng, dst.num_slots, 3.0)
    need = [1 + extra_ids] * num_requests
    return Workload(f"state_{seed}", seed, src, dst, plen, split_tables(st, need), split_tables(dt, need))
