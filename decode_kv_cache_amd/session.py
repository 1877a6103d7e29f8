"""Device-side set-up of a workload's two pools: allocate the KV tensors (and
fp32 scales), fill them with the seeded synthetic values and register them
with libkvx.  Plumbing only -- no transfer arithmetic happens here."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import kvx
from . import workloads as W


@dataclass
class Side:
    spec: W.PoolSpec
    kv: torch.Tensor                 # uint8 [phys_layers, 2, region_bytes]
    sc: Optional[torch.Tensor]       # float32 [phys_layers, 2, num_blocks] or None
    pool: kvx.Pool

    def region(self, layer: int, kv: int) -> torch.Tensor:
        return self.kv[self.spec.phys(layer), kv]


def register(spec: W.PoolSpec, kv: torch.Tensor, sc: Optional[torch.Tensor]) -> kvx.Pool:
    return kvx.kvx_pool_create(kv=kv, scales=sc, num_layers=spec.num_layers, num_blocks=spec.num_blocks,
                               block_size=spec.block_size, num_heads=spec.num_heads,
                               head_dim=spec.head_dim, elem_bytes=spec.elem_bytes, layout=spec.layout,
                               phys=spec.phys, sliding_window=spec.window)


def device_side(spec: W.PoolSpec, seed: int, tag: int, device="cuda", values=None) -> Side:
    """Pool on the device.  ``values``: None -> seeded N(0,1) values of the
    pool's dtype generated on the device; a (kv, scales) pair of host numpy
    arrays (uint8, uint32 bits) -> uploaded as is."""
    if values is None:
        kv, sc = W.alloc_pool(spec, device)
        W.fill_pool(spec, kv, sc, seed, tag)
    else:
        hkv, hsc = values
        kv = torch.from_numpy(np.ascontiguousarray(hkv)).to(device)
        sc = (torch.from_numpy(np.ascontiguousarray(hsc).view(np.int32)).to(device).view(torch.float32)
              if hsc is not None else None)
    return Side(spec, kv, sc, register(spec, kv, sc))


def scale_bits(sc: torch.Tensor) -> np.ndarray:
    """Host copy of fp32 scales as uint32 bit patterns."""
    return sc.view(torch.int32).cpu().numpy().view(np.uint32)


@dataclass
class StateSide:
    spec: W.StateSpec
    regions: list                    # two uint8 tensors [layers, num_slots * slot_bytes[r]]
    pool: kvx.StatePool


def state_device_side(spec: W.StateSpec, seed: int, tag: int, device="cuda", values=None) -> StateSide:
    """State pool on the device: seeded values of the pool's dtype, or the
    given pair of host uint8 arrays."""
    if values is None:
        regions = W.alloc_state_pool(spec, device)
        W.fill_state_pool(spec, regions, seed, tag)
    else:
        regions = [torch.from_numpy(np.ascontiguousarray(v)).to(device) for v in values]
    pool = kvx.kvx_state_pool_create(regions=regions, num_slots=spec.num_slots, slot_bytes=spec.slot_bytes)
    return StateSide(spec, regions, pool)


def group_side(spec, seed: int, tag: int, device="cuda", values=None):
    """Side of either pool kind."""
    if isinstance(spec, W.StateSpec):
        return state_device_side(spec, seed, tag, device, values)
    return device_side(spec, seed, tag, device, values)
