"""Maximum sizes on the GPU.  One layer whose work list needs more
workgroups than one launch may have along x (2^22): a latent region of
4,200,000 blocks of 256 token rows of 16 bytes (17.2 GB per pool), moved
block i -> block i, so the plan is one triple of 17.2 GB cut into 4,200,000
pieces of 4 KiB and pushed as two launches.  Checked against the plain
definition, which needs no oracle at this size: the first n token rows of
the destination region equal the source's, byte for byte, and the rows past
n keep their old bytes (n leaves the last block 100 rows short)."""
import numpy as np
import pytest
import torch

from decode_kv_cache_amd import kvx
from decode_kv_cache_amd import session as S
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_work_list_past_one_launch():
    nb, bs, row = 4_200_000, 256, 16
    spec = W.PoolSpec(1, nb, bs, 1, row // 2, W.BF16, regions=1)
    need = spec.pool_bytes * 2
    free, _ = torch.cuda.mem_get_info()
    if free < need + (8 << 30):
        pytest.skip(f"needs {need >> 30} GiB of device memory, {free >> 30} GiB free")
    print("test_work_list_past_one_launch: pools of", spec.pool_bytes, "bytes", flush=True)
    gs = S.device_side(spec, 7001, 1)
    gd = S.device_side(spec, 7001, 2)
    n = nb * bs - 100
    ids = np.arange(nb, dtype=np.int32)
    plan = kvx.kvx_plan(gs.pool, gd.pool, [n], [ids], [ids])
    shape = plan.launch_shape()
    assert shape["piece_bytes"] == 4096 and shape["pieces"] == -(-n * row // 4096) > (1 << 22)
    src_region, dst_region = gs.kv[0, 0], gd.kv[0, 0]
    tail_before = dst_region[n * row:].clone()
    src_head = src_region[:1 << 20].clone()
    assert not torch.equal(dst_region[:n * row], src_region[:n * row])   # distinct seeded fills
    kvx.kvx_push_layer(plan, 0)
    torch.cuda.synchronize()
    assert torch.equal(dst_region[:n * row], src_region[:n * row])
    assert torch.equal(dst_region[n * row:], tail_before)
    assert torch.equal(src_region[:1 << 20], src_head)
    plan.close()
    del gs, gd
    torch.cuda.empty_cache()
