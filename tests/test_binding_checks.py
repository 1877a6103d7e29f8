"""The Python binding refuses tensors the kernels cannot address safely: host
tensors, tensors on another device, strided views, the wrong element type
and regions too small for the pool's blocks.  Such a tensor would otherwise
reach a kernel as a raw pointer and be written out of bounds.  The host-tensor
refusals run on the CPU; the rest need device tensors."""
import pytest
import torch

from decode_kv_cache_amd import kvx

GEOM = dict(num_layers=2, num_blocks=8, block_size=4, num_heads=2, head_dim=8, elem_bytes=2)
BLOCK = 4 * 2 * 8 * 2   # bytes per block per region


def test_pool_create_refuses_host_tensor():
    kv = torch.zeros((2, 2, 8 * BLOCK), dtype=torch.uint8)
    with pytest.raises(ValueError, match="host tensor"):
        kvx.kvx_pool_create(kv=kv, **GEOM)


def test_pool_create_refuses_non_tensor():
    with pytest.raises(ValueError, match="torch tensor"):
        kvx.kvx_pool_create(kv=[0] * 10, **GEOM)


def test_state_pool_create_refuses_host_tensors():
    regs = [torch.zeros((2, 4 * 64), dtype=torch.uint8), torch.zeros((2, 4 * 128), dtype=torch.uint8)]
    with pytest.raises(ValueError, match="host tensor"):
        kvx.kvx_state_pool_create(regions=regs, num_slots=4, slot_bytes=(64, 128))
    with pytest.raises(ValueError, match="two regions"):
        kvx.kvx_state_pool_create(regions=regs[:1], num_slots=4, slot_bytes=(64, 128))


def test_pack_unpack_refuse_host_staging():
    stg = torch.zeros(1 << 12, dtype=torch.uint8)
    # the staging buffer is checked before the plan is touched
    with pytest.raises(ValueError, match="host tensor"):
        kvx.kvx_pack(None, 0, 1, stg)
    with pytest.raises(ValueError, match="host tensor"):
        kvx.kvx_unpack(None, 0, 1, stg)


@pytest.mark.gpu
def test_device_tensor_refusals():
    dev = torch.device("cuda", torch.cuda.current_device())
    kv = torch.zeros((2, 2, 8 * BLOCK), dtype=torch.uint8, device=dev)
    pool = kvx.kvx_pool_create(kv=kv, **GEOM)     # the well-formed pool registers
    pool.close()
    with pytest.raises(ValueError, match="contiguous"):
        kvx.kvx_pool_create(kv=torch.zeros((2, 2, 16 * BLOCK), dtype=torch.uint8, device=dev)[:, :, ::2], **GEOM)
    with pytest.raises(ValueError, match="uint8"):
        kvx.kvx_pool_create(kv=kv.view(torch.int16), **GEOM)
    with pytest.raises(ValueError, match="need"):
        kvx.kvx_pool_create(kv=kv[:, :, :7 * BLOCK].contiguous(), **GEOM)
    with pytest.raises(ValueError, match="slabs"):
        kvx.kvx_pool_create(kv=kv[:1].contiguous(), **GEOM)
    with pytest.raises(ValueError, match="slabs"):
        kvx.kvx_pool_create(kv=kv, phys=lambda l: l + 1, **GEOM)
    with pytest.raises(ValueError, match="region bytes"):
        kvx.kvx_pool_create(kv=kv.view(2, 2, 4, -1), **GEOM)
    sc = torch.zeros((2, 2, 8), dtype=torch.float32, device=dev)
    kvx.kvx_pool_create(kv=kv, scales=sc, **GEOM).close()
    with pytest.raises(ValueError, match="float32"):
        kvx.kvx_pool_create(kv=kv, scales=sc.view(torch.int32), **GEOM)
    with pytest.raises(ValueError, match="scales must be"):
        kvx.kvx_pool_create(kv=kv, scales=sc[:, :, :7].contiguous(), **GEOM)
    with pytest.raises(ValueError, match="contiguous"):
        kvx.kvx_pool_create(kv=kv, scales=torch.zeros((2, 2, 16), dtype=torch.float32, device=dev)[:, :, ::2],
                            **GEOM)
    regs = [torch.zeros((2, 4 * 64), dtype=torch.uint8, device=dev),
            torch.zeros((2, 4 * 128), dtype=torch.uint8, device=dev)]
    kvx.kvx_state_pool_create(regions=regs, num_slots=4, slot_bytes=(64, 128)).close()
    with pytest.raises(ValueError, match="regions\\[1\\]"):
        kvx.kvx_state_pool_create(regions=[regs[0], regs[1][:, :256].contiguous()], num_slots=4,
                                  slot_bytes=(64, 128))
    stg = torch.zeros(1 << 12, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        kvx.kvx_pack(None, 0, 1, stg[::2])
    with pytest.raises(ValueError, match="contiguous"):
        kvx.kvx_unpack(None, 0, 1, stg[::2])
