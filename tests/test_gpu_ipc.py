"""The consumer pool in another process: the pytest process owns the
destination (decode-side) KV cache, a spawned producer process receives it
through a CUDA IPC handle (torch shares device tensors that way), registers
it as its destination pool, plans the transfer and pushes every layer.  This
is the one-GPU part of a push into a separate serving instance ([MORI] §6
and [PUSH] step 3: the producer writes into memory the consumer registered;
on a node the same pointers would come from the peer GPU).  Every byte must
equal the oracle's push; bytes outside the planned slots keep the consumer's
own values.  The shared allocation stays far below 2 GiB."""
import numpy as np
import pytest
import torch
import torch.multiprocessing as _mp

import oracle as O
import oracle_pins as P
from decode_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

SPEC = W.PoolSpec(2, 256, 16, 8, 128, W.BF16)   # 2 layers x K/V x 256 blocks of 32 KiB: 32 MiB
SEED = 4242


def case():
    rng = np.random.Generator(np.random.PCG64(SEED))
    plen = [1500, 900, 1200]
    need = [W.alloc_blocks(p, SPEC.block_size) for p in plen]
    return W.Workload("ipc_push", SEED, SPEC, SPEC, plen,
                      W.split_tables(W.geometric_run_table(rng, SPEC.num_blocks, 3.0), need),
                      W.split_tables(W.geometric_run_table(rng, SPEC.num_blocks, 3.0), need))


def producer(handoff, done, release):
    """Runs in the spawned process: its own source pool, the consumer's pool
    from the IPC-shared tensor, one plan, every layer pushed.  Every
    reference to the shared tensor is dropped before reporting, so the
    owning process sees it released."""
    import gc

    import torch

    from decode_kv_cache_amd import kvx
    from decode_kv_cache_amd import session as S
    try:
        dst_kv = handoff.get(timeout=120)
        wl = case()
        hs = W.host_values(wl.src, wl.seed, 1)
        gs = S.device_side(wl.src, wl.seed, 1, values=hs)
        L, NB = SPEC.num_layers, SPEC.num_blocks
        dst = kvx.kvx_pool_create(kv=dst_kv, num_layers=L, num_blocks=NB, block_size=SPEC.block_size,
                                  num_heads=SPEC.num_heads, head_dim=SPEC.head_dim, elem_bytes=SPEC.elem_bytes,
                                  layout=SPEC.layout)
        toks = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
        side = torch.cuda.Stream()
        plan = kvx.kvx_plan(gs.pool, dst, toks, wl.src_tables, wl.dst_tables, stream=side)
        for l in range(L):
            kvx.kvx_push_layer(plan, l, stream=side)
        side.synchronize()
        plan.close()
        dst.close()
        del plan, dst, dst_kv
        gc.collect()
        done.put("pushed")
    except Exception as e:   # reported to the parent
        done.put(f"error: {e!r}")
    release.wait(120)


def test_push_into_a_pool_owned_by_another_process():
    wl = case()
    hs, hd = W.host_values(wl.src, wl.seed, 1), W.host_values(wl.dst, wl.seed, 2)
    dst_kv = torch.from_numpy(np.ascontiguousarray(hd[0])).cuda()
    torch.cuda.synchronize()
    ctx = _mp.get_context("spawn")
    handoff, done, release = ctx.Queue(), ctx.Queue(), ctx.Event()
    print("starting the producer process", flush=True)
    proc = ctx.Process(target=producer, args=(handoff, done, release))
    proc.start()
    handoff.put(dst_kv)
    try:
        msg = done.get(timeout=180)
        assert msg == "pushed", msg
        torch.cuda.synchronize()
        src, dst = P.pools(O, wl)
        toks = [n - 1 for n in wl.prompt_lens]
        exp = dst.copy()
        O.push(src, exp, O.make_plan(src.geom, dst.geom,
                                     [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)]))
        assert np.array_equal(dst_kv.cpu().numpy(), exp.kv)
    finally:
        release.set()
        proc.join(60)
        if proc.is_alive():
            proc.kill()
            proc.join(10)
    assert proc.exitcode == 0, proc.exitcode
