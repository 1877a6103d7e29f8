"""Random cases that combine the geometry options: one or two regions, a
sliding window or none, equal or different block sizes per side, scales
(equal block sizes only), both layouts, and null (-1) entries where a
sliding window drops blocks.  Inputs only: which blocks a window drops is
decided with the band mask of the attention definition, not with the
library's or the oracle's rule."""
import numpy as np
import torch

from decode_kv_cache_amd import workloads as W


def _seen_blocks(n, w, bs):
    """Block positions holding a position that the query at position n sees
    under a window of w positions (all of them for w = 0)."""
    nb = -(-n // bs)
    if w <= 0:
        return set(range(nb))
    m = torch.ones(n + 1, n + 1, dtype=torch.bool).tril().triu(-(w - 1))
    return {int(k) // bs for k in torch.nonzero(m[n]).flatten() if int(k) // bs < nb}


def combo_cases(count, seed0, *, max_tokens=60, head_dims=(16, 32)):
    rng = np.random.Generator(np.random.PCG64(seed0))
    for i in range(count):
        regions = int(rng.choice([1, 2]))
        mixed = bool(rng.random() < 0.35)
        bs = int(rng.choice([1, 2, 3, 4, 8, 16]))
        bsd = int(rng.choice([x for x in (1, 2, 3, 4, 8, 16) if x != bs])) if mixed else bs
        window = int(rng.choice([0, 0, 1, 2, 5, bs + 1, 17, 40]))
        scales = (not mixed) and bool(rng.random() < 0.3)
        nblk = int(3 * max_tokens // min(bs, bsd) + 40)
        wl = W.random_case(20000 + seed0 + i, layout=["NHD", "HND"][int(rng.integers(0, 2))],
                           elem_bytes=int(rng.choice([1, 2])), num_layers=int(rng.integers(1, 3)),
                           num_blocks=nblk, block_size=bs, dst_block_size=bsd,
                           num_heads=1 if regions == 1 else int(rng.integers(1, 4)),
                           head_dim=int(rng.choice(head_dims)), has_scales=scales,
                           num_requests=int(rng.integers(1, 4)), max_tokens=max_tokens,
                           run_mean=float(rng.choice([1.5, 4.0])), extra_ids=int(rng.integers(0, 2)),
                           regions=regions, window=window)
        if window and rng.random() < 0.5:
            st, dt = [], []
            for p, s, d in zip(wl.prompt_lens, wl.src_tables, wl.dst_tables):
                n = max(0, p - 1)
                s, d = s.copy(), d.copy()
                ks, kd = _seen_blocks(n, window, bs), _seen_blocks(n, window, bsd)
                for j in range(-(-n // bs)):
                    if j not in ks:
                        s[j] = -1
                for j in range(-(-n // bsd)):
                    if j not in kd:
                        d[j] = -1
                st.append(s)
                dt.append(d)
            wl = W.Workload(wl.name + "_null", wl.seed, wl.src, wl.dst, wl.prompt_lens, st, dt)
        yield wl
