#!/usr/bin/env python3
"""Benchmark: paged-KV block transfer GB/s (read + write) on one MI355X.

Default workload (qwen32b_push): Qwen3-32B-shaped KV -- 64 layers, K and V,
8 KV heads, head_dim 128, block 16, bf16 -- one 8192-token prompt (8191 tokens
move; the consumer recomputes the last one), block tables of contiguous runs
with geometric length (mean 4) in pools of 4096 blocks.  One step = the
layerwise push: kvx_push_layer(layer, ready[layer]) on a side stream for each
of the 64 layers, ready[layer] being the (already fired) event of that
layer's compute.

Other workloads (--workload), one JSON line each:
  batched_push   64 prompts uniform in [1024, 16384], fragmented tables (mean
                 run 2), each layer's push waiting on a synthetic compute
                 kernel of that layer running concurrently on the compute stream
  tp4_share      NHD 8 heads -> HND 2-head slice (TP4 rank 0), 32 x 4096 tokens
  multiturn_fp8  fp8 KV + fp32 per-block scales, 32 sessions, turns 2..8 copy
                 the decode side's retained prefix back to the prefill pool
  pack_unpack    the default workload through a contiguous staging buffer
  qwen32b_reblock  the default KV with 64-slot consumer blocks (16-slot producer)
  xfer_pipeline  batched_push's requests driven through the transfer state
                 machine (kvx_xfer), layer by layer
  tiny_push      2 layers, one 200-token prompt (launch-bound; no claim)
  dsr1_mla_push  DeepSeek-R1-shaped MLA: 61 layers of one 576-element latent
                 region, token-granular blocks, 8 x 8192-token prompts
  gptoss_swa_push  gpt-oss-120b-shaped: 36 layers alternating full attention
                 and a 128-position sliding window (only the blocks the next
                 query still sees move), 8 x 8192-token prompts
  qwen3next_state_push  Qwen3-Next-shaped hybrid: 12 full-attention layers
                 and 36 gated-delta-net layers whose conv (48 KiB) and
                 recurrent (1 MiB) state slots move, 16 x 8192-token prompts

Prints ONE JSON line on stdout.  Everything else goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV block transfer GB/s (read+write) on 1 MI355X + % of HBM peak"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD published peak
PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 1 << 30
WORKLOAD_NAMES = ["qwen32b_push", "batched_push", "tp4_share", "multiturn_fp8", "pack_unpack", "qwen32b_reblock",
                  "xfer_pipeline", "tiny_push", "dsr1_mla_push", "gptoss_swa_push", "qwen3next_state_push"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The dominant kernel of each workload's bench line, as named in profiles/
# (the kernel that the workload's --counters run launches).
COUNTER_KERNEL = {"qwen32b_push": "many_kernel", "qwen32b_reblock": "many_kernel", "tiny_push": "many_kernel",
                  "multiturn_fp8": "many_kernel",
                  "tp4_share": "heads_kernel", "pack_unpack": "many_kernel", "dsr1_mla_push": "many_kernel",
                  "gptoss_swa_push": "many_kernel", "qwen3next_state_push": "many_kernel"}


def counter_ratio(workload: str, kernel: str = None):
    """Measured HBM bytes over algorithmic bytes of the dominant kernel's
    launches, from the committed rocprofv3 --pmc summary (FETCH_SIZE and
    WRITE_SIZE passes, each scaled by the counter's reading for a plain copy
    of known size); None when there is no summary or the kernel sources
    changed since it was taken."""
    from decode_kv_cache_amd.profiling import kernel_source_digest
    kernel = kernel or COUNTER_KERNEL.get(workload, "push_kernel")
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0] if v.strip() else ""
    if kv.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    try:
        return float(kv["calibrated_hbm_bytes_per_launch"]) / float(kv["algorithmic_bytes_per_launch"])
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def cpu_info():
    cores = len(os.sched_getaffinity(0))
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, os.cpu_count(), model


def cpu_baseline(what: str, pass_fn, bytes_per_pass: int, seconds: float, setup_s: float):
    """Time the oracle's own copy routine, single-threaded, for ~`seconds`."""
    passes = 0
    t0 = time.perf_counter()
    while True:
        pass_fn()
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores, ncpu, model = cpu_info()
    return {"value": round(bytes_per_pass * passes / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}; {passes} passes in {el:.1f} s (single thread; the host has {cores} usable cores, "
                      f"{ncpu} total, {model}); oracle plan {setup_s * 1e3:.1f} ms"}


def oracle_pools(wl, gs, gd, layers):
    """Host copies of the sampled layers of both pools as oracle pools."""
    import oracle as O
    from decode_kv_cache_amd import session as S

    def geom(spec, n):
        return O.Geometry(n, spec.num_blocks, spec.block_size, spec.num_heads, spec.head_dim, spec.elem_bytes,
                          spec.layout, spec.has_scales, spec.regions, spec.window)

    def pool(spec, side):
        kv = np.stack([side.kv[spec.phys(l)].cpu().numpy() for l in layers])
        sc = np.stack([S.scale_bits(side.sc[spec.phys(l)]) for l in layers]) if side.sc is not None else None
        return O.Pool(geom(spec, len(layers)), kv, sc)
    return pool(wl.src, gs), pool(wl.dst, gd)


def steady_plan_ms(kvx, src, dst, tokens, src_tables, dst_tables, stream, reps=5, runs=False):
    """Median host time of kvx_plan (build, upload enqueue) once the process
    is warm; the first plan of a process also pays one-time runtime set-up."""
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        p = kvx.kvx_plan(src, dst, tokens, src_tables, dst_tables, runs=runs, stream=stream)
        ts.append((time.perf_counter() - t0) * 1e3)
        p.close()
    return float(np.median(ts))


class Timer:
    """Events on one stream around a region."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def inputs_digest(tables, sides, prompt_lens) -> str:
    """SHA-256 (first 16 hex digits) of a run's inputs: every block table,
    the prompt lengths, and the first MiB of every physical region (and all
    scales) of every pool, source and destination pre-fill alike.  Enough to
    show that two runs used the same seeded bytes without copying whole pools
    to the host; taken before anything is pushed."""
    h = hashlib.sha256()
    for t in tables:
        h.update(np.ascontiguousarray(t, dtype=np.int32).tobytes())
    h.update(np.asarray(prompt_lens, dtype=np.int64).tobytes())
    for side in sides:
        if hasattr(side, "kv"):
            regions = [side.kv[p, r] for p in range(side.kv.shape[0]) for r in range(side.kv.shape[1])]
            if side.sc is not None:
                h.update(side.sc.cpu().numpy().tobytes())
        else:
            regions = [reg[l] for reg in side.regions for l in range(reg.shape[0])]
        for reg in regions:
            h.update(reg[:1 << 20].cpu().numpy().tobytes())
    return h.hexdigest()[:16]


def roofline(bytes_per_launch: int, avg_us: float, kernel: str, workload: str, extra=None):
    """The line's roofline object.  `traffic` is HBM bytes per launch: the
    counter summary's measured-over-algorithmic ratio for this kernel and
    workload times the launch's algorithmic bytes."""
    ach = bytes_per_launch / (avg_us * 1e-6) / 1e9
    ratio = counter_ratio(workload)
    r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(ach / HBM_PEAK_GBS, 4),
         "traffic": None if ratio is None else round(ratio * bytes_per_launch),
         "traffic_over_algorithmic": None if ratio is None else round(ratio, 4), "kernel": kernel,
         "avg_launch_us": round(avg_us, 3), "algorithmic_bytes_per_launch": bytes_per_launch}
    if extra:
        r.update(extra)
    return r


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def workload(W, name: str, args):
    """The named workload's generator with the command line's overrides
    (--seed for any workload, --tp-rank for tp4_share, --phys-layers for the
    batched_push geometry)."""
    ctor = {**W.WORKLOADS, **W.HYBRID_WORKLOADS}[name]
    kw = {}
    if args.seed is not None:
        kw["seed"] = args.seed
    if name == "tp4_share" and args.tp_rank is not None:
        kw["tp_rank"] = args.tp_rank
    if name == "batched_push" and args.phys_layers is not None:
        kw["phys_layers"] = args.phys_layers
    return ctor(**kw)


def timed_steps(torch, stream, step, steps, warmup):
    """W untimed steps; then `steps` steps between two events on `stream`,
    after a synchronize on both sides (the span); then `steps` more with an
    event between consecutive steps (the per-step spans).  (span ms,
    per-step spans ms).  The events between steps are left out of the span:
    each costs a few microseconds of the stream's time (about 9 us, 1.3%, on
    a queue step of the Qwen3-32B-shaped push)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    return a.elapsed_time(b), per


def span_stats(per_step_ms, how="a second pass of the steps, an event between consecutive steps") -> dict:
    a = np.asarray(per_step_ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 4), "min_ms": round(float(a.min()), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "mean_ms": round(float(a.mean()), 4),
            "steps": int(a.size), "pass": how}


def worklist_bytes(plan) -> int:
    """Device work-list bytes a plan uploads: 32 B per cut piece (twice for a
    one-wave plan, which keeps a destination-ordered copy), or two run tables
    of 16 B per triple plus their run indexes; 16 B per planned block either
    way (the scale copies' block pairs)."""
    sh = plan.launch_shape()
    ntrip = len(plan.triples(0, 0))
    regions = 2 if plan.src.regions == 2 else 1
    blocks = len(plan.runs()) if plan.src.block_size == plan.dst.block_size else 0
    if sh["run_table"]:
        chunks = sh["pieces"] // regions
        return 2 * 16 * ntrip + 2 * 4 * (-(-chunks // 8)) + 16 * blocks
    pieces = sh["pieces"] // regions
    copies = 2 if sh["lanes"] == 64 else 1
    return copies * 32 * pieces + 16 * blocks


def launch_groups(pairs):
    """(plan, layer) pairs as the launches they take once writes back up:
    each plan's layers (plans in order of first appearance, layers in the
    pairs' order) in runs of up to 32, one kvx_push_many launch each (with
    per-block scales, that launch and the small scale launch behind it)."""
    per_plan = {}
    for p, l in pairs:
        per_plan.setdefault(id(p), (p, []))[1].append(l)
    out = []
    for p, ls in per_plan.values():
        out += [(p, ls[i:i + 32]) for i in range(0, len(ls), 32)]
    return out


def launch_group_us(torch, kvx, side, pairs, rounds=3):
    """Kernel time per launch group once writes back up, from the launches'
    own dispatch timestamps (kvx_push_many_timed over one group's layers):
    (mean us per group, mean algorithmic bytes per group, groups)."""
    ls = launch_groups(pairs)
    ev = []
    for _ in range(rounds):
        for p, layers in ls:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            kvx.kvx_push_many_timed([p] * len(layers), layers, a, b, stream=side)
            ev.append((a, b))
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    nbytes = [sum(p.bytes_per_layer()) * len(layers) for p, layers in ls] * rounds
    return float(np.mean(us)), float(np.mean(nbytes)), len(ls)


class QueueStep:
    """The layerwise step through one write queue on `side`: for each (plan,
    layer) pair, kvx_queue_push(plan, layer, ready[i]), then kvx_queue_flush."""

    def __init__(self, kvx, side, pairs, ready):
        self.kvx, self.side, self.pairs, self.ready = kvx, side, pairs, ready
        self.q = kvx.Queue(side)

    def __call__(self):
        for i, (p, l) in enumerate(self.pairs):
            self.q.push(p, l, ready=self.ready[i])
        self.q.flush()

    def timed(self, torch, steps, warmup):
        """(span ms, per-step ms, launch groups per step, kernel launches per step)."""
        w0, g0, n0 = self.q.stats3()
        span, per = timed_steps(torch, self.side, self, steps, warmup)
        w1, g1, n1 = self.q.stats3()
        nsteps = (w1 - w0) / len(self.pairs)
        return span, per, (g1 - g0) / nsteps, (n1 - n0) / nsteps

    def launch_us(self, torch, rounds=3):
        return launch_group_us(torch, self.kvx, self.side, self.pairs, rounds)

    def close(self):
        self.q.close()


# ---------------------------------------------------------------------------
# oracle leg: parity of the timed path (verification step before timing) and
# the CPU baseline; the only part of this file that touches oracle/
# ---------------------------------------------------------------------------
def oracle_geom(O, spec, n_layers=None):
    return O.Geometry(spec.num_layers if n_layers is None else n_layers, spec.num_blocks, spec.block_size,
                      spec.num_heads, spec.head_dim, spec.elem_bytes, spec.layout, spec.has_scales, spec.regions,
                      spec.window)


def snap_layers(S, side, layers):
    """Host copies (regions, scale bits) of the sampled layers' physical slabs."""
    out = {}
    for l in layers:
        p = side.spec.phys(l)
        out[p] = (side.kv[p].cpu().numpy().copy(),
                  S.scale_bits(side.sc[p]).copy() if side.sc is not None else None)
    return out


def parity_push_layers(O, S, wl, gs, gd, src_snap, dst_snap, toks, layers, label):
    """Every byte of the sampled layers' regions (and scales) against the
    oracle's push of the pre-step source onto the pre-step destination; the
    source must be unchanged."""
    op = O.make_plan(oracle_geom(O, wl.src), oracle_geom(O, wl.dst),
                     [O.Request(n, s, d) for n, s, d in zip(toks, wl.src_tables, wl.dst_tables)])
    nbytes, bad = 0, []
    for l in layers:
        p = wl.src.phys(l)
        skv, ssc = src_snap[p]
        dkv, dsc = dst_snap[p]
        for r in range(wl.src.regions):
            exp = dkv[r].copy()
            O.push_region(skv[r], exp, op.triples)
            got = gd.kv[p, r].cpu().numpy()
            nbytes += got.size
            if not np.array_equal(got, exp):
                bad.append(f"layer {l} region {r}")
            if not np.array_equal(gs.kv[p, r].cpu().numpy(), skv[r]):
                bad.append(f"layer {l} region {r}: source changed")
            if ssc is not None:
                es = dsc[r].copy()
                O.push_scales(ssc[r], es, op.pairs)
                if not np.array_equal(S.scale_bits(gd.sc[p, r]), es):
                    bad.append(f"layer {l} region {r} scales")
    return parity_record(bad, f"{label}: every byte of layers {layers} (K/V regions"
                              f"{' and scales' if wl.src.has_scales else ''}) against the oracle", nbytes)


def parity_record(bad, what, nbytes):
    r = {"result": "fail" if bad else "pass", "checked": what, "bytes_compared": int(nbytes)}
    if bad:
        r["mismatches"] = bad[:8]
    log(f"parity: {r['result']} ({what}; {nbytes} bytes)" + (f" MISMATCH {bad[:4]}" if bad else ""))
    return r


def bench_push(args, torch, kvx, S, W):
    """qwen32b_push (default), tiny_push and qwen32b_reblock: the layerwise
    push.  The step: for each layer, kvx_queue_push(layer, ready[layer]) on
    the side stream's write queue (the layer's write goes out once its event
    has fired), then kvx_queue_flush; ready[layer] is the (already fired)
    event of that layer's compute."""
    from decode_kv_cache_amd import bench_support as B
    wl = workload(W, args.workload, args)
    gs, gd = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, stream=side)
    plan_ms = steady_plan_ms(kvx, gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, side)
    rd, wr = plan.bytes_per_layer()
    L = wl.src.num_layers
    layer_bytes = rd + wr
    step_bytes = layer_bytes * L
    nruns = len(plan.runs()) if wl.src.block_size == wl.dst.block_size else None
    ntrip = len(plan.triples())
    log(f"plan: {nruns} runs, {ntrip} triples/region, {layer_bytes} B per layer, "
        f"{step_bytes} B per step, host plan {plan_ms:.2f} ms")

    if args.counters:   # the queue's launches once writes back up: kvx_push_many of 32 layers per launch
        counters_run(torch, kvx, plan, side, 1, layer_bytes * min(L, 32),
                     launch=lambda _l: kvx.kvx_push_many([plan] * L, list(range(L)), stream=side))
        plan.close()
        return None
    digest = inputs_digest(wl.src_tables + wl.dst_tables, [gs, gd], wl.prompt_lens)

    # One ready event per layer, recorded on the compute stream.  The headline
    # step uses events that have already fired (the layer's compute is done).
    ready = [torch.cuda.Event() for _ in range(L)]
    for e in ready:
        e.record(compute)
    torch.cuda.synchronize()
    step = QueueStep(kvx, side, [(plan, l) for l in range(L)], ready)

    # Verification step on the freshly filled pools, through the timed path.
    parity = None
    if not args.no_parity:
        import oracle as O
        layers = sorted({0, 1, L // 2 + 5, L - 1} & set(range(L)))
        src_snap, dst_snap = snap_layers(S, gs, layers), snap_layers(S, gd, layers)
        step()
        torch.cuda.synchronize()
        parity = parity_push_layers(O, S, wl, gs, gd, src_snap, dst_snap, tokens, layers,
                                    "one step through kvx_queue on the fresh pools")
        del src_snap, dst_snap

    span_ms, per_step, groups_per_step, launches_per_step = step.timed(torch, args.steps, args.warmup)
    ms_per_step = span_ms / args.steps
    gbs = step_bytes * args.steps / (span_ms * 1e-3) / 1e9
    stats = span_stats(per_step)
    log(f"queue step: span {span_ms:.3f} ms for {args.steps} steps ({ms_per_step * 1e3:.1f} us/step, median "
        f"{stats['median_ms'] * 1e3:.1f}, min {stats['min_ms'] * 1e3:.1f}, p90 {stats['p90_ms'] * 1e3:.1f}); "
        f"{groups_per_step:.2f} launch groups, {launches_per_step:.2f} launches per step: {gbs:.1f} GB/s = "
        f"{100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f} GB/s")

    # Cold caches: each step after a 1 GiB fill of a scratch buffer on the
    # side stream, which leaves none of the step's bytes in the L2s or the
    # 256 MB MALL, timed from an event behind the fill to one behind the
    # step.  Its counterpart is the span's second pass, which also has an
    # event between consecutive steps.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    marks = []
    for i in range(args.steps):
        B.fill(scratch, i & 0xFF, stream=side)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(side)
        step()
        b.record(side)
        marks.append((a, b))
    torch.cuda.synchronize()
    cold = np.array([a.elapsed_time(b) for a, b in marks])
    del scratch, marks
    cold_stats = span_stats(cold, "each step after a 1 GiB fill of a scratch buffer on the side stream (outside "
                                  "the timed interval); compare span.median_ms")
    cold_stats["GBs_at_median"] = round(step_bytes / (cold_stats["median_ms"] * 1e-3) / 1e9, 1)
    log(f"cold-cache steps: median {cold_stats['median_ms'] * 1e3:.1f} us ({cold_stats['GBs_at_median']} GB/s) "
        f"against {stats['median_ms'] * 1e3:.1f} us in the span's second pass")

    # Kernel measurement for the roofline.  Once writes back up, the queue's
    # groups are kvx_push_many launches of 32 layers each (two per step); the
    # same launches, each timed from its own dispatch timestamps.
    k_avg_us, k_bytes, _ = step.launch_us(torch)
    log(f"batched push kernel: {k_avg_us:.2f} us per launch of {min(L, 32)} layers (dispatch timestamps)")

    # Secondary: one kvx_push_layer launch per layer on the side stream.
    def layer_step():
        for l in range(L):
            kvx.kvx_push_layer(plan, l, ready=ready[l], stream=side)
    lspan, lper = timed_steps(torch, side, layer_step, args.steps, 2)
    layer_gbs = step_bytes * args.steps / (lspan * 1e-3) / 1e9
    kd0 = [torch.cuda.Event(enable_timing=True) for _ in range(L)]
    kd1 = [torch.cuda.Event(enable_timing=True) for _ in range(L)]
    for l in range(L):
        kvx.kvx_push_layer_timed(plan, l, kd0[l], kd1[l], ready=ready[l], stream=side)
    torch.cuda.synchronize()
    layer_kernel_us = float(np.mean([kd0[l].elapsed_time(kd1[l]) for l in range(L)]) * 1e3)
    log(f"one kvx_push_layer launch per layer: {layer_gbs:.1f} GB/s ({lspan / args.steps * 1e3 / L:.2f} us per "
        f"layer; dispatch timestamps {layer_kernel_us:.2f} us per launch)")

    # Secondary: fresh events (recorded on the compute stream right before each
    # push, so each kvx_push_layer enqueues a cross-stream wait).
    def fresh_step():
        for l in range(L):
            ready[l].record(compute)
            kvx.kvx_push_layer(plan, l, ready=ready[l], stream=side)
    fresh_step()
    with Timer(torch, side) as t:
        for _ in range(args.steps):
            fresh_step()
    fresh_gbs = step_bytes * args.steps / (t.ms * 1e-3) / 1e9
    for e in ready:
        e.record(compute)
    torch.cuda.synchronize()
    log(f"kvx_push_layer with fresh per-layer events: {fresh_gbs:.1f} GB/s")

    # Secondary: the per-layer step captured once in a HIP graph and replayed.
    kvx.kvx_plan_wait(plan)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for l in range(L):
            kvx.kvx_push_layer(plan, l, stream=torch.cuda.current_stream())
    with torch.cuda.stream(side):   # replay() launches on the current stream
        graph.replay()
        with Timer(torch, side) as t:
            for _ in range(args.steps):
                graph.replay()
    graph_gbs = step_bytes * args.steps / (t.ms * 1e-3) / 1e9
    log(f"per-layer step replayed from a HIP graph: {graph_gbs:.1f} GB/s")
    del graph

    # Secondary: all layers in one kvx_push_many call.
    many_plans, many_layers = [plan] * L, list(range(L))
    kvx.kvx_push_many(many_plans, many_layers, stream=side)
    with Timer(torch, side) as t:
        for _ in range(args.steps):
            kvx.kvx_push_many(many_plans, many_layers, stream=side)
    many_gbs = step_bytes * args.steps / (t.ms * 1e-3) / 1e9
    log(f"all layers in one kvx_push_many call: {many_gbs:.1f} GB/s")

    # Secondary: layers alternating over two side streams, plan built with
    # KVX_PLAN_OVERLAP.
    oplan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, overlap=True, stream=side)
    two_gbs = two_stream_rate(torch, kvx, oplan, ready, side, L, args.steps, step_bytes)
    log(f"layers alternating over two side streams (overlap plan): {two_gbs:.1f} GB/s")
    oplan.close()

    # Ceiling, same run: the same bytes without a block table.  Per layer, K
    # and V each as one contiguous segment of the plan's payload bytes
    # (layer l's regions of both pools), so no byte is served from a cache.
    ceiling = None
    if wl.src.block_size == wl.dst.block_size and wl.src.regions == 2:
        seg = rd // 2
        assert seg <= wl.src.region_bytes and seg <= wl.dst.region_bytes and seg % 16 == 0
        sp = [[gs.region(l, r).data_ptr() for r in range(2)] for l in range(L)]
        dp = [[gd.region(l, r).data_ptr() for r in range(2)] for l in range(L)]
        lay_src = [torch.tensor(sp[l], dtype=torch.int64, device="cuda") for l in range(L)]
        lay_dst = [torch.tensor(dp[l], dtype=torch.int64, device="cuda") for l in range(L)]
        half = -(-L // 2)
        grp_src = [torch.tensor([x for l in ls for x in sp[l]], dtype=torch.int64, device="cuda")
                   for ls in (range(0, half), range(half, L))]
        grp_dst = [torch.tensor([x for l in ls for x in dp[l]], dtype=torch.int64, device="cuda")
                   for ls in (range(0, half), range(half, L))]

        def plain_per_layer():
            for l in range(L):
                B.copy_segments(lay_src[l], lay_dst[l], seg, 0, stream=side)

        def plain_stream():
            for g in range(2):
                B.copy_segments(grp_src[g], grp_dst[g], seg, 1, stream=side)
        c_layer, _ = timed_steps(torch, side, plain_per_layer, args.steps, 2)
        c_stream, _ = timed_steps(torch, side, plain_stream, args.steps, 2)
        # the chip's plain-copy rate: the step's read bytes as one contiguous
        # segment of each pool, rotating over four windows so that no window
        # repeats within four steps (the pools are scratch by now)
        tot = rd * L
        win = min(gs.kv.numel(), gd.kv.numel()) // 4 // 4096 * 4096
        assert tot <= win and tot % 16 == 0
        wins = [(torch.tensor([gs.kv.data_ptr() + w * win], dtype=torch.int64, device="cuda"),
                 torch.tensor([gd.kv.data_ptr() + w * win], dtype=torch.int64, device="cuda")) for w in range(4)]
        turn = [0]

        def plain_contiguous():
            s_, d_ = wins[turn[0] % 4]
            turn[0] += 1
            B.copy_segments(s_, d_, tot, 1, stream=side)
        c_contig, _ = timed_steps(torch, side, plain_contiguous, args.steps, 2)
        # the same runs squeezed into a dense window on each side (block i of
        # the table -> the rank of its ID among the table's IDs), same queue step
        def dense_tables(tables, bs):
            used = [np.asarray(t[:-(-n // bs)], dtype=np.int64) for t, n in zip(tables, tokens)]
            ranks = np.argsort(np.argsort(np.concatenate(used))).astype(np.int32)
            cuts = np.cumsum([0] + [len(u) for u in used])
            return [ranks[cuts[i]:cuts[i + 1]] for i in range(len(used))]
        wplan = kvx.kvx_plan(gs.pool, gd.pool, tokens, dense_tables(wl.src_tables, wl.src.block_size),
                             dense_tables(wl.dst_tables, wl.dst.block_size), stream=side)

        wstep = QueueStep(kvx, side, [(wplan, l) for l in range(L)], ready)
        c_window, _ = timed_steps(torch, side, wstep, args.steps, 2)
        wstep.close()
        wplan.close()
        cl = step_bytes * args.steps / (c_layer * 1e-3) / 1e9
        cs = step_bytes * args.steps / (c_stream * 1e-3) / 1e9
        cw = step_bytes * args.steps / (c_window * 1e-3) / 1e9
        cc = step_bytes * args.steps / (c_contig * 1e-3) / 1e9
        ceiling = {
            "plain_copy_per_layer_GBs": round(cl, 1),
            "plain_copy_per_layer": f"{L} launches, one per layer: K and V each one contiguous segment of "
                                    f"{seg} B, one-wave workgroups of 32 KiB chunks",
            "plain_copy_streamed_GBs": round(cs, 1),
            "plain_copy_streamed": f"2 launches of {half} layers: the same segments as 4 KiB chunks of four-wave "
                                   f"workgroups (the launch shape of the queue's batched groups)",
            "plain_copy_contiguous_GBs": round(cc, 1),
            "plain_copy_contiguous": f"one launch per step: the step's {tot} read bytes as one contiguous segment of "
                                     f"each pool, 4 KiB chunks of four-wave workgroups (four rotating windows)",
            "value_over_plain_copy_contiguous": round(gbs / cc, 4),
            "dense_window_queue_GBs": round(cw, 1),
            "dense_window_queue": "the same runs renumbered into a dense window of each pool, same queue step",
            "value_over_plain_copy_streamed": round(gbs / cs, 4),
            "value_over_plain_copy_per_layer": round(gbs / cl, 4),
        }
        log(f"ceiling: plain copy per layer {cl:.1f}, streamed {cs:.1f}, contiguous {cc:.1f}, dense-window queue step "
        f"{cw:.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        layers = list(range(min(32, L)))
        src, dst = oracle_pools(wl, gs, gd, layers)
        t0 = time.perf_counter()
        oplan = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in
                                                 zip(tokens, wl.src_tables, wl.dst_tables)])
        setup = time.perf_counter() - t0
        cpu = cpu_baseline(f"oracle push (numpy copy of each triple) of {len(layers)} of {L} layers",
                           lambda: O.push(src, dst, oplan), len(layers) * sum(oplan.bytes_per_layer()),
                           args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s ({cpu['sample']})")

    step.close()
    plan.close()
    return {
        "value": gbs, "ms_per_step": ms_per_step, "dtype": "u8", "parity": parity, "span": stats,
        "config": {"workload": wl.name, "seed": wl.seed, "inputs_sha256_16": digest, "layers": L,
                   "kv_heads": wl.src.num_heads, "head_dim": wl.src.head_dim,
                   "block_size": wl.src.block_size, "payload_dtype": wl.src.dtype, "layout": wl.src.layout,
                   "prompt_tokens": wl.prompt_lens, "tokens_moved": tokens, "pool_blocks": wl.src.num_blocks,
                   "dst_block_size": wl.dst.block_size, "dst_pool_blocks": wl.dst.num_blocks,
                   "merged_runs": nruns, "triples_per_region": ntrip, "bytes_per_step": step_bytes,
                   "step": f"{L} x kvx_queue_push(layer, ready[layer]) then kvx_queue_flush on one side stream; "
                           f"each write goes out after its layer's (fired) event",
                   "launch_groups_per_step": round(groups_per_step, 3),
                   "kernel_launches_per_step": round(launches_per_step, 3),
                   "host_plan_ms": round(plan_ms, 3),
                   "push_layer_per_launch_GBs": round(layer_gbs, 1),
                   "push_layer_span_us_per_layer": round(lspan / args.steps * 1e3 / L, 3),
                   "push_layer_kernel_us_dispatch_stamps": round(layer_kernel_us, 3),
                   "fresh_event_push_layer_GBs": round(fresh_gbs, 1),
                   "graph_replay_push_layer_GBs": round(graph_gbs, 1),
                   "two_stream_push_layer_GBs": None if two_gbs is None else round(two_gbs, 1),
                   "push_many_all_layers_GBs": round(many_gbs, 1),
                   "cold_cache_steps": cold_stats},
        "ceiling": ceiling,
        "roofline": roofline(round(k_bytes), k_avg_us, "kvx::copy_many_kernel<0> (kvx_queue groups / kvx_push_many)",
                             args.workload,
                             {"layers_per_launch": min(L, 32),
                              "measured": f"dispatch timestamps of each launch: kvx_push_many_timed over {min(L, 32)} "
                                          f"layers (one launch), {-(-L // 32)} per step, 3 rounds",
                              "span_us_per_launch": round(ms_per_step * 1e3 / -(-L // 32), 3)}),
        "cpu_baseline": cpu,
    }


def bench_hybrid(args, torch, kvx, S, W):
    """Layer groups of other shapes (MLA, sliding window, state slots): one
    step pushes every model layer, in model order, from its group's plan."""
    wl = workload(W, args.workload, args)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    sides, plans, gbytes = [], [], []
    for gi, g in enumerate(wl.groups):
        gs, gd = S.group_side(g.src, wl.seed, 1 + 10 * gi), S.group_side(g.dst, wl.seed, 2 + 10 * gi)
        sides.append((gs, gd))
    torch.cuda.synchronize()
    digest = inputs_digest([t for g in wl.groups for t in g.src_tables + g.dst_tables],
                           [x for pair in sides for x in pair], wl.prompt_lens)
    plan_ms = 0.0
    for gi, g in enumerate(wl.groups):
        gs, gd = sides[gi]
        plans.append(kvx.kvx_plan(gs.pool, gd.pool, tokens, g.src_tables, g.dst_tables, stream=side))
        plan_ms += steady_plan_ms(kvx, gs.pool, gd.pool, tokens, g.src_tables, g.dst_tables, side)
    groups_cfg = []
    for gi, g in enumerate(wl.groups):
        rd, wr = plans[gi].bytes_per_layer()
        gbytes.append(rd + wr)
        nl = sum(1 for x, _ in wl.layer_map if x == gi)
        ntrip = [len(plans[gi].triples(0, r)) for r in range(2 if isinstance(g.src, W.StateSpec) else g.src.regions)]
        groups_cfg.append({"group": g.name, "layers": nl, "bytes_per_layer": rd + wr, "triples_per_region": ntrip,
                           "pool": repr(g.src)})
        log(f"group {g.name}: {nl} layers, {rd + wr} B per layer, triples per region {ntrip}")
    M = len(wl.layer_map)
    step_bytes = sum(gbytes[gi] for gi, _ in wl.layer_map)
    log(f"{M} model layers, {step_bytes} B per step, host plans {plan_ms:.2f} ms")

    if args.counters:   # the queue's launches once writes back up: kvx_push_many over every model layer
        pl, ly = [plans[gi] for gi, _ in wl.layer_map], [l for _, l in wl.layer_map]
        counters_run(torch, kvx, None, side, 1, step_bytes, launch=lambda _l: kvx.kvx_push_many(pl, ly, stream=side),
                     what="bytes_per_call")
        for p in plans:
            p.close()
        return None
    ready = [torch.cuda.Event() for _ in range(M)]
    for e in ready:
        e.record(compute)
    torch.cuda.synchronize()
    step = QueueStep(kvx, side, [(plans[gi], l) for gi, l in wl.layer_map], ready)

    # Verification step on the fresh pools, through the timed path: the first
    # and last layer of every group against the oracle.
    parity = None
    if not args.no_parity:
        import oracle as O
        sample = []
        for gi in range(len(wl.groups)):
            ls = [l for x, l in wl.layer_map if x == gi]
            sample += [(gi, ls[0]), (gi, ls[-1])]

        def snap(side_, layer):
            if isinstance(side_, S.StateSide):
                return [side_.regions[r][layer].cpu().numpy().copy() for r in range(2)], None
            ph = side_.spec.phys(layer)
            return ([side_.kv[ph, r].cpu().numpy().copy() for r in range(side_.spec.regions)],
                    [S.scale_bits(side_.sc[ph, r]).copy() for r in range(side_.spec.regions)]
                    if side_.sc is not None else None)
        snaps = {k: (snap(sides[k[0]][0], k[1]), snap(sides[k[0]][1], k[1])) for k in sample}
        step()
        torch.cuda.synchronize()
        bad, nbytes = [], 0
        for gi, l in sample:
            g = wl.groups[gi]
            reqs = [O.Request(n, a, b) for n, a, b in zip(tokens, g.src_tables, g.dst_tables)]
            if isinstance(g.src, W.StateSpec):
                op = O.make_state_plan(O.StateGeometry(g.src.num_layers, g.src.num_slots, tuple(g.src.slot_bytes)),
                                       O.StateGeometry(g.dst.num_layers, g.dst.num_slots, tuple(g.dst.slot_bytes)),
                                       reqs)
            else:
                op = O.make_plan(oracle_geom(O, g.src), oracle_geom(O, g.dst), reqs)
            (skv, ssc), (dkv, dsc) = snaps[(gi, l)]
            (gkv, gsc), (s_after, _) = snap(sides[gi][1], l), snap(sides[gi][0], l)
            for r in range(len(skv)):
                tr = op.triples[r] if isinstance(op, O.StatePlan) else op.triples
                exp = dkv[r].copy()
                O.push_region(skv[r], exp, tr)
                nbytes += exp.size
                if not np.array_equal(gkv[r], exp):
                    bad.append(f"group {g.name} layer {l} region {r}")
                if not np.array_equal(s_after[r], skv[r]):
                    bad.append(f"group {g.name} layer {l} region {r}: source changed")
                if ssc is not None:
                    es = dsc[r].copy()
                    O.push_scales(ssc[r], es, op.pairs)
                    if not np.array_equal(gsc[r], es):
                        bad.append(f"group {g.name} layer {l} region {r} scales")
        parity = parity_record(bad, "one step through kvx_queue on the fresh pools: every byte of the first and "
                                    "last layer of each group against the oracle", nbytes)
        del snaps

    span_ms, per_step, groups_per_step, launches_per_step = step.timed(torch, args.steps, args.warmup)
    ms_per_step = span_ms / args.steps
    gbs = step_bytes * args.steps / (span_ms * 1e-3) / 1e9
    stats = span_stats(per_step)
    log(f"queue step: span {span_ms:.3f} ms for {args.steps} steps ({ms_per_step * 1e3:.1f} us/step, median "
        f"{stats['median_ms'] * 1e3:.1f}); {launches_per_step:.2f} launches per step: {gbs:.1f} GB/s "
        f"= {100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f} GB/s")
    k_avg_us, k_bytes, k_launches = step.launch_us(torch)

    # Secondary: one kvx_push_layer launch per model layer.
    def layer_step():
        for i, (gi, l) in enumerate(wl.layer_map):
            kvx.kvx_push_layer(plans[gi], l, ready=ready[i], stream=side)
    lspan, _ = timed_steps(torch, side, layer_step, args.steps, 2)
    layer_gbs = step_bytes * args.steps / (lspan * 1e-3) / 1e9
    log(f"one kvx_push_layer launch per model layer: {layer_gbs:.1f} GB/s")

    # Per group: kvx_push_layer kernel durations from dispatch timestamps.
    n_chk = min(3, args.steps)
    per_group = {gi: [] for gi in range(len(wl.groups))}
    evs = []
    for _ in range(n_chk):
        for i, (gi, l) in enumerate(wl.layer_map):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            kvx.kvx_push_layer_timed(plans[gi], l, a, b, ready=ready[i], stream=side)
            evs.append((gi, a, b))
    torch.cuda.synchronize()
    for gi, a, b in evs:
        per_group[gi].append(a.elapsed_time(b) * 1e3)
    for gi, g in enumerate(wl.groups):
        us = float(np.mean(per_group[gi]))
        groups_cfg[gi]["push_layer_kernel_us_dispatch_stamps"] = round(us, 3)
        groups_cfg[gi]["push_layer_kernel_GBs"] = round(gbytes[gi] / (us * 1e-6) / 1e9, 1)
        log(f"group {g.name}: kvx_push_layer kernel {us:.2f} us per launch (dispatch stamps), "
            f"{groups_cfg[gi]['push_layer_kernel_GBs']} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        sample = list(range(min(8, M)))
        work = []
        setup = 0.0
        nbytes = 0
        for i in sample:
            gi, l = wl.layer_map[i]
            g = wl.groups[gi]
            gs, gd = sides[gi]
            reqs = [O.Request(n, s, d) for n, s, d in zip(tokens, g.src_tables, g.dst_tables)]
            t0 = time.perf_counter()
            if isinstance(g.src, W.StateSpec):
                geo = O.StateGeometry(1, g.src.num_slots, tuple(g.src.slot_bytes))
                src = O.StatePool(geo, [gs.regions[r][l:l + 1].cpu().numpy() for r in range(2)])
                dst = O.StatePool(geo, [gd.regions[r][l:l + 1].cpu().numpy() for r in range(2)])
                op = O.make_state_plan(geo, geo, reqs)
                work.append((O.push_state, src, dst, op))
            else:
                src, dst = oracle_pools(W.Workload(g.name, wl.seed, g.src, g.dst, [], [], []), gs, gd, [l])
                op = O.make_plan(src.geom, dst.geom, reqs)
                work.append((O.push, src, dst, op))
            setup += time.perf_counter() - t0
            nbytes += sum(op.bytes_per_layer())

        def one_pass():
            for fn, src, dst, op in work:
                fn(src, dst, op)
        cpu = cpu_baseline(f"oracle push of model layers {sample[0]}..{sample[-1]} of {M}", one_pass, nbytes,
                           args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s ({cpu['sample']})")

    step.close()
    for p in plans:
        p.close()
    return {
        "value": gbs, "ms_per_step": ms_per_step, "dtype": "u8", "parity": parity, "span": stats,
        "config": {"workload": wl.name, "seed": wl.seed, "inputs_sha256_16": digest, "model_layers": M,
                   "prompt_tokens": wl.prompt_lens, "tokens_moved": tokens,
                   "groups": groups_cfg, "bytes_per_step": step_bytes, "host_plan_ms": round(plan_ms, 3),
                   "step": f"{M} x kvx_queue_push in model order, then kvx_queue_flush, on one side stream; each "
                           f"write goes out after its layer's (fired) event",
                   "launch_groups_per_step": round(groups_per_step, 3),
                   "kernel_launches_per_step": round(launches_per_step, 3),
                   "push_layer_per_launch_GBs": round(layer_gbs, 1)},
        "roofline": roofline(round(k_bytes), k_avg_us, "kvx::copy_many_kernel<0> (kvx_queue groups)",
                             args.workload, {"measured": "dispatch timestamps of each launch (kvx_push_many_timed "
                                                         "over up to 32 layers of one layer group); bytes and "
                                                         f"duration per launch averaged over {k_launches} launches"}),
        "cpu_baseline": cpu,
    }


def two_stream_rate(torch, kvx, plan, ready, side, L, steps, step_bytes):
    """The step with layers alternating between two side streams (already-
    fired events): the next layer's workgroups fill in behind this layer's
    last ones.  Whole-step rate only: the kernels overlap, so no per-launch
    duration exists."""
    sides = [side, torch.cuda.Stream()]
    for _ in range(2):
        for l in range(L):
            kvx.kvx_push_layer(plan, l, ready=ready[l], stream=sides[l % 2])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(sides[0])
    sides[1].wait_event(a)
    for _ in range(steps):
        for l in range(L):
            kvx.kvx_push_layer(plan, l, ready=ready[l], stream=sides[l % 2])
    j = torch.cuda.Event()
    j.record(sides[1])
    sides[0].wait_event(j)
    b.record(sides[0])
    torch.cuda.synchronize()
    return step_bytes * steps / (a.elapsed_time(b) * 1e-3) / 1e9


def counters_run(torch, kvx, plan, side, L, bytes_per_launch, launch=None, what="bytes_per_launch"):
    """Kernels for a counter pass: kvxb_copy of CALIB_BYTES (known traffic:
    CALIB_BYTES read + CALIB_BYTES written) three times, then two steps of
    `launch(layer)` over every layer (default: the layerwise push).  The
    printed line gives the algorithmic bytes of each `launch` call, or of
    each kernel launch where those are all alike."""
    from decode_kv_cache_amd import bench_support as B
    if launch is None:
        def launch(l):
            kvx.kvx_push_layer(plan, l, stream=side)
    buf = torch.empty(2 * CALIB_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        B.copy(buf[CALIB_BYTES:], buf[:CALIB_BYTES], CALIB_BYTES, stream=side)
    for _ in range(2):
        for l in range(L):
            launch(l)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": True, "calib_copy_bytes": CALIB_BYTES, "calls": 2 * L,
                      what: bytes_per_launch}), flush=True)


def bench_batched(args, torch, kvx, S, W):
    """batched_push: 64 requests; layer l's push (kvx_push_layer on a side
    stream) waits for a synthetic compute kernel of layer l running
    concurrently on the compute stream.  The compute kernel spins on FMAs and
    then writes a canary into layer l's planned source blocks, so a push that
    did not wait for it is caught.  Ways of sharing the chip, each measured
    (push alone, compute alone, both):
      bounded    one compute workgroup per CU, so push workgroups co-reside
      full       the compute grid fills every CU's wave slots (as attention or
                 a GEMM does)
      full_split the full compute grid on a stream masked to 7/8 of the CUs,
                 the push on a stream masked to the other 1/8 (full_split4:
                 3/4 and 1/4)
    The line's value is the --compute-mode variant (default: bounded, the
    footprint of a tiled GEMM or attention kernel whose LDS tiles hold it to
    one workgroup per CU); every variant is measured and reported in the
    same line."""
    from decode_kv_cache_amd import bench_support as B
    wl = workload(W, "batched_push", args)
    gs, gd = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, stream=side)
    plan_ms = steady_plan_ms(kvx, gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, side)
    rd, wr = plan.bytes_per_layer()
    L = wl.src.num_layers
    step_bytes = (rd + wr) * L
    nruns = len(plan.runs())
    log(f"plan: {nruns} runs for {sum(tokens)} tokens, {rd + wr} B per layer, host plan {plan_ms:.1f} ms")
    if args.counters:   # --runs: the run-table plan's kernel instead
        cplan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, runs=True, stream=side) \
            if args.runs else plan
        counters_run(torch, kvx, cplan, side, L, rd + wr)
        plan.close()
        return None
    digest = inputs_digest(wl.src_tables + wl.dst_tables, [gs, gd], wl.prompt_lens)
    bb = wl.src.block_size * wl.src.num_heads * wl.src.head_dim * wl.src.elem_bytes
    used = np.concatenate([t[:-(-n // wl.src.block_size)] for t, n in zip(wl.src_tables, tokens)])
    blocks = torch.from_numpy(used.astype(np.int32)).cuda()
    props = torch.cuda.get_device_properties(0)
    ncu = props.multi_processor_count
    full_grid = ncu * props.max_threads_per_multi_processor // 256
    sink = torch.empty(full_grid * 256, dtype=torch.float32, device="cuda")
    ready = [torch.cuda.Event() for _ in range(L)]
    splits = {"full_split": max(1, ncu // 8), "full_split4": max(1, ncu // 4)}
    masked = {}

    def streams(mode):
        # CU masks must be contiguous ranges of CU indices here (the runtime
        # refuses interleaved ones): the push takes the top `split` CUs
        if mode not in splits:
            return compute, side
        if mode not in masked:
            split = splits[mode]
            masked[mode] = (B.CuMaskStream(range(ncu - split), ncu), B.CuMaskStream(range(ncu - split, ncu), ncu))
        return masked[mode][0].torch, masked[mode][1].torch

    def compute_layer(cs, grid, l, iters):
        B.layer_compute(sink, iters, grid, gs.region(l, 0), gs.region(l, 1), blocks, bb, 0xC0DE0000 + l,
                        stream=cs)

    def both_step(cs, ps, grid, iters):
        for l in range(L):
            compute_layer(cs, grid, l, iters)
            ready[l].record(cs)
            kvx.kvx_push_layer(plan, l, ready=ready[l], stream=ps)

    def measure(mode):
        cs, ps = streams(mode)
        grid = ncu if mode == "bounded" else full_grid

        def push_only():
            for l in range(L):
                kvx.kvx_push_layer(plan, l, stream=ps)
        push_only()
        with Timer(torch, ps) as t:
            for _ in range(args.steps):
                push_only()
        t_p = t.ms / args.steps
        # calibrate the compute kernel to about one layer's push time (five
        # launches timed after two untimed ones, so clock ramp-up does not skew it)
        probe = 4000 if grid > ncu else 20000
        for _ in range(2):
            compute_layer(cs, grid, 0, probe)
        with Timer(torch, cs) as t:
            for _ in range(5):
                compute_layer(cs, grid, 0, probe)
        iters = max(100, int(probe * (t_p / L) / (t.ms / 5)))

        def compute_only():
            for l in range(L):
                compute_layer(cs, grid, l, iters)
        compute_only()
        with Timer(torch, cs) as t:
            for _ in range(args.steps):
                compute_only()
        t_c = t.ms / args.steps
        both_step(cs, ps, grid, iters)
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        marks[0].record(cs)
        for i in range(args.steps):
            both_step(cs, ps, grid, iters)
            j = torch.cuda.Event()
            j.record(ps)
            cs.wait_event(j)
            marks[i + 1].record(cs)
        torch.cuda.synchronize()
        per = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)])
        t_b = marks[0].elapsed_time(marks[-1]) / args.steps
        eff = (t_c + t_p - t_b) / min(t_c, t_p)
        r = {"mode": mode, "compute_grid": grid, "compute_iters": iters,
             "push_cus": splits.get(mode, ncu), "compute_cus": ncu - splits.get(mode, 0),
             "push_alone_ms": round(t_p, 3), "push_alone_GBs": round(step_bytes / (t_p * 1e-3) / 1e9, 1),
             "compute_alone_ms": round(t_c, 3), "overlapped_ms": round(t_b, 3),
             "overlapped_GBs": round(step_bytes / (t_b * 1e-3) / 1e9, 1),
             "overlap_efficiency": round(eff, 3),
             "span": span_stats(per, "the overlapped steps, an event between consecutive steps")}
        log(f"{mode}: push alone {t_p:.2f} ms ({r['push_alone_GBs']} GB/s), compute alone {t_c:.2f} ms, "
            f"overlapped {t_b:.2f} ms -> {r['overlapped_GBs']} GB/s, overlap efficiency {eff:.2f}")
        return r, per

    mode = args.compute_mode
    # Verification step on the fresh pools, in the timed configuration: the
    # pushes run beside the compute kernels, each gated by its layer's event.
    parity = None
    if not args.no_parity:
        import oracle as O
        slabs = [0, wl.src.n_phys - 1]
        dst_snap = snap_layers(S, gd, slabs)
        cs, ps = streams(mode)
        both_step(cs, ps, ncu if mode == "bounded" else full_grid, 1000)
        torch.cuda.synchronize()
        # aliased logical layers rewrite a slab with the same bytes: the last
        # push of each slab read the source as its own compute left it, which
        # is the source as it stands now
        src_after = snap_layers(S, gs, slabs)
        parity = parity_push_layers(O, S, wl, gs, gd, src_after, dst_snap, tokens, slabs,
                                    f"one overlapped step ({mode} compute beside the pushes) on the fresh pools")
        del dst_snap, src_after

    results = {}
    for m in ("bounded", "full", "full_split", "full_split4"):
        if m == mode:
            continue
        results[m] = measure(m)[0]
    results[mode], per = measure(mode)
    main = results[mode]
    for pair in masked.values():
        for s_ in pair:
            s_.close()
    # Run tables instead of cut pieces (KVX_PLAN_RUNS), push alone, same pools.
    rplan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, runs=True, stream=side)
    rplan_ms = steady_plan_ms(kvx, gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, side, runs=True)

    def runs_only():
        for l in range(L):
            kvx.kvx_push_layer(rplan, l, stream=side)
    runs_only()
    with Timer(torch, side) as t:
        for _ in range(args.steps):
            runs_only()
    t_r = t.ms / args.steps
    run_table = {"taken": rplan.launch_shape()["run_table"], "host_plan_ms": round(rplan_ms, 3),
                 "worklist_bytes": worklist_bytes(rplan), "push_alone_ms": round(t_r, 3),
                 "push_alone_GBs": round(step_bytes / (t_r * 1e-3) / 1e9, 1),
                 "pieces_worklist_bytes": worklist_bytes(plan), "pieces_host_plan_ms": round(plan_ms, 3),
                 "pieces_push_alone_GBs": main["push_alone_GBs"],
                 "traffic_over_algorithmic": counter_ratio("batched_push", "run_kernel")}
    log(f"run tables: host plan {rplan_ms:.2f} ms (pieces {plan_ms:.2f}), work list {run_table['worklist_bytes']} B "
        f"(pieces {run_table['pieces_worklist_bytes']}), push alone {run_table['push_alone_GBs']} GB/s")
    rplan.close()
    # canary delivered: layer L-1's pushed destination holds its compute's canary
    d0 = int(wl.dst_tables[0][0])
    got = gd.region(L - 1, 0)[d0 * bb:d0 * bb + 4].cpu().numpy().view(np.uint32)[0]
    canary_ok = bool(got == ((0xC0DE0000 + L - 1) & 0xFFFFFFFF))
    t_b = main["overlapped_ms"]
    gbs = step_bytes / (t_b * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        layers = [0, 1]
        src, dst = oracle_pools(wl, gs, gd, layers)
        t0 = time.perf_counter()
        oplan = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in
                                                 zip(tokens, wl.src_tables, wl.dst_tables)])
        setup = time.perf_counter() - t0
        cpu = cpu_baseline(f"oracle push of {len(layers)} of {L} layers", lambda: O.push(src, dst, oplan),
                           len(layers) * sum(oplan.bytes_per_layer()), args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s")
    plan.close()
    return {
        "value": gbs, "ms_per_step": t_b, "dtype": "u8", "parity": parity, "span": span_stats(per),
        "config": {"workload": wl.name, "seed": wl.seed, "inputs_sha256_16": digest, "layers": L,
                   "physical_layer_slabs": wl.src.n_phys,
                   "kv_heads": wl.src.num_heads, "head_dim": wl.src.head_dim, "block_size": wl.src.block_size,
                   "payload_dtype": wl.src.dtype, "requests": len(tokens), "tokens_moved_total": int(sum(tokens)),
                   "pool_blocks": wl.src.num_blocks, "merged_runs": nruns, "bytes_per_step": step_bytes,
                   "step": f"{L} x (synthetic compute of layer l on the compute stream, its event, "
                           f"kvx_push_layer(l) on a side stream)",
                   "compute_mode": mode, "cu_sharing_knob": {
                       "bounded": "compute grid bounded to one workgroup per CU; no CU mask",
                       "full": "compute grid fills every CU's wave slots; no CU mask",
                       "full_split": f"CU masks: compute on {ncu - splits['full_split']} CUs, push on "
                                     f"{splits['full_split']}",
                       "full_split4": f"CU masks: compute on {ncu - splits['full_split4']} CUs, push on "
                                      f"{splits['full_split4']}"}[mode],
                   "variants": results, "canary_delivered": canary_ok, "host_plan_ms": round(plan_ms, 2),
                   "run_table_plan": run_table},
        "roofline": roofline(rd + wr, main["push_alone_ms"] * 1e3 / L, "kvx::copy_kernel<0> (kvx_push_layer)",
                             wl.name, {"note": "push alone on its stream, span over its launches"}),
        "cpu_baseline": cpu,
    }


def bench_tp4(args, torch, kvx, S, W):
    """tp4_share: TP4 rank 0's 2-head slice NHD -> HND of every layer: one
    head-slice write per layer through the side stream's write queue
    (kvx_queue_push_heads), then a flush."""
    wl = workload(W, "tp4_share", args)
    gs, gd = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    digest = inputs_digest(wl.src_tables + wl.dst_tables, [gs, gd], wl.prompt_lens)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, stream=side)
    L = wl.src.num_layers
    nh = wl.dst.num_heads
    rank = wl.extra["tp_rank"]
    row = wl.src.head_dim * wl.src.elem_bytes
    per_layer = 2 * 2 * sum(tokens) * nh * row   # K and V, read + write
    step_bytes = per_layer * L

    per_launch = min(L, 32)
    launches = -(-L // per_launch)
    q = kvx.Queue(side)

    def step():   # one head-slice write per layer through the queue
        for l in range(L):
            q.push_heads(plan, l, rank * nh, 0, nh)
        q.flush()

    def layers_step():   # every layer's share in one call, 32 layers per launch
        kvx.kvx_copy_heads_layers(plan, 0, L, rank * nh, 0, nh, stream=side)

    def layer_step():
        for l in range(L):
            kvx.kvx_copy_heads(plan, l, rank * nh, 0, nh, stream=side)
    if args.counters:
        counters_run(torch, kvx, plan, side, 1, per_layer * per_launch, launch=lambda _l: layers_step())
        q.close()
        plan.close()
        return None
    parity = None
    if not args.no_parity:   # verification step on the fresh pools against the oracle
        import oracle as O
        layers = [0, L - 1]
        pre_s, pre_d = snap_layers(S, gs, layers), snap_layers(S, gd, layers)
        step()
        torch.cuda.synchronize()
        reqs = [O.Request(n, a, b) for n, a, b in zip(tokens, wl.src_tables, wl.dst_tables)]
        op = O.make_plan(oracle_geom(O, wl.src), oracle_geom(O, wl.dst), reqs)
        sr, dr = O.head_rows(op, rank * nh, 0, nh, reqs)
        bad, nbytes = [], 0
        for l in layers:
            for kv in (0, 1):
                exp = pre_d[l][0][kv].copy()
                O.copy_heads_region(pre_s[l][0][kv], exp, wl.src.head_dim * wl.src.elem_bytes, sr, dr)
                got = gd.kv[l, kv].cpu().numpy()
                nbytes += got.size
                if not np.array_equal(got, exp):
                    bad.append(f"layer {l} region {kv}")
        parity = parity_record(bad, f"one step through kvx_queue_push_heads on the fresh pools: every byte of "
                                    f"layers {layers} of the consumer against the oracle's head transform "
                                    f"(TP rank {rank})", nbytes)
        del pre_s, pre_d
    span_ms, per_step = timed_steps(torch, side, step, args.steps, args.warmup)
    ms = span_ms / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    w0, g0, n0 = q.stats3()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    w1, g1, n1 = q.stats3()
    log(f"queue step: {ms * 1e3:.1f} us per step, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%), "
        f"{(n1 - n0) / args.steps:.2f} launches per step")
    mspan, _ = timed_steps(torch, side, layers_step, args.steps, 1)
    many_ms = mspan / args.steps
    many_gbs = step_bytes / (many_ms * 1e-3) / 1e9
    log(f"kvx_copy_heads_layers, {launches} launches of {per_launch} layers: {many_gbs:.1f} GB/s")
    lspan, _ = timed_steps(torch, side, layer_step, args.steps, 1)
    layer_gbs = step_bytes * args.steps / (lspan * 1e-3) / 1e9
    log(f"one kvx_copy_heads launch per layer: {layer_gbs:.1f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        layers = [0, 1, 2, 3]
        src, dst = oracle_pools(wl, gs, gd, layers)
        reqs = [O.Request(n, s, d) for n, s, d in zip(tokens, wl.src_tables, wl.dst_tables)]
        t0 = time.perf_counter()
        oplan = O.make_plan(src.geom, dst.geom, reqs)
        setup = time.perf_counter() - t0

        def one():
            for l in range(len(layers)):
                O.copy_heads(src, dst, oplan, reqs, l, rank * nh, 0, nh)
        cpu = cpu_baseline(f"oracle copy_heads (numpy row gather/scatter) of {len(layers)} of {L} layers", one,
                           len(layers) * per_layer, args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s")
    q.close()
    plan.close()
    return {
        "value": gbs, "ms_per_step": ms, "dtype": "u8", "parity": parity, "span": span_stats(per_step),
        "config": {"workload": wl.name, "seed": wl.seed, "inputs_sha256_16": digest, "layers": L,
                   "src": "NHD, 8 KV heads", "dst": f"HND, {nh} KV heads",
                   "tp_rank": rank, "tp_size": wl.extra["tp_size"], "head_dim": wl.src.head_dim,
                   "block_size": wl.src.block_size, "payload_dtype": wl.src.dtype, "requests": len(tokens),
                   "tokens_moved": tokens[0], "bytes_per_step": step_bytes,
                   "step": f"{L} x kvx_queue_push_heads(layer, rank {rank} slice) then kvx_queue_flush on one "
                           f"side stream; the writes have no pending events, so they leave in merged launches",
                   "kernel_launches_per_step": round((n1 - n0) / args.steps, 3),
                   "launch_groups_per_step": round((g1 - g0) / args.steps, 3),
                   "copy_heads_layers_GBs": round(many_gbs, 1),
                   "copy_heads_per_layer_GBs": round(layer_gbs, 1)},
        "roofline": roofline(per_layer * per_launch, many_ms * 1e3 / launches,
                             "kvx::heads_many_kernel (kvx_queue_push_heads groups / kvx_copy_heads_layers)",
                             wl.name, {"measured": f"span of back-to-back kvx_copy_heads_layers launches of "
                                                   f"{per_launch} layers"}),
        "cpu_baseline": cpu,
    }


def bench_multiturn(args, torch, kvx, S, W):
    """multiturn_fp8: turns 2..8, each copies every session's retained prefix
    (2048 (t-1) tokens, reused because it reaches the 512-token threshold)
    from the decode pool back to the prefill pool: every layer's write
    through the side stream's write queue, one flush per turn."""
    wl = workload(W, "multiturn_fp8", args)
    ex = wl.extra
    dec, pre = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    digest = inputs_digest(list(ex["decode_tables"]) + [t for k in sorted(ex["prefill_tables"])
                                                        for t in ex["prefill_tables"][k]], [dec, pre], wl.prompt_lens)
    side = torch.cuda.Stream()
    L = wl.src.num_layers
    plans, step_bytes, plan_ms = [], 0, 0.0
    for t in range(1, ex["turns"] + 1):
        reusable = ex["growth"] * (t - 1)
        if t == 1 or not kvx.kvx_should_reuse(reusable, ex["threshold"]):
            continue
        t0 = time.perf_counter()
        p = kvx.kvx_plan(dec.pool, pre.pool, [reusable] * ex["sessions"], ex["decode_tables"],
                         ex["prefill_tables"][t], runs=args.runs, stream=side)
        plan_ms += (time.perf_counter() - t0) * 1e3
        plans.append((t, p))
        step_bytes += sum(p.bytes_per_layer()) * L

    # The step: each turn's layers through the side stream's write queue (the
    # decode side holds every layer already, so the writes are ready at
    # once), then a flush: the turns write the same prefill pool, so each
    # turn's writes go out behind the previous turn's.
    q = kvx.Queue(side)

    def step():
        for _, p in plans:
            for l in range(L):
                q.push(p, l)
            q.flush()

    def layer_step():
        for _, p in plans:
            for l in range(L):
                kvx.kvx_push_layer(p, l, stream=side)
    if args.counters:   # a step's batched launches: kvx_push_many over every layer of each turn
        counters_run(torch, kvx, None, side, len(plans), step_bytes // len(plans),
                     launch=lambda i: kvx.kvx_push_many([plans[i][1]] * L, list(range(L)), stream=side),
                     what="bytes_per_call")
        q.close()
        for _, p in plans:
            p.close()
        return None
    parity = None
    if not args.no_parity:   # verification step: turns 2..8 replayed on the oracle for sampled layers
        import oracle as O
        layers = [0, L - 1]
        dsnap, psnap = snap_layers(S, dec, layers), snap_layers(S, pre, layers)
        step()
        torch.cuda.synchronize()
        g = oracle_geom(O, wl.src)
        state = {l: (psnap[l][0].copy(), psnap[l][1].copy()) for l in layers}
        for t, _ in plans:
            reqs = [O.reuse_request(t, ex["growth"], ex["threshold"], ex["decode_tables"][s_],
                                    ex["prefill_tables"][t][s_]) for s_ in range(ex["sessions"])]
            op = O.make_plan(g, g, reqs)
            for l in layers:
                for kv in (0, 1):
                    O.push_region(dsnap[l][0][kv], state[l][0][kv], op.triples)
                    O.push_scales(dsnap[l][1][kv], state[l][1][kv], op.pairs)
        bad, nbytes = [], 0
        for l in layers:
            got = pre.kv[l].cpu().numpy()
            nbytes += got.size
            if not np.array_equal(got, state[l][0]):
                bad.append(f"layer {l} payload")
            if not np.array_equal(S.scale_bits(pre.sc[l]), state[l][1]):
                bad.append(f"layer {l} scales")
            if not np.array_equal(dec.kv[l].cpu().numpy(), dsnap[l][0]):
                bad.append(f"layer {l}: decode pool changed")
        parity = parity_record(bad, f"one step through kvx_queue (turns {[t for t, _ in plans]}) on the fresh pools: every byte and "
                                    f"scale of prefill-pool layers {layers} against the oracle's turn-by-turn "
                                    f"replay", nbytes)
        del dsnap, psnap, state
    for _ in range(args.warmup):
        step()
    with Timer(torch, side) as t:
        for _ in range(args.steps):
            step()
    ms = t.ms / args.steps
    # per-turn spans: a second pass, an event behind each turn's flush
    nt = len(plans)
    w0, g0, n0 = q.stats3()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps * nt + 1)]
    marks[0].record(side)
    for i in range(args.steps):
        for j, (_, p) in enumerate(plans):
            for l in range(L):
                q.push(p, l)
            q.flush()
            marks[i * nt + j + 1].record(side)
    torch.cuda.synchronize()
    w1, g1, n1 = q.stats3()
    launches_per_step = (n1 - n0) / args.steps
    k_us, k_bytes, k_groups = launch_group_us(torch, kvx, side, [(p, l) for _, p in plans for l in range(L)])
    lspan, _ = timed_steps(torch, side, layer_step, args.steps, 1)
    layer_gbs = step_bytes * args.steps / (lspan * 1e-3) / 1e9
    log(f"queue: {launches_per_step:.1f} launches per step; batched launch groups {k_us:.1f} us each; "
        f"one kvx_push_layer launch per layer: {layer_gbs:.1f} GB/s")
    spans = np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps * nt)]).reshape(args.steps, nt)
    per_step = spans.sum(axis=1)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    turn_bytes = [sum(p.bytes_per_layer()) * L for _, p in plans]
    per_turn = [{"turn": t, "median_ms": round(float(np.median(spans[:, j])), 4),
                 "min_ms": round(float(spans[:, j].min()), 4), "p90_ms": round(float(np.percentile(spans[:, j], 90)), 4),
                 "GBs_at_median": round(turn_bytes[j] / (np.median(spans[:, j]) * 1e-3) / 1e9, 1)}
                for j, (t, _) in enumerate(plans)]
    log(f"multiturn: {ms:.2f} ms per step (turns {[t for t, _ in plans]}), {gbs:.1f} GB/s "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}%); per turn median ms {[x['median_ms'] for x in per_turn]}")
    # The other kind of work list (run tables or cut pieces), same pools and step.
    alt = []
    alt_ms = 0.0
    for t, _ in plans:
        t0 = time.perf_counter()
        alt.append(kvx.kvx_plan(dec.pool, pre.pool, [ex["growth"] * (t - 1)] * ex["sessions"], ex["decode_tables"],
                                ex["prefill_tables"][t], runs=not args.runs, stream=side))
        alt_ms += (time.perf_counter() - t0) * 1e3

    def alt_step():
        for p in alt:
            for l in range(L):
                kvx.kvx_push_layer(p, l, stream=side)
    alt_span, _ = timed_steps(torch, side, alt_step, args.steps, 1)
    alt_gbs = step_bytes * args.steps / (alt_span * 1e-3) / 1e9
    other = {"work_list": "cut pieces" if args.runs else "run tables (KVX_PLAN_RUNS)",
             "taken": [p.launch_shape()["run_table"] for p in alt],
             "GBs_one_launch_per_layer": round(alt_gbs, 1),
             "this_line_GBs_one_launch_per_layer": round(layer_gbs, 1),
             "host_plan_ms_all_turns": round(alt_ms, 2),
             "worklist_bytes": sum(worklist_bytes(p) for p in alt),
             "this_line_worklist_bytes": sum(worklist_bytes(p) for _, p in plans)}
    log(f"with {other['work_list']}: {alt_gbs:.1f} GB/s, host plans {alt_ms:.2f} ms (this line {plan_ms:.2f}), "
        f"work lists {other['worklist_bytes']} B (this line {other['this_line_worklist_bytes']})")
    for p in alt:
        p.close()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        layers = [0]
        src, dst = oracle_pools(wl, dec, pre, layers)
        t_last = plans[-1][0]
        t0 = time.perf_counter()
        reqs = [O.reuse_request(t_last, ex["growth"], ex["threshold"], ex["decode_tables"][s],
                                ex["prefill_tables"][t_last][s]) for s in range(ex["sessions"])]
        oplan = O.make_plan(src.geom, dst.geom, reqs)
        setup = time.perf_counter() - t0
        cpu = cpu_baseline(f"oracle push (payload + scales) of turn {t_last}, {len(layers)} of {L} layers",
                           lambda: O.push(src, dst, oplan), sum(oplan.bytes_per_layer()) * len(layers),
                           args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s")
    turns = [t for t, _ in plans]
    q.close()
    for _, p in plans:
        p.close()
    return {
        "value": gbs, "ms_per_step": ms, "dtype": "u8", "parity": parity,
        "span": span_stats(per_step, "a second pass of the steps, an event between consecutive turns"),
        "config": {"workload": wl.name, "seed": wl.seed, "inputs_sha256_16": digest, "layers": L,
                   "kv_heads": wl.src.num_heads, "head_dim": wl.src.head_dim, "per_turn": per_turn,
                   "work_list": "run tables (KVX_PLAN_RUNS)" if args.runs else "cut pieces",
                   "other_work_list": other,
                   "block_size": wl.src.block_size, "payload_dtype": wl.src.dtype, "scales": "fp32 per block",
                   "sessions": ex["sessions"], "turns_copied": turns, "threshold_tokens": ex["threshold"],
                   "bytes_per_step": step_bytes,
                   "step": f"turns 2..8: {L} x kvx_queue_push (decode -> prefill, no event) per turn, then "
                           f"kvx_queue_flush, on one side stream",
                   "kernel_launches_per_step": round(launches_per_step, 2),
                   "push_layer_per_launch_GBs": round(layer_gbs, 1),
                   "host_plan_ms_all_turns": round(plan_ms, 2)},
        "roofline": roofline(round(k_bytes), k_us, "kvx::copy_many_kernel<0> + kvx::scale_many_kernel<0> (kvx_queue "
                             "groups)", wl.name,
                             {"measured": f"dispatch timestamps of each launch group (kvx_push_many_timed over up to "
                                          f"32 layers of one turn: the payload launch and the small scale launch "
                                          f"behind it), {k_groups} groups per step, 3 rounds; sizes grow with the "
                                          f"turn"}),
        "cpu_baseline": cpu,
    }


def bench_pack(args, torch, kvx, S, W):
    """pack_unpack: the default workload's 64 layers gathered into a staging
    buffer and scattered from it into the consumer pool."""
    wl = workload(W, "qwen32b_push", args)
    gs, gd = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    digest = inputs_digest(wl.src_tables + wl.dst_tables, [gs, gd], wl.prompt_lens)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    side = torch.cuda.Stream()
    plan = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, stream=side)
    L = wl.src.num_layers
    nbytes = kvx.kvx_staging_bytes(plan, 0, L)
    stg = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    step_bytes = 4 * nbytes  # pack reads + writes nbytes, unpack reads + writes nbytes

    def step():
        kvx.kvx_pack(plan, 0, L, stg, stream=side)
        kvx.kvx_unpack(plan, 0, L, stg, stream=side)
    if args.counters:   # each of a step's 4 launches (32 layers) reads and writes nbytes / 2
        counters_run(torch, kvx, plan, side, 1, nbytes, launch=lambda _l: step())
        plan.close()
        return None
    parity = None
    if not args.no_parity:   # verification step: staging and consumer pool of sampled layers vs the oracle
        import oracle as O
        layers = [0, 37, L - 1]
        pre_s, pre_d = snap_layers(S, gs, layers), snap_layers(S, gd, layers)
        step()
        torch.cuda.synchronize()
        g1s, g1d = oracle_geom(O, wl.src, 1), oracle_geom(O, wl.dst, 1)
        op = O.make_plan(g1s, g1d, [O.Request(n, a, b) for n, a, b in zip(tokens, wl.src_tables, wl.dst_tables)])
        per = nbytes // L
        bad, cmp = [], 0
        for l in layers:
            src1 = O.Pool(g1s, pre_s[l][0][None], None)
            exp_stg = O.pack(src1, op, 0, 1)
            got_stg = stg[l * per:(l + 1) * per].cpu().numpy()
            cmp += got_stg.size
            if not np.array_equal(got_stg, exp_stg):
                bad.append(f"layer {l} staging")
            exp = O.Pool(g1d, pre_d[l][0][None].copy(), None)
            O.unpack(exp_stg, exp, op, 0, 1)
            got = gd.kv[l].cpu().numpy()
            cmp += got.size
            if not np.array_equal(got, exp.kv[0]):
                bad.append(f"layer {l} consumer pool")
        parity = parity_record(bad, f"one step on the fresh pools: staging of layers {layers} against the oracle's "
                                    f"pack, their consumer regions against the oracle's unpack", cmp)
        del pre_s, pre_d
    span_ms, per_step = timed_steps(torch, side, step, args.steps, args.warmup)
    ms = span_ms / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"pack+unpack: {ms * 1e3:.1f} us per step for {nbytes} staged bytes, {gbs:.1f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        layers = list(range(8))
        src, dst = oracle_pools(wl, gs, gd, layers)
        t0 = time.perf_counter()
        oplan = O.make_plan(src.geom, dst.geom, [O.Request(n, s, d) for n, s, d in
                                                 zip(tokens, wl.src_tables, wl.dst_tables)])
        setup = time.perf_counter() - t0

        def one():
            O.unpack(O.pack(src, oplan, 0, len(layers)), dst, oplan, 0, len(layers))
        cpu = cpu_baseline(f"oracle pack + unpack of {len(layers)} of {L} layers", one,
                           4 * O.staging_bytes(oplan, 0, len(layers)), args.cpu_seconds, setup)
        log(f"cpu baseline: {cpu['value']} GB/s")
    plan.close()
    # a plan without scales packs and unpacks up to 32 layers per launch (kvx.h)
    assert not wl.src.has_scales
    launches = 2 * -(-L // 32)
    return {
        "value": gbs, "ms_per_step": ms, "dtype": "u8", "parity": parity, "span": span_stats(per_step),
        "config": {"workload": "pack_unpack", "seed": wl.seed, "inputs_sha256_16": digest, "geometry": "qwen32b_push", "layers": L, "staging_bytes": nbytes,
                   "bytes_per_step": step_bytes,
                   "step": f"kvx_pack of {L} layers then kvx_unpack of {L} layers ({launches} launches)"},
        "roofline": roofline(step_bytes // launches, ms * 1e3 / launches,
                             "kvx::copy_many_kernel<1>/<2> (kvx_pack / kvx_unpack)", "pack_unpack"),
        "cpu_baseline": cpu,
    }


def bench_xfer(args, torch, kvx, S, W):
    """xfer_pipeline: batched_push's 64 requests driven through the transfer
    state machine: all requests prefilled, half registered up front and half
    after the forward pass (deferred writes); per layer one synthetic compute
    kernel then one save of that layer for all requests with the layer's
    event; seal; poll until every request is done.  Compared with the same
    bytes moved by one multi-request plan per layer."""
    from decode_kv_cache_amd import bench_support as B
    wl = workload(W, "batched_push", args)
    gs, gd = S.device_side(wl.src, wl.seed, 1), S.device_side(wl.dst, wl.seed, 2)
    digest = inputs_digest(wl.src_tables + wl.dst_tables, [gs, gd], wl.prompt_lens)
    tokens = [kvx.kvx_tokens_to_move(p, 0) for p in wl.prompt_lens]
    R, L = len(tokens), wl.src.num_layers
    side = torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    sink = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    bb = wl.src.block_size * wl.src.num_heads * wl.src.head_dim * wl.src.elem_bytes
    ref = kvx.kvx_plan(gs.pool, gd.pool, tokens, wl.src_tables, wl.dst_tables, stream=side)
    step_bytes = sum(ref.bytes_per_layer()) * L

    def run(step_no):
        x = kvx.Xfer(gs.pool, stream=side)
        t_host = 0.0
        now = float(step_no)
        for r in range(R):
            if r % 2 == 0:
                x.register(r, 0, gd.pool, wl.dst_tables[r], now)
            x.prefill(r, 0, tokens[r], wl.src_tables[r], now)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(compute)
        side.wait_event(a)
        for l in range(L):
            B.layer_compute(sink, 1000, 64, stream=compute)
            ev = torch.cuda.Event()
            ev.record(compute)
            t0 = time.perf_counter()
            x.save_layer_many(l, range(R), [0] * R, now, ready=ev)
            t_host += time.perf_counter() - t0
        for r in range(R):
            x.seal(r, 0)
        t0 = time.perf_counter()
        for r in range(1, R, 2):
            x.register(r, 0, gd.pool, wl.dst_tables[r], now)
        t_host += time.perf_counter() - t0
        j = torch.cuda.Event()
        j.record(side)
        compute.wait_event(j)
        b.record(compute)
        done = 0
        for _ in range(100):
            x.poll(now)
            done += len(x.pop_finished())
            if done == R:
                break
            torch.cuda.synchronize()
        if done != R:
            raise RuntimeError(f"xfer pipeline: {R - done} requests did not finish")
        ms = a.elapsed_time(b)
        x.close()
        return ms, t_host

    parity = None
    if not args.no_parity:   # the first run on the fresh pools: sampled slabs against the oracle
        import oracle as O
        slabs = [0, wl.src.n_phys - 1]
        pre_s, pre_d = snap_layers(S, gs, slabs), snap_layers(S, gd, slabs)
        run(0)
        torch.cuda.synchronize()
        parity = parity_push_layers(O, S, wl, gs, gd, pre_s, pre_d, tokens, slabs,
                                    "the first run through the transfer state machine on the fresh pools")
        del pre_s, pre_d
    else:
        run(0)
    res = [run(i + 1) for i in range(args.steps)]
    ms = float(np.mean([r[0] for r in res]))
    host_us = float(np.mean([r[1] for r in res])) * 1e6 / (R * L)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    # same bytes through one multi-request plan per layer, no state machine
    for l in range(L):
        kvx.kvx_push_layer(ref, l, stream=side)
    with Timer(torch, side) as t:
        for _ in range(args.steps):
            for l in range(L):
                kvx.kvx_push_layer(ref, l, stream=side)
    raw = step_bytes / (t.ms / args.steps * 1e-3) / 1e9
    log(f"xfer pipeline: {ms:.2f} ms per step, {gbs:.1f} GB/s; host {host_us:.2f} us per (request, layer) saved; "
        f"one plan per layer without the state machine: {raw:.1f} GB/s")
    ref.close()
    return {
        "value": gbs, "ms_per_step": ms, "dtype": "u8", "parity": parity, "span": span_stats([r[0] for r in res], "per step of the timed run (host-paced saves)"),
        "config": {"workload": "xfer_pipeline", "seed": wl.seed, "inputs_sha256_16": digest, "geometry": "batched_push", "requests": R, "layers": L,
                   "bytes_per_step": step_bytes,
                   "step": f"{R} requests x {L} layers through kvx_xfer (half registered after the forward pass), "
                           f"one synthetic compute kernel per layer",
                   "host_us_per_save": round(host_us, 3), "one_plan_per_layer_GBs": round(raw, 1)},
        "roofline": roofline(step_bytes // (R * L), ms * 1e3 / (R * L), "kvx::copy_many_kernel<0> (kvx_push_many via kvx_xfer)",
                             "xfer_pipeline", {"note": "per (request, layer) write, span of the whole step"}),
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen32b_push", choices=WORKLOAD_NAMES)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the verification step against the oracle")
    ap.add_argument("--runs", action="store_true",
                    help="batched_push --counters and multiturn_fp8: plans keep run tables (KVX_PLAN_RUNS)")
    ap.add_argument("--compute-mode", default="bounded", choices=["bounded", "full", "full_split", "full_split4"],
                    help="batched_push: how the compute stand-in shares the chip with the push")
    ap.add_argument("--counters", action="store_true",
                    help="short run for rocprofv3 --pmc: a 1 GiB plain copy (calibration) x3, then 2 steps")
    ap.add_argument("--seed", type=int, default=None, help="workload seed (default: the workload's own)")
    ap.add_argument("--tp-rank", type=int, default=None, choices=range(4), help="tp4_share: the TP4 rank timed")
    ap.add_argument("--phys-layers", type=int, default=None,
                    help="batched_push geometry: physical layer slabs behind the 64 layers (1..24, default 16)")
    args = ap.parse_args()
    if args.phys_layers is not None and not 1 <= args.phys_layers <= 24:
        print("bench.py: --phys-layers must be in 1..24 (each slab is 8 GiB over both pools)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py: libkvx runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the transfer shards per request, layer and head slice; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_kv_cache_amd import kvx
    from decode_kv_cache_amd import session as S
    from decode_kv_cache_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name} {getattr(dev, 'gcnArchName', '')} CUs={dev.multi_processor_count} "
        f"mem={dev.total_memory / 2**30:.0f} GiB; workload {args.workload}")
    fn = {"qwen32b_push": bench_push, "tiny_push": bench_push, "qwen32b_reblock": bench_push,
          "batched_push": bench_batched, "xfer_pipeline": bench_xfer,
          "tp4_share": bench_tp4, "multiturn_fp8": bench_multiturn, "pack_unpack": bench_pack,
          "dsr1_mla_push": bench_hybrid, "gptoss_swa_push": bench_hybrid,
          "qwen3next_state_push": bench_hybrid}[args.workload]
    if args.counters and fn is bench_xfer:
        print("bench.py: --counters is not available for xfer_pipeline", file=sys.stderr)
        sys.exit(2)
    r = fn(args, torch, kvx, S, W)
    if r is None:
        return
    # Every step copies: what it reads (payload and scales) it writes once.
    if "bytes_per_step" in r["config"]:
        r["config"]["bytes_read_per_step"] = r["config"]["bytes_written_per_step"] = r["config"]["bytes_per_step"] // 2
    out = {
        "metric": METRIC, "value": round(r["value"], 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": r["dtype"], "data": "synthetic",
        "pct_of_hbm_peak": round(100 * r["value"] / HBM_PEAK_GBS, 2),
        "parity": (r.get("parity") or {}).get("result", "skipped"), "parity_detail": r.get("parity"),
        "span": r.get("span"), "ceiling": r.get("ceiling"),
        "config": r["config"], "roofline": r["roofline"], "cpu_baseline": r["cpu_baseline"],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
