#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over one batch: the cache
append of every sequence's new token (slot_mapping write) followed by paged
decode attention over each sequence's context (the decode kernel, plus the
merge or reduction kernel when contexts are split), issued as one call
(pkv_paged_decode_attention_appending: the MFMA decode kernels write the
new rows themselves; before the vector kernel the append kernel runs
first).  The block tables,
context lengths and slot mapping come from the native block pool, built
before the timed region (its host cost per step is measured separately).

Per workload:
  - timed region: K steps back to back (nothing recorded between kernels);
    `value` = algorithmic KV bytes per step / mean step time;
  - profiled pass: at least 50 steps whose decode and merge/reduction kernels
    are bracketed by events their own dispatch stamps: the decode kernel
    alone, t_attn = decode + merge/reduction (the roofline figure), and the
    period between successive steps' decode starts, each as mean and
    p10/p50/p90;
  - the same step replayed from a HIP graph, and the streaming-read probe
    over the same byte count (the achievable read rate).

The headline is the 32K-token shared-prefix workload (the largest that fits
one GPU); the other decode workloads follow under "configs".  Prints one
JSON line.  Inputs are seeded synthetic data of the workloads' shapes.  To
keep every timed step reading cold HBM rather than the 256 MB Infinity Cache,
the caches are replicated and the steps rotate over the replicas.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c5_long_shared_bf16",
                    help="the headline workload (default: the 32K-token shared-prefix one, "
                         "the largest single-GPU workload)")
    ap.add_argument("--others", default="c2_qwen3_8b_bf16,c3_llama2_7b_f16,c4_llama3_70b_fp8,"
                                        "c6_llama3_70b_int8",
                    help="comma-separated workloads timed after the headline and reported "
                         "under 'configs' ('' for none)")
    ap.add_argument("--algo", default="auto", choices=["auto", "vector", "mfma"])
    ap.add_argument("--step", default="appending", choices=["appending", "two-calls"],
                    help="appending: one call that appends the new rows and decodes "
                         "(pkv_paged_decode_attention_appending; the MFMA decode kernels "
                         "write the rows themselves, the vector path launches the append "
                         "first); "
                         "two-calls: pkv_paged_cache_append, then the decode")
    ap.add_argument("--partition", type=int, default=-1, help="-1: the workload's own setting")
    ap.add_argument("--replicas", type=int, default=0, help="0: enough to exceed 4x the MALL")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time the multi-query workloads, swapping and prefix caching")
    ap.add_argument("--multiquery", action="store_true",
                    help="also time the multi-query workloads (prompt chunks, draft "
                         "verification) and add them under 'multiquery' (implied by "
                         "--all-configs)")
    ap.add_argument("--mq-only", default="",
                    help="time only this multi-query workload (a key of synth.MQ_CONFIGS) and "
                         "print its figures: for profiling one multi-query kernel")
    ap.add_argument("--swap", action="store_true",
                    help="also time swapping half the sequences to pinned host memory and "
                         "back (implied by --all-configs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (10 times): the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_elem_bytes(kv):
    return {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}[kv]


DT_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3, "int8": 4}
PROFILES = os.path.join(ROOT, "profiles")


# the source file that defines each decode kernel
KERNEL_FILES = {"decode_stream_kernel": "pkv_decode_stream.hip",
                "decode_split_merge_kernel": "pkv_decode_stream.hip",
                "decode_mfma_kernel": "pkv_decode_mfma.hip",
                "decode_vec_kernel": "pkv_decode_vec.hip",
                "decode_reduce_kernel": "pkv_decode_vec.hip",
                "cache_append_kernel": "pkv_append.hip",
                "multiquery_mfma_kernel": "pkv_multiquery.hip",
                "multiquery_stream_kernel": "pkv_multiquery.hip",
                "multiquery_reduce_kernel": "pkv_multiquery.hip",
                "multiquery_split_merge_kernel": "pkv_multiquery.hip"}


def kernel_source_hash(kernel):
    """sha256 over the file that defines `kernel` (with its launch code) and
    every header it includes, followed through csrc/ and include/: what a
    counter profile of that kernel was taken of.  Changes elsewhere in the
    library (other kernels, the host pool, argument checks) leave it alone."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "paged_kv_cache_363_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    seen, todo = [], [KERNEL_FILES[kernel]]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        path = next((os.path.join(d, name) for d in (csrc, inc)
                     if os.path.exists(os.path.join(d, name))), None)
        if path is None:
            continue   # a system header
        seen.append(name)
        with open(path, "rb") as f:
            todo += re.findall(rb'#include "([^"]+)"', f.read())
        todo = [t.decode() if isinstance(t, bytes) else t for t in todo]
    h = hashlib.sha256()
    for name in sorted(seen):
        path = next(os.path.join(d, name) for d in (csrc, inc) if os.path.exists(os.path.join(d, name)))
        with open(path, "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def decode_path(cfg, algo, partition):
    """(kernel name, kernel family, partition tokens) of the decode call a
    step makes; partition 0 = the balanced schedule."""
    import paged_kv_cache_363_amd as pkv
    kv = DT_CODE[cfg.kv_dtype]
    a = algo if algo != "auto" else pkv.decode_algo_for(cfg.num_q_heads, cfg.num_kv_heads,
                                                        cfg.head_dim, DT_CODE[cfg.q_dtype], kv)
    if a == "mfma" and partition == 0 and cfg.num_seqs <= 2048:
        return "decode_stream_kernel", a, 0
    # the fixed partition such a call uses (an f32 cache never takes the
    # balanced schedule, so the helper reports the fixed choice)
    ps = pkv.decode_partition_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                   cfg.max_blocks_per_seq, DT_CODE["f32"], partition)
    if a == "mfma" and ps < cfg.max_blocks_per_seq * 16 and cfg.num_seqs <= 2048:
        # several fixed partitions: the persistent grid in partition mode
        return "decode_stream_kernel", a, ps
    return ("decode_mfma_kernel" if a == "mfma" else "decode_vec_kernel"), a, ps


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter
    summary (profiles/<kernel>_<workload>_traffic.json), or None when there is
    none or the kernel's sources (kernel_source_hash) changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def setup(cfg, dev):
    import numpy as np
    import torch
    import paged_kv_cache_363_amd as pkv
    from synth import gen
    from synth.scenario import build_state, table_array

    ctx = gen.context_lens(cfg)
    nb = gen.num_blocks(cfg, ctx)
    pool = pkv.BlockPool(nb, cfg.block_size, gen.free_order(cfg, nb))
    t0 = time.perf_counter()
    st = build_state(cfg, pool, ctx)
    t_pool = time.perf_counter() - t0
    kv_t = {"fp8": torch.uint8, "int8": torch.int8}.get(cfg.kv_dtype) or gen.TORCH_DTYPE[cfg.kv_dtype]
    shape = (nb, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    kc = torch.zeros(shape, dtype=kv_t, device=dev)
    vc = torch.zeros(shape, dtype=kv_t, device=dev)
    k_scale, v_scale = gen.kv_scales(cfg, ctx)
    for s, p0, slots in st["prefill"]:
        if not slots:
            continue
        k, v = gen.seq_kv(cfg, s, p0 + len(slots))
        pkv.paged_cache_append(kc, vc, k[p0:].to(dev), v[p0:].to(dev),
                               torch.tensor(slots, dtype=torch.int64, device=dev),
                               k_scale, v_scale)
    kn, vn = gen.step_kv(cfg)
    torch.cuda.synchronize()
    return dict(ctx=ctx, nb=nb, pool=pool, state=st, k_cache=kc, v_cache=vc,
                block_tables=torch.from_numpy(table_array(cfg, st["tables"])).to(dev),
                context_lens=torch.from_numpy(ctx).to(dev), q=gen.queries(cfg).to(dev),
                k_new=kn.to(dev), v_new=vn.to(dev),
                slots=torch.from_numpy(st["step_slots"]).to(dev),
                k_scale=k_scale, v_scale=v_scale, t_pool_build=t_pool)


def host_bookkeeping_us(cfg, st):
    """Host time of one decode step's block bookkeeping (slots, new blocks,
    copy-on-write) for the whole batch: one pkv_batch_append_slots call on the
    decode layout, timed over successive steps from the workload's state."""
    import numpy as np
    import paged_kv_cache_363_amd as pkv
    from synth import gen
    from synth.scenario import build_state
    nb = st["nb"]
    ctx = st["ctx"]
    pool = pkv.BlockPool(nb, cfg.block_size, gen.free_order(cfg, nb))
    state = build_state(cfg, pool, ctx)
    reps = 20
    mb = cfg.max_blocks_per_seq + -(-reps // cfg.block_size) + 1
    rows = np.full((cfg.num_seqs, mb), -1, np.int32)
    for s, t in enumerate(state["tables"]):
        rows[s, :len(t)] = t
    nblk = np.array([len(t) for t in state["tables"]], np.int32)
    lens = np.asarray(ctx, np.int32).copy()
    slots = np.empty(cfg.num_seqs, np.int64)
    t0 = time.perf_counter()
    for _ in range(reps):
        pool.batch_append_slots(rows, nblk, lens, slot_mapping=slots)
    return (time.perf_counter() - t0) / reps * 1e6


PROBE_TILE = 4096   # bytes per tile of the streaming-read probe


def time_stream_probe(kv_bytes, R, K, dev):
    """The library's streaming-read probe over the workload's byte count: the
    read rate this GPU achieves for paged decode's access pattern (4 KiB tiles
    in a shuffled order, contiguous shares per wave, four tiles in flight).
    R disjoint regions of kv_bytes (rounded to whole tiles), each read in its
    own shuffled order and rotated like the cache replicas; the mean of K
    launches, each between two events its dispatch stamps, as the decode
    kernel is timed.
    Returns (ms per launch, GB/s)."""
    import torch
    import paged_kv_cache_363_amd as pkv
    nt = max(1, kv_bytes // PROBE_TILE)
    buf = torch.empty(R * nt * PROBE_TILE, dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4099)
    ids = [(torch.randperm(nt, device=dev, generator=gen) + r * nt).to(torch.int32)
           for r in range(R)]
    sink = torch.empty(256 * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(4):
        pkv.stream_read_probe(buf, ids[i % R], sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for pair in evs:       # create the underlying HIP events before handing them over
        for e in pair:
            e.record(stream)
    torch.cuda.synchronize()
    for i, pair in enumerate(evs):
        pkv.stream_read_probe(buf, ids[i % R], sink, events=pair)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / K
    del buf, ids, sink
    torch.cuda.empty_cache()
    return ms, nt * PROBE_TILE / (ms * 1e-3) / 1e9


def pct(xs, q):
    """q-th percentile (0..100) of xs, linear interpolation."""
    import numpy as np
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def summary_ms(xs):
    return {"mean": round(sum(xs) / len(xs), 5), "p10": round(pct(xs, 10), 5),
            "p50": round(pct(xs, 50), 5), "p90": round(pct(xs, 90), 5), "n": len(xs)}


PROFILE_STEPS = 50   # steps of the profiled pass (percentiles), at least


def time_config(cfg, args, dev, partition, with_cpu=True):
    import numpy as np
    import torch
    import paged_kv_cache_363_amd as pkv

    log(f"setup {cfg.name}")
    st = setup(cfg, dev)
    log("setup done")
    eb = kv_elem_bytes(cfg.kv_dtype)
    ctx = st["ctx"].astype(np.int64)
    kv_bytes = int(ctx.sum()) * 2 * cfg.num_kv_heads * cfg.head_dim * eb
    cache_bytes = 2 * st["k_cache"].numel() * st["k_cache"].element_size()
    R = args.replicas or max(1, min(8, math.ceil(4 * MALL_BYTES / max(kv_bytes, 1))))
    kcs, vcs = [st["k_cache"]], [st["v_cache"]]
    for _ in range(R - 1):
        kcs.append(st["k_cache"].clone())
        vcs.append(st["v_cache"].clone())
    ps = partition
    if ps == 0 and args.algo == "auto":
        # the schedule a serving loop would pick from its host-side lengths
        ps = pkv.decode_partition_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                       cfg.head_dim, cfg.max_blocks_per_seq,
                                       DT_CODE[cfg.kv_dtype], 0, context_lens=st["ctx"])
    kernel, algo, part = decode_path(cfg, args.algo, ps)
    has_reduce = kernel == "decode_stream_kernel" or part < cfg.max_blocks_per_seq * 16
    ws = pkv.alloc_workspace(st["q"], st["k_cache"], st["block_tables"], ps)
    out = torch.empty_like(st["q"])
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        r = i % R
        if args.step == "two-calls":
            pkv.paged_cache_append(kcs[r], vcs[r], st["k_new"], st["v_new"], st["slots"],
                                   st["k_scale"], st["v_scale"])
            pkv.paged_decode_attention(st["q"], kcs[r], vcs[r], st["block_tables"],
                                       st["context_lens"], cfg.scale, st["k_scale"],
                                       st["v_scale"], partition_size=ps, out=out, workspace=ws,
                                       algo=args.algo, events=evs)
        else:
            pkv.paged_decode_attention_appending(
                st["q"], st["k_new"], st["v_new"], st["slots"], kcs[r], vcs[r],
                st["block_tables"], st["context_lens"], cfg.scale, st["k_scale"], st["v_scale"],
                partition_size=ps, out=out, workspace=ws, algo=args.algo, events=evs)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done ({R} replicas)")
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # Timed region: K whole steps back to back, nothing recorded between the
    # kernels (an event record on the stream costs ~3 us of GPU time).
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    step_ms = total_ms / K
    # Profiled pass: at least PROFILE_STEPS steps, each decode kernel launched
    # with start/stop events its own dispatch stamps (no event records between
    # the kernels), and the merge/reduction kernel's end stamped the same way.
    # Per step: the decode kernel alone, t_attn = decode + merge/reduction, and
    # the period from one step's decode start to the next one's (one append,
    # decode and merge each): the step time distribution.
    Kp = max(K, PROFILE_STEPS)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(Kp)]
    for trio in evs:       # create the underlying HIP events before handing them over
        for e in trio:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(Kp):
        a, b, c = evs[i]
        step(i, (a, b, c if has_reduce else None))
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b, _ in evs]
    attn_ms = ([a.elapsed_time(c) for a, _, c in evs] if has_reduce else list(dec_ms))
    red_ms = [x - y for x, y in zip(attn_ms, dec_ms)]
    period_ms = [evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(Kp - 1)]
    # The same steps captured into one HIP graph and replayed (the launch
    # path a serving loop can use; every kernel here is capturable).  Each
    # graph launch leaves the GPU idle for several microseconds before the
    # graph's first kernel (kernel trace of the Qwen3-8B-shaped step: 8.4 us,
    # against none between eager launches or inside a graph), so one graph
    # holds G >= 8 steps, rotating over the cache replicas, and the figure
    # is per step.
    g_step_ms = None
    G = R * -(-8 // R)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(G):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-K // G))
        t_start.record(stream)
        for _ in range(reps):
            graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        g_step_ms = t_start.elapsed_time(t_end) / (reps * G)
        del graph
    except RuntimeError as e:   # reported, never silently replaced
        log(f"graph capture failed: {e}")
    dec_avg = sum(dec_ms) / Kp
    attn_avg = sum(attn_ms) / Kp
    probe_ms, probe_gbs = time_stream_probe(kv_bytes, R, K, dev)
    log(f"streaming-read probe: {probe_ms:.4f} ms, {probe_gbs:.1f} GB/s")
    res = dict(
        config=cfg.name, kv_bytes=kv_bytes, replicas=R, cache_bytes_per_replica=cache_bytes,
        kernel=kernel, algo=algo, partition=part, has_reduce=has_reduce,
        ms_per_step=step_ms, wall_ms_per_step=wall / K * 1e3,
        decode_kernel_ms=dec_avg, reduce_kernel_ms=attn_avg - dec_avg, t_attn_ms=attn_avg,
        decode_ms_stats=summary_ms(dec_ms), t_attn_ms_stats=summary_ms(attn_ms),
        reduce_ms_stats=summary_ms(red_ms), step_period_ms_stats=summary_ms(period_ms),
        step_gbs=kv_bytes / (step_ms * 1e-3) / 1e9,
        graph_ms_per_step=g_step_ms, graph_steps=G,
        decode_kernel_gbs=kv_bytes / (dec_avg * 1e-3) / 1e9,
        t_attn_gbs=kv_bytes / (attn_avg * 1e-3) / 1e9,
        tokens_per_s=cfg.num_seqs / (step_ms * 1e-3),
        probe_ms=probe_ms, probe_gbs=probe_gbs,
        t_pool_build_s=st["t_pool_build"])
    log(f"timed {K} steps: {step_ms:.4f} ms/step; {Kp} profiled: decode kernel "
        f"{dec_avg:.4f} ms, decode + merge/reduction {attn_avg:.4f} ms")
    res["host_bookkeeping_us_per_step"] = host_bookkeeping_us(cfg, st)
    if with_cpu and args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(cfg, st, args.cpu_budget, out)
        log("cpu baseline done")
    del kcs, vcs, ws, out, st
    torch.cuda.empty_cache()
    return res


def roofline_obj(cfg, res):
    """The roofline object of one workload: t_attn (decode kernel + merge or
    reduction) against the HBM peak on the algorithmic KV bytes, with the
    decode kernel's own fraction beside it and the counter traffic of the
    decode kernel (and of the reduction, when one runs)."""
    traffic = measured_traffic(cfg.name, res["kernel"])
    red_kernel = reduce_kernel_of(res)
    red_traffic = measured_traffic(cfg.name, red_kernel) if red_kernel else None
    return {"bound": "hbm", "achieved": round(res["t_attn_gbs"], 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(res["t_attn_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": res["kernel"] + (f" + {red_kernel}" if red_kernel else ""),
            "t_attn_ms": round(res["t_attn_ms"], 5),
            "decode_kernel_ms": round(res["decode_kernel_ms"], 5),
            "reduce_kernel_ms": round(res["reduce_kernel_ms"], 5),
            "decode_only_frac": round(res["decode_kernel_gbs"] / HBM_PEAK_GBS, 4),
            "decode_only_gbs": round(res["decode_kernel_gbs"], 2),
            "reduce_traffic": red_traffic,
            "algorithmic_bytes_per_launch": res["kv_bytes"],
            "pct_of_peak": round(100 * res["t_attn_gbs"] / HBM_PEAK_GBS, 2),
            "target_pct": 70.0 if cfg.name in LONG_CONTEXT else None}


def reduce_kernel_of(res):
    """The merge or reduction kernel a step runs after the decode kernel."""
    if not res["has_reduce"]:
        return None
    if res["kernel"] == "decode_stream_kernel" and res["partition"] == 0:
        return "decode_split_merge_kernel"
    return "decode_reduce_kernel"


# the workloads the 70%-of-peak bar applies to (long contexts)
LONG_CONTEXT = ("c2_qwen3_8b_bf16", "c4_llama3_70b_fp8", "c5_long_shared_bf16")


def config_obj(cfg, res):
    """One workload's figures for the JSON line."""
    return {"workload": cfg.name, "description": cfg.description, "algo": res["algo"],
            "kernel": res["kernel"], "partition": res["partition"],
            "kv_bytes_per_step": res["kv_bytes"],
            "step_gbs": round(res["step_gbs"], 2),
            "pct_hbm_peak_step": round(100 * res["step_gbs"] / HBM_PEAK_GBS, 2),
            "ms_per_step": round(res["ms_per_step"], 5),
            "decode_tokens_per_s": round(res["tokens_per_s"], 1),
            "roofline": roofline_obj(cfg, res),
            "decode_kernel_ms": res["decode_ms_stats"],
            "t_attn_ms": res["t_attn_ms_stats"],
            "step_period_ms": res["step_period_ms_stats"],
            "graph_ms_per_step": (round(res["graph_ms_per_step"], 5)
                                  if res["graph_ms_per_step"] else None),
            "achievable_read_gbs": round(res["probe_gbs"], 2),
            "t_attn_frac_of_achievable": round(res["t_attn_gbs"] / res["probe_gbs"], 4),
            "replicas": res["replicas"]}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/f16 MFMA, published peak


def time_multiquery(mq, args, dev):
    """One multi-query call (several rows per sequence attending causally) on
    a decode workload's cache: K calls back to back, then a pass with events
    around the attention kernel.  Algorithmic bytes: every context token's K
    and V once; flops: 4 d per (row, q-head, visible token)."""
    import numpy as np
    import torch
    import paged_kv_cache_363_amd as pkv
    from synth import CONFIGS, gen
    cfg = CONFIGS[mq.base]
    log(f"setup {mq.name}")
    st = setup(cfg, dev)
    pkv.paged_cache_append(st["k_cache"], st["v_cache"], st["k_new"], st["v_new"], st["slots"],
                           st["k_scale"], st["v_scale"])
    ctx = st["ctx"].astype(np.int64)
    ql = gen.query_lens(mq, st["ctx"])
    qs = gen.query_start(ql)
    rows = int(qs[-1])
    q = gen.mq_queries(mq, cfg, rows).to(dev)
    qs_dev = torch.from_numpy(qs).to(dev)
    max_q = int(ql.max(initial=0))
    eb = kv_elem_bytes(cfg.kv_dtype)
    kv_bytes = int(ctx.sum()) * 2 * cfg.num_kv_heads * cfg.head_dim * eb
    visible = sum(int(ctx[s]) * int(ql[s]) - int(ql[s]) * (int(ql[s]) - 1) // 2
                  for s in range(cfg.num_seqs))      # sum over rows of (position + 1)
    flops = 4 * cfg.head_dim * cfg.num_q_heads * visible
    R = max(1, min(8, math.ceil(4 * MALL_BYTES / max(kv_bytes, 1))))
    kcs, vcs = [st["k_cache"]], [st["v_cache"]]
    for _ in range(R - 1):
        kcs.append(st["k_cache"].clone())
        vcs.append(st["v_cache"].clone())
    # the host planner weighs the balanced schedule against one fixed pass
    # with the batch's lengths, as a serving loop holding them would
    ps = pkv.multiquery_partition_size(cfg.num_seqs, max_q, cfg.num_q_heads, cfg.num_kv_heads,
                                       cfg.max_blocks_per_seq, 0, context_lens=st["ctx"],
                                       kv_dtype=DT_CODE[cfg.kv_dtype])
    n = pkv.multiquery_workspace_size(rows, cfg.num_seqs, max_q, cfg.num_q_heads,
                                      cfg.num_kv_heads, cfg.head_dim, cfg.max_blocks_per_seq, ps)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def call(i, evs=None):
        r = i % R
        pkv.paged_multiquery_attention(q, kcs[r], vcs[r], st["block_tables"], st["context_lens"],
                                       qs_dev, max_q, cfg.scale, st["k_scale"], st["v_scale"],
                                       partition_size=ps, out=out, workspace=ws, events=evs)

    for i in range(max(2, args.warmup // 4)):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call(0)
    torch.cuda.synchronize()
    K = max(3, min(args.steps, int(2.0 / max(time.perf_counter() - t0, 1e-6))))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(K):
        call(i)
    b.record(stream)
    torch.cuda.synchronize()
    call_ms = a.elapsed_time(b) / K
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for trio in evs:
        for e in trio:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        call(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = sum(x.elapsed_time(y) for x, y, _ in evs) / K
    red_ms = sum(y.elapsed_time(z) for _, y, z in evs) / K
    gbs = kv_bytes / (kern_ms * 1e-3) / 1e9
    tflops = flops / (kern_ms * 1e-3) / 1e12
    mfma_bound = flops / kv_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
            if mfma_bound else
            {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)})
    log(f"{mq.name}: {K} calls, {call_ms:.4f} ms/call, attention kernel {kern_ms:.4f} ms")
    res = {"description": mq.description, "rows": rows, "max_rows_per_seq": max_q,
           "partition": ps, "ms_per_call": round(call_ms, 5), "kernel_ms": round(kern_ms, 5),
           "reduce_ms": round(red_ms, 5), "rows_per_s": round(rows / (call_ms * 1e-3), 1),
           "kv_gbs_call": round(kv_bytes / (call_ms * 1e-3) / 1e9, 2),
           "kv_gbs_kernel": round(gbs, 2), "tflops_kernel": round(tflops, 2),
           "flop_per_byte": round(flops / kv_bytes, 2), "kv_bytes": kv_bytes, "flops": flops,
           "calls": K, "replicas": R, "roofline": roof}
    del kcs, vcs, st
    torch.cuda.empty_cache()
    return res


def time_swap(cfg, args, dev):
    """Swap half of the workload's sequences to pinned host memory and back
    (pkv_seq_swap bookkeeping, pkv_swap_blocks copies): GB/s each way over the
    K and V bytes moved, each direction timed over several repetitions."""
    import torch
    import paged_kv_cache_363_amd as pkv
    log(f"setup swap {cfg.name}")
    st = setup(cfg, dev)
    pool, tables = st["pool"], st["state"]["tables"]
    moved = list(range(0, cfg.num_seqs, 2))
    n = sum(len(tables[s]) for s in moved)
    host = pkv.BlockPool(n, cfg.block_size)
    shape = (n,) + tuple(st["k_cache"].shape[1:])
    hk = torch.empty(shape, dtype=st["k_cache"].dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=st["k_cache"].dtype, pin_memory=True)
    t0 = time.perf_counter()
    out_pairs, host_tables = [], {}
    for s in moved:
        host_tables[s], pr = pool.seq_swap(host, tables[s])
        out_pairs += pr
    t_book = time.perf_counter() - t0
    p_out = torch.tensor(out_pairs, dtype=torch.int32, device=dev)
    p_in = torch.tensor([(b, a) for a, b in out_pairs], dtype=torch.int32, device=dev)
    block_bytes = st["k_cache"][0].numel() * st["k_cache"].element_size()
    moved_bytes = 2 * n * block_bytes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    reps = 5
    pkv.swap_blocks(hk, hv, st["k_cache"], st["v_cache"], p_out)
    pkv.swap_blocks(st["k_cache"], st["v_cache"], hk, hv, p_in)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        pkv.swap_blocks(hk, hv, st["k_cache"], st["v_cache"], p_out)
    ev[1].record()
    for _ in range(reps):
        pkv.swap_blocks(st["k_cache"], st["v_cache"], hk, hv, p_in)
    ev[2].record()
    torch.cuda.synchronize()
    out_ms = ev[0].elapsed_time(ev[1]) / reps
    in_ms = ev[1].elapsed_time(ev[2]) / reps
    res = {"workload": cfg.name, "sequences": len(moved), "blocks": n,
           "bytes_each_way": moved_bytes,
           "out_ms": round(out_ms, 4), "in_ms": round(in_ms, 4),
           "out_gbs": round(moved_bytes / (out_ms * 1e-3) / 1e9, 2),
           "in_gbs": round(moved_bytes / (in_ms * 1e-3) / 1e9, 2),
           "host_bookkeeping_ms": round(t_book * 1e3, 3)}
    log(f"swap: {res['out_gbs']} GB/s out, {res['in_gbs']} GB/s in")
    del hk, hv, st
    torch.cuda.empty_cache()
    return res


def time_prefix_cache(cfg):
    """Host cost of prefix-cached table creation on a shared-prefix workload:
    the first request's prompt blocks are registered, then every request
    (prefix + its own tail) is created through the cache and released, over
    several rounds.  Reports the tokens served from the cache and the host
    microseconds per request."""
    import numpy as np
    import paged_kv_cache_363_amd as pkv
    from synth import gen
    ctx = gen.context_lens(cfg)
    P = cfg.shared_prefix
    rs = np.random.default_rng(cfg.seed)
    prefix = [int(x) for x in rs.integers(0, 32000, P)]
    prompts = [prefix + [int(x) for x in rs.integers(0, 32000, int(ctx[s]) - 1 - P)]
               for s in range(cfg.num_seqs)]
    nb = gen.num_blocks(cfg, ctx)
    pool = pkv.BlockPool(nb, cfg.block_size, gen.free_order(cfg, nb))
    toks = [np.asarray(t, np.int32) for t in prompts]
    first, _ = pool.seq_create_cached(toks[0], len(prompts[0]), cfg.max_blocks_per_seq)
    pool.register_blocks(toks[0], len(prompts[0]), first)
    pool.seq_free(first)
    rounds, hit_tokens, total_tokens = 5, 0, 0
    t0 = time.perf_counter()
    for _ in range(rounds):
        tables = []
        for t in toks:
            tab, c = pool.seq_create_cached(t, len(t), cfg.max_blocks_per_seq)
            hit_tokens += c
            total_tokens += len(t)
            tables.append(tab)
        for tab in tables:
            pool.seq_free(tab)
    dt = time.perf_counter() - t0
    n = rounds * len(toks)
    return {"workload": cfg.name, "requests": n, "shared_prefix_tokens": P,
            "cached_token_fraction": round(hit_tokens / total_tokens, 4),
            "host_us_per_request": round(dt / n * 1e6, 2),
            "cached_blocks": pool.cached_blocks()}


def cpu_baseline(cfg, st, budget_s, gpu_out):
    """The fp64 oracle on the host, two legs on the same workload's sequences
    (longest context first):
      - single-threaded, on a bounded sample (until budget_s is spent);
      - each sequence's rows (one per q-head) shared among the host's
        threads (oracle.default_threads: OMP_NUM_THREADS, else the CPU
        count, at most 16), on as many sequences as fit the same budget.
    Reported: oracle KV GB/s and decode tokens/s per leg.  The rows the
    oracle computed are compared with the GPU output of the timed steps."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from harness import allclose_report, oracle_setup
    from oracle import oracle as orc
    from synth import gen
    ctx = st["ctx"]
    order = [int(s) for s in np.argsort(-ctx, kind="stable")]
    o = oracle_setup(cfg, order)
    qb = gen.bits(o["q"])
    eb = kv_elem_bytes(cfg.kv_dtype)
    per_seq = [int(ctx[s]) * 2 * cfg.num_kv_heads * cfg.head_dim * eb for s in range(cfg.num_seqs)]
    worst, ok_all = 0.0, True

    def run(seqs, threads):
        nonlocal worst, ok_all
        t0 = time.perf_counter()
        ref = orc.paged_decode(qb[seqs], cfg.q_dtype, o["k_cache"], o["v_cache"], cfg.kv_dtype,
                               o["block_tables"][seqs], o["ctx"][seqs], cfg.scale, o["k_scale"],
                               o["v_scale"], threads=threads)
        dt = time.perf_counter() - t0
        got = gpu_out[seqs].float().cpu().numpy().astype(np.float64)
        ok, _, err = allclose_report(got, ref, 2e-3, 1e-2)
        ok_all &= ok
        worst = max(worst, err)
        return dt

    # single thread: one sequence at a time until the budget is spent
    done, t1 = 0, 0.0
    for s in order:
        t1 += run([s], 1)
        done += 1
        if t1 >= budget_s:
            break
    b1 = sum(per_seq[s] for s in order[:done])
    # all threads: one sequence per call (its H_q rows shared among them),
    # longest first, until the same budget is spent
    nt = orc.default_threads()
    doneN, tN = 0, 0.0
    for s in order:
        tN += run([s], nt)
        doneN += 1
        if tN >= budget_s:
            break
    bN = sum(per_seq[s] for s in order[:doneN])
    return {"value": round(bN / tN / 1e9, 4), "unit": "GB/s", "cores": nt, "kind": "oracle",
            "tokens_per_s": round(doneN / tN, 3),
            "sample": f"{doneN} of {cfg.num_seqs} sequences of {cfg.name} (longest first), all "
                      f"q-heads, {tN:.1f} s of fp64 oracle with its rows shared among {nt} "
                      f"threads",
            "single_thread": {
                "value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                "tokens_per_s": round(done / t1, 3),
                "sample": f"{done} of {cfg.num_seqs} sequences of {cfg.name} (longest first), "
                          f"all q-heads, {t1:.1f} s of single-threaded fp64 oracle"},
            "gpu_rows_match_oracle": ok_all, "max_abs_err": worst}


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, ten times: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the counter's scale
    (2^30 bytes read and written per dispatch)."""
    import torch
    n = 2 ** 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 10}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the decode path has "
                                   "no multi-GPU mode in this build", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import paged_kv_cache_363_amd as pkv  # noqa: F401  (fails loudly if libpkv.so is missing)
    from synth import CONFIGS
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = "cuda:0"
    if args.mq_only:
        from synth import MQ_CONFIGS
        res = time_multiquery(MQ_CONFIGS[args.mq_only], args, dev)
        print(json.dumps({"multiquery_workload": args.mq_only, **res}), flush=True)
        return
    cfg = CONFIGS[args.config]
    ps = cfg.partition_size if args.partition < 0 else args.partition
    res = time_config(cfg, args, dev, ps)
    line = {
        "metric": "paged-decode effective KV GB/s (% of MI355X HBM peak) and decode tokens/s",
        "value": round(res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype if cfg.kv_dtype == cfg.q_dtype else f"{cfg.q_dtype}+{cfg.kv_dtype}-kv",
        "data": "synthetic",
        "config": {"workload": cfg.name, "description": cfg.description,
                   "num_seqs": cfg.num_seqs, "num_q_heads": cfg.num_q_heads,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "partition": res["partition"],
                   "algo": res["algo"], "kv_bytes_per_step": res["kv_bytes"],
                   "replicas": res["replicas"], "step": args.step},
        "decode_tokens_per_s": round(res["tokens_per_s"], 1),
        "pct_hbm_peak_step": round(100 * res["step_gbs"] / HBM_PEAK_GBS, 2),
        "roofline": roofline_obj(cfg, res),
        "step_period_ms": res["step_period_ms_stats"],
        "t_attn_ms": res["t_attn_ms_stats"],
        "decode_kernel_ms": res["decode_ms_stats"],
        "achievable_read": {
            "gbs": round(res["probe_gbs"], 2), "ms": round(res["probe_ms"], 5),
            "t_attn_frac": round(res["t_attn_gbs"] / res["probe_gbs"], 4),
            "probe": "pkv_stream_read_probe over the same bytes: shuffled 4 KiB tiles, "
                     "contiguous shares per wave, 4 tiles in flight, 256 x 4 waves, "
                     "timed by dispatch-stamped events like the decode kernel"},
        "graph": ({"ms_per_step": round(res["graph_ms_per_step"], 5),
                   "step_gbs": round(res["kv_bytes"] / (res["graph_ms_per_step"] * 1e-3) / 1e9, 2),
                   "steps_per_graph": res["graph_steps"]}
                  if res["graph_ms_per_step"] else None),
        "host_bookkeeping_us_per_step": round(res["host_bookkeeping_us_per_step"], 1),
        "cpu_baseline": res.get("cpu_baseline"),
    }
    others = [n for n in args.others.split(",") if n and n != cfg.name]
    if others:
        line["configs"] = {}
        for name in others:
            c = CONFIGS[name]
            r = time_config(c, args, dev, c.partition_size, with_cpu=False)
            line["configs"][name] = config_obj(c, r)
    if args.all_configs or args.swap:
        line["swap"] = time_swap(cfg, args, dev)
    if args.all_configs:
        line["prefix_cache"] = time_prefix_cache(CONFIGS["c5_long_shared_bf16"])
    if args.all_configs or args.multiquery:
        from synth import MQ_CONFIGS
        line["multiquery"] = {name: time_multiquery(m, args, dev) for name, m in MQ_CONFIGS.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
