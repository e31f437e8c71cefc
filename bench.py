#!/usr/bin/env python3
"""Benchmark: one compression event per step over every layer of a model-shaped KV cache.

A step is the whole path for one batch of synthetic input already resident in HBM:
(beacon update when the workload has one,) scoring, top-K selection and compaction of
every (layer, sequence, KV head).  Default workload: R1-Distill-Qwen-7B attention
geometry, 28 layers, 28 query / 4 KV heads, head_dim 128, one 16,384-token trace,
window 32, 16 beacons per KV head, budget 4096.

Prints one JSON line (rank 0, one GPU):
  value       cached KV tokens compressed per second (sum over sequences of L_b per step,
              a token counted once across layers and heads)
  roofline    the dominant kernel group's algorithmic bytes / measured duration vs 8 TB/s
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # Enough untimed steps that the GPU has reached its working clocks before the timed
    # ones (a cold start under-reports short events by about a tenth).
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="qwen7b_16k")
    p.add_argument("--cpu-units", type=int, default=-1,
                   help="at most this many units in the CPU-oracle sample (0: skip; -1: no limit; "
                        "each pool process stops after about 15 s of oracle work either way)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy five times (a known-size reference for the "
                            "FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--window", type=int, default=None,
                   help="override the workload's recent window W (queries per head, always-kept keys)")
    p.add_argument("--beacons", type=int, default=None, help="override the beacons per KV head (live and slots)")
    p.add_argument("--budget", type=int, default=None, help="override the kept keys per KV head")
    p.add_argument("--aggregation", default="max", choices=["max", "mean"],
                   help="score aggregation over the observation rows (the method: max; Table 2: mean)")
    p.add_argument("--steady-state", type=int, default=0, metavar="CYCLES",
                   help="time CYCLES steady-state cycles (append a chunk of t_new tokens, refresh beacons, compress "
                        "back to the budget) instead of one event")
    p.add_argument("--decode", action="store_true",
                   help="time one decoding step of attention over the full caches and over the compacted ones")
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def score_kernel_names(head_dim: int, n_obs: int) -> tuple:
    """The two kernels one bkv_score call launches for this geometry, by the library's own
    dispatch rules: the register-row stats pass up to 256 padded observation rows (4 waves),
    8 waves up to 512 at head_dim 128, 3 blocks per wave up to 384 at head_dim 64, else the
    LDS-staged stats pass; the 4-wave finish where two workgroups' staged rows and
    statistics fit in one CU's 160 KiB of LDS, else the 8-wave finish."""
    obs_pad = -(-n_obs // 32) * 32
    if obs_pad <= 256:
        stats = "qs_stats_kernel<D,BPW>"
    elif head_dim == 128 and obs_pad <= 512:
        stats = "qs_stats_kernel8<D>"
    elif head_dim == 64 and obs_pad <= 384:
        stats = "qs_stats_kernel_wide<D,3>"
    else:
        stats = "score_kernel<D,false>"
    lds = obs_pad * head_dim * 2 + 4 * 4 * obs_pad * 4
    finish = "score_kernel<D,true>" if 2 * lds <= 160 * 1024 else "finish8_kernel<D>"
    return stats, finish


def alg_bytes(w, lens):
    """Algorithmic HBM bytes of one event per kernel group: K rows read once and the
    observation queries (score), scores read and positions written (select), kept K/V rows
    read and written plus positions (compact), pool read and beacons written (fps)."""
    D, G = w.head_dim, w.group
    n_obs = G * w.window + w.nb_max
    per_layer_heads = w.n_kv_heads
    score = select = compact = fps = 0
    for L in lens:
        L = int(L)
        N = min(w.budget, L)
        u = w.n_layers * per_layer_heads
        score += u * (L * D * 2 + n_obs * D * 2)
        select += u * (L * 4 + N * 4)
        compact += u * (4 * N * D * 2 + N * 4)
        if w.runs_fps:
            fps += u * ((w.nb_init + G * w.t_new) * D * 2 + w.nb_max * D * 2)
    return {"score": score, "select": select, "compact": compact, "update_beacons": fps}


def event_bytes(w, lens):
    """Algorithmic HBM bytes of one whole event: K read once, the observation rows, the kept
    K/V rows read and written, the kept positions once, and (with a beacon update) the pool
    read and the beacons written.  The score vector written by the scorer and read back by
    the selection is traffic of splitting the event into stages, not of the method, and is
    not counted (the per-stage figures above do count it)."""
    D, G = w.head_dim, w.group
    n_obs = G * w.window + w.nb_max
    total = 0
    for L in lens:
        L = int(L)
        N = min(w.budget, L)
        u = w.n_layers * w.n_kv_heads
        total += u * (L * D * 2 + n_obs * D * 2 + 4 * N * D * 2 + N * 4)
        if w.runs_fps:
            total += u * ((w.nb_init + G * w.t_new) * D * 2 + w.nb_max * D * 2)
    return total


def score_flops(w, lens):
    n_obs = w.group * w.window + w.nb_max
    return sum(2.0 * n_obs * int(L) * w.head_dim * w.n_layers * w.n_kv_heads for L in lens)


SCORER_SOURCES = ("score.hip", "score_qs.hip", "score_common.h")


def scorer_digest():
    """sha256 over the scorer's sources, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in SCORER_SOURCES:
        with open(os.path.join(ROOT, "attention_guided_eviction_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_ceiling(dev, gib=2, reps=5):
    """Read+write copy rate of a plain device copy of `gib` GiB (2*gib GiB moved), median of reps."""
    import statistics
    import torch
    n = gib << 28   # float32 elements
    src = torch.ones(n, device=dev)
    dst = torch.empty(n, device=dev)
    dst.copy_(src)
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * gib * (1 << 30) / (statistics.median(times) * 1e-3) / 1e9


def _profile_values(path):
    """key = value lines of a committed profile summary (comment lines skipped)."""
    vals = {}
    if not os.path.exists(path):
        return vals
    with open(path) as f:
        for line in f:
            m = re.match(r"\s*([a-z_0-9]+) = (\S+)\s*$", line)
            if m:
                vals[m.group(1)] = m.group(2)
    return vals


def score_counters(workload):
    """MFMA / VALU busy fractions of the scorer's two passes from the committed counter
    summary for this workload, or None when there is none or the scorer source has changed
    since the counters were taken."""
    vals = _profile_values(os.path.join(ROOT, "profiles", f"score_counters_{workload}.md"))
    if vals.get("scorer_sha256") != scorer_digest():
        return None
    keys = ("mfma_busy_stats", "mfma_busy_finish", "valu_busy_stats", "valu_busy_finish", "coexec_stats",
            "coexec_finish")
    if not all(k in vals for k in keys):
        return None
    return {k: float(vals[k]) for k in keys} | {"source": f"profiles/score_counters_{workload}.md"}


def score_traffic(workload):
    """HBM bytes per bkv_score call from the committed counter summary for this workload,
    or None when there is none or the scorer source has changed since it was taken."""
    vals = _profile_values(os.path.join(ROOT, "profiles", f"score_traffic_{workload}.txt"))
    if vals.get("scorer_sha256") != scorer_digest() or "traffic_bytes_per_call" not in vals:
        return None
    return float(vals["traffic_bytes_per_call"])


# ---- CPU oracle baseline ---------------------------------------------------------------------
# The float64 oracle runs units (layer, sequence, KV head) in a process pool, one BLAS thread
# per process.  The pool is forked before anything touches the GPU (its processes hold no GPU
# state) and is sized to the host cores this job may use, at most CPU_POOL_MAX (the CPU share
# of one GPU on the measurement host).

CPU_POOL_MAX = 16


def cpu_pool_size():
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(cores, CPU_POOL_MAX))


def _oracle_worker_init():
    import threadpoolctl
    import torch
    torch.set_num_threads(1)
    threadpoolctl.threadpool_limits(1)


def _oracle_units(job):
    """Worker: build the inputs of its units (untimed), wait for every worker, then time the
    oracle over them.  Returns (cached rows, oracle seconds, seconds of each unit)."""
    w, units, barrier = job
    from synth import unit_inputs, bf16_bits
    from oracle import bkv_oracle as O
    prepared = []
    for l, b, h in units:
        u = unit_inputs(w, l, b, h, "cpu")
        prepared.append((bf16_bits(u["k"]), bf16_bits(u["v"]), bf16_bits(u["q"]), bf16_bits(u["beacons"]),
                         u["nb"], u["L"]))
    barrier.wait()
    t0 = time.perf_counter()
    rows = 0
    each = []
    for kb, vb, qb, bb, nb, L in prepared:
        t1 = time.perf_counter()
        if w.runs_fps:
            bb, nb, _ = O.update_beacons(bb, nb, qb[:, w.q_len - w.t_new:], w.nb_max)
        O.compress_unit(kb, vb, qb, bb, nb, w.window, w.budget)
        rows += L
        each.append(time.perf_counter() - t1)
    return rows, time.perf_counter() - t0, each


class CpuBaseline:
    """The oracle's pool, created at start-up (before the GPU is initialised)."""

    def __init__(self, size):
        import multiprocessing as mp
        self.size = size
        self.ctx = mp.get_context("fork")
        self.manager = self.ctx.Manager()
        self.pool = self.ctx.Pool(size, initializer=_oracle_worker_init)

    def close(self):
        self.pool.close()
        self.pool.join()
        self.manager.shutdown()

    def run(self, w, n_units, budget_s=15.0):
        """A bounded sample of the workload's units in seeded random order: three units
        timed alone first (their median is the single-process seconds per unit), then about
        budget_s seconds of oracle work per process, all processes together.  tokens/s = rows
        per wall second of the pooled run / (layers x KV heads)."""
        import numpy as np
        rng = np.random.default_rng(1)
        per_layer = w.batch * w.n_kv_heads
        order = []
        for u_id in rng.permutation(w.units):
            l, rem = divmod(int(u_id), per_layer)
            order.append((l, *divmod(rem, w.n_kv_heads)))
        if n_units > 0:
            order = order[:n_units]
        calib = order[:3]
        rows1, t1, each = self.pool.apply(_oracle_units, ((w, calib, self.manager.Barrier(1)),))
        per_unit = float(np.median(each))
        rest = order[len(calib):]
        k = max(1, min(int(budget_s / max(per_unit, 1e-6)), -(-len(rest) // self.size)))
        shares = [rest[i * k:(i + 1) * k] for i in range(self.size)]
        shares = [sh for sh in shares if sh]
        if shares:
            barrier = self.manager.Barrier(len(shares))
            res = self.pool.map(_oracle_units, [(w, sh, barrier) for sh in shares], chunksize=1)
        else:
            shares = [calib]
            res = [(rows1, t1, each)]
        rows = sum(r[0] for r in res)
        wall = max(r[1] for r in res)
        done = sum(len(sh) for sh in shares)
        tokens_per_s = rows / wall / (w.n_layers * w.n_kv_heads)
        return {"value": tokens_per_s, "unit": "tokens/s", "cores": len(shares), "kind": "oracle",
                "os_cpu_count": os.cpu_count(), "pool_size": self.size, "processes_used": len(shares),
                "single_process_s_per_unit": round(per_unit, 4),
                "single_process_s_all_units": round(per_unit * w.units, 1),
                "sample": f"{done} of {w.units} (layer, sequence, KV head) units of {w.name} in seeded random order, "
                          f"{len(shares)} processes x up to {k} units (at most ~{budget_s:.0f} s of oracle work each, "
                          f"one BLAS thread per process), {rows} cached rows in {wall:.2f} s wall; float64 NumPy beacon "
                          f"update, scores, "
                          f"top-K and compaction; inputs built before the timed region; rows/s divided by "
                          f"layers x KV heads"}


def decode_bench(args, w, log):
    """Decode attention (one new query per head, all layers) over the workload's full caches
    and over the caches one compression event leaves, HIP events around each."""
    import torch
    from synth import layer_tensors, seq_lengths
    from attention_guided_eviction_amd import bkv
    from attention_guided_eviction_amd.event import CompressionEvent, EventConfig
    dev = torch.device("cuda:0")
    layers = [layer_tensors(w, l, dev) for l in range(w.n_layers)]
    inp = {key: [lt[key] for lt in layers] for key in layers[0]}
    del layers
    lens = seq_lengths(w)
    seq = torch.from_numpy(lens).to(dev)
    cfg = EventConfig(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, w.q_len, w.window,
                      w.nb_max, w.budget, w.t_new)
    ev = CompressionEvent(cfg, seq, dev)
    ev.run(inp["k"], inp["v"], inp["q"], inp["beacons"], inp["n_beacons"])
    q = [t[:, :, -1].contiguous() for t in inp["q"]]
    out = [torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev) for _ in q]
    kept = torch.clamp(seq, max=w.budget)
    res = {}
    for name, k, v, cap, sl, n_rows in (("full", inp["k"], inp["v"], w.capacity, seq, lens.sum()),
                                        ("compacted", ev.k_out, ev.v_out, w.budget, kept,
                                         sum(min(int(x), w.budget) for x in lens))):
        shape = bkv.CacheShape(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, cap, sl)
        ws = bkv.alloc_workspace(bkv.decode_workspace_bytes(shape), dev)
        call = bkv.prepare_decode_attention(shape, q, k, v, out, ws)
        for _ in range(args.warmup):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        nbytes = float(n_rows) * w.n_layers * w.n_kv_heads * w.head_dim * 2 * 2
        res[name] = {"ms_per_step": round(ms, 4), "cached_rows": int(n_rows), "alg_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "alg_frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] decode over {name} caches: {ms:.3f} ms per step")
    out_line = {"metric": "decode attention over the full vs the compacted cache (one step, all layers)",
                "workload": w.name, "budget": w.budget, "results": res,
                "speedup_from_compression": round(res["full"]["ms_per_step"] / res["compacted"]["ms_per_step"], 2)}
    print(json.dumps(out_line), flush=True)


def steady_state(args, w, log):
    """Steady-state cycles of the workload's geometry: every sequence at the budget, a chunk
    of t_new tokens appended, beacons refreshed, the cache compressed back to the budget."""
    import torch
    from attention_guided_eviction_amd.loop import LoopConfig, SteadyStateLoop
    if args.window is not None:
        w = w.replace(window=args.window)
    if args.beacons is not None:
        w = w.replace(nb_init=args.beacons, nb_max=args.beacons)
    if args.budget is not None:
        w = w.replace(budget=args.budget)
    T = w.t_new if w.t_new > 0 else 128
    cfg = LoopConfig(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.budget, w.window, w.nb_max, T,
                     args.aggregation)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    n, B, Hkv, Hq, D = w.n_layers, w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    rnd = lambda *s: torch.randn(*s, generator=gen, device=dev).to(torch.bfloat16)
    loop = SteadyStateLoop(cfg, dev)
    loop.start([rnd(B, Hkv, w.budget, D) for _ in range(n)], [rnd(B, Hkv, w.budget, D) for _ in range(n)],
               [rnd(B, Hkv, max(w.nb_max, 1), D) for _ in range(n)],
               [torch.full((B, Hkv), w.nb_max, dtype=torch.int32, device=dev) for _ in range(n)])
    chunks = [([rnd(B, Hkv, T, D) for _ in range(n)], [rnd(B, Hkv, T, D) for _ in range(n)],
               [rnd(B, Hq, T, D) for _ in range(n)]) for _ in range(2)]
    for i in range(args.warmup):
        loop.cycle(*chunks[i % 2])
    torch.cuda.synchronize()
    # Appending the chunk is the decoding engine's work; only compress() is timed.
    total = 0.0
    for i in range(args.steady_state):
        loop.append(*chunks[i % 2])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        loop.compress()
        b.record()
        torch.cuda.synchronize()
        total += a.elapsed_time(b)
    ms = total / args.steady_state
    tokens = B * cfg.capacity
    out = {
        "metric": "cached KV tokens compressed/sec per GPU, steady state (append, refresh beacons, compress)",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steady_state,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name} steady state", "layers": n, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "batch": B, "seq_len": f"{cfg.capacity} compressed to {w.budget} every {T} tokens",
                   "window": w.window, "beacons": w.nb_max, "budget": w.budget, "aggregation": args.aggregation},
    }
    log(f"[bench] steady state: {ms:.3f} ms per compression cycle")
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards by "
              f"(layer, sequence, KV head) with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    from synth import WORKLOADS, seq_lengths
    from attention_guided_eviction_amd import bkv
    from attention_guided_eviction_amd.event import CompressionEvent, EventConfig

    def log(*a):
        if not args.quiet:
            print(*a, file=sys.stderr, flush=True)

    w = WORKLOADS[args.workload]
    if args.steady_state > 0:
        return steady_state(args, w, log)
    if args.decode:
        return decode_bench(args, w, log)
    cpu = CpuBaseline(cpu_pool_size()) if args.cpu_units != 0 else None
    if args.window is not None:
        w = w.replace(window=args.window)
    if args.beacons is not None:
        w = w.replace(nb_init=args.beacons, nb_max=args.beacons)
    if args.budget is not None:
        w = w.replace(budget=args.budget)
    bkv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    from synth import layer_tensors
    layers = [layer_tensors(w, l, dev) for l in range(w.n_layers)]
    inp = {key: [lt[key] for lt in layers] for key in layers[0]}
    lens = seq_lengths(w)
    seq_len = torch.from_numpy(lens).to(dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs for {w.name} built in {time.time() - t0:.1f}s")
    cfg = EventConfig(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, w.q_len, w.window,
                      w.nb_max, w.budget, w.t_new, args.aggregation)
    ev = CompressionEvent(cfg, seq_len, dev)
    stream = torch.cuda.current_stream()
    k, v, q, bc, nb = inp["k"], inp["v"], inp["q"], inp["beacons"], inp["n_beacons"]

    ev.bind(k, v, q, bc, nb)
    for _ in range(args.warmup):
        ev.step()
    torch.cuda.synchronize()

    # whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        ev.step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.steps} steps, {ms:.3f} ms/step")

    # Per-call durations on the same stream: one full event first keeps the GPU busy while
    # the host enqueues the timed calls, so the events bracket GPU time only.
    names = (["update_beacons"] if w.runs_fps else []) + ["score", "select", "compact"]
    per = {}
    for name in names:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev.step()
        a.record(stream)
        for _ in range(args.steps):
            ev.calls[name]()
        b.record(stream)
        torch.cuda.synchronize()
        per[name] = a.elapsed_time(b) / args.steps
    log("[bench] per call ms: " + ", ".join(f"{n} {t:.3f}" for n, t in per.items()))

    tokens = float(lens.sum())
    ab = alg_bytes(w, lens)
    total_bytes = event_bytes(w, lens)
    dom = max(per, key=per.get)
    achieved = ab[dom] / (per[dom] * 1e-3) / 1e9
    # The committed counter summary holds for the workload as named, max aggregation.
    as_named = args.window is None and args.beacons is None and args.budget is None and args.aggregation == "max"
    traffic = score_traffic(w.name) if dom == "score" and as_named else None
    stats_kernel, finish_kernel = score_kernel_names(w.head_dim, w.group * w.window + w.nb_max)
    roof = {"kernel": {"score": f"{stats_kernel} (stats) + {finish_kernel} (finish): one bkv_score call",
                       "select": "select_topk_kernel (bkv_select_topk)",
                       "compact": "compact_kernel (bkv_compact)",
                       "update_beacons": "fps_kernel (bkv_update_beacons)"}[dom],
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "ms_per_launch": round(per[dom], 4), "alg_bytes_per_launch": ab[dom]}
    if dom == "score":
        tf = score_flops(w, lens) / (per[dom] * 1e-3) / 1e12
        roof["mfma_tflops_one_pass"] = round(tf, 1)
    out = {
        "metric": "cached KV tokens compressed/sec per GPU; achieved HBM GB/s as % of peak",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "batch": w.batch, "seq_len": int(lens.max()) if w.ragged is None
                   else f"ragged {w.ragged[0]}-{w.ragged[1]} (sum {int(lens.sum())})",
                   "window": w.window, "beacons": w.nb_max, "budget": w.budget, "beacon_update_queries": w.t_new,
                   "aggregation": args.aggregation},
        "hbm_alg_gbs": round(total_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_alg_frac_of_peak": round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "per_call_ms": {n: round(t, 4) for n, t in per.items()},
        # every stage against HBM: its algorithmic bytes (alg_bytes) over its live duration
        "per_call_gbs": {n: {"alg_bytes": ab[n], "achieved": round(ab[n] / (t * 1e-3) / 1e9, 1),
                             "frac": round(ab[n] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)} for n, t in per.items()},
        "roofline": roof,
        # utilisation of the scorer's passes from the committed counter summary (same scorer
        # sources and workload only)
        "mfma_busy": score_counters(w.name) if dom == "score" and as_named else None,
    }
    # Same-run ceiling: a plain read+write device copy of 4 GiB moved.
    ceil = copy_ceiling(dev)
    out["copy_ceiling_gbs"] = round(ceil, 1)
    out["hbm_alg_frac_of_copy_ceiling"] = round(total_bytes / (ms * 1e-3) / 1e9 / ceil, 4)
    log(f"[bench] copy ceiling {ceil:.0f} GB/s")
    if args.copy_calibration:
        n = 1 << 28   # 1 GiB of float32
        src = torch.ones(n, device=dev)
        dst = torch.empty(n, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if cpu is not None:
        log(f"[bench] CPU oracle on a sample ({cpu.size} processes) ...")
        out["cpu_baseline"] = cpu.run(w, args.cpu_units)
        cpu.close()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
