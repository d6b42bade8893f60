#!/usr/bin/env python3
"""Benchmark of the fused evict+attend decode step on one MI355X.

Default workload: the Llama-3-8B shape at a 32K context (32 layers, 32 query /
8 KV heads, head_dim 128, vocab 128256, batch 16, 32768-token synthetic
prefill, budgets 1024 / 2048, protected window 128, FP16 window 256). After
the first decode step (which attends over the whole prefill and evicts down
to the budget; timed and reported separately) and `--warmup` steps, exactly
`--steps` steady decode steps are timed. Each step is the whole hot path: the
logits reducer (confidence and budget) and the fused attend+evict kernel.
Inputs for the timed steps are generated and resident in HBM beforehand.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA, MI355X
METRIC = "decode steps/s + KV GB/s (fraction of HBM peak) for fused evict+attend step"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(w, st, steps, S):
    """Bytes the method must move per launch of the fused kernel (averaged over
    the timed steps): KV rows read, per-row state, query/output/new-row
    traffic, and rows moved by compaction or age-out."""
    L, B, Hq, d = w["num_layers"], w["batch"], w["num_q_heads"], w["head_dim"]
    kv = st["kv_bytes"] / steps
    per_row_state = 8 if w["policy"] == "kvpop" else 12      # pos + (prio) | pos + ema read + ema write
    state = st["rows_attended"] / steps * per_row_state
    io = 2 * (L * B * Hq * d * 2) + S * (2 * d * 2) + S * (4 * d)
    old_row = (2 * d + 8) if w["old_int8"] else 4 * d
    moved = st["rows_moved"] / steps * 2 * old_row
    return kv, kv + state + io + moved


def kernel_source_hash():
    """sha256 over the fused kernel's sources, to tie stored counter figures to the code they measured."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kv_cache_eviction_04_amd", "csrc")
    h = hashlib.sha256()
    for name in ("kernels.hip", "device.h", "layout.h"):
        with open(os.path.join(root, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload):
    """HBM bytes per fused-kernel launch from the committed counter summary of this workload, or None
    when there is none or the kernel's sources changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"fused_step_kernel.{workload}.hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _oracle_rows_worker(args):
    """Confidence and base budget of (row, step) tasks: the oracle as it stands."""
    from oracle import confidence as OCONF
    cfg, tasks = args
    t0 = time.perf_counter()
    out = {}
    for key, z in tasks:
        c = OCONF.confidence(z, cfg.w_entropy, cfg.w_margin, cfg.w_pmax)
        out[key] = OCONF.gate(c, cfg.tau, cfg.n_low, cfg.n_high, cfg.gate_literal)
    return out, time.perf_counter() - t0


def _oracle_segments_worker(args):
    """Steps of a group of segments, from their read-back state, with the base
    budgets of the confidence phase: the oracle's own per-segment step, as
    OracleCache.step calls it."""
    from oracle import cache as OC
    from oracle import confidence as OCONF
    cfg, t0_pos, states, steps = args
    L, B, H, G = cfg.num_layers, cfg.batch, cfg.num_kv_heads, cfg.group
    t0 = time.perf_counter()
    for i, x in enumerate(steps):
        t = t0_pos + i
        for s, seg in states.items():
            l, b, h = s // (B * H), (s // H) % B, s % H
            qg, kn, vn = x["q"][l][b][h * G:(h + 1) * G], x["k"][l][b][h], x["v"][l][b][h]
            if cfg.policy == "conf":
                bud = OCONF.layer_budget(x["base"][b], l, L, cfg.pyramid)
                OC.conf_segment_step(seg, t, qg, kn, vn, bud, cfg, segment_id=s)
            else:
                OC.kvpop_segment_step(seg, t, qg, kn, vn, float(x["prio"][l][b][h]), cfg)
    return time.perf_counter() - t0


def host_cores():
    """Host cores this process may use: its CPU affinity, capped by the
    OMP_NUM_THREADS share when the environment sets one."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def cpu_baseline(w, gpu, seed, first_input_step, budget_s):
    """Time the CPU oracle (as it stands) on a bounded, exact sample of the same
    workload: a subset of segments continued from the GPU's current state, on
    every host core through a process pool (segments are independent given
    their row's budget). The pool first computes the sampled rows' confidence
    for every sampled step, then runs the segments in groups."""
    import copy
    import multiprocessing as mp

    import numpy as np
    import torch

    from kv_cache_eviction_04_amd import synth
    from oracle import cache as OC

    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    rows = sorted({0, B - 1})
    layers = sorted({0, L // 2, L - 1})
    segs = [(l * B + b) * H + h for l in layers for b in rows for h in range(H)]
    cfg = OC.Config.from_dict(w)
    cores = host_cores()
    states = {}
    for s in segs:
        ro = {k: v.cpu().numpy() for k, v in gpu.read_cache(s, 1).items()}
        seg = OC.Segment(w["head_dim"])
        n = int(ro["len"][0])
        seg.pos = ro["pos"][0, :n].astype(np.int64)
        seg.is8 = ro["is_int8"][0, :n].astype(bool)
        seg.k16, seg.v16 = ro["k16"][0, :n].copy(), ro["v16"][0, :n].copy()
        seg.k8, seg.v8 = ro["k8"][0, :n].copy(), ro["v8"][0, :n].copy()
        seg.ks, seg.vs = ro["k_scale"][0, :n].copy(), ro["v_scale"][0, :n].copy()
        seg.ema = ro["ema"][0, :n].astype(np.float64)
        seg.prio = ro["prio"][0, :n].copy()
        states[s] = seg
    t_pos = gpu.position
    # the sample: enough steps for about budget_s seconds of single-core work
    # (the per-segment step cost is measured on one step first)
    dev = torch.device("cuda", 0)
    lbs = sorted({(l, b) for l in layers for b in rows})

    def host_step(i):
        x = synth.step_inputs(w, seed, first_input_step + i, dev)
        li = torch.tensor([l for l, _ in lbs], device=dev)
        bi = torch.tensor([b for _, b in lbs], device=dev)
        q, k, v = (x[n][li, bi].cpu().numpy() for n in ("q", "k", "v"))
        pr = x["prio"][li, bi].cpu().numpy() if x["prio"] is not None else None
        nest = {n: {l: {} for l, _ in lbs} for n in ("q", "k", "v", "prio")}
        for j, (l, b) in enumerate(lbs):
            nest["q"][l][b], nest["k"][l][b], nest["v"][l][b] = q[j], k[j], v[j]
            if pr is not None:
                nest["prio"][l][b] = pr[j]
        logits = None if x["logits"] is None else {b: x["logits"][b].cpu().numpy() for b in rows}
        return dict(q=nest["q"], k=nest["k"], v=nest["v"], prio=nest["prio"] if pr is not None else None,
                    logits=logits)

    probe = host_step(0)
    t0 = time.perf_counter()
    base_probe = None
    if cfg.policy == "conf":
        base_probe, _ = _oracle_rows_worker((cfg, [((b, 0), probe["logits"][b]) for b in rows]))
    t_conf1 = time.perf_counter() - t0
    one = dict(probe, base={b: base_probe[(b, 0)] for b in rows} if base_probe else None)
    probe_states = {s: states[s] for s in segs[:4]}
    t_seg1 = _oracle_segments_worker((cfg, t_pos, copy.deepcopy(probe_states), [one])) / 4
    per_step_serial = t_seg1 * len(segs) + t_conf1
    n_steps = max(2, min(100, int(budget_s / max(per_step_serial, 1e-6))))
    steps = [probe] + [host_step(i) for i in range(1, n_steps)]

    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_rows_worker, [(cfg, [])] * cores)  # start the workers before timing
        t0 = time.perf_counter()
        bases = {}
        if cfg.policy == "conf":
            tasks = [((b, i), st["logits"][b]) for i, st in enumerate(steps) for b in rows]
            chunks = [tasks[j::cores] for j in range(cores)]
            for out, _ in pool.map(_oracle_rows_worker, [(cfg, c) for c in chunks if c]):
                bases.update(out)
        t_conf = time.perf_counter() - t0
        for i, st in enumerate(steps):
            st["base"] = {b: bases[(b, i)] for b in rows} if bases else None
            st["logits"] = None
        groups = [segs[j::cores] for j in range(cores) if segs[j::cores]]
        t0 = time.perf_counter()
        pool.map(_oracle_segments_worker, [(cfg, t_pos, {s: states[s] for s in g}, steps) for g in groups])
        t_seg = time.perf_counter() - t0
    S = L * B * H
    # wall time per step on `cores` processes, extrapolated from the sampled
    # segments (and rows) to every segment (and row) of the workload
    per_step = (t_seg / n_steps) * (S / len(segs)) + (t_conf / n_steps) * (B / len(rows))
    return {
        "value": 1.0 / per_step,
        "unit": "steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{n_steps} steady steps of {len(segs)} of {S} segments (batch rows {rows}, layers {layers}, "
                   f"all {H} KV heads) continued from the GPU state, plus confidence for {len(rows)} of {B} rows; "
                   f"float64 NumPy oracle in {cores} worker processes (segments and (row, step) confidences "
                   f"spread over them); per-step wall time extrapolated x{S}/{len(segs)} (segments) and "
                   f"x{B}/{len(rows)} (rows)"),
        "seconds": t_seg + t_conf,
        "steps_timed": n_steps,
    }


def hbm_ceiling(dev, nbytes=3 << 29, reps=10):
    """The HBM bandwidth plain streaming kernels attain on this part, beside
    its peak: the library's probe kernel reading (and copying) nbytes, and
    torch's device copy of the same buffer, each timed with events."""
    import torch

    from kv_cache_eviction_04_amd import confkv
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    read_ms = timed(lambda: confkv.bandwidth_probe(src, sink, copy=False))
    copy_ms = timed(lambda: confkv.bandwidth_probe(src, dst, copy=True))
    torch_ms = timed(lambda: dst.copy_(src))
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "read_ms": read_ms, "read_gbps": nbytes / (read_ms * 1e-3) / 1e9,
            "copy_ms": copy_ms, "copy_gbps": 2 * nbytes / (copy_ms * 1e-3) / 1e9,
            "torch_copy_gbps": 2 * nbytes / (torch_ms * 1e-3) / 1e9,
            "kernels": "confkv_bandwidth_probe read and copy (16-byte loads, 8 in flight per lane); torch copy_; "
                       "copies count bytes read + written"}


def kv_footprint(gpu, w):
    """Bytes of K/V rows the cache retains now: 4d per FP16 row, 2d + 8 per
    INT8 row (codes and two fp32 scales), summed over every segment."""
    import torch
    d = w["head_dim"]
    total = rows = 0
    chunk = max(1, (64 << 20) // max(gpu.rows_max, 1))
    for first in range(0, gpu.S, chunk):
        n = min(chunk, gpu.S - first)
        ro = gpu.read_cache(first, n, fields=("is_int8",))
        live = torch.arange(gpu.rows_max, device=ro["len"].device)[None, :] < ro["len"][:, None]
        is8 = (ro["is_int8"] != 0) & live
        n8 = int(is8.sum())
        n_all = int(live.sum())
        total += n8 * (2 * d + 8) + (n_all - n8) * 4 * d
        rows += n_all
    return {"bytes": total, "gb": total / 1e9, "rows": rows, "position": gpu.position}


def kvpop_prefill_leg(gpu, w, S, seed, dev):
    """KVpop masked prefill at sequence length S on the cache `gpu` (a KVpop
    configuration), then its future-attention target pass, five timed calls
    each. Algorithmic FLOPs count 4*d per allowed (query head, key) pair for
    the prefill (QK and PV multiply-adds) and 2*d per counted pair for the
    target."""
    import torch

    from kv_cache_eviction_04_amd import confkv

    B, Hq, H, d = w["batch"], w["num_q_heads"], w["num_kv_heads"], w["head_dim"]
    gq = torch.Generator(device=dev).manual_seed(seed + 1)
    pq = torch.randn((B, Hq, S, d), generator=gq, device=dev).half()
    pk_ = torch.randn((B, H, S, d), generator=gq, device=dev).half()
    pv_ = torch.randn((B, H, S, d), generator=gq, device=dev).half()
    pp = torch.rand((B, H, S), generator=gq, device=dev)
    pout = torch.empty_like(pq)
    s_, wnd, kk = w["num_sink"], w["protect_last"], w["kvpop_k"]
    pairs = 0
    for qq in range(S):
        pairs += min(s_, qq + 1) + max(0, qq - max(s_, qq - wnd) + 1) + min(kk, max(0, qq - wnd - s_))
    flops = 4.0 * d * pairs * B * Hq
    _, _, ws = gpu.kvpop_prefill(pq, pk_, pv_, pp, out=pout)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 5
    e0.record()
    for _ in range(n):
        gpu.kvpop_prefill(pq, pk_, pv_, pp, out=pout, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    if gpu.status() != confkv.OK:
        log("device status after the prefill is not OK")
        sys.exit(1)
    prefill = {"seq_len": S, "batch": B, "ms_per_layer": ms, "allowed_pairs_per_head": pairs,
               "tflops": flops / (ms * 1e-3) / 1e12, "peak_tflops": MFMA_FP16_PEAK_TFLOPS,
               "frac": flops / (ms * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS}
    log(f"kvpop prefill S={S} B={B}: {ms:.3f} ms per layer, {prefill['tflops']:.0f} TFLOP/s "
        f"({100 * prefill['frac']:.1f}% of fp16 MFMA peak)")
    # the transposed pass: 2*d FLOPs per counted (query head, key) pair
    plse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    gpu.kvpop_prefill(pq, pk_, pv_, pp, out=pout, lse=plse, workspace=ws)
    tgt = gpu.kvpop_future_target(pq, pk_, plse)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        gpu.kvpop_future_target(pq, pk_, plse, out=tgt)
    e1.record()
    torch.cuda.synchronize()
    tms = e0.elapsed_time(e1) / n
    tpairs = sum(max(0, S - t - wnd) for t in range(S))
    tflops = 2.0 * d * tpairs * B * Hq
    prefill["future_target"] = {"ms_per_layer": tms, "counted_pairs_per_head": tpairs,
                                "tflops": tflops / (tms * 1e-3) / 1e12,
                                "frac": tflops / (tms * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS}
    log(f"kvpop future target S={S} B={B}: {tms:.3f} ms per layer, "
        f"{prefill['future_target']['tflops']:.0f} TFLOP/s")
    del plse, tgt
    del pq, pk_, pv_, pp, pout, ws
    torch.cuda.empty_cache()
    return prefill


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-len", type=int, default=16384,
                    help="sequence length of the KVpop masked-prefill measurement (0 skips it)")
    ap.add_argument("--no-kvpop-leg", action="store_true",
                    help="other workloads: skip the KVpop prefill measurement on a cache of the KVpop shape")
    ap.add_argument("--split-steps", type=int, default=50,
                    help="steps of the per-layer call sequence (attend per layer, then evict) timed after the "
                         "fused steps; 0 skips it")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference kernel for HBM counter scaling)")
    ap.add_argument("--spread-steps", type=int, default=200,
                    help="steps timed one by one (an event at every step boundary) for p10/p50/p90; 0 skips it")
    ap.add_argument("--graph-steps", type=int, default=None,
                    help="steps captured into one hipGraph and replayed (default: 512 for the launch-bound toy "
                         "and GPT-2 shapes, 0 for the others)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the plain-copy HBM ceiling measurement")
    ap.add_argument("--run-to", type=int, default=0,
                    help="after the measurements, keep decoding (untimed) until this many tokens have been "
                         "generated after the prefill, then report the retained K/V footprint there")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this library runs the decode step on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_eviction_04_amd import confkv, synth

    dev = torch.device("cuda", 0)
    w = synth.workload(args.workload)
    L, B, Hq, H, d = w["num_layers"], w["batch"], w["num_q_heads"], w["num_kv_heads"], w["head_dim"]
    S = L * B * H

    if args.calib_copy:
        # one elementwise kernel that reads exactly 1 GiB and writes exactly 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("calibration kernel (neg): 1 GiB read + 1 GiB written")
        del src, dst

    ceiling = None
    if not args.no_ceiling:
        ceiling = hbm_ceiling(dev)
        log(f"streaming over {ceiling['bytes'] / 2**30:.2f} GiB: read {ceiling['read_gbps']:.0f} GB/s, copy "
            f"{ceiling['copy_gbps']:.0f} GB/s (read + write; torch copy {ceiling['torch_copy_gbps']:.0f} GB/s)")

    log(f"workload {args.workload}: L{L} B{B} Hq{Hq} Hkv{H} d{d} prefill {w['prefill']}")
    t0 = time.perf_counter()
    pk = pv = None
    if w["prefill"]:
        pk, pv = synth.prefill(w, args.seed, dev)
    gpu = confkv.Cache(w, pk, pv, device=dev)
    torch.cuda.synchronize()
    del pk, pv
    torch.cuda.empty_cache()
    log(f"init done in {time.perf_counter() - t0:.1f}s, state {gpu.state_bytes / 2**30:.2f} GiB")

    step_i = 0
    out = torch.empty((L, B, Hq, d), dtype=torch.float16, device=dev)

    def run_step(x):
        gpu.step(x["logits"], x["q"], x["k"], x["v"], x["prio"], out=out)

    # first decode step: attends over the whole prefill, then evicts to the budget
    x = synth.step_inputs(w, args.seed, step_i, dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_step(x)
    e1.record()
    torch.cuda.synchronize()
    first_ms = e0.elapsed_time(e1)
    step_i += 1
    first_stats = gpu.stats(reset=True)
    log(f"first step {first_ms:.3f} ms, KV read {first_stats['kv_bytes'] / 1e9:.2f} GB")

    fill = 0
    if w["policy"] == "kvpop":  # reach the steady state: sinks + window + k rows
        fill = w["num_sink"] + w["protect_last"] + w["kvpop_k"]
    for i in range(fill + args.warmup):
        run_step(synth.step_inputs(w, args.seed, step_i, dev))
        step_i += 1
    inputs = [synth.step_inputs(w, args.seed, step_i + i, dev) for i in range(args.steps)]
    torch.cuda.synchronize()
    gpu.stats(reset=True)
    # Event pairs around the fused kernel only: each record costs stream time,
    # so the reducer is timed in a pass of its own after the timed region.
    gpu.profile(True, kernels=("step",))
    gpu.profile_read(reset=True)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for x in inputs:
        run_step(x)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_i += args.steps
    gpu.profile(False)
    prof = gpu.profile_read(reset=True)
    st = gpu.stats(reset=True)
    rc = gpu.status()
    if rc != confkv.OK:
        log(f"device status {rc}")
        sys.exit(1)

    ms_per_step = wall * 1e3 / args.steps
    steps_per_s = args.steps / wall
    kv_per_step, alg_per_launch = algorithmic_bytes(w, st, args.steps, S)
    kv_gbps = kv_per_step / (ms_per_step * 1e-3) / 1e9
    fused_avg_ms = prof["fused_ms"] / max(prof["fused_launches"], 1)
    reduce_avg_ms = None
    if w["policy"] != "kvpop":  # the reducer's duration, over a few more steps
        red_inputs = [synth.step_inputs(w, args.seed, step_i + i, dev) for i in range(20)]
        torch.cuda.synchronize()
        gpu.profile(True, kernels=("reduce",))
        for x in red_inputs:
            run_step(x)
        gpu.profile(False)
        red = gpu.profile_read(reset=True)
        step_i += len(red_inputs)
        gpu.stats(reset=True)
        reduce_avg_ms = red["reduce_ms"] / max(red["reduce_launches"], 1)
    # The distribution of step times: one event at every step boundary on the
    # stream the steps run on (each record costs a little stream time, so this
    # is a pass of its own after the timed region).
    spread = None
    if args.spread_steps > 0:
        sp_in = [synth.step_inputs(w, args.seed, step_i + i, dev) for i in range(args.spread_steps)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.spread_steps + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i, x in enumerate(sp_in):
            run_step(x)
            evs[i + 1].record()
        torch.cuda.synchronize()
        step_i += args.spread_steps
        gpu.stats(reset=True)
        ts = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.spread_steps))
        q = lambda f: ts[min(len(ts) - 1, int(f * (len(ts) - 1) + 0.5))]  # noqa: E731
        spread = {"steps": len(ts), "p10_ms": q(0.1), "p50_ms": q(0.5), "p90_ms": q(0.9),
                  "mean_ms": sum(ts) / len(ts), "min_ms": ts[0], "max_ms": ts[-1]}
        log(f"step time p10/p50/p90 {spread['p10_ms']:.4f}/{spread['p50_ms']:.4f}/{spread['p90_ms']:.4f} ms "
            f"over {len(ts)} steps")
        del sp_in

    # The same steps captured into one hipGraph and replayed once: the step's
    # two launches per step without the host's launch overhead. The position
    # is a launch argument, so one graph covers one run of consecutive
    # positions (the library's host position advances during the capture).
    graph = None
    n_graph = args.graph_steps if args.graph_steps is not None else (
        512 if args.workload in ("toy", "gpt2_small") else 0)
    if n_graph > 0:
        g_in = [synth.step_inputs(w, args.seed, step_i + i, dev) for i in range(2 * n_graph)]
        e_in = g_in[:n_graph]
        torch.cuda.synchronize()
        t_e = time.perf_counter()
        for x in e_in:  # eager reference over the same number of steps
            run_step(x)
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - t_e) * 1e3 / n_graph
        step_i += n_graph
        cg = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(cg, stream=cap):
                for x in g_in[n_graph:]:
                    run_step(x)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cg.replay()
        e1.record()
        torch.cuda.synchronize()
        step_i += n_graph
        graph_ms = e0.elapsed_time(e1) / n_graph
        if gpu.status() != confkv.OK:
            log("device status after the graph replay is not OK")
            sys.exit(1)
        gpu.stats(reset=True)
        graph = {"steps": n_graph, "graph_ms_per_step": graph_ms, "graph_steps_per_s": 1e3 / graph_ms,
                 "eager_wall_ms_per_step": eager_ms}
        log(f"hipGraph of {n_graph} steps: {graph_ms * 1e3:.1f} us/step ({1e3 / graph_ms:.0f} steps/s) against "
            f"{eager_ms * 1e3:.1f} us/step issued one by one")
        del g_in, e_in, cg

    achieved = alg_per_launch / (fused_avg_ms * 1e-3) / 1e9
    log(f"{steps_per_s:.1f} steps/s ({ms_per_step:.4f} ms/step), KV {kv_gbps:.0f} GB/s; fused kernel "
        f"{fused_avg_ms * 1e3:.1f} us avg -> {achieved:.0f} GB/s algorithmic"
        + ("" if reduce_avg_ms is None else f"; reducer {reduce_avg_ms * 1e3:.1f} us"))

    # The same step as a model's layer loop issues it: one attend launch per
    # layer, then the reducer and the evict launch. Python issues 33 calls a
    # step, so the wall clock is host-bound; the device time per step is the
    # sum of the kernels' event-timed durations.
    split = None
    if args.split_steps > 0:
        sp_inputs = [synth.step_inputs(w, args.seed, step_i + i, dev) for i in range(args.split_steps + 1)]

        def run_split(x):
            for l in range(L):
                gpu.attend(l, x["q"][l], x["k"][l], x["v"][l], None if x["prio"] is None else x["prio"][l],
                           out=out[l])
            gpu.evict(x["logits"])

        run_split(sp_inputs[0])
        torch.cuda.synchronize()
        gpu.profile(True)
        for k in gpu.KERNELS:
            gpu.profile_kernel(k, reset=True)
        t_sp = time.perf_counter()
        for x in sp_inputs[1:]:
            run_split(x)
        torch.cuda.synchronize()
        sp_wall = time.perf_counter() - t_sp
        gpu.profile(False)
        step_i += args.split_steps + 1
        att_ms, att_n = gpu.profile_kernel("attend")
        ev_ms, ev_n = gpu.profile_kernel("evict")
        red_ms, red_n = gpu.profile_kernel("reduce")
        dev_ms = (att_ms + ev_ms + red_ms) / args.split_steps
        if gpu.status() != confkv.OK:
            log("device status after the per-layer steps is not OK")
            sys.exit(1)
        split = {
            "steps": args.split_steps,
            "device_ms_per_step": dev_ms,
            "device_steps_per_s": 1e3 / dev_ms,
            "attend_avg_us": att_ms / max(att_n, 1) * 1e3,
            "evict_avg_us": ev_ms / max(ev_n, 1) * 1e3,
            "reducer_avg_us": red_ms / red_n * 1e3 if red_n else None,
            "launches_per_step": L + 1 + (1 if red_n else 0),
            "wall_ms_per_step": sp_wall * 1e3 / args.split_steps,
        }
        log(f"per-layer calls: {dev_ms:.4f} ms/step of kernels (attend {split['attend_avg_us']:.1f} us x {L}, "
            f"evict {split['evict_avg_us']:.1f} us), wall {split['wall_ms_per_step']:.3f} ms/step")

    # The next-token draw from this step's logits (greedy and inverse-CDF),
    # timed with events on the stream it runs on.
    sampling = None
    if w["policy"] == "conf":
        x = synth.step_inputs(w, args.seed, step_i, dev)
        u = torch.rand((B,), generator=torch.Generator(device=dev).manual_seed(args.seed), device=dev)
        tok = torch.empty((B,), dtype=torch.int32, device=dev)
        sampling = {"logits_bytes": B * w["vocab"] * 4}
        for name, uu in (("greedy", None), ("draw", u)):
            gpu.sample(x["logits"], uu, out=tok)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 50
            e0.record()
            for _ in range(n):
                gpu.sample(x["logits"], uu, out=tok)
            e1.record()
            torch.cuda.synchronize()
            sampling[f"{name}_us"] = e0.elapsed_time(e1) * 1e3 / n
        if gpu.status() != confkv.OK:
            log("device status after sampling is not OK")
            sys.exit(1)
        log(f"sampling: greedy {sampling['greedy_us']:.1f} us, draw {sampling['draw_us']:.1f} us per call "
            f"({sampling['logits_bytes'] / 1e6:.1f} MB of logits)")

    # KVpop prefill with the multi-query mask at the pages' 16384-token
    # training length, one layer per call. A KVpop workload measures it on its
    # own cache; any other workload on a cache of the KVpop Qwen3-8B shape made
    # for it (its state is a few GB), so the default run reports it too.
    prefill = None
    if args.prefill_len > 0 and (w["policy"] == "kvpop" or not args.no_kvpop_leg):
        if w["policy"] == "kvpop":
            prefill = kvpop_prefill_leg(gpu, w, args.prefill_len, args.seed, dev)
        else:
            kw = synth.workload("kvpop_qwen3_8b")
            kpk, kpv = synth.prefill(kw, args.seed, dev)
            kgpu = confkv.Cache(kw, kpk, kpv, device=dev)
            prefill = kvpop_prefill_leg(kgpu, kw, args.prefill_len, args.seed, dev)
            prefill["workload"] = "kvpop_qwen3_8b"
            del kgpu, kpk, kpv
            torch.cuda.empty_cache()

    if args.run_to > 0:
        target = w["prefill"] + args.run_to
        log(f"decoding on to position {target} (from {gpu.position}) for the footprint")
        while gpu.position < target:
            run_step(synth.step_inputs(w, args.seed, step_i, dev))
            step_i += 1
            if step_i % 4096 == 0:
                torch.cuda.synchronize()
                log(f"... position {gpu.position}")
        torch.cuda.synchronize()
        if gpu.status() != confkv.OK:
            log("device status after the run is not OK")
            sys.exit(1)
    footprint = kv_footprint(gpu, w)
    log(f"retained K/V at position {footprint['position']}: {footprint['gb']:.3f} GB in {footprint['rows']} rows")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, gpu, args.seed, step_i, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.4g} steps/s ({cpu['seconds']:.1f} s wall on {cpu['cores']} processes, "
            f"about {cpu['seconds'] * cpu['cores']:.0f} s of CPU work)")

    res = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA, fp32 accumulate; " + ("fp16 window + int8 K/V" if w["old_int8"] else "fp16 K/V"),
        "data": "synthetic",
        "config": {
            "workload": args.workload, "layers": L, "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": d,
            "vocab": w["vocab"], "prefill": w["prefill"], "policy": w["policy"],
            "n_low": w.get("n_low"), "n_high": w.get("n_high"), "protect_last": w["protect_last"],
            "fp16_window": w["fp16_window"], "num_sink": w["num_sink"], "kvpop_k": w["kvpop_k"],
            "pyramid": w["pyramid"], "kv_storage": "fp16 window + int8 older rows" if w["old_int8"] else "fp16",
            "seed": args.seed,
        },
        "kv_gb_per_s": kv_gbps,
        "kv_frac_of_hbm_peak": kv_gbps / HBM_PEAK_GBPS,
        "kv_bytes_per_step": kv_per_step,
        "tokens_per_s": steps_per_s * B,
        "first_step_ms": first_ms,
        "first_step_kv_bytes": first_stats["kv_bytes"],
        "reducer_us": None if reduce_avg_ms is None else reduce_avg_ms * 1e3,
        "rows_evicted_per_step": st["rows_evicted"] / args.steps,
        "rows_moved_per_step": st["rows_moved"] / args.steps,
        "step_time_spread": spread,
        "hbm_ceiling": ceiling,
        "kv_footprint": footprint,
        "graph": graph,
        "roofline": {
            "bound": "hbm",
            "kernel": "fused_step_kernel",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": stored_traffic(args.workload),
            "bytes_per_launch": alg_per_launch,
            "avg_launch_us": fused_avg_ms * 1e3,
        },
        "cpu_baseline": cpu,
        "per_layer_calls": split,
        "sampling": sampling,
        "kvpop_prefill": prefill,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
