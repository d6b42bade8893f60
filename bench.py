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


def cpu_baseline(w, gpu, seed, first_input_step, budget_s):
    """Time the CPU oracle (as it stands) on a bounded, exact sample of the same
    workload: a subset of segments continued from the GPU's current state."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from kv_cache_eviction_04_amd import synth
    from oracle import cache as OC
    from oracle import confidence as OCONF

    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    rows = sorted({0, B - 1})
    layers = sorted({0, L // 2, L - 1})
    segs = [(l * B + b) * H + h for l in layers for b in rows for h in range(H)]
    cfg = OC.Config.from_dict(w)
    oc = OC.OracleCache(cfg, segs)
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
        oc.segs[s] = seg
    oc.t = gpu.position
    dev = torch.device("cuda", 0)
    t_seg = t_conf = 0.0
    n_steps = 0
    with threadpool_limits(limits=1):
        while t_seg + t_conf < budget_s:
            x = synth.step_inputs(w, seed, first_input_step + n_steps, dev)
            xs = {k: (None if v is None else v.cpu().numpy()) for k, v in x.items()}
            base = None
            if cfg.policy == "conf":
                t0 = time.perf_counter()
                base = {}
                for b in rows:
                    c = OCONF.confidence(xs["logits"][b], cfg.w_entropy, cfg.w_margin, cfg.w_pmax)
                    base[b] = OCONF.gate(c, cfg.tau, cfg.n_low, cfg.n_high, cfg.gate_literal)
                t_conf += time.perf_counter() - t0
            t0 = time.perf_counter()
            oc.step(logits=xs["logits"] if cfg.policy == "conf" else None, q=xs["q"], k_new=xs["k"],
                    v_new=xs["v"], prio=xs["prio"], base_override=base)
            t_seg += time.perf_counter() - t0
            n_steps += 1
    S = L * B * H
    # oc.step computes the confidence of its rows itself; t_conf times that same work on its own, so
    # the segment part is (t_seg - t_conf) and the confidence part scales with the batch rows.
    per_step = ((t_seg - t_conf) / n_steps) * (S / len(segs)) + (t_conf / n_steps) * (B / len(rows))
    return {
        "value": 1.0 / per_step,
        "unit": "steps/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{n_steps} steady steps of {len(segs)} of {S} segments (batch rows {rows}, layers {layers}, "
                   f"all {H} KV heads) continued from the GPU state, plus confidence for {len(rows)} of {B} rows; "
                   f"per-step time extrapolated x{S}/{len(segs)} (segments) and x{B}/{len(rows)} (rows); "
                   f"float64 NumPy, one thread"),
        "seconds": t_seg + t_conf,
        "steps_timed": n_steps,
    }


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
                    help="KVpop workloads: sequence length of the masked-prefill measurement (0 skips it)")
    ap.add_argument("--split-steps", type=int, default=50,
                    help="steps of the per-layer call sequence (attend per layer, then evict) timed after the "
                         "fused steps; 0 skips it")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference kernel for HBM counter scaling)")
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
    # training length, one layer per call: algorithmic FLOPs count 4*d per
    # allowed (query head, key) pair (QK and PV multiply-adds).
    prefill = None
    if w["policy"] == "kvpop" and args.prefill_len > 0:
        S = args.prefill_len
        gq = torch.Generator(device=dev).manual_seed(args.seed + 1)
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

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, gpu, args.seed, step_i, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.4g} steps/s ({cpu['seconds']:.1f}s of CPU work)")

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
        "dtype": "f32",
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
