"""Host-side checks of bench.py's contract (no GPU): multi-GPU runs are
refused, the algorithmic byte count of a launch, and the tie between the
stored HBM-traffic figure and the kernel sources it was measured on."""

import os
import re
import subprocess
import sys

import bench
from kv_cache_eviction_04_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_a_steady_llama_step():
    # Steady state of the Llama-3-8B 32K shape: 1025 rows per segment, 257 in
    # the FP16 window (512 B each) and 768 INT8 rows (256 B of codes + 8 B of
    # scales), one aged-out row moved per segment.
    w = synth.workload("llama3_8b_32k")
    S = w["num_layers"] * w["batch"] * w["num_kv_heads"]
    steps = 10
    kv_seg = 257 * 512 + 768 * 264
    st = {"kv_bytes": kv_seg * S * steps, "rows_attended": 1025 * S * steps, "rows_moved": S * steps}
    kv, total = bench.algorithmic_bytes(w, st, steps, S)
    assert kv == kv_seg * S == 1369440256
    q_and_out = 2 * (32 * 16 * 32 * 128 * 2)             # q read, out written (fp16)
    new_row = S * (2 * 128 * 2) + S * (4 * 128)          # k_new/v_new read, written into the ring
    state = 1025 * S * 12                                # pos read, EMA read and written
    moved = S * 2 * 264                                  # a moved row, read and written at the old-row size
    assert total == kv + state + q_and_out + new_row + moved
    assert abs(total / 1.435e9 - 1.0) < 2e-3             # the per-launch figure the measurements quote


def test_stored_traffic_is_tied_to_the_kernel_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "fused_step_kernel.llama3_8b_32k.hbm_traffic.md")
    text = open(path).read()
    recorded = re.search(r"kernel_source_sha256: `([0-9a-f]{64})`", text).group(1)
    figure = float(re.search(r"traffic_bytes_per_launch: `(\d+)`", text).group(1))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: recorded)
    assert bench.stored_traffic("llama3_8b_32k") == figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.stored_traffic("llama3_8b_32k") is None
    assert bench.stored_traffic("no_such_workload") is None


def test_cpu_baseline_workers_reproduce_the_oracle_step():
    # The baseline's pool runs the oracle's confidence per (row, step) and its
    # per-segment step per segment; together they must equal OracleCache.step.
    import copy

    import numpy as np
    import torch

    from oracle import cache as OC

    for name, over in (("toy", dict(prefill=100)), ("kvpop_qwen3_8b", dict(num_layers=1, batch=2, protect_last=8,
                                                                          fp16_window=8, kvpop_k=20))):
        w = synth.workload(name, **over)
        cfg = OC.Config.from_dict(w)
        S = w["num_layers"] * w["batch"] * w["num_kv_heads"]
        rng = np.random.default_rng(0)
        ref = OC.OracleCache(cfg)
        P0 = w["prefill"]
        rows_of = {s: (rng.standard_normal((P0, w["head_dim"])), rng.standard_normal((P0, w["head_dim"])))
                   for s in range(S)}
        ref.init(P0, lambda s: rows_of[s])
        states = {s: copy.deepcopy(ref.segs[s]) for s in range(S)}
        steps = []
        for i in range(6):
            x = {k: (None if v is None else v.numpy()) for k, v in
                 synth.step_inputs(w, 1, i, torch.device("cpu")).items()}
            steps.append(x)
            ref.step(logits=x["logits"], q=x["q"], k_new=x["k"], v_new=x["v"], prio=x["prio"])
        if cfg.policy == "conf":
            tasks = [((b, i), x["logits"][b]) for i, x in enumerate(steps) for b in range(w["batch"])]
            bases, _ = bench._oracle_rows_worker((cfg, tasks))
            for i, x in enumerate(steps):
                x["base"] = {b: bases[(b, i)] for b in range(w["batch"])}
        bench._oracle_segments_worker((cfg, P0, states, steps))
        for s in range(S):
            assert states[s].pos.tolist() == ref.segs[s].pos.tolist()
            assert np.array_equal(states[s].ema, ref.segs[s].ema)


def test_host_cores_respects_the_thread_share(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.host_cores() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.setenv("OMP_NUM_THREADS", "")
    assert bench.host_cores() == len(os.sched_getaffinity(0))
