"""GPU parity at the full sizes of the three large workloads, in the launch
configuration the benchmark times (every segment of the shape in one launch),
checked in lockstep on a sample of segments the oracle can follow one by one.

* Llama-3-8B shape at a 32K context: the first step attends over all 32769
  rows of every segment (HBM-staged) and radix-selects ~31.7K victims; the
  later steps are the LDS-staged steady state.
* Qwen-32B shape: 64 layers, batch 64, G = 5, pyramidal budgets, the whole
  4096-step stream with checks spread over it.
* KVpop on the Qwen3-8B shape: fill-up to the 2048-row budget, the first
  evictions, and the history-free closed form of the kept set.
* The per-layer calls (attend per layer with automatic split-K, then evict)
  on the Llama-3-8B shape at 32K: the first step splits 32769 rows per
  segment 32 ways.
"""

import pytest
import torch

from gpu_lockstep import DEV, Lockstep, log
from kv_cache_eviction_04_amd import confkv, synth
from oracle import kvpop as KP

pytestmark = pytest.mark.gpu


def segments(w, picks):
    B, H = w["batch"], w["num_kv_heads"]
    return sorted({(l * B + b) * H + h for l, b, h in picks})


def drive(ls, total, checked):
    worst = 0.0
    for i in range(total):
        r = ls.step(check=i in checked)
        if r:
            worst = max(worst, r["worst_out"])
            log(f"{ls.w['name']}: step {i} (t {r['t']}) checked, out err {r['worst_out']:.2e}")
    assert ls.gpu.status() == confkv.OK
    log(f"{ls.w['name']}: worst score err {ls.worst_score:.2e}, own-score victim flips {ls.own_flips}")
    return worst


def release_prefill(ls):
    ls.prefill = None
    torch.cuda.empty_cache()


def test_llama3_8b_32k_full_size():
    w = synth.workload("llama3_8b_32k")
    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    segs = segments(w, [(0, 0, 0), (0, B - 1, H - 1), (L // 2, 3, 2), (L - 1, 0, 5), (L - 1, B - 1, 7)])
    ls = Lockstep(w, 0, segs)
    release_prefill(ls)
    worst = drive(ls, 48, {0, 1, 2, 46, 47})
    log(f"llama3_8b_32k full size: worst out err {worst:.2e}")


def test_qwen32b_full_size_stream():
    w = synth.workload("qwen32b")
    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    segs = segments(w, [(0, 0, 0), (0, B - 1, H - 1), (L // 2, 17, 3), (L - 1, 0, 0), (L - 1, B - 1, 7)])
    ls = Lockstep(w, 1, segs)
    release_prefill(ls)
    n = w["steps"]
    worst = drive(ls, n, {0, 1, 2, n // 4, n // 2, 3 * n // 4, n - 1})
    log(f"qwen32b full size: {n} steps, worst out err {worst:.2e}")


def test_kvpop_qwen3_8b_full_size_fill_and_evict():
    w = synth.workload("kvpop_qwen3_8b")
    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    picks = [(0, 0, 0), (L // 2, 3, 4), (L - 1, B - 1, H - 1)]
    segs = segments(w, picks)
    seed = 2
    ls = Lockstep(w, seed, segs)
    s_, wnd, k = w["num_sink"], w["protect_last"], w["kvpop_k"]
    full = s_ + wnd + k                      # the budget is reached at step full - 1
    total = full + 560
    drive(ls, total, {0, 1, wnd, wnd + 1, full - 1, full, full + 1, total - 2, total - 1})
    # history-free closed form at the last step, for the sampled segments
    t = ls.gpu.position - 1
    prio = {}
    for step in range(wnd, t + 1):
        prio[step - wnd] = synth.step_inputs(w, seed, step, DEV)["prio"].cpu().numpy()
    for seg, (l, b, h) in zip(segs, sorted(picks, key=lambda p: (p[0] * B + p[1]) * H + p[2])):
        want = KP.kept_closed_form(t, lambda p: prio[p][l, b, h], s_, wnd, k)
        ro = ls.gpu.read_cache(seg, 1)
        n = int(ro["len"][0])
        assert ro["pos"][0, :n].tolist() == want, f"segment {seg}"
    log(f"kvpop full size: {total} steps, closed form holds at t {t}")


def test_llama3_8b_32k_full_size_per_layer_calls():
    w = synth.workload("llama3_8b_32k")
    L, B, H = w["num_layers"], w["batch"], w["num_kv_heads"]
    segs = segments(w, [(0, 0, 0), (L // 2, B - 1, 4), (L - 1, 7, 7)])
    ls = Lockstep(w, 3, segs, split=0)
    release_prefill(ls)
    worst = drive(ls, 6, {0, 1, 5})
    assert max(ls.splits_used) >= 2
    log(f"llama3_8b_32k per-layer calls: splits used {sorted(ls.splits_used)}, worst out err {worst:.2e}")


def test_kvpop_qwen3_8b_whole_stream_closed_form():
    """The KVpop stream at its stated length (131072 decode steps), on the GPU
    alone: at checkpoints along the stream the kept set of each sampled
    segment equals the history-free closed form, which static priorities make
    exact ("Resumen Técnico: KVpop" §2.3 and §2.4). The priorities the step
    consumes are gathered on the device as the stream runs."""
    w = synth.workload("kvpop_qwen3_8b")
    L, B, Hq, H, d = w["num_layers"], w["batch"], w["num_q_heads"], w["num_kv_heads"], w["head_dim"]
    s_, wnd, k = w["num_sink"], w["protect_last"], w["kvpop_k"]
    picks = [(0, 0, 0), (L // 2, 3, 4), (L - 1, B - 1, H - 1)]
    seed = 7
    total = w["steps"]
    checks = {s_ + wnd + k + 1000, total // 4 - 1, total // 2 - 1, total - 1}
    gpu = confkv.Cache(w, None, None)
    li = torch.tensor([p[0] for p in picks], device=DEV)
    bi = torch.tensor([p[1] for p in picks], device=DEV)
    hi = torch.tensor([p[2] for p in picks], device=DEV)
    pbuf = torch.empty((total, len(picks)), dtype=torch.float32, device=DEV)
    out = torch.empty((L, B, Hq, d), dtype=torch.float16, device=DEV)
    for step in range(total):
        x = synth.step_inputs(w, seed, step, DEV)
        gpu.step(None, x["q"], x["k"], x["v"], x["prio"], out=out)
        pbuf[step] = x["prio"][li, bi, hi]
        if step in checks:
            t = gpu.position - 1
            # the priority of position p arrives with the inputs of step p + w
            pr = pbuf[: t + 1].cpu().numpy()
            for j, (l, b, h) in enumerate(picks):
                seg = (l * B + b) * H + h
                want = KP.kept_closed_form(t, lambda p: pr[p + wnd, j], s_, wnd, k)
                ro = gpu.read_cache(seg, 1)
                n = int(ro["len"][0])
                assert ro["pos"][0, :n].tolist() == want, f"t {t} segment {seg}"
            log(f"kvpop whole stream: closed form holds at t {t} for {len(picks)} segments")
    assert gpu.status() == confkv.OK
