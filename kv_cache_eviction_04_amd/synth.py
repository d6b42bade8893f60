"""Seeded synthetic workloads and step inputs.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic. Both the GPU path and the CPU oracle are fed from it: the
GPU consumes the tensors directly and the oracle consumes device-to-host
copies of exactly those tensors, so the two never need the same random bits.

Workloads (the shapes of the pages' evaluation settings; synthetic values):
  toy              1 layer, 4 MHA heads, d 64, batch 1, vocab 1000
  gpt2_small       12 layers, 12 MHA heads, d 64, vocab 50257, batch 1, 1024-token prefill, pyramidal budgets
  llama3_8b_32k    32 layers, 32 q / 8 kv heads, d 128, vocab 128256, batch 16, 32768-token prefill
  qwen32b          64 layers, 40 q / 8 kv heads, d 128, vocab 152064, batch 64, 512-token prompt, pyramidal
  kvpop_qwen3_8b   36 layers, 32 q / 8 kv heads, d 128, batch 8, fixed budget s + w + k = 4 + 256 + 1788

q, k, v and prefill rows are N(0,1) rounded to fp16. Logits are fp32
N(0,1) * s with one s per (step, batch row): s = hi with probability p_hi,
else lo (bursty difficulty). KVpop priorities are U(0,1) fp32.
"""

from __future__ import annotations

import copy

import torch

_COMMON = dict(tau=0.6, alpha=0.5, ema_beta=0.9, w_entropy=0.4, w_margin=0.3, w_pmax=0.3,
               gate_literal=False, pyramid=False, num_sink=0, kvpop_k=0, old_int8=True,
               softmax_scale=0.0, policy="conf")

WORKLOADS = {
    "toy": dict(_COMMON, num_layers=1, batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64, vocab=1000,
                prefill=0, steps=512, n_low=64, n_high=128, protect_last=16, fp16_window=32,
                logit_law=((8.0, 0.8), (0.5, 0.2))),
    "gpt2_small": dict(_COMMON, num_layers=12, batch=1, num_q_heads=12, num_kv_heads=12, head_dim=64,
                       vocab=50257, prefill=1024, steps=4096, n_low=256, n_high=512, protect_last=64,
                       fp16_window=128, pyramid=True, logit_law=((8.0, 0.8), (0.5, 0.2))),
    "llama3_8b_32k": dict(_COMMON, num_layers=32, batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          vocab=128256, prefill=32768, steps=512, n_low=1024, n_high=2048, protect_last=128,
                          fp16_window=256, logit_law=((10.0, 0.9), (0.3, 0.1))),
    "qwen32b": dict(_COMMON, num_layers=64, batch=64, num_q_heads=40, num_kv_heads=8, head_dim=128,
                    vocab=152064, prefill=512, steps=4096, n_low=512, n_high=1024, protect_last=64,
                    fp16_window=256, pyramid=True, logit_law=((8.0, 0.8), (0.5, 0.2))),
    "kvpop_qwen3_8b": dict(_COMMON, policy="kvpop", num_layers=36, batch=8, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, vocab=0, prefill=0, steps=131072, num_sink=4, protect_last=256,
                           fp16_window=256, kvpop_k=1788, old_int8=False, logit_law=None),
}


def workload(name: str, **overrides) -> dict:
    w = copy.deepcopy(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    return w


def capacity(w: dict) -> int:
    """Old-region rows per segment that the workload can need: the prefill,
    or the largest budget (+1 for the row aged out in the same step)."""
    if w["policy"] == "kvpop":
        bmax = w["num_sink"] + w["protect_last"] + w["kvpop_k"]
    else:
        top = max(w["n_low"], w["n_high"])
        bmax = (3 * top) // 2 if w.get("pyramid") and w["num_layers"] > 1 else top
    need = max(w.get("prefill", 0), bmax + 1, w["num_sink"] + w["protect_last"] + 1)
    return int(need)


def _seed(seed: int, *tags: int) -> int:
    """Mix (seed, tags...) into a 63-bit generator seed (splitmix64 steps)."""
    x = (seed * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    for t in tags:
        x = (x ^ (t + 0x632BE59BD9B4E019)) & 0xFFFFFFFFFFFFFFFF
        x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed: int, *tags: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *tags))
    return g


_STREAM_LOGITS, _STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_PRIO, _STREAM_PRE_K, _STREAM_PRE_V, _STREAM_S = range(8)


def prefill(w: dict, seed: int, device, layers=None):
    """Prefill K, V as fp16 [L][B][Hkv][P0][d] (or only the given layers)."""
    L, B, H, d, P0 = w["num_layers"], w["batch"], w["num_kv_heads"], w["head_dim"], w["prefill"]
    layers = range(L) if layers is None else layers
    K = torch.empty((len(layers), B, H, P0, d), dtype=torch.float16, device=device)
    V = torch.empty_like(K)
    for i, l in enumerate(layers):
        K[i] = torch.randn((B, H, P0, d), generator=_gen(device, seed, _STREAM_PRE_K, l), device=device,
                           dtype=torch.float16)
        V[i] = torch.randn((B, H, P0, d), generator=_gen(device, seed, _STREAM_PRE_V, l), device=device,
                           dtype=torch.float16)
    return K, V


def step_inputs(w: dict, seed: int, step: int, device):
    """Inputs of decode step ``step`` (0-based): dict with logits [B][V] fp32
    (None for KVpop), q [L][B][Hq][d], k/v [L][B][Hkv][d] fp16 and prio
    [L][B][Hkv] fp32 (None for CONF-KV)."""
    L, B, Hq, H, d = w["num_layers"], w["batch"], w["num_q_heads"], w["num_kv_heads"], w["head_dim"]
    out = {}
    if w["policy"] == "conf":
        (hi, p_hi), (lo, _) = w["logit_law"]
        u = torch.rand((B,), generator=_gen(device, seed, _STREAM_S, step), device=device)
        s = torch.where(u < p_hi, torch.full_like(u, hi), torch.full_like(u, lo))
        z = torch.randn((B, w["vocab"]), generator=_gen(device, seed, _STREAM_LOGITS, step), device=device)
        out["logits"] = (z * s[:, None]).contiguous()
        out["prio"] = None
    else:
        out["logits"] = None
        out["prio"] = torch.rand((L, B, H), generator=_gen(device, seed, _STREAM_PRIO, step), device=device)
    out["q"] = torch.randn((L, B, Hq, d), generator=_gen(device, seed, _STREAM_Q, step), device=device,
                           dtype=torch.float16)
    out["k"] = torch.randn((L, B, H, d), generator=_gen(device, seed, _STREAM_K, step), device=device,
                           dtype=torch.float16)
    out["v"] = torch.randn((L, B, H, d), generator=_gen(device, seed, _STREAM_V, step), device=device,
                           dtype=torch.float16)
    return out
