"""The no-allocation KVpop prefill (confkv_kvpop_prefill_noalloc) against the
workspace entry point it varies (confkv_kvpop_prefill), through the C ABI.

Both enqueue the same kernels; only the workspace differs (the library's
static per-GPU array instead of the caller's buffer), so their outputs and
LSEs must be identical bit for bit. The existing entry point is itself held
to the oracle by the KVpop prefill tests. Two calls in a row, the second on a
smaller input, show that nothing of the first call's scratch leaks into the
second; a call whose workspace would exceed the array is refused.
"""

import pytest
import torch

from gpu_lockstep import DEV, log
from kv_cache_eviction_04_amd import confkv, synth

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, S, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, Hq, S, d), generator=g, device=DEV).half()
    k = torch.randn((B, Hkv, S, d), generator=g, device=DEV).half()
    v = torch.randn((B, Hkv, S, d), generator=g, device=DEV).half()
    p = torch.rand((B, Hkv, S), generator=g, device=DEV).contiguous()
    return q, k, v, p


def test_noalloc_prefill_matches_the_workspace_entry_point():
    B, Hq, Hkv, d = 2, 32, 8, 128
    w = synth.workload("kvpop_qwen3_8b", num_layers=1, batch=B)
    gpu = confkv.Cache(w)
    for call, (S, seed) in enumerate(((5000, 11), (1777, 12))):   # second call smaller
        log(f"no-alloc prefill: call {call}, S {S}, B {B}, Hq {Hq}, Hkv {Hkv}, d {d}")
        q, k, v, p = _inputs(B, Hq, Hkv, S, d, seed)
        lse_ref = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
        out_ref, lse_ref, _ = gpu.kvpop_prefill(q, k, v, p, lse=lse_ref)
        out = torch.full((B, Hq, S, d), float("nan"), dtype=torch.float16, device=DEV)
        lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
        gpu.kvpop_prefill_noalloc(q, k, v, p, out, lse)
        torch.cuda.synchronize()
        assert gpu.status() == confkv.OK
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), f"call {call}: outputs differ"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), f"call {call}: LSEs differ"


def test_noalloc_prefill_refuses_more_than_its_scratch():
    # B*Hkv = 64 segments: S = 16384 needs exactly the 16 MiB; S = 16500 more
    B, Hkv = 8, 8
    w = synth.workload("kvpop_qwen3_8b", num_layers=1, batch=B)
    gpu = confkv.Cache(w)
    L = confkv.lib()
    assert L.confkv_kvpop_prefill_workspace(gpu.h, 16384) == 16 << 20
    assert L.confkv_kvpop_prefill_workspace(gpu.h, 16500) > 16 << 20
    S, d, Hq = 16500, 128, 32
    q = torch.zeros((B, Hq, S, d), dtype=torch.float16, device=DEV)
    kv = torch.zeros((B, Hkv, S, d), dtype=torch.float16, device=DEV)
    p = torch.zeros((B, Hkv, S), dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(confkv.ConfKVError) as e:
        gpu.kvpop_prefill_noalloc(q, kv, kv, p, out)
    assert e.value.code == confkv.ECAPACITY
    assert gpu.status() == confkv.OK
