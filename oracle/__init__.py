"""CPU oracle for the confidence-gated KV-cache eviction decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. The GPU library shares no
code, header, table or constant generator with it.

This is a plain, slow, obviously-correct NumPy implementation, computed in
float64 except where the method fixes another precision (the INT8 quantizer
is emulated with exact IEEE float32 operations). It follows the steps of the
method in the order the pages give them.

Sources (cited by page title and section throughout):

* [CONF-KV abstract] "CONF-KV: Confidence-Aware KV Cache Eviction with
  Mixed-Precision Storage for Long-Horizon LLMs", abstract (chatpaper.ai).
* [Conf-KV post] "Conf-KV: confidence-aware KV-cache eviction with mixed
  FP16/INT8 storage" (rcap.io blog post): the method paragraphs, the
  decoding-loop pseudocode, and the caveats list.
* [KVpop summary] "Resumen Técnico: KVpop — Compresión de Caché de
  Clave-Valor con Poda Predictiva en Línea" (gist.science): §2.1
  architecture and budget, §2.3 delayed scoring, §2.4 inference efficiency.

Where the pages are silent or contradict each other the reading taken is
stated at the function that depends on it.

Modules:
    confidence  next-token distribution -> confidence c -> gated budget
    attention   decode attention (two-pass, blockwise online, split+LSE)
    quant       per-token absmax INT8 quantizer (float32-exact)
    policy      EMA, recency, composite score, protected-window eviction
    kvpop       sink + window + top-k fixed budget over static priorities
    cache       the whole per-step loop over every (layer, batch, kv-head)
    sampling    the next token from p = softmax(logits): greedy or inverse-CDF
    kvpop_prefill  KVpop's multi-query mask and masked prefill attention
"""

from . import confidence, attention, quant, policy, kvpop, cache, sampling, kvpop_prefill  # noqa: F401
