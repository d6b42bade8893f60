"""The per-step decode loop over every (layer, batch row, KV head) segment.

[Conf-KV post], decoding-loop pseudocode, in its order: run the model with the
cache (here: append this step's key/value row and attend), take the softmax
of the logits, compute the confidence c, pick the budget from c against tau,
then for each layer update the attention-mass EMA, and if the layer holds
more rows than the budget, score and evict the lowest rows outside the
protected window; finally store rows older than the FP16 window as INT8.

[KVpop summary] §2.1-2.4 replaces confidence, EMA and score by the fixed
budget B = s + w + k over static priorities (see ``kvpop``).

Readings where the pages are silent (each is listed in the design doc):
* batch rows are independent decode streams: c and the budget are per row;
* budget and eviction are per segment (layer, batch row, KV head); query heads
  h*G .. h*G+G-1 share KV head h;
* the new row is appended before attention and attends to itself; its EMA
  starts at 0 and is updated in the same step like every other present row;
* the INT8 store runs every step, whether or not anything was evicted, and
  after the eviction; rows with pos <= t - W are INT8 afterwards;
* prefill rows take positions 0..P0-1, start with EMA 0, are neither attended
  nor evicted at initialization, and those with pos <= P0-1-W are stored INT8
  at once; the first decode row has position P0;
* scale of the attention scores 1/sqrt(d) unless given.

Segment order is seg = (l * B + b) * Hkv + h.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import attention, confidence, kvpop, policy, quant


@dataclass
class Config:
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    vocab: int = 0
    policy: str = "conf"          # "conf" | "kvpop"
    n_low: int = 0
    n_high: int = 0
    protect_last: int = 0         # P (CONF-KV) / w (KVpop)
    fp16_window: int = 0          # W
    num_sink: int = 0             # s
    tau: float = 0.6
    alpha: float = 0.5
    ema_beta: float = 0.9
    w_entropy: float = confidence.W_ENTROPY
    w_margin: float = confidence.W_MARGIN
    w_pmax: float = confidence.W_PMAX
    gate_literal: bool = False
    pyramid: bool = False
    kvpop_k: int = 0
    old_int8: bool = True
    softmax_scale: float = 0.0
    ranker: str = "score"         # "score": alpha*ema + (1-alpha)*recency; "random": SplitMix64 ranks
    seed: int = 0                 # seed of the random ranker

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale else 1.0 / math.sqrt(self.head_dim)

    @property
    def window(self) -> int:
        """Rows newer than this age stay FP16. KVpop keeps its protected
        window w in FP16 and moves a row out of it when it leaves protection."""
        return self.protect_last if self.policy == "kvpop" else self.fp16_window

    @classmethod
    def from_dict(cls, d: dict) -> "Config":
        names = cls.__dataclass_fields__.keys()
        return cls(**{k: v for k, v in d.items() if k in names})


class Segment:
    """Logical contents of one segment, rows in ascending position order."""

    def __init__(self, d: int):
        self.d = d
        self.pos = np.zeros(0, dtype=np.int64)
        self.is8 = np.zeros(0, dtype=bool)
        self.k16 = np.zeros((0, d), dtype=np.float16)
        self.v16 = np.zeros((0, d), dtype=np.float16)
        self.k8 = np.zeros((0, d), dtype=np.int8)
        self.v8 = np.zeros((0, d), dtype=np.int8)
        self.ks = np.zeros(0, dtype=np.float32)
        self.vs = np.zeros(0, dtype=np.float32)
        self.ema = np.zeros(0, dtype=np.float64)
        self.prio = np.zeros(0, dtype=np.float32)

    def __len__(self):
        return int(self.pos.size)

    def append(self, pos, k16, v16, ema=0.0, prio=np.nan):
        self.append_rows(np.array([pos]), np.asarray(k16).reshape(1, self.d), np.asarray(v16).reshape(1, self.d),
                         ema, prio)

    def append_rows(self, pos, K16, V16, ema=0.0, prio=np.nan):
        """Append FP16 rows (positions must exceed every present one)."""
        n, d = len(pos), self.d
        self.pos = np.concatenate([self.pos, np.asarray(pos, np.int64)])
        self.is8 = np.concatenate([self.is8, np.zeros(n, bool)])
        self.k16 = np.concatenate([self.k16, np.asarray(K16, np.float16).reshape(n, d)])
        self.v16 = np.concatenate([self.v16, np.asarray(V16, np.float16).reshape(n, d)])
        self.k8 = np.concatenate([self.k8, np.zeros((n, d), np.int8)])
        self.v8 = np.concatenate([self.v8, np.zeros((n, d), np.int8)])
        self.ks = np.concatenate([self.ks, np.zeros(n, np.float32)])
        self.vs = np.concatenate([self.vs, np.zeros(n, np.float32)])
        self.ema = np.concatenate([self.ema, np.full(n, float(ema))])
        self.prio = np.concatenate([self.prio, np.full(n, np.float32(prio), np.float32)])

    def keep(self, mask):
        for name in ("pos", "is8", "k16", "v16", "k8", "v8", "ks", "vs", "ema", "prio"):
            setattr(self, name, getattr(self, name)[mask])

    def remove(self, idx):
        mask = np.ones(len(self), dtype=bool)
        mask[np.asarray(idx, dtype=np.int64)] = False
        self.keep(mask)

    def dequantized(self):
        """K-hat, V-hat as float64: FP16 rows widened, INT8 rows fl32(code*scale)."""
        K = self.k16.astype(np.float64)
        V = self.v16.astype(np.float64)
        if self.is8.any():
            i8 = self.is8
            K[i8] = quant.dequantize(self.k8[i8], self.ks[i8]).astype(np.float64)
            V[i8] = quant.dequantize(self.v8[i8], self.vs[i8]).astype(np.float64)
        return K, V

    def store_int8_upto(self, limit_pos):
        """Quantize every row still in FP16 with pos <= limit_pos."""
        sel = np.nonzero((~self.is8) & (self.pos <= limit_pos))[0]
        for i in sel:
            self.k8[i], self.ks[i] = quant.quantize_row(self.k16[i])
            self.v8[i], self.vs[i] = quant.quantize_row(self.v16[i])
            self.k16[i] = 0
            self.v16[i] = 0
            self.is8[i] = True


@dataclass
class SegmentRecord:
    """What one segment's step produced (for comparison with the GPU)."""
    out: np.ndarray            # [G, d] float64 attention output
    lse: np.ndarray            # [G]
    pos: np.ndarray            # positions present during attention (ascending)
    mass: np.ndarray           # per present row (CONF-KV)
    score32: np.ndarray        # the oracle's own ranking value per present row, float32 (never an override)
    budget: int
    victims: np.ndarray        # evicted positions


@dataclass
class StepRecord:
    t: int
    conf: dict = field(default_factory=dict)       # b -> c
    base: dict = field(default_factory=dict)       # b -> base budget
    seg: dict = field(default_factory=dict)        # seg -> SegmentRecord


def conf_segment_step(seg: Segment, t, qg, k_new, v_new, budget, cfg: Config, score_override=None,
                      segment_id=0):
    """One CONF-KV step of one segment, in the pseudocode's order. With the
    random ranker the EMA is still kept; only the ranking value changes."""
    seg.append(t, k_new, v_new, ema=0.0)
    K, V = seg.dequantized()
    o, lse, p = attention.attend_two_pass(qg, K, V, cfg.scale)
    mass = attention.attention_mass(p)
    seg.ema = policy.ema_update(seg.ema, mass, cfg.ema_beta)
    if cfg.ranker == "random":
        score32 = policy.random_rank(cfg.seed, t, segment_id, seg.pos)
    else:
        score32 = policy.composite_score(seg.ema, policy.recency(seg.pos, t), cfg.alpha).astype(np.float32)
    rank_by = score32 if score_override is None else np.asarray(score_override, np.float32)
    present = seg.pos.copy()
    victims = policy.select_victims(seg.pos, rank_by, t, budget, cfg.num_sink, cfg.protect_last)
    seg.remove(victims)
    if cfg.old_int8:
        seg.store_int8_upto(t - cfg.window)
    return SegmentRecord(o, lse, present, mass, score32, int(budget), present[victims])


def kvpop_segment_step(seg: Segment, t, qg, k_new, v_new, prio_leaving, cfg: Config, prio_override=None):
    """One KVpop step of one segment: append, attend, score the row that
    leaves the window (delayed scoring), keep the top-k long-range rows."""
    w = cfg.protect_last
    seg.append(t, k_new, v_new)
    K, V = seg.dequantized()
    o, lse, p = attention.attend_two_pass(qg, K, V, cfg.scale)
    leaving = np.nonzero(seg.pos == t - w)[0]
    if leaving.size and t - w >= cfg.num_sink:
        seg.prio[leaving[0]] = np.float32(prio_leaving)
    own = seg.prio.copy()
    rank_by = own if prio_override is None else np.asarray(prio_override, np.float32)
    present = seg.pos.copy()
    victims = kvpop.long_range_victims(seg.pos, rank_by, t, cfg.num_sink, w, cfg.kvpop_k)
    seg.remove(victims)
    if cfg.old_int8:
        seg.store_int8_upto(t - cfg.window)
    return SegmentRecord(o, lse, present, np.zeros(0), own, kvpop.budget(cfg.num_sink, w, cfg.kvpop_k),
                         present[victims])


class OracleCache:
    """All (or a chosen subset of) segments of a model's KV cache."""

    def __init__(self, cfg: Config, segments=None):
        self.cfg = cfg
        L, B, H = cfg.num_layers, cfg.batch, cfg.num_kv_heads
        self.seg_ids = list(range(L * B * H)) if segments is None else sorted(int(s) for s in segments)
        self.segs = {s: Segment(cfg.head_dim) for s in self.seg_ids}
        self.t = 0

    def coords(self, seg: int):
        H, B = self.cfg.num_kv_heads, self.cfg.batch
        return seg // (B * H), (seg // H) % B, seg % H

    def rows(self):
        return sorted({self.coords(s)[1] for s in self.seg_ids})

    def init(self, prefill_len: int, rows_of=None):
        """rows_of(seg) -> (K16 [P0, d], V16 [P0, d]) for each simulated segment."""
        for s in self.seg_ids:
            seg = self.segs[s]
            if prefill_len:
                K, V = rows_of(s)
                seg.append_rows(np.arange(prefill_len), K[:prefill_len], V[:prefill_len])
                if self.cfg.old_int8:
                    seg.store_int8_upto(prefill_len - 1 - self.cfg.window)
        self.t = prefill_len

    def step(self, logits=None, q=None, k_new=None, v_new=None, prio=None, overrides=None, base_override=None):
        """One decode step. q [L][B][Hq][d], k_new/v_new [L][B][Hkv][d] (fp16),
        logits [B][V] (fp32, CONF-KV), prio [L][B][Hkv] (fp32, KVpop).
        overrides: optional seg -> ranking values per present row (lockstep
        checks hand in the GPU's own scores). base_override: b -> base budget."""
        cfg = self.cfg
        t = self.t
        rec = StepRecord(t)
        G = cfg.group
        if cfg.policy == "conf":
            for b in self.rows():
                c = confidence.confidence(np.asarray(logits[b]), cfg.w_entropy, cfg.w_margin, cfg.w_pmax)
                rec.conf[b] = c
                rec.base[b] = confidence.gate(c, cfg.tau, cfg.n_low, cfg.n_high, cfg.gate_literal)
            if base_override:
                rec.base.update(base_override)
        for s in self.seg_ids:
            l, b, h = self.coords(s)
            qg = np.asarray(q[l][b][h * G:(h + 1) * G], dtype=np.float16)
            kn = np.asarray(k_new[l][b][h], dtype=np.float16)
            vn = np.asarray(v_new[l][b][h], dtype=np.float16)
            ov = None if overrides is None else overrides.get(s)
            if cfg.policy == "conf":
                bud = confidence.layer_budget(rec.base[b], l, cfg.num_layers, cfg.pyramid)
                rec.seg[s] = conf_segment_step(self.segs[s], t, qg, kn, vn, bud, cfg, ov, segment_id=s)
            else:
                rec.seg[s] = kvpop_segment_step(self.segs[s], t, qg, kn, vn, float(prio[l][b][h]), cfg, ov)
        self.t = t + 1
        return rec
