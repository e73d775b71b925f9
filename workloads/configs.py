"""The five named workload shapes.

Shapes follow the layers the pages evaluate on (Mistral-7B, Yi-34B, Llama-70B and a
Llama-7B-sized MHA layer; KVCache reuse 01, CacheBlend §1.6 experiment table; QCFuse
summary §4 results) and chunk counts of 5/15/35 (CacheBlend problem definition page,
§2.6 F1-vs-chunk-count figure). Chunk length 512 and query lengths are choices of
this workload set; the pages never state them.

Selection specs:
  ("pct", p)         N = ceil(p * L_ctx / 100) selected context tokens per request.
  ("taper", [(a,b)]) one ratio a/b per simulated layer, N_l = ceil(a * L_ctx / b).
  ("quota", alpha)   per-chunk quotas drawn as ceil(alpha * u * T), u ~ U(0,1)
                     (Cache-Craft per-chunk N = ceil(CFO * |C|) form, KVCache reuse 01 §2.3.3).
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    dtype: str              # "f32" or "bf16": storage type of every tensor
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_base: float
    n_chunks: int           # chunks per request
    chunk_tokens: int
    query_len: int
    n_req: int = 1
    n_layers: int = 1
    select: Tuple = ("pct", 15)
    outlier_p: float = 0.0          # per context token probability of K x outlier_scale
    outlier_scale: float = 4.0
    head_scale: Optional[Tuple[float, float]] = None   # per-layer per-KV-head U(lo, hi) scales
    shared_chunks: Optional[int] = None                # chunks common to all requests
    anchors_k: int = 4
    placed_at: Optional[List[int]] = field(default=None, hash=False, compare=False)

    @property
    def ctx_len(self) -> int:
        return self.n_chunks * self.chunk_tokens

    @property
    def total_len(self) -> int:
        return self.ctx_len + self.query_len

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = [
    Config(0, "tiny_f32", "f32", 4, 2, 64, 10000.0, 3, 128, 16,
           select=("pct", 15)),
    Config(1, "mistral7b_layer", "bf16", 32, 8, 128, 10000.0, 5, 512, 32,
           select=("pct", 15), outlier_p=0.02),
    Config(2, "yi34b_layer_x4req", "bf16", 56, 8, 128, 10000.0, 15, 512, 48,
           n_req=4, select=("pct", 10), shared_chunks=11),
    Config(3, "llama70b_8layers", "bf16", 64, 8, 128, 10000.0, 35, 512, 64,
           n_layers=8, select=("taper", [(14 - l, 70) for l in range(8)]),
           head_scale=(0.5, 2.0)),
    Config(4, "llama7b_mha_quota", "bf16", 32, 32, 128, 10000.0, 64, 512, 64,
           select=("quota", 0.35)),
]


def get_config(key) -> Config:
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(key)
