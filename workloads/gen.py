"""Seeded generators for the fusion-step inputs.

Every named tensor draws from its own stream,
``numpy.random.default_rng(SeedSequence(seed, spawn_key=(tensor_id, *extra)))``,
so a tensor regenerates bit-identically on its own, whatever else is drawn.
Values are ``standard_normal`` float32, optionally scaled, then stored either as
float32 ("f32" workloads) or as bfloat16 bit patterns in uint16 (round to nearest
even), which is exactly what the device receives.

Layout conventions (shared by every consumer):
  chunk store   [S, Hkv, D]        S = distinct chunk tokens, chunk id c at rows c*T..c*T+T-1
  chunk table   [n_req, n_chunks, 4] int32: (src_row, n_tokens, dst_row, orig_pos)
  q_crit        [n_req, Lq, Hq, D]  critical-layer query projections, before rotary embedding
  q/k/v fresh   [n_req, L, H, D]    position-indexed fresh projections, before rotary embedding
  quotas        [n_req, n_chunks] int32 (only for per-chunk-quota workloads)
The cached K in a chunk store stands for keys that were rotated at the chunk's
original positions orig_pos + t when the chunk was precomputed.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .configs import Config, get_config

_TENSOR_IDS = {
    "k_store": 1, "v_store": 2, "k_crit": 3, "q_crit": 4, "q_new": 5, "k_new": 6,
    "v_new": 7, "outlier": 8, "perm": 9, "head_scale": 10, "crit_scale": 11, "quota": 12,
}


def rng_for(seed: int, name: str, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS[name], *extra)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def store_as(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def normal(seed: int, name: str, shape, *extra: int) -> np.ndarray:
    return rng_for(seed, name, *extra).standard_normal(size=shape, dtype=np.float32)


@dataclass
class Workload:
    """All inputs of one fusion-step workload (one or more simulated layers)."""
    cfg: Config
    seed: int
    chunks: np.ndarray                    # [n_req, n_chunks, 4] int32
    store_rows: int
    k_crit: np.ndarray                    # [S, Hkv, D]
    q_crit: np.ndarray                    # [n_req, Lq, Hq, D]
    quotas: Optional[np.ndarray] = None   # [n_req, n_chunks] int32
    outlier_rows: Optional[np.ndarray] = None   # bool [S]
    _layers: Dict[int, dict] = field(default_factory=dict, repr=False)

    @property
    def dtype(self) -> str:
        return self.cfg.dtype

    def layer(self, l: int = 0) -> dict:
        """Per-layer tensors: k_store, v_store [S,Hkv,D]; q_new [n_req,L,Hq,D]; k_new, v_new [n_req,L,Hkv,D]."""
        if l not in self._layers:
            self._layers.clear()   # keep at most one layer resident: large layers are hundreds of MB
            self._layers[l] = _make_layer(self, l)
        return self._layers[l]

    def selection_spec(self, l: int = 0):
        """('count', num, den) meaning N = ceil(num * L_ctx / den), or ('quota', quotas)."""
        kind = self.cfg.select[0]
        if kind == "pct":
            return ("count", int(self.cfg.select[1]), 100)
        if kind == "taper":
            a, b = self.cfg.select[1][l]
            return ("count", int(a), int(b))
        if kind == "quota":
            return ("quota", self.quotas)
        raise ValueError(kind)


def _chunk_tables(cfg: Config, seed: int):
    T = cfg.chunk_tokens
    if cfg.shared_chunks is not None and cfg.n_req > 1:
        n_shared = cfg.shared_chunks
        n_priv = cfg.n_chunks - n_shared
        n_distinct = n_shared + n_priv * cfg.n_req
        tables = []
        for r in range(cfg.n_req):
            ids = list(range(n_shared)) + [n_shared + n_priv * r + i for i in range(n_priv)]
            perm = rng_for(seed, "perm", r).permutation(len(ids))
            ids = [ids[i] for i in perm]
            tables.append([(cid * T, T, c * T, 0) for c, cid in enumerate(ids)])
    else:
        n_distinct = cfg.n_chunks * cfg.n_req
        tables = []
        for r in range(cfg.n_req):
            tables.append([((r * cfg.n_chunks + c) * T, T, c * T, 0) for c in range(cfg.n_chunks)])
    return np.asarray(tables, dtype=np.int32), n_distinct * T


def make_workload(config, seed: Optional[int] = None) -> Workload:
    cfg = get_config(config) if not isinstance(config, Config) else config
    seed = cfg.index if seed is None else seed
    chunks, S = _chunk_tables(cfg, seed)
    Hq, Hkv, D = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    outlier = None
    kc = normal(seed, "k_crit", (S, Hkv, D))
    if cfg.outlier_p > 0:
        outlier = rng_for(seed, "outlier").random(S) < cfg.outlier_p
        kc[outlier] *= cfg.outlier_scale
    if cfg.head_scale is not None:
        lo, hi = cfg.head_scale
        kc *= rng_for(seed, "crit_scale").uniform(lo, hi, size=Hkv).astype(np.float32)[None, :, None]
    qc = normal(seed, "q_crit", (cfg.n_req, cfg.query_len, Hq, D))
    quotas = None
    if cfg.select[0] == "quota":
        alpha = float(cfg.select[1])
        u = rng_for(seed, "quota").random((cfg.n_req, cfg.n_chunks))
        quotas = np.ceil(alpha * u * cfg.chunk_tokens).astype(np.int32)
    return Workload(cfg=cfg, seed=seed, chunks=chunks, store_rows=S,
                    k_crit=store_as(kc, cfg.dtype), q_crit=store_as(qc, cfg.dtype),
                    quotas=quotas, outlier_rows=outlier)


def _make_layer(w: Workload, l: int) -> dict:
    cfg, seed, S = w.cfg, w.seed, w.store_rows
    Hq, Hkv, D, L, nr = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.total_len, cfg.n_req
    ks = normal(seed, "k_store", (S, Hkv, D), l)
    vs = normal(seed, "v_store", (S, Hkv, D), l)
    qn = normal(seed, "q_new", (nr, L, Hq, D), l)
    kn = normal(seed, "k_new", (nr, L, Hkv, D), l)
    vn = normal(seed, "v_new", (nr, L, Hkv, D), l)
    if w.outlier_rows is not None:
        ks[w.outlier_rows] *= cfg.outlier_scale
        # the same tokens keep a large key when their K is freshly recomputed
        for r in range(nr):
            for (src, n, dst, _o) in w.chunks[r]:
                m = w.outlier_rows[src:src + n]
                kn[r, dst:dst + n][m] *= cfg.outlier_scale
    if cfg.head_scale is not None:
        lo, hi = cfg.head_scale
        sc = rng_for(seed, "head_scale", l).uniform(lo, hi, size=(2, Hkv)).astype(np.float32)
        ks *= sc[0][None, :, None]
        kn *= sc[0][None, None, :, None]
        vs *= sc[1][None, :, None]
        vn *= sc[1][None, None, :, None]
    return {"k_store": store_as(ks, cfg.dtype), "v_store": store_as(vs, cfg.dtype),
            "q_new": store_as(qn, cfg.dtype), "k_new": store_as(kn, cfg.dtype),
            "v_new": store_as(vn, cfg.dtype)}


def make_custom(*, dtype="f32", n_q_heads=4, n_kv_heads=2, head_dim=64, rope_base=10000.0,
                chunk_lens=(16, 24), orig_pos=None, query_len=4, n_req=1, seed=1234,
                select=("pct", 25), extra_store_rows=0, anchors_k=2) -> Workload:
    """A small workload with ragged chunk lengths and arbitrary original positions.

    Chunk c of request r sits at store rows [src, src+T_c) (requests use disjoint
    rows, plus ``extra_store_rows`` unused rows at the end) and at fused rows
    [n_c, n_c+T_c), n_c = sum of the earlier lengths.
    """
    lens = [int(t) for t in chunk_lens]
    n_chunks = len(lens)
    orig = [0] * n_chunks if orig_pos is None else [int(o) for o in orig_pos]
    tables, src = [], 0
    for _r in range(n_req):
        rows, dst = [], 0
        for c in range(n_chunks):
            rows.append((src, lens[c], dst, orig[c]))
            src += lens[c]
            dst += lens[c]
        tables.append(rows)
    S = src + extra_store_rows
    L_ctx = sum(lens)
    cfg = Config(-1, "custom", dtype, n_q_heads, n_kv_heads, head_dim, rope_base, n_chunks,
                 max(lens), query_len, n_req=n_req, select=select, anchors_k=anchors_k)
    chunks = np.asarray(tables, dtype=np.int32)
    kc = normal(seed, "k_crit", (S, n_kv_heads, head_dim))
    qc = normal(seed, "q_crit", (n_req, query_len, n_q_heads, head_dim))
    quotas = None
    if select[0] == "quota":
        u = rng_for(seed, "quota").random((n_req, n_chunks))
        quotas = np.ceil(float(select[1]) * u * np.asarray(lens)[None, :]).astype(np.int32)
    w = Workload(cfg=cfg, seed=seed, chunks=chunks, store_rows=S,
                 k_crit=store_as(kc, dtype), q_crit=store_as(qc, dtype), quotas=quotas)
    L = L_ctx + query_len
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    w._layers[0] = {
        "k_store": store_as(normal(seed, "k_store", (S, Hkv, D), 0), dtype),
        "v_store": store_as(normal(seed, "v_store", (S, Hkv, D), 0), dtype),
        "q_new": store_as(normal(seed, "q_new", (n_req, L, Hq, D), 0), dtype),
        "k_new": store_as(normal(seed, "k_new", (n_req, L, Hkv, D), 0), dtype),
        "v_new": store_as(normal(seed, "v_new", (n_req, L, Hkv, D), 0), dtype),
    }
    return w
