"""fp64 oracle for the per-layer KV-cache fusion step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. Nothing here is shared with the HIP path.

What is computed (sources are the five pages on non-prefix KV-cache reuse):
  * full KV reuse after adjusting position encodings -- CacheBlend problem
    definition page, §2.4 "Full KV Reuse";
  * per-layer selective recompute: mask to the selected tokens, compute their
    Q/K/V, extend K/V with the reused cache of the other tokens, attend selected
    x all tokens -- KVCache reuse 01, §1.3.4 (CacheBlend selective recompute flow);
  * query-centric selection: attention of the query's Q against one critical
    middle layer's K, top-N context tokens -- QCFuse summary (zh) §2.A
    "critical-layer attention profiling" and (ja) §2 system workflow;
  * key-norm anchors per chunk -- QCFuse summary (zh) §2.A "anchor-based
    lightweight query probing";
  * location-aware sparse attention over a discrete token index table with a
    strict causal constraint -- QCFuse summary (zh) §2.A last bullet;
  * N rounded up, N = ceil(ratio * |C|) -- Cache-Craft CSDN article §2.1 and
    KVCache reuse 01 §2.3.3; ties keep the lower index, as a stable sort by
    descending score does -- Cache-Craft CSDN article §2.2.2 token selection.

Readings where the pages are silent (all documented with the design notes):
  rotary pairs are half-split (i, i + d/2); theta_i = base^(-2i/d); logits are
  scaled by 1/sqrt(d); cached K holds keys rotated at orig_pos + t, so moving a
  chunk to fused row n_c rotates it by delta_c = n_c - orig_pos; the scoring
  softmax runs over context keys only and is summed unweighted over all query
  heads and query rows; query rows are always recomputed and sit at [L_ctx, L);
  query head h uses KV head h // g; key j is visible to a recomputed row at
  absolute position p iff j <= p.

Every array here is float64 (inputs are upcast from the exact bits the device
receives). Rounding to the storage type happens only where the fused cache is
stored. Nothing is blocked, fused or reordered beyond the definitions.
"""
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "to_f64", "round_to_storage", "bf16_round", "storage_bits", "rope_theta", "rope",
    "chunk_layout", "fuse_rerotate", "key_norms", "extract_anchors", "critical_scores",
    "select_count", "select_topn", "select_topn_quota", "row_positions", "scatter_kv",
    "sparse_causal_attn", "fused_layer", "kv_deviation", "hkvd_filter", "gradual_filter_layers",
    "anchor_prefix", "anchor_probe", "query_centric_layers", "chunk_attention_stats",
    "cache_context_impact", "preceding_chunk_scores", "prefix_overlap", "cachecraft_count",
]


# ----------------------------------------------------------------------------- storage types

def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Upcast stored values: float32 arrays directly, bfloat16 bit patterns (uint16) via float32."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (one rounding step).

    bfloat16 keeps 8 significant bits; values are rounded on the grid 2^(e-8) where
    x = m * 2^e with 0.5 <= |m| < 1 (e clamped at the smallest normal exponent).
    """
    x = np.asarray(x, dtype=np.float64)
    _m, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    return np.rint(x / q) * q


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


def storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of values that already lie on the storage grid."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.view(np.uint32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- rotary embedding

def rope_theta(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d) for i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate every pair (x_i, x_{i+d/2}) by the angle pos * theta_i.

    x: [..., d]; pos: scalar or array broadcastable to x.shape[:-1].
    (x_i, x_{i+d/2}) -> (x_i cos - x_{i+d/2} sin, x_i sin + x_{i+d/2} cos).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ----------------------------------------------------------------------------- S1: re-rotation

def chunk_layout(chunks: np.ndarray) -> Tuple[int, List[Tuple[int, int, int, int]]]:
    """Concatenate chunks in request order: chunk c lands at n_c = sum of earlier lengths.

    chunks: [n_chunks, 4] rows (src_row, n_tokens, dst_row, orig_pos). The table's
    dst_row must equal n_c. Returns (L_ctx, [(src, T, n_c, delta_c)]) with
    delta_c = n_c - orig_pos (the position shift the cached keys must undergo).
    """
    out, n = [], 0
    for src, T, dst, orig in np.asarray(chunks).tolist():
        if dst != n:
            raise ValueError("chunks must tile the context in request order")
        out.append((int(src), int(T), n, n - int(orig)))
        n += int(T)
    return n, out


def fuse_rerotate(k_store, v_store, chunks, L: int, dtype: str, base: float):
    """Full KV reuse with position re-alignment (CacheBlend problem definition, §2.4).

    K_fused[n_c + t] = round(R(delta_c) K_store[src_c + t]); V_fused[n_c + t] = V_store[src_c + t].
    Returns float64 arrays [L, Hkv, d]; rows >= L_ctx are NaN (not written by this stage).
    """
    ks, vs = to_f64(k_store, dtype), to_f64(v_store, dtype)
    L_ctx, lay = chunk_layout(chunks)
    kf = np.full((L,) + ks.shape[1:], np.nan)
    vf = np.full((L,) + vs.shape[1:], np.nan)
    for src, T, n, delta in lay:
        kf[n:n + T] = round_to_storage(rope(ks[src:src + T], delta, base), dtype)
        vf[n:n + T] = vs[src:src + T]
    return kf, vf


# ----------------------------------------------------------------------------- S2a: anchors

def key_norms(k_crit_store, dtype: str) -> np.ndarray:
    """L2 norm of each cached key over all KV heads and head dimensions."""
    k = to_f64(k_crit_store, dtype)
    return np.sqrt(np.sum(k.reshape(k.shape[0], -1) ** 2, axis=1))


def extract_anchors(k_crit_store, chunks, k: int, dtype: str) -> np.ndarray:
    """Per chunk, the k tokens with the largest key norm (QCFuse summary (zh) §2.A, anchors).

    Order is (-norm, t): larger norms first, the lower token offset wins a tie.
    Returns [n_chunks, k] int32 token offsets within each chunk.
    """
    norms = key_norms(k_crit_store, dtype)
    out = []
    for src, T, _dst, _orig in np.asarray(chunks).tolist():
        nt = norms[src:src + T]
        order = sorted(range(T), key=lambda t: (-nt[t], t))
        out.append(order[:k])
    return np.asarray(out, dtype=np.int32)


def anchor_prefix(k_store, v_store, chunks, anchors, dtype: str, base: float):
    """Anchors as a compact prefix for the query probe (QCFuse summary (zh) §2.A: the anchors are
    injected into the query's forward pass as a lightweight prefix).

    Reading: the anchors of each chunk in ascending token order, chunks in request order, occupy
    prefix rows a = 0 .. A-1 (A = n_chunks * k). A key cached at position orig_c + t moves to row a:
    K_pre[a] = round(R(a - orig_c - t) K_store[src_c + t]); V_pre[a] = V_store[src_c + t].
    anchors: [n_chunks, k] token offsets. Returns float64 (K_pre, V_pre) [A, Hkv, d].
    """
    ks, vs = to_f64(k_store, dtype), to_f64(v_store, dtype)
    kp, vp = [], []
    a = 0
    for (src, _T, _dst, orig), anc in zip(np.asarray(chunks).tolist(), np.asarray(anchors).tolist()):
        for t in sorted(int(x) for x in anc):
            kp.append(round_to_storage(rope(ks[src + t], a - int(orig) - t, base), dtype))
            vp.append(vs[src + t])
            a += 1
    d = ks.shape[-1]
    shape = (a, ks.shape[1], d)
    return np.asarray(kp).reshape(shape), np.asarray(vp).reshape(shape)


def anchor_probe(k_pre, v_pre, q_new, k_new, v_new, dtype: str, base: float):
    """The query's forward pass over the anchor prefix: the Lq query rows sit at rows A .. A+Lq-1
    after the A prefix rows; their K/V are stored there (K rotated at its row) and every query row
    attends causally to the prefix and the query rows up to itself.
    q_new, k_new, v_new: stored values [Lq, H, d]. Returns (O [Lq, Hq, d], LSE [Lq, Hq])."""
    A = k_pre.shape[0]
    Lq = np.asarray(q_new).shape[0]
    kf = np.concatenate([k_pre, np.full((Lq,) + k_pre.shape[1:], np.nan)])
    vf = np.concatenate([v_pre, np.full((Lq,) + v_pre.shape[1:], np.nan)])
    rp = (A + np.arange(Lq)).astype(np.int32)
    kf, vf = scatter_kv(kf, vf, k_new, v_new, rp, dtype, base)
    return sparse_causal_attn(q_new, rp, kf, vf, dtype, base)


def query_centric_layers(q_layers, k_layers, chunks, n_kv_heads: int, dtype: str, base: float,
                         n_select: int, mode: str):
    """The query-centric baselines the QCFuse pages compare against (QCFuse summary (zh) §4
    results; (ja) §3): QCAll scores every layer with that layer's own query and cached keys and
    recomputes each layer's own top-N; QCLast scores only the last layer and uses its top-N for
    every layer. q_layers[l]: [Lq, Hq, d]; k_layers[l]: the layer's chunk store.
    Returns (scores [n_layers or 1][L_ctx], selections [n_layers][N])."""
    if mode == "all":
        sc = [critical_scores(q, k, chunks, n_kv_heads, dtype, base) for q, k in zip(q_layers, k_layers)]
        return np.asarray(sc), [select_topn(s, n_select) for s in sc]
    if mode == "last":
        s = critical_scores(q_layers[-1], k_layers[-1], chunks, n_kv_heads, dtype, base)
        sel = select_topn(s, n_select)
        return s[None], [sel for _ in q_layers]
    raise ValueError(mode)


# ----------------------------------------------------------------------------- S2b: scoring

def critical_scores(q_crit, k_crit_store, chunks, n_kv_heads: int, dtype: str, base: float) -> np.ndarray:
    """Query-centric token scores from one critical layer (QCFuse summary (zh) §2.A).

    k'_j = R(delta_c) K_crit[src_c + t] for j = n_c + t (the key re-aligned to the fused
    layout, not rounded); q_{i,h} = R(L_ctx + i) Q_crit[i, h] (the query follows the chunks).
    x = q . k' / sqrt(d); softmax over the L_ctx context keys for every (h, i);
    s_j = sum over all query heads h and query rows i of the probability of key j.
    q_crit: [Lq, Hq, d]. Returns s [L_ctx].
    """
    q = to_f64(q_crit, dtype)
    kc = to_f64(k_crit_store, dtype)
    Lq, Hq, d = q.shape
    g = Hq // n_kv_heads
    L_ctx, lay = chunk_layout(chunks)
    kp = np.empty((L_ctx, n_kv_heads, d))
    for src, T, n, delta in lay:
        kp[n:n + T] = rope(kc[src:src + T], delta, base)
    qr = rope(q, (L_ctx + np.arange(Lq))[:, None], base)      # [Lq, Hq, d]
    s = np.zeros(L_ctx)
    for h in range(Hq):
        x = qr[:, h, :] @ kp[:, h // g, :].T / math.sqrt(d)  # [Lq, L_ctx]
        x = x - x.max(axis=1, keepdims=True)
        p = np.exp(x)
        p = p / p.sum(axis=1, keepdims=True)
        s += p.sum(axis=0)
    return s


# ----------------------------------------------------------------------------- S2c: selection

def select_count(num: int, den: int, L_ctx: int) -> int:
    """N = ceil(num * L_ctx / den) in exact integer arithmetic (Cache-Craft's ceil rounding)."""
    num, den, L_ctx = int(num), int(den), int(L_ctx)
    if den <= 0 or num < 0:
        raise ValueError("ratio must be non-negative with a positive denominator")
    return -((-num * L_ctx) // den)


def select_topn(scores: Sequence[float], N: int) -> np.ndarray:
    """The N best indices by (-score, index), returned in ascending index order."""
    s = [float(v) for v in scores]
    order = sorted(range(len(s)), key=lambda j: (-s[j], j))
    return np.asarray(sorted(order[:N]), dtype=np.int32)


def select_topn_quota(scores: Sequence[float], chunks, quotas: Sequence[int]) -> np.ndarray:
    """Per-chunk quotas (Cache-Craft per-chunk argtop_N, KVCache reuse 01 §2.3.3):
    top quota_c of each chunk's own tokens by (-score, index); chunks concatenated in order."""
    _L, lay = chunk_layout(chunks)
    parts = []
    for (src, T, n, _delta), qc in zip(lay, quotas):
        if qc > T:
            raise ValueError("quota exceeds chunk length")
        parts.append(n + select_topn(np.asarray(scores)[n:n + T], int(qc)))
    return np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, np.int32)


def row_positions(sel, L_ctx: int, Lq: int) -> np.ndarray:
    """Recomputed rows: the selected context positions, then every query position."""
    return np.concatenate([np.asarray(sel, dtype=np.int64), L_ctx + np.arange(Lq)]).astype(np.int32)


# ----------------------------------------------------------------------------- S3: scatter

def scatter_kv(k_fused, v_fused, k_new, v_new, row_pos, dtype: str, base: float):
    """Overwrite the recomputed rows (KVCache reuse 01 §1.3.4, 'extend K_i and V_i').

    K_fused[row_pos[r]] = round(R(row_pos[r]) K_new[r]); V_fused[row_pos[r]] = V_new[r].
    k_new, v_new: stored values [R, Hkv, d] (compact, K before rotation). Returns copies.
    """
    kf, vf = np.array(k_fused, dtype=np.float64), np.array(v_fused, dtype=np.float64)
    kn, vn = to_f64(k_new, dtype), to_f64(v_new, dtype)
    rp = np.asarray(row_pos, dtype=np.int64)
    kf[rp] = round_to_storage(rope(kn, rp[:, None], base), dtype)
    vf[rp] = vn
    return kf, vf


# ----------------------------------------------------------------------------- CacheBlend gradual filtering

def kv_deviation(k_fused, v_fused, k_new, v_new, row_pos, n_rows: int, dtype: str, base: float):
    """KV deviation of recomputed tokens (KVCache reuse 01, §1.3.2: the absolute difference between
    a token's reused KV and its recomputed KV; §1.3.3 ranks tokens by it).

    Reading: for each of the first n_rows recomputed rows r, at absolute position p = row_pos[r],
    the Euclidean norm, over every KV head and dimension, of (recomputed K - reused K) together
    with (recomputed V - reused V). The recomputed K is the value the cache would store,
    round(R(p) K_new[r]); the reused K/V are the cache's rows at p after re-rotation and before the
    scatter. k_fused, v_fused: float64 [L, Hkv, d]; k_new, v_new: stored values [>= n_rows, Hkv, d]
    (compact, K before rotation). Returns float64 [n_rows].
    """
    n = int(n_rows)
    rp = np.asarray(row_pos, dtype=np.int64)[:n]
    kf, vf = np.asarray(k_fused, dtype=np.float64), np.asarray(v_fused, dtype=np.float64)
    kn = round_to_storage(rope(to_f64(np.asarray(k_new)[:n], dtype), rp[:, None], base), dtype)
    vn = to_f64(np.asarray(v_new)[:n], dtype)
    dk = kn - kf[rp]
    dv = vn - vf[rp]
    return np.sqrt((dk * dk).sum(axis=(1, 2)) + (dv * dv).sum(axis=(1, 2)))


def hkvd_filter(dev, row_pos, n_prev: int, n_keep: int) -> np.ndarray:
    """Next layer's recomputed rows under gradual filtering (KVCache reuse 01, §1.3.3: layer i keeps,
    among the tokens layer i-1 selected, the given share with the highest KV deviation).

    row_pos holds the previous selection (n_prev context positions, ascending) followed by the query
    rows. The n_keep context rows of highest deviation (float64, ties to the lower row) are kept in
    ascending order, followed by the same query rows.
    """
    rp = np.asarray(row_pos, dtype=np.int64)
    keep = select_topn(np.asarray(dev, dtype=np.float64)[:n_prev], int(n_keep))
    return np.concatenate([rp[:n_prev][keep], rp[n_prev:]]).astype(np.int32)


# ----------------------------------------------------------------------------- S4: attention

def sparse_causal_attn(q_new, row_pos, k_fused, v_fused, dtype: str, base: float,
                       rows: Optional[Sequence[int]] = None):
    """Location-aware sparse causal attention (QCFuse summary (zh) §2.A; KVCache reuse 01 §1.3.4).

    For recomputed row r at absolute position p = row_pos[r] and query head h:
    q = R(p) Q_new[r, h]; keys j <= p of KV head h // g; O = softmax(q . K_j / sqrt(d)) V_j.
    q_new: stored [R, Hq, d]; k_fused, v_fused: float64 [L, Hkv, d] (values on the storage grid).
    rows: optional subset of r to evaluate. Returns (O [n_rows, Hq, d], LSE [n_rows, Hq]).
    """
    q = to_f64(q_new, dtype)
    R, Hq, d = q.shape
    Hkv = k_fused.shape[1]
    g = Hq // Hkv
    rp = np.asarray(row_pos, dtype=np.int64)
    rows = range(R) if rows is None else rows
    # keys and values of one KV head as contiguous [L, d] arrays (a copy, no arithmetic)
    kh = [np.ascontiguousarray(np.asarray(k_fused, dtype=np.float64)[:, kv, :]) for kv in range(Hkv)]
    vh = [np.ascontiguousarray(np.asarray(v_fused, dtype=np.float64)[:, kv, :]) for kv in range(Hkv)]
    outs, lses = [], []
    for r in rows:
        p = int(rp[r])
        qr = rope(q[r], p, base)                                  # [Hq, d]
        o = np.empty((Hq, d))
        lse = np.empty(Hq)
        for kv in range(Hkv):
            # the g query heads h = kv*g .. kv*g+g-1 of this KV head, one column each
            x = kh[kv][:p + 1] @ qr[kv * g:(kv + 1) * g].T / math.sqrt(d)   # [p+1, g]
            m = x.max(axis=0)
            e = np.exp(x - m)
            o[kv * g:(kv + 1) * g] = (e / e.sum(axis=0)).T @ vh[kv][:p + 1]
            lse[kv * g:(kv + 1) * g] = m + np.log(e.sum(axis=0))
        outs.append(o)
        lses.append(lse)
    return np.asarray(outs).reshape(len(outs), Hq, d), np.asarray(lses).reshape(len(lses), Hq)


# ----------------------------------------------------------------------------- Cache-Craft selection

def chunk_attention_stats(q_new, k_cache, chunks, n_kv_heads: int, dtype: str, base: float, rows=None):
    """Per-token inter-chunk attention of a full causal prefill (Cache-Craft: inter-attention is the
    sum of attention weights between chunks, KVCache reuse 01 §2.3.1; the per-token table is what
    the token selection sums, Cache-Craft CSDN article §2.2.2).

    For context token t (query, rotated at t) and chunk j: inter[t, j] = sum over query heads h of the
    softmax probability, over the keys s <= t of the context, of the keys s in chunk j. The keys are
    the prefill's cache rows (k_cache: stored values [>= L_ctx, Hkv, d], already rotated at their
    positions); q_new: stored [>= L_ctx, Hq, d] before rotation. rows: optional subset of tokens.
    Returns float64 [n_rows, n_chunks]; every row sums to Hq.
    """
    L_ctx, lay = chunk_layout(chunks)
    q = to_f64(np.asarray(q_new)[:L_ctx], dtype)
    kc = to_f64(np.asarray(k_cache)[:L_ctx], dtype)
    Hq, d = q.shape[1], q.shape[2]
    g = Hq // n_kv_heads
    rows = np.arange(L_ctx) if rows is None else np.asarray(rows, dtype=np.int64)
    qr = rope(q[rows], rows[:, None], base)                              # [n, Hq, d]
    chunk_of = np.empty(L_ctx, dtype=np.int64)
    for c, (_src, T, n, _delta) in enumerate(lay):
        chunk_of[n:n + T] = c
    inter = np.zeros((len(rows), len(lay)))
    visible = np.arange(L_ctx)[None, :] <= rows[:, None]                # key s <= token t
    for h in range(Hq):
        x = qr[:, h, :] @ kc[:, h // g, :].T / math.sqrt(d)             # [n, L_ctx]
        x = np.where(visible, x, -np.inf)
        x = x - x.max(axis=1, keepdims=True)
        p = np.exp(x)
        p = p / p.sum(axis=1, keepdims=True)
        for c in range(len(lay)):
            inter[:, c] += p[:, chunk_of == c].sum(axis=1)
    return inter


def preceding_chunk_scores(inter, chunks) -> np.ndarray:
    """Token score for recompute selection (KVCache reuse 01 §2.3.3: T(C_i) = argtop_N of
    sum_{j<i} inter(C_j, t)): the attention mass token t of chunk i puts on the chunks before it."""
    L_ctx, lay = chunk_layout(chunks)
    inter = np.asarray(inter, dtype=np.float64)
    s = np.zeros(L_ctx)
    for c, (_src, T, n, _delta) in enumerate(lay):
        s[n:n + T] = inter[n:n + T, :c].sum(axis=1)
    return s


def cache_context_impact(inter, chunks) -> np.ndarray:
    """CCI per chunk (Cache-Craft CSDN article §2.2.1: CCI = sigmoid(sum inter / sum intra); KVCache
    reuse 01 §2.3.1 with inter and intra normalised alike, which leaves the ratio unchanged).
    sum inter: the chunk's tokens' attention on earlier chunks; sum intra: on their own chunk."""
    _L, lay = chunk_layout(chunks)
    inter = np.asarray(inter, dtype=np.float64)
    out = []
    for c, (_src, T, n, _delta) in enumerate(lay):
        a = inter[n:n + T, :c].sum()
        b = inter[n:n + T, c].sum()
        out.append(1.0 / (1.0 + math.exp(-a / b)))
    return np.asarray(out)


def prefix_overlap(inter_to_old, old_prefix: Sequence[int], new_prefix: Sequence[int]) -> float:
    """Adjusted prefix overlap beta' of one chunk (Cache-Craft CSDN article §2.2.1; KVCache reuse 01
    §2.3.2): beta' = (sum of the chunk's inter-attention on old-prefix chunks also in the new prefix)
    x (1 - gamma) / (sum on all old-prefix chunks), gamma = Kendall tau distance between the shared
    chunks' order in the old and the new prefix (discordant pairs / all pairs; 0 below two shared).
    inter_to_old[c]: the chunk's inter-attention on old-prefix chunk id c. Reading: an empty old
    prefix (no attention outside the chunk was recorded) gives beta' = 0."""
    old = [int(c) for c in old_prefix]
    new = [int(c) for c in new_prefix]
    den = sum(float(inter_to_old[c]) for c in old)
    if den <= 0.0:
        return 0.0
    shared = [c for c in old if c in new]
    num = sum(float(inter_to_old[c]) for c in shared)
    n = len(shared)
    gamma = 0.0
    if n >= 2:
        pos_new = {c: i for i, c in enumerate(new)}
        disc = sum(1 for i in range(n) for j in range(i + 1, n) if pos_new[shared[i]] > pos_new[shared[j]])
        gamma = disc / (n * (n - 1) / 2)
    return num * (1.0 - gamma) / den


def cachecraft_count(alpha: float, cci: float, beta: float, n_tokens: int) -> int:
    """Tokens to recompute in one chunk: N = ceil(alpha * CCI * (1 - beta') * |C|) (Cache-Craft CSDN
    article §2.1; CFO = alpha * CCI * (1 - beta'), §2.2.1), evaluated in float64 in this order and
    clamped to [0, |C|]."""
    x = float(alpha) * float(cci) * (1.0 - float(beta)) * float(n_tokens)
    return int(min(max(math.ceil(x), 0), int(n_tokens)))


# ----------------------------------------------------------------------------- fused layer

def fused_layer(*, k_store, v_store, chunks, L: int, q_new, k_new, v_new, dtype: str, base: float,
                n_kv_heads: int, q_crit=None, k_crit_store=None, n_select: Optional[int] = None,
                quotas=None, row_pos=None, attn_rows=None, hkvd_prev=None, hkvd_n_prev=None):
    """One layer of the fusion step: S1, then (S2 when a critical-layer query is given), S3, S4.

    q_new, k_new, v_new are position-indexed fresh projections [L, H, d]; the recomputed
    rows are gathered from them at row_pos. Without q_crit, row_pos must be given -- or, for
    gradual filtering, the previous layer's rows hkvd_prev (hkvd_n_prev context rows first): then
    the n_select of them with the highest KV deviation at this layer are recomputed.
    Returns a dict with k_fused, v_fused, row_pos, scores (or None), dev (or None), out, lse.
    """
    L_ctx, _ = chunk_layout(chunks)
    Lq = L - L_ctx
    kf, vf = fuse_rerotate(k_store, v_store, chunks, L, dtype, base)
    scores = None
    dev = None
    if hkvd_prev is not None:
        prev = np.asarray(hkvd_prev, dtype=np.int64)
        npv = int(hkvd_n_prev)
        dev = kv_deviation(kf, vf, np.asarray(k_new)[prev[:npv]], np.asarray(v_new)[prev[:npv]],
                           prev, npv, dtype, base)
        row_pos = hkvd_filter(dev, prev, npv, int(n_select))
    elif q_crit is not None:
        scores = critical_scores(q_crit, k_crit_store, chunks, n_kv_heads, dtype, base)
        if quotas is not None:
            sel = select_topn_quota(scores, chunks, quotas)
        else:
            sel = select_topn(scores, int(n_select))
        row_pos = row_positions(sel, L_ctx, Lq)
    rp = np.asarray(row_pos, dtype=np.int64)
    kf, vf = scatter_kv(kf, vf, np.asarray(k_new)[rp], np.asarray(v_new)[rp], rp, dtype, base)
    out, lse = sparse_causal_attn(np.asarray(q_new)[rp], rp, kf, vf, dtype, base, rows=attn_rows)
    return {"k_fused": kf, "v_fused": vf, "row_pos": rp.astype(np.int32), "scores": scores,
            "dev": dev, "out": out, "lse": lse}


def gradual_filter_layers(*, layers, chunks, L: int, dtype: str, base: float, n_kv_heads: int,
                          counts: Sequence[int], q_crit=None, k_crit_store=None, row_pos0=None,
                          attn_rows=None):
    """Layer-by-layer recompute with gradual filtering (KVCache reuse 01, §1.3.3 and §1.3.4).

    layers[l] holds layer l's k_store, v_store, q_new, k_new, v_new. Layer 0 recomputes counts[0]
    tokens chosen by the critical-layer score (or the given row_pos0): the first-layer attention
    deviation of the page needs a full prefill of that layer, so the query-centric score stands in
    for it (a reading). Layer l > 0 keeps the counts[l] tokens of layer l-1's selection with the
    highest KV deviation at layer l (counts must not increase). Returns one fused_layer result
    per layer.
    """
    res = []
    prev, npv = None, None
    for l, lay in enumerate(layers):
        kw = dict(k_store=lay["k_store"], v_store=lay["v_store"], chunks=chunks, L=L,
                  q_new=lay["q_new"], k_new=lay["k_new"], v_new=lay["v_new"], dtype=dtype, base=base,
                  n_kv_heads=n_kv_heads, n_select=int(counts[l]), attn_rows=attn_rows)
        if l == 0:
            if row_pos0 is not None:
                r = fused_layer(row_pos=row_pos0, **kw)
            else:
                r = fused_layer(q_crit=q_crit, k_crit_store=k_crit_store, **kw)
        else:
            if counts[l] > npv:
                raise ValueError("gradual filtering keeps a subset: counts must not increase")
            r = fused_layer(hkvd_prev=prev, hkvd_n_prev=npv, **kw)
        res.append(r)
        prev = r["row_pos"]
        npv = len(prev) - (L - chunk_layout(chunks)[0])
    return res
