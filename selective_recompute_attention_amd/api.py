"""Python binding with the names of the C ABI (argument marshalling only).

Every function takes caller-allocated torch tensors on the GPU (inputs and outputs), converts
them to device pointers and sizes, and calls the matching ``sra_*`` entry point on the current
torch stream. All computation happens in the HIP kernels of libsra.so.
"""
import ctypes
from typing import Optional

import numpy as np
import torch

from ._lib import (DTYPE_BF16, DTYPE_F32, Chunk, LayerArgs, SRAError, Shape, check, hip_runtime, lib)  # noqa: F401

__all__ = ["make_shape", "select_count", "workspace_size", "anchor_workspace_size", "fuse_rerotate", "extract_anchors", "anchor_prefix",
           "stats_workspace_size", "chunk_attention_stats", "prefix_overlap", "cachecraft_count",
           "score_select", "select_topn", "select_topn_nested", "scatter_kv", "hkvd_select", "sparse_causal_attn", "fused_layer",
           "fused_layer_static",
           "pipelined_layers", "create_events", "destroy_events", "check_rows", "chunk_array", "SRAError"]


def make_shape(n_q_heads: int, n_kv_heads: int, head_dim: int, dtype, rope_base: float = 10000.0) -> Shape:
    if dtype in (torch.bfloat16, "bf16"):
        dt = DTYPE_BF16
    elif dtype in (torch.float32, "f32"):
        dt = DTYPE_F32
    else:
        dt = int(dtype)
    return Shape(int(n_q_heads), int(n_kv_heads), int(head_dim), dt, float(rope_base))


def chunk_array(chunks) -> ctypes.Array:
    """int array [..., 4] (src_row, n_tokens, dst_row, orig_pos) -> contiguous C array of sra_chunk."""
    a = np.ascontiguousarray(np.asarray(chunks, dtype=np.int32).reshape(-1, 4))
    arr = (Chunk * len(a))()
    ctypes.memmove(arr, a.ctypes.data, a.nbytes)
    return arr


def _quota_array(quotas):
    if quotas is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(quotas, dtype=np.int32).reshape(-1))
    arr = (ctypes.c_int32 * len(a))(*a.tolist())
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsra must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def select_count(num: int, den: int, ctx_len: int) -> int:
    out = ctypes.c_int32(0)
    check(lib().sra_select_count(int(num), int(den), int(ctx_len), ctypes.byref(out)))
    return int(out.value)


def workspace_size(shape: Shape, n_req: int, n_chunks: int, L: int, R: int, Lq: int) -> int:
    n = lib().sra_workspace_size(ctypes.byref(shape), n_req, n_chunks, L, R, Lq)
    if n == 0:
        raise SRAError(2, "invalid sizes for sra_workspace_size")
    return int(n)


def fuse_rerotate(shape, k_store, v_store, chunks, k_fused, v_fused, stream=None):
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = (ch.shape[0], ch.shape[1]) if ch.ndim == 3 else (1, ch.shape[0])
    check(lib().sra_fuse_rerotate(ctypes.byref(shape), n_req, _ptr(k_store), _ptr(v_store), k_store.shape[0],
                                  chunk_array(ch), n_chunks, _ptr(k_fused), _ptr(v_fused),
                                  k_fused.shape[-3], _stream(stream)))


def anchor_workspace_size(chunks) -> int:
    """Bytes of workspace sra_extract_anchors needs: 8 per chunk token."""
    return 8 * int(np.asarray(chunks, dtype=np.int64).reshape(-1, 4)[:, 1].sum())


def extract_anchors(shape, k_store, chunks, k, anchor_rows, ws, norms=None, stream=None):
    ch = np.asarray(chunks, dtype=np.int32).reshape(-1, 4)
    check(lib().sra_extract_anchors(ctypes.byref(shape), _ptr(k_store), k_store.shape[0], chunk_array(ch),
                                    len(ch), int(k), _ptr(anchor_rows), _ptr(norms), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def anchor_prefix(shape, k_store, v_store, chunks, anchor_rows, k_probe, v_probe, stream=None):
    """Anchor probe prefix rows [0, n_chunks * k) of k_probe/v_probe [n_req][L_probe][Hkv][d]
    (sra_anchor_prefix); anchor_rows: [n_req][n_chunks][k] int32 on the device."""
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = ch.shape[0], ch.shape[1]
    carr = chunk_array(ch)
    check(lib().sra_anchor_prefix(ctypes.byref(shape), n_req, _ptr(k_store), _ptr(v_store), k_store.shape[0],
                                  ctypes.cast(carr, ctypes.POINTER(Chunk)), n_chunks, _ptr(anchor_rows),
                                  anchor_rows.shape[-1], _ptr(k_probe), _ptr(v_probe), k_probe.shape[-3],
                                  _stream(stream)))


def stats_workspace_size(shape: Shape, n_req: int, ctx_len: int, n_chunks: int) -> int:
    return int(lib().sra_stats_workspace_size(ctypes.byref(shape), n_req, ctx_len, n_chunks))


def chunk_attention_stats(shape, q_fresh, k_cache, chunks, ws, inter=None, token_scores=None, cci=None,
                          stream=None):
    """Per-token, per-chunk attention statistics of a full causal prefill (sra_chunk_attention_stats):
    inter [n_req][L_ctx][n_chunks], token_scores [n_req][L_ctx], cci [n_req][n_chunks] (float32, each
    optional). q_fresh [n_req][q_rows][Hq][d] before rotation; k_cache [n_req][k_rows][Hkv][d] rotated."""
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = ch.shape[0], ch.shape[1]
    carr = chunk_array(ch)
    check(lib().sra_chunk_attention_stats(ctypes.byref(shape), n_req, _ptr(q_fresh), q_fresh.shape[1],
                                          _ptr(k_cache), k_cache.shape[1], ctypes.cast(carr, ctypes.POINTER(Chunk)),
                                          n_chunks, _ptr(inter), _ptr(token_scores), _ptr(cci), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)))


def prefix_overlap(inter_to_old, old_ids, new_ids) -> float:
    """beta' of one chunk (sra_prefix_overlap); inter_to_old[i] belongs to old_ids[i]."""
    n_old, n_new = len(old_ids), len(new_ids)
    a = (ctypes.c_double * max(n_old, 1))(*[float(x) for x in inter_to_old])
    o = (ctypes.c_int32 * max(n_old, 1))(*[int(x) for x in old_ids])
    n = (ctypes.c_int32 * max(n_new, 1))(*[int(x) for x in new_ids])
    out = ctypes.c_double()
    check(lib().sra_prefix_overlap(a, o, n_old, n, n_new, ctypes.byref(out)))
    return float(out.value)


def cachecraft_count(alpha: float, cci: float, beta: float, n_tokens: int) -> int:
    """N = ceil(alpha * cci * (1 - beta) * n_tokens), clamped (sra_cachecraft_count)."""
    out = ctypes.c_int32()
    check(lib().sra_cachecraft_count(float(alpha), float(cci), float(beta), int(n_tokens), ctypes.byref(out)))
    return int(out.value)


def score_select(shape, q_crit, k_crit_store, chunks, n_select, quotas, scores, row_pos, ws, stream=None):
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = ch.shape[0], ch.shape[1]
    _qa, qp = _quota_array(quotas)
    check(lib().sra_score_select(ctypes.byref(shape), n_req, _ptr(q_crit), q_crit.shape[1], _ptr(k_crit_store),
                                 k_crit_store.shape[0], chunk_array(ch), n_chunks,
                                 -1 if n_select is None else int(n_select), qp, _ptr(scores), _ptr(row_pos),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def select_topn(scores, n_select, quotas, chunks, Lq, row_pos, stream=None):
    n_req, ctx_len = scores.shape
    _qa, qp = _quota_array(quotas)
    if chunks is not None:
        ch = np.asarray(chunks, dtype=np.int32)
        carr, n_chunks = chunk_array(ch), ch.shape[1]
    else:
        carr, n_chunks = None, 0
    check(lib().sra_select_topn(_ptr(scores), n_req, ctx_len, -1 if n_select is None else int(n_select), qp,
                                carr, n_chunks, int(Lq), _ptr(row_pos), _stream(stream)))


def select_topn_nested(scores, prev_rows, n_prev, Lq, n_select, row_pos, stream=None):
    """Nested Top-N among the first n_prev rows of prev_rows [n_req][>= n_prev + Lq]: level l writes
    row_pos[l] [n_req][n_select[l] + Lq]; see sra_select_topn_nested."""
    n_req, ctx_len = scores.shape
    n_levels = len(n_select)
    if len(row_pos) != n_levels:
        raise ValueError("one row_pos tensor per level")
    counts = (ctypes.c_int32 * n_levels)(*[int(n) for n in n_select])
    outs = (ctypes.c_void_p * n_levels)(*[_ptr(r) for r in row_pos])
    check(lib().sra_select_topn_nested(_ptr(scores), n_req, ctx_len, _ptr(prev_rows), prev_rows.stride(0),
                                       int(n_prev), int(Lq), n_levels, counts, outs, _stream(stream)))


def scatter_kv(shape, k_new, v_new, row_pos, k_fused, v_fused, stream=None):
    n_req, R = row_pos.shape
    check(lib().sra_scatter_kv(ctypes.byref(shape), n_req, _ptr(k_new), _ptr(v_new), _ptr(row_pos), R,
                               _ptr(k_fused), _ptr(v_fused), k_fused.shape[-3], _stream(stream)))


def hkvd_select(shape, k_fused, v_fused, k_new, v_new, row_pos_prev, n_prev, n_keep, dev, row_pos_next,
                stream=None):
    """KV deviation of the previous rows' first n_prev context rows (dev [n_req][n_prev] float32) and the
    next layer's rows (row_pos_next [n_req][n_keep + R_prev - n_prev]): see sra_hkvd_select."""
    n_req, R_prev = row_pos_prev.shape
    check(lib().sra_hkvd_select(ctypes.byref(shape), n_req, _ptr(k_fused), _ptr(v_fused), k_fused.shape[-3],
                                _ptr(k_new), _ptr(v_new), _ptr(row_pos_prev), R_prev, int(n_prev), int(n_keep),
                                _ptr(dev), _ptr(row_pos_next), _stream(stream)))


def sparse_causal_attn(shape, q_new, row_pos, k_fused, v_fused, out, lse, ws, stream=None, fallback=None):
    """fallback: optional int32 [n_req][Hkv], 1 where a group was recomputed exactly (fp16 range)."""
    n_req, R = row_pos.shape
    check(lib().sra_sparse_causal_attn(ctypes.byref(shape), n_req, _ptr(q_new), _ptr(row_pos), R,
                                       _ptr(k_fused), _ptr(v_fused), k_fused.shape[-3], _ptr(out), _ptr(lse),
                                       _ptr(fallback), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def _layer_args(shape, *, chunks, k_store, v_store, q_fresh, k_fresh, v_fresh, row_pos, k_fused, v_fused,
                out, lse=None, q_crit=None, k_crit_store=None, n_select=None, quotas=None, scores=None,
                anchors_k=0, anchor_rows=None, anchor_norms=None, hkvd_prev=None, hkvd_prev_ctx=0,
                hkvd_dev=None, stage_events=None, store_rows=None, attn_fallback=None):
    """A filled sra_layer_args and the host arrays it points to (keep both alive during the call)."""
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = ch.shape[0], ch.shape[1]
    carr = chunk_array(ch)
    qa, qp = _quota_array(quotas)
    L = k_fused.shape[-3]
    Lq = q_crit.shape[1] if q_crit is not None else L - int(ch[0, :, 1].sum())
    a = LayerArgs()
    a.shape = shape
    a.n_req, a.n_chunks, a.chunks = n_req, n_chunks, ctypes.cast(carr, ctypes.POINTER(Chunk))
    a.query_len, a.total_len = Lq, L
    a.k_store, a.v_store = _ptr(k_store), _ptr(v_store)
    a.store_rows = k_store.shape[0] if store_rows is None else int(store_rows)
    a.q_crit = _ptr(q_crit)
    a.k_crit_store = _ptr(k_crit_store)
    a.crit_store_rows = k_crit_store.shape[0] if k_crit_store is not None else 0
    a.n_select = -1 if n_select is None else int(n_select)
    a.chunk_quota = qp
    a.scores = _ptr(scores)
    a.anchors_k, a.anchor_rows, a.anchor_norms = int(anchors_k), _ptr(anchor_rows), _ptr(anchor_norms)
    a.hkvd_prev, a.hkvd_dev = _ptr(hkvd_prev), _ptr(hkvd_dev)
    a.hkvd_prev_rows = hkvd_prev.shape[1] if hkvd_prev is not None else 0
    a.hkvd_prev_ctx = int(hkvd_prev_ctx)
    a.q_fresh, a.k_fresh, a.v_fresh = _ptr(q_fresh), _ptr(k_fresh), _ptr(v_fresh)
    a.row_pos, a.n_rows = _ptr(row_pos), row_pos.shape[1]
    a.k_fused, a.v_fused, a.out, a.lse = _ptr(k_fused), _ptr(v_fused), _ptr(out), _ptr(lse)
    if stage_events is not None:
        a.stage_events = ctypes.cast(stage_events, ctypes.POINTER(ctypes.c_void_p))
    a.attn_fallback = _ptr(attn_fallback)
    return a, (carr, qa)


def fused_layer(shape, *, ws, stream=None, **kw):
    """One layer (sra_fused_layer). Keyword arguments as the fields of sra_layer_args:
    chunks, k_store, v_store, q_fresh, k_fresh, v_fresh, row_pos, k_fused, v_fused, out; optional lse,
    q_crit, k_crit_store, n_select, quotas, scores; anchors_k > 0 with anchor_rows
    [n_req][n_chunks][anchors_k] (int32) and optional anchor_norms [crit_store_rows] (float32);
    hkvd_prev [n_req][hkvd_prev_ctx + Lq] (int32) to select by gradual filtering (the n_select
    previous context rows of highest KV deviation, written to hkvd_dev [n_req][hkvd_prev_ctx]);
    stage_events: optional ctypes array of 8 hipEvent_t handles; attn_fallback: optional int32
    [n_req][Hkv] report of groups recomputed exactly (fp16 range)."""
    a, keep = _layer_args(shape, **kw)
    check(lib().sra_fused_layer(ctypes.byref(a), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    del keep


def fused_layer_static(shape, *, stream=None, **kw):
    """One layer (sra_fused_layer_static): as fused_layer, with the library's static scratch instead of
    a workspace (no device allocation; calls on one GPU must not overlap)."""
    a, keep = _layer_args(shape, **kw)
    check(lib().sra_fused_layer_static(ctypes.byref(a), _stream(stream)))
    del keep


def create_events(n: int = 4):
    """n hipEvent_t handles (timing disabled) for pipelined_layers; release with destroy_events."""
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        e = ctypes.c_void_p()
        if hip_runtime().hipEventCreateWithFlags(ctypes.byref(e), 2) != 0:   # hipEventDisableTiming
            raise RuntimeError("hipEventCreateWithFlags failed")
        arr[i] = e.value
    return arr


def destroy_events(arr):
    for e in arr:
        if e:
            hip_runtime().hipEventDestroy(ctypes.c_void_p(e))


def pipelined_layers(shape, layers, host_k, host_v, k_buf, v_buf, events, ws, stream=None, copy_stream=None):
    """Layers in order with each layer's chunk store prefetched from pinned host memory on
    copy_stream while the previous layer runs (sra_pipelined_layers). layers: one dict of
    fused_layer keyword arguments per layer, without k_store/v_store (store_rows given instead);
    host_k/host_v: pinned host tensors per layer; k_buf/v_buf: n_buf >= 2 device buffers each (bytes
    of the largest store; n_buf >= len(layers) keeps the copy stream from ever waiting); events:
    create_events(2 * n_buf)."""
    n = len(layers)
    args = (LayerArgs * n)()
    keep = []
    for l, kw in enumerate(layers):
        a, k = _layer_args(shape, k_store=None, v_store=None, **kw)
        args[l] = a
        keep.append(k)
    hk = (ctypes.c_void_p * n)(*[t.data_ptr() for t in host_k])
    hv = (ctypes.c_void_p * n)(*[t.data_ptr() for t in host_v])
    nb = len(k_buf)
    kb = (ctypes.c_void_p * nb)(*[t.data_ptr() for t in k_buf])
    vb = (ctypes.c_void_p * nb)(*[t.data_ptr() for t in v_buf])
    nbytes = min(t.numel() * t.element_size() for t in list(k_buf) + list(v_buf))
    cs = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
    check(lib().sra_pipelined_layers(args, n, hk, hv, nbytes, kb, vb, nb, events, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream), cs))
    del keep


def check_rows(row_pos, L: int, stream=None) -> int:
    """Synchronous; returns -1 when valid, else raises SRAError (status SRA_E_ROWS)."""
    n_req, R = row_pos.shape
    bad = ctypes.c_int32(-1)
    check(lib().sra_check_rows(_ptr(row_pos), n_req, R, int(L), ctypes.byref(bad), _stream(stream)))
    return int(bad.value)
