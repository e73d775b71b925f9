"""Python binding with the names of the C ABI (argument marshalling only).

Every function takes caller-allocated torch tensors on the GPU (inputs and outputs), converts
them to device pointers and sizes, and calls the matching ``sra_*`` entry point on the current
torch stream. All computation happens in the HIP kernels of libsra.so.
"""
import ctypes
from typing import Optional

import numpy as np
import torch

from ._lib import (DTYPE_BF16, DTYPE_F32, Chunk, LayerArgs, SRAError, Shape, check, lib)  # noqa: F401

__all__ = ["make_shape", "select_count", "workspace_size", "anchor_workspace_size", "fuse_rerotate", "extract_anchors",
           "score_select", "select_topn", "scatter_kv", "hkvd_select", "sparse_causal_attn", "fused_layer",
           "check_rows", "chunk_array", "SRAError"]


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


def sparse_causal_attn(shape, q_new, row_pos, k_fused, v_fused, out, lse, ws, stream=None):
    n_req, R = row_pos.shape
    check(lib().sra_sparse_causal_attn(ctypes.byref(shape), n_req, _ptr(q_new), _ptr(row_pos), R,
                                       _ptr(k_fused), _ptr(v_fused), k_fused.shape[-3], _ptr(out), _ptr(lse),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def fused_layer(shape, *, chunks, k_store, v_store, q_fresh, k_fresh, v_fresh, row_pos, k_fused, v_fused,
                out, ws, lse=None, q_crit=None, k_crit_store=None, n_select=None, quotas=None, scores=None,
                anchors_k=0, anchor_rows=None, anchor_norms=None, hkvd_prev=None, hkvd_prev_ctx=0,
                hkvd_dev=None, stage_events=None, stream=None):
    """stage_events: optional ctypes array of 8 hipEvent_t handles (see sra_layer_args).
    anchors_k > 0 also extracts key-norm anchors of every (request, chunk) into anchor_rows
    [n_req][n_chunks][anchors_k] (int32) and, when given, anchor_norms [crit_store_rows] (float32).
    hkvd_prev [n_req][hkvd_prev_ctx + Lq] (int32) selects by gradual filtering: the n_select previous
    context rows of highest KV deviation (written to hkvd_dev [n_req][hkvd_prev_ctx]) are recomputed."""
    ch = np.asarray(chunks, dtype=np.int32)
    n_req, n_chunks = ch.shape[0], ch.shape[1]
    carr = chunk_array(ch)
    _qa, qp = _quota_array(quotas)
    L = k_fused.shape[-3]
    Lq = q_crit.shape[1] if q_crit is not None else L - int(ch[0, :, 1].sum())
    a = LayerArgs()
    a.shape = shape
    a.n_req, a.n_chunks, a.chunks = n_req, n_chunks, ctypes.cast(carr, ctypes.POINTER(Chunk))
    a.query_len, a.total_len = Lq, L
    a.k_store, a.v_store, a.store_rows = _ptr(k_store), _ptr(v_store), k_store.shape[0]
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
    check(lib().sra_fused_layer(ctypes.byref(a), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def check_rows(row_pos, L: int, stream=None) -> int:
    """Synchronous; returns -1 when valid, else raises SRAError (status SRA_E_ROWS)."""
    n_req, R = row_pos.shape
    bad = ctypes.c_int32(-1)
    check(lib().sra_check_rows(_ptr(row_pos), n_req, R, int(L), ctypes.byref(bad), _stream(stream)))
    return int(bad.value)
