"""The C ABI without a GPU: the library loads, exports every declared symbol, and reports every
host-detectable error with its status code before touching the device.

Device pointers here are fake (aligned, non-NULL integers); every call below fails validation
on the host, so no HIP call is made with them.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from selective_recompute_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sra.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libsra.so not built")

FAKE = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(16)]   # distinct, 16-byte aligned


def shape(hq=32, hkv=8, d=128, dtype=L.DTYPE_BF16, base=10000.0):
    return L.Shape(hq, hkv, d, dtype, base)


def chunks(rows):
    a = np.asarray(rows, dtype=np.int32).reshape(-1, 4)
    arr = (L.Chunk * len(a))()
    ctypes.memmove(arr, a.ctypes.data, a.nbytes)
    return arr


def last_error():
    return L.lib().sra_last_error().decode()


def test_every_declared_symbol_is_exported():
    names = re.findall(r"^\s*(?:int|size_t|const char\*)\s+(sra_\w+)\s*\(", open(HEADER).read(), re.M)
    assert len(names) >= 12
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L._SIGS), "binding declarations must mirror the header"


def test_error_strings():
    lib = L.lib()
    for code in range(10):
        assert lib.sra_error_string(code)
    assert lib.sra_error_string(0) == b"success"


@pytest.mark.parametrize("num,den,ctx", [(15, 100, 384), (9, 70, 17920), (10, 100, 7680), (0, 5, 9),
                                         (100, 100, 2560), (1, 3, 10), (7, 70, 17920), (35, 100, 1)])
def test_select_count_matches_oracle(num, den, ctx):
    out = ctypes.c_int32(-7)
    assert L.lib().sra_select_count(num, den, ctx, ctypes.byref(out)) == L.SRA_OK
    assert out.value == O.select_count(num, den, ctx)


def test_select_count_errors():
    out = ctypes.c_int32()
    lib = L.lib()
    assert lib.sra_select_count(1, 0, 10, ctypes.byref(out)) == L.SRA_E_SHAPE
    assert lib.sra_select_count(-1, 10, 10, ctypes.byref(out)) == L.SRA_E_SHAPE
    assert lib.sra_select_count(11, 10, 10, ctypes.byref(out)) == L.SRA_E_SHAPE
    assert lib.sra_select_count(1, 10, 10, None) == L.SRA_E_NULL


def test_workspace_size_is_monotone_and_rejects_bad_sizes():
    lib = L.lib()
    s = shape()
    a = lib.sra_workspace_size(ctypes.byref(s), 1, 5, 2592, 416, 32)
    b = lib.sra_workspace_size(ctypes.byref(s), 4, 5, 2592, 416, 32)
    assert a > 0 and b > a and a % 256 == 0
    assert lib.sra_workspace_size(ctypes.byref(shape(hq=30, hkv=8)), 1, 5, 2592, 416, 32) == 0
    assert lib.sra_workspace_size(ctypes.byref(shape(d=96)), 1, 5, 2592, 416, 32) == 0
    assert lib.sra_workspace_size(None, 1, 5, 2592, 416, 32) == 0
    assert lib.sra_workspace_size(ctypes.byref(s), 1, 5, 10, 4, 11) == 0


def test_fuse_rerotate_host_errors():
    lib = L.lib()
    ok = chunks([[0, 4, 0, 0], [4, 4, 4, 0]])
    st = None
    call = lambda sh, ch, n, ks=FAKE[0], vs=FAKE[1], kf=FAKE[2], vf=FAKE[3], rows=8, Ln=10: \
        lib.sra_fuse_rerotate(ctypes.byref(sh), 1, ks, vs, rows, ch, n, kf, vf, Ln, st)
    assert call(shape(hq=30), ok, 2) == L.SRA_E_SHAPE
    assert call(shape(d=80), ok, 2) == L.SRA_E_SHAPE
    assert call(shape(dtype=5), ok, 2) == L.SRA_E_DTYPE
    assert call(shape(), ok, 2, ks=None) == L.SRA_E_NULL
    assert call(shape(), ok, 2, kf=ctypes.c_void_p(0x10000008)) == L.SRA_E_SHAPE     # misaligned
    assert call(shape(), chunks([[0, 4, 0, 0], [4, 4, 5, 0]]), 2) == L.SRA_E_CHUNKS   # gap
    assert "dst_row" in last_error()
    assert call(shape(), chunks([[0, 4, 0, 0], [6, 4, 4, 0]]), 2) == L.SRA_E_CHUNKS   # past store end
    assert call(shape(), ok, 2, Ln=7) == L.SRA_E_SHAPE                               # L < L_ctx
    # the store overlaps the fused output
    assert call(shape(), ok, 2, kf=FAKE[0]) == L.SRA_E_ALIAS
    assert lib.sra_fuse_rerotate(ctypes.byref(shape()), 1, FAKE[0], FAKE[1], 8, None, 2, FAKE[2], FAKE[3],
                                 10, None) == L.SRA_E_NULL


def test_score_select_host_errors():
    lib = L.lib()
    ch = chunks([[0, 64, 0, 0], [64, 64, 64, 0]])
    s = shape()
    need = lib.sra_workspace_size(ctypes.byref(s), 1, 2, 136, 20, 8)
    call = lambda n_select=12, quota=None, ws=FAKE[4], wsb=need, Lq=8, sh=s: lib.sra_score_select(
        ctypes.byref(sh), 1, FAKE[0], Lq, FAKE[1], 128, ch, 2, n_select, quota, FAKE[2], FAKE[3], ws, wsb, None)
    assert call(n_select=129) == L.SRA_E_SHAPE              # N > L_ctx
    assert call(n_select=-1) == L.SRA_E_SHAPE
    assert call(Lq=0) == L.SRA_E_SHAPE
    assert call(ws=None) == L.SRA_E_WORKSPACE
    assert call(wsb=256) == L.SRA_E_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10000010)) == L.SRA_E_WORKSPACE   # not 256-byte aligned
    bad_q = (ctypes.c_int32 * 2)(65, 1)
    assert call(quota=ctypes.cast(bad_q, ctypes.POINTER(ctypes.c_int32))) == L.SRA_E_SHAPE
    assert call(Lq=300, sh=shape(hq=64, hkv=8)) == L.SRA_E_LIMIT       # Lq * g > 2048


def test_quota_totals_must_match_across_requests():
    lib = L.lib()
    ch = chunks([[0, 8, 0, 0], [8, 8, 8, 0], [16, 8, 0, 0], [24, 8, 8, 0]])
    q = (ctypes.c_int32 * 4)(2, 3, 3, 3)
    rc = lib.sra_select_topn(FAKE[0], 2, 16, -1, ctypes.cast(q, ctypes.POINTER(ctypes.c_int32)), ch, 2, 4,
                             FAKE[1], None)
    assert rc == L.SRA_E_SHAPE and "selects" in last_error()


def test_attention_and_scatter_host_errors():
    lib = L.lib()
    s = shape()
    assert lib.sra_sparse_causal_attn(ctypes.byref(s), 1, FAKE[0], FAKE[1], 10, FAKE[2], FAKE[3], 20, FAKE[4],
                                      None, None, None, 0, None) == L.SRA_E_WORKSPACE
    assert lib.sra_sparse_causal_attn(ctypes.byref(s), 1, FAKE[0], FAKE[1], 30, FAKE[2], FAKE[3], 20, FAKE[4],
                                      None, None, FAKE[5], 1 << 30, None) == L.SRA_E_SHAPE       # R > L
    assert lib.sra_sparse_causal_attn(ctypes.byref(s), 1, FAKE[0], FAKE[1], 10, FAKE[2], FAKE[3], 20, FAKE[2],
                                      None, None, FAKE[5], 1 << 30, None) == L.SRA_E_ALIAS       # out is k_fused
    assert lib.sra_sparse_causal_attn(ctypes.byref(s), 1, FAKE[0], FAKE[1], 10, FAKE[2], FAKE[3], 20, FAKE[4],
                                      None, FAKE[4], FAKE[5], 1 << 30, None) == L.SRA_E_ALIAS    # fallback is out
    assert lib.sra_scatter_kv(ctypes.byref(s), 1, FAKE[0], FAKE[1], None, 4, FAKE[2], FAKE[3], 20,
                              None) == L.SRA_E_NULL
    assert lib.sra_scatter_kv(ctypes.byref(s), 1, FAKE[0], FAKE[1], FAKE[6], 4, FAKE[0], FAKE[3], 20,
                              None) == L.SRA_E_ALIAS
    assert lib.sra_check_rows(None, 1, 4, 10, None, None) == L.SRA_E_NULL


def test_anchor_host_errors():
    lib = L.lib()
    s = shape()
    ch = chunks([[0, 8, 0, 0]])
    ws = FAKE[2]
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 8, ch, 1, 9, FAKE[1], None, ws, 64, None) == L.SRA_E_SHAPE
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 8, ch, 1, 0, FAKE[1], None, ws, 64, None) == L.SRA_E_SHAPE
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 8, ch, 1, 65, FAKE[1], None, ws, 64, None) == L.SRA_E_LIMIT
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 7, ch, 1, 2, FAKE[1], None, ws, 64, None) == L.SRA_E_CHUNKS
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 8, ch, 1, 2, FAKE[1], None, ws, 56, None) == L.SRA_E_WORKSPACE
    assert lib.sra_extract_anchors(ctypes.byref(s), FAKE[0], 8, ch, 1, 2, FAKE[1], None, None, 64, None) == L.SRA_E_WORKSPACE


def test_fused_layer_host_errors():
    lib = L.lib()
    ch = chunks([[0, 64, 0, 0], [64, 64, 64, 0]])
    a = L.LayerArgs()
    a.shape = shape()
    a.n_req, a.n_chunks, a.chunks = 1, 2, ctypes.cast(ch, ctypes.POINTER(L.Chunk))
    a.query_len, a.total_len = 8, 136
    a.k_store, a.v_store, a.store_rows = FAKE[0], FAKE[1], 128
    a.q_fresh, a.k_fresh, a.v_fresh = FAKE[2], FAKE[3], FAKE[4]
    a.row_pos, a.n_rows = FAKE[5], 20
    a.k_fused, a.v_fused, a.out = FAKE[6], FAKE[7], FAKE[8]
    a.q_crit, a.k_crit_store, a.crit_store_rows, a.n_select = FAKE[9], FAKE[10], 128, 13   # 13 + 8 != 20
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[11], 1 << 30, None) == L.SRA_E_SHAPE
    a.total_len = 137
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[11], 1 << 30, None) == L.SRA_E_SHAPE
    a.total_len, a.n_select = 136, 12
    a.out = FAKE[6]
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[11], 1 << 30, None) == L.SRA_E_ALIAS
    a.out = FAKE[8]
    assert lib.sra_fused_layer(ctypes.byref(a), None, 0, None) == L.SRA_E_WORKSPACE
    assert lib.sra_fused_layer(None, None, 0, None) == L.SRA_E_NULL


def test_hkvd_host_errors():
    lib = L.lib()
    s = shape()
    ok_args = [FAKE[0], FAKE[1], 100, FAKE[2], FAKE[3], FAKE[4], 40, 30, 20, FAKE[5], FAKE[6], None]
    def call(**kw):
        a = list(ok_args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.sra_hkvd_select(ctypes.byref(s), 1, *a)
    assert call(a9=None) == L.SRA_E_NULL                     # dev
    assert call(a10=None) == L.SRA_E_NULL                    # row_pos_next
    assert call(a8=31) == L.SRA_E_SHAPE                      # n_keep > n_prev
    assert call(a7=41) == L.SRA_E_SHAPE                      # n_prev > R_prev
    assert call(a6=101) == L.SRA_E_SHAPE                     # R_prev > L
    assert call(a10=FAKE[4]) == L.SRA_E_ALIAS                # next rows written over the previous rows
    assert call(a0=None) == L.SRA_E_NULL
    # the fused layer's filtering mode
    ch = chunks([[0, 64, 0, 0], [64, 64, 64, 0]])
    a = L.LayerArgs()
    a.shape = shape()
    a.n_req, a.n_chunks, a.chunks = 1, 2, ctypes.cast(ch, ctypes.POINTER(L.Chunk))
    a.query_len, a.total_len = 8, 136
    a.k_store, a.v_store, a.store_rows = FAKE[0], FAKE[1], 128
    a.q_fresh, a.k_fresh, a.v_fresh = FAKE[2], FAKE[3], FAKE[4]
    a.row_pos, a.n_rows = FAKE[5], 20
    a.k_fused, a.v_fused, a.out = FAKE[6], FAKE[7], FAKE[8]
    a.hkvd_prev, a.hkvd_prev_rows, a.hkvd_prev_ctx, a.hkvd_dev, a.n_select = FAKE[9], 38, 30, FAKE[10], 12
    a.q_crit, a.k_crit_store, a.crit_store_rows = FAKE[11], FAKE[12], 128
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[13], 1 << 30, None) == L.SRA_E_SHAPE   # with q_crit
    a.q_crit = None
    a.hkvd_dev = None
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[13], 1 << 30, None) == L.SRA_E_NULL
    a.hkvd_dev = FAKE[10]
    a.hkvd_prev_rows = 37                                                                  # != ctx + Lq
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[13], 1 << 30, None) == L.SRA_E_SHAPE
    a.hkvd_prev_rows, a.n_select = 38, 31                                                  # keeps more than given
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[13], 1 << 30, None) == L.SRA_E_SHAPE
    a.n_select, a.hkvd_prev = 12, FAKE[5]                                                  # prev == row_pos
    assert lib.sra_fused_layer(ctypes.byref(a), FAKE[13], 1 << 30, None) == L.SRA_E_ALIAS


def test_pipelined_layers_host_errors():
    lib = L.lib()
    ch = chunks([[0, 64, 0, 0], [64, 64, 64, 0]])
    a = (L.LayerArgs * 2)()
    for i in range(2):
        a[i].shape = shape()
        a[i].n_req, a[i].n_chunks, a[i].chunks = 1, 2, ctypes.cast(ch, ctypes.POINTER(L.Chunk))
        a[i].query_len, a[i].total_len = 8, 136
        a[i].store_rows = 128
        a[i].q_fresh, a[i].k_fresh, a[i].v_fresh = FAKE[2], FAKE[3], FAKE[4]
        a[i].row_pos, a[i].n_rows = FAKE[5], 20
        a[i].k_fused, a[i].v_fused, a[i].out = FAKE[6], FAKE[7], FAKE[8]
    P = ctypes.c_void_p
    hk = (P * 2)(0x1000, 0x2000)
    hv = (P * 2)(0x3000, 0x4000)
    nb = 128 * 8 * 128 * 2
    kb = (P * 2)(0xA0000000, 0xA4000000)
    vb = (P * 2)(0xA8000000, 0xAC000000)
    ev = (P * 4)(1, 2, 3, 4)
    args = [a, 2, hk, hv, nb, kb, vb, 2, ev, FAKE[11], 1 << 30, None, None]
    def call(i=None, v=None):
        x = list(args)
        if i is not None:
            x[i] = v
        return lib.sra_pipelined_layers(*x)
    assert call(8, None) == L.SRA_E_NULL                                   # events
    assert call(7, 1) == L.SRA_E_SHAPE                                     # one buffer pair
    assert call(1, 0) == L.SRA_E_SHAPE                                     # no layers
    assert call(4, nb - 2) == L.SRA_E_SHAPE                                # stores larger than the buffers
    assert call(5, (P * 2)(0xA0000000, 0xA0000100)) == L.SRA_E_ALIAS       # buffers overlap
    assert call(2, (P * 2)(0x1000, None)) == L.SRA_E_NULL                  # a host store
    a[1].row_pos, a[1].n_rows = FAKE[5], 137                               # layer 1 invalid: nothing enqueued
    assert call() == L.SRA_E_SHAPE


def test_anchor_prefix_host_errors():
    lib = L.lib()
    s = shape()
    ch = chunks([[0, 8, 0, 0], [8, 8, 8, 0]])
    base = [ctypes.byref(s), 1, FAKE[0], FAKE[1], 16, ch, 2, FAKE[2], 4, FAKE[3], FAKE[4], 12, None]
    def call(i=None, v=None):
        x = list(base)
        if i is not None:
            x[i] = v
        return lib.sra_anchor_prefix(*x)
    assert call(11, 7) == L.SRA_E_SHAPE          # prefix of 8 rows does not fit 7
    assert call(8, 9) == L.SRA_E_SHAPE           # k > n_tokens
    assert call(8, 65) == L.SRA_E_LIMIT
    assert call(4, 15) == L.SRA_E_CHUNKS         # second chunk reads outside the store
    assert call(7, None) == L.SRA_E_NULL
    assert call(9, FAKE[0]) == L.SRA_E_ALIAS     # probe cache over the store


def test_cachecraft_host_helpers_match_oracle():
    import selective_recompute_attention_amd as sra
    rng = np.random.default_rng(9)
    for _ in range(500):
        a, c, b = float(rng.uniform(0, 1)), float(rng.uniform(0, 1)), float(rng.choice([0.0, 0.25, rng.uniform(0, 1)]))
        n = int(rng.integers(0, 600))
        assert sra.cachecraft_count(a, c, b, n) == O.cachecraft_count(a, c, b, n)
    for _ in range(300):
        ids = list(rng.permutation(12)[:int(rng.integers(0, 8))])
        new = list(rng.permutation(12)[:int(rng.integers(0, 10))])
        att = {int(i): float(rng.uniform(0, 2)) for i in range(12)}
        got = sra.prefix_overlap([att[i] for i in ids], ids, new)
        assert got == O.prefix_overlap(att, ids, new)


def test_stats_host_errors():
    lib = L.lib()
    ch = chunks([[0, 8, 0, 0], [8, 8, 8, 0]])
    s = shape()
    ws_need = lib.sra_stats_workspace_size(ctypes.byref(s), 1, 16, 2)
    assert ws_need > 0
    ok = [ctypes.byref(s), 1, FAKE[0], 20, FAKE[1], 20, ch, 2, FAKE[2], FAKE[3], FAKE[4], FAKE[5], ws_need, None]
    def call(i=None, v=None):
        x = list(ok)
        if i is not None:
            x[i] = v
        return lib.sra_chunk_attention_stats(*x)
    assert call(12, ws_need - 8) == L.SRA_E_WORKSPACE
    assert call(3, 15) == L.SRA_E_SHAPE            # queries do not cover the context
    assert call(4, None) == L.SRA_E_NULL
    sf = shape(dtype=L.DTYPE_F32)
    assert call(0, ctypes.byref(sf)) == L.SRA_E_DTYPE
    assert call(8, FAKE[5]) == L.SRA_E_ALIAS        # inter written over the workspace
    out = ctypes.c_int32()
    assert lib.sra_cachecraft_count(0.5, 0.5, 0.0, -1, ctypes.byref(out)) == L.SRA_E_SHAPE
    assert lib.sra_prefix_overlap(None, None, 2, None, 0, ctypes.byref(ctypes.c_double())) == L.SRA_E_NULL
