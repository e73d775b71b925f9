"""ctypes declarations of libsra.so (the C ABI in include/sra.h).

Loading fails loudly with an ImportError-like exception when the library has not been built:
there is no fallback implementation.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# SRA_LIB_PATH selects another build of the same library (the host-sanitized one, for instance)
LIB_PATH = os.environ.get("SRA_LIB_PATH") or os.path.join(_PKG, "libsra.so")

SRA_OK = 0
SRA_E_NULL = 1
SRA_E_SHAPE = 2
SRA_E_CHUNKS = 3
SRA_E_ALIAS = 4
SRA_E_WORKSPACE = 5
SRA_E_DTYPE = 6
SRA_E_ROWS = 7
SRA_E_HIP = 8
SRA_E_LIMIT = 9
DTYPE_BF16 = 0
DTYPE_F32 = 1


class Shape(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_double)]


class Chunk(ctypes.Structure):
    _fields_ = [("src_row", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("dst_row", ctypes.c_int32), ("orig_pos", ctypes.c_int32)]


class LayerArgs(ctypes.Structure):
    _fields_ = [
        ("shape", Shape), ("n_req", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
        ("chunks", ctypes.POINTER(Chunk)), ("query_len", ctypes.c_int32), ("total_len", ctypes.c_int32),
        ("k_store", ctypes.c_void_p), ("v_store", ctypes.c_void_p), ("store_rows", ctypes.c_int64),
        ("q_crit", ctypes.c_void_p), ("k_crit_store", ctypes.c_void_p), ("crit_store_rows", ctypes.c_int64),
        ("n_select", ctypes.c_int32), ("chunk_quota", ctypes.POINTER(ctypes.c_int32)),
        ("scores", ctypes.c_void_p),
        ("anchors_k", ctypes.c_int32), ("anchor_rows", ctypes.c_void_p), ("anchor_norms", ctypes.c_void_p),
        ("hkvd_prev", ctypes.c_void_p), ("hkvd_prev_rows", ctypes.c_int32), ("hkvd_prev_ctx", ctypes.c_int32),
        ("hkvd_dev", ctypes.c_void_p),
        ("q_fresh", ctypes.c_void_p), ("k_fresh", ctypes.c_void_p), ("v_fresh", ctypes.c_void_p),
        ("row_pos", ctypes.c_void_p), ("n_rows", ctypes.c_int32),
        ("k_fused", ctypes.c_void_p), ("v_fused", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
        ("attn_fallback", ctypes.c_void_p),
    ]


_c = ctypes
_P = ctypes.c_void_p
_SIGS = {
    "sra_select_count": (_c.c_int, [_c.c_int64, _c.c_int64, _c.c_int32, _c.POINTER(_c.c_int32)]),
    "sra_workspace_size": (_c.c_size_t, [_c.POINTER(Shape), _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32]),
    "sra_error_string": (_c.c_char_p, [_c.c_int]),
    "sra_last_error": (_c.c_char_p, []),
    "sra_fuse_rerotate": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _P, _c.c_int64, _c.POINTER(Chunk),
                                     _c.c_int32, _P, _P, _c.c_int32, _P]),
    "sra_extract_anchors": (_c.c_int, [_c.POINTER(Shape), _P, _c.c_int64, _c.POINTER(Chunk), _c.c_int32,
                                       _c.c_int32, _P, _P, _P, _c.c_size_t, _P]),
    "sra_anchor_prefix": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _P, _c.c_int64, _c.POINTER(Chunk),
                                     _c.c_int32, _P, _c.c_int32, _P, _P, _c.c_int32, _P]),
    "sra_chunk_attention_stats": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _c.c_int32, _P, _c.c_int32,
                                             _c.POINTER(Chunk), _c.c_int32, _P, _P, _P, _P, _c.c_size_t, _P]),
    "sra_stats_workspace_size": (_c.c_size_t, [_c.POINTER(Shape), _c.c_int32, _c.c_int32, _c.c_int32]),
    "sra_prefix_overlap": (_c.c_int, [_c.POINTER(_c.c_double), _c.POINTER(_c.c_int32), _c.c_int32,
                                      _c.POINTER(_c.c_int32), _c.c_int32, _c.POINTER(_c.c_double)]),
    "sra_cachecraft_count": (_c.c_int, [_c.c_double, _c.c_double, _c.c_double, _c.c_int32, _c.POINTER(_c.c_int32)]),
    "sra_score_select": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _c.c_int32, _P, _c.c_int64,
                                    _c.POINTER(Chunk), _c.c_int32, _c.c_int32, _c.POINTER(_c.c_int32),
                                    _P, _P, _P, _c.c_size_t, _P]),
    "sra_select_topn": (_c.c_int, [_P, _c.c_int32, _c.c_int32, _c.c_int32, _c.POINTER(_c.c_int32),
                                   _c.POINTER(Chunk), _c.c_int32, _c.c_int32, _P, _P]),
    "sra_select_topn_nested": (_c.c_int, [_P, _c.c_int32, _c.c_int32, _P, _c.c_int32, _c.c_int32, _c.c_int32,
                                          _c.c_int32, _c.POINTER(_c.c_int32), _c.POINTER(_P), _P]),
    "sra_scatter_kv": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _P, _P, _c.c_int32, _P, _P,
                                  _c.c_int32, _P]),
    "sra_hkvd_select": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _P, _c.c_int32, _P, _P, _P, _c.c_int32,
                                   _c.c_int32, _c.c_int32, _P, _P, _P]),
    "sra_sparse_causal_attn": (_c.c_int, [_c.POINTER(Shape), _c.c_int32, _P, _P, _c.c_int32, _P, _P,
                                          _c.c_int32, _P, _P, _P, _P, _c.c_size_t, _P]),
    "sra_fused_layer": (_c.c_int, [_c.POINTER(LayerArgs), _P, _c.c_size_t, _P]),
    "sra_fused_layer_static": (_c.c_int, [_c.POINTER(LayerArgs), _P]),
    "sra_check_rows": (_c.c_int, [_P, _c.c_int32, _c.c_int32, _c.c_int32, _c.POINTER(_c.c_int32), _P]),
    "sra_pipelined_layers": (_c.c_int, [_c.POINTER(LayerArgs), _c.c_int32, _c.POINTER(_P), _c.POINTER(_P),
                                        _c.c_size_t, _c.POINTER(_P), _c.POINTER(_P), _c.c_int32, _c.POINTER(_P),
                                        _P, _c.c_size_t, _P, _P]),
}

_hip = None


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime, for the few calls the binding makes itself (event handles)."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventCreateWithFlags.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        _hip = h
    return _hip

_lib = None


class SRAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises RuntimeError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m selective_recompute_attention_amd.build` (no fallback exists)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def check(status: int) -> None:
    if status != SRA_OK:
        l = lib()
        raise SRAError(status, f"{l.sra_error_string(status).decode()}: {l.sra_last_error().decode()}")
