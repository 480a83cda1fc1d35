"""ctypes view of libbsa's C ABI (include/bsa.h): structs, prototypes, loading.

Argument marshalling only.  The shared library is built in-tree by
``block_sparse_attention_02_amd.build``; importing this module without it
raises, so nothing silently falls back to another implementation.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK = 0
BSA_ERR_ARG = 1
BSA_ERR_SHAPE = 2
BSA_ERR_UNSUPPORTED = 3
BSA_ERR_WORKSPACE = 4
BSA_ERR_INDEX = 5
BSA_ERR_HIP = 6

BSA_BF16 = 0
BSA_F32 = 1

BSA_SEL_BLOCK = 0
BSA_SEL_TOKEN = 1

STATUS_NAMES = {
    0: "BSA_OK", 1: "BSA_ERR_ARG", 2: "BSA_ERR_SHAPE", 3: "BSA_ERR_UNSUPPORTED",
    4: "BSA_ERR_WORKSPACE", 5: "BSA_ERR_INDEX", 6: "BSA_ERR_HIP",
}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f32 = ctypes.c_float
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pf32 = ctypes.POINTER(ctypes.c_float)


class TDesc(ctypes.Structure):
    _fields_ = [("B", _i64), ("N", _i64), ("H", _i64), ("D", _i64),
                ("sB", _i64), ("sN", _i64), ("sH", _i64)]


class RouteArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("d", TDesc), ("dt", _i32),
                ("perm", _p), ("block_len", _p), ("J", _i32), ("M", _i32),
                ("R", _i32), ("kmax", _i32), ("scale", _f32),
                ("q2k_idx", _p), ("q2k_num", _p),
                ("qbar", _p), ("kbar", _p), ("E", _p), ("item_order", _p), ("perm_bh_stride", _i64)]


class QOuterArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("out", _p),
                ("dq", TDesc), ("dkv", TDesc), ("dout", TDesc),
                ("dt", _i32), ("scale", _f32), ("mode", _i32),
                ("perm", _p), ("block_len", _p), ("J", _i32), ("M", _i32),
                ("q2k_idx", _p), ("q2k_num", _p), ("kmax", _i32),
                ("blk_idx", _p), ("blk_cnt", _p), ("S", _i32), ("BS", _i32), ("causal", _i32),
                ("lse", _p), ("item_order", _p),
                ("k_sum", _p), ("v_sum", _p), ("b_sum", _p),
                ("coarse", _p), ("gate", _p), ("perm_bh_stride", _i64), ("order_long", _i32)]


class Segment(ctypes.Structure):
    _fields_ = [("video", _i32), ("T", _i32), ("H", _i32), ("W", _i32)]


H3_MAX_SEGMENTS = 16


class H3RouteArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("d", TDesc), ("dt", _i32),
                ("perm", _p), ("block_len", _p), ("J", _i32), ("M", _i32),
                ("num_prefix", _i32), ("nregions", _i32), ("spans", _p), ("budgets", _p),
                ("kmax", _i32), ("scale", _f32), ("q2k_idx", _p), ("q2k_num", _p),
                ("qbar", _p), ("kbar", _p), ("item_order", _p), ("no_fill", _i32)]


class ReblockArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("d", TDesc), ("dt", _i32), ("M", _i32), ("ridge", _f32),
                ("perm", _p), ("block_len", _p), ("moment", _p), ("factor", _p), ("features", _p),
                ("levels", _p), ("dirs", _p)]


class CoarseArgs(ctypes.Structure):
    _fields_ = [("v", _p), ("d", TDesc), ("dt", _i32), ("perm", _p), ("block_len", _p),
                ("J", _i32), ("M", _i32), ("E", _p), ("vbar", _p), ("C", _p)]


class SummaryArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("d", TDesc), ("dt", _i32),
                ("perm", _p), ("block_len", _p), ("J", _i32), ("M", _i32), ("scale", _f32),
                ("anchor", _p), ("anchor_out", _p), ("k_sum", _p), ("v_sum", _p), ("b_sum", _p)]


class KvOuterArgs(ctypes.Structure):
    _fields_ = [("q", _p), ("k", _p), ("v", _p), ("dq", TDesc), ("dkv", TDesc),
                ("dt", _i32), ("scale", _f32), ("causal", _i32),
                ("q2k", _p), ("q2k_cnt", _p), ("k_sel", _i32), ("BK", _i32),
                ("o_buf", _p), ("lse_buf", _p), ("nslot", _p), ("chunk_cap", _i32)]


class KvOuterLayout(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("max_edges", ctypes.c_int64), ("max_chunks", ctypes.c_int64),
                ("chunk_cap", ctypes.c_int64), ("off_count", ctypes.c_size_t), ("off_rowptr", ctypes.c_size_t),
                ("off_nchunk", ctypes.c_size_t), ("off_chunks", ctypes.c_size_t), ("off_edges", ctypes.c_size_t),
                ("bytes", ctypes.c_size_t)]


class CombineArgs(ctypes.Structure):
    _fields_ = [("o_buf", _p), ("lse_buf", _p), ("nslot", _p), ("k_sel", _i32), ("Hkv", _i32),
                ("dout", TDesc), ("out", _p), ("lse", _p)]


# name -> (restype, argtypes); every symbol declared in include/bsa.h
PROTOTYPES = {
    "bsa_last_error": (ctypes.c_char_p, []),
    "bsa_version": (ctypes.c_char_p, []),
    "bsa_check": (_i32, [_p]),
    "bsa_tile_dims": (_i32, [_i32] * 6 + [ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "vsa_tile_index": (_i32, [_i32] * 6 + [_p, _p, _p, _p]),
    "vsa_budget": (_i32, [ctypes.c_double, _i32]),
    "vsa_pool_route_topk_ws": (_i32, [ctypes.POINTER(RouteArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "vsa_pool_route_topk": (_i32, [ctypes.POINTER(RouteArgs), _p, ctypes.c_size_t, _p]),
    "bsa_qouter_ws": (_i32, [ctypes.POINTER(QOuterArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "bsa_forward_qouter": (_i32, [ctypes.POINTER(QOuterArgs), _p, ctypes.c_size_t, _p]),
    "bsa_forward_qouter_static": (_i32, [ctypes.POINTER(QOuterArgs), _p]),
    "h3_tile_dims": (_i32, [ctypes.POINTER(Segment), _i32, _i32, _i32, _i32] + [ctypes.POINTER(_i32)] * 6),
    "h3_tile_index": (_i32, [ctypes.POINTER(Segment), _i32, _i32, _i32, _i32, _p, _p, _p, _p]),
    "h3_pool_route_topk_ws": (_i32, [ctypes.POINTER(H3RouteArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "h3_pool_route_topk": (_i32, [ctypes.POINTER(H3RouteArgs), _p, ctypes.c_size_t, _p]),
    "spark_reblock_dims": (_i32, [_i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "spark_reblock_ws": (_i32, [ctypes.POINTER(ReblockArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "spark_reblock": (_i32, [ctypes.POINTER(ReblockArgs), _p, ctypes.c_size_t, _p]),
    "vsa_coarse_ws": (_i32, [ctypes.POINTER(CoarseArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "vsa_coarse": (_i32, [ctypes.POINTER(CoarseArgs), _p, ctypes.c_size_t, _p]),
    "spark_summaries_ws": (_i32, [ctypes.POINTER(SummaryArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "spark_summaries": (_i32, [ctypes.POINTER(SummaryArgs), _p, ctypes.c_size_t, _p]),
    "bsa_kvouter_ws": (_i32, [ctypes.POINTER(KvOuterArgs), ctypes.POINTER(ctypes.c_size_t)]),
    "bsa_forward_kvouter": (_i32, [ctypes.POINTER(KvOuterArgs), _p, ctypes.c_size_t, _p]),
    "bsa_kvouter_index_layout": (_i32, [ctypes.POINTER(KvOuterArgs), ctypes.POINTER(KvOuterLayout)]),
    "bsa_combine": (_i32, [ctypes.POINTER(CombineArgs), _p]),
}


class BsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


_lib = None


def load(path=None):
    """Load libbsa.so (cached).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError("libbsa.so is not built (%s); run block_sparse_attention_02_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def check(status):
    """Raise BsaError for a non-OK status, with the library's message."""
    if status != BSA_OK:
        raise BsaError(status, load().bsa_last_error().decode("utf-8", "replace"))
