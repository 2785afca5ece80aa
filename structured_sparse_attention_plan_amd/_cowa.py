"""ctypes binding of libcowa.so — one Python function per C entry point of cowa.h.

Argument marshalling only: the structs below mirror cowa.h field by field, and every
function returns the C status (0 = COWA_OK).  The library is loaded from this package's
directory; a missing library raises ImportError (there is no fallback path).
"""

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcowa.so")

COWA_OK = 0
COWA_ERR_INVALID_ARG = -1
COWA_ERR_UNSUPPORTED = -2
COWA_ERR_WORKSPACE_TOO_SMALL = -3
COWA_ERR_PLAN_MISMATCH = -4
COWA_ERR_HIP = -5

COWA_BAND_COMPLEMENTARY, COWA_BAND_DUPLICATED, COWA_BAND_DENSE = 0, 1, 2
COWA_DTYPE_BF16, COWA_DTYPE_F32 = 0, 1
COWA_OP_FWD, COWA_OP_BWD, COWA_OP_DECODE, COWA_OP_MALA_BWD, COWA_OP_MALA_FWD = 0, 1, 2, 3, 4
COWA_BWD_DELTA, COWA_BWD_DQ, COWA_BWD_DKDV, COWA_BWD_ALL = 1, 2, 4, 7

EXPORTS = ("cowa_status_string", "cowa_window_make", "cowa_plan_blocks", "cowa_tile_sizes",
           "cowa_workspace_size", "cowa_fwd", "cowa_mala_fwd", "cowa_bwd", "cowa_mala_bwd", "cowa_decode", "cowa_decode_varlen",
           "cowa_wcache_layout", "cowa_wcache_append", "cowa_wcache_decode", "cowa_decode_noalloc")
COWA_DECODE_SCRATCH_BYTES = 16 << 20

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_pi32 = ctypes.POINTER(ctypes.c_int32)


class cowa_window(ctypes.Structure):
    _fields_ = [("sink", _i32), ("near_w", _i32), ("gap", _i32), ("lr", _i32), ("band_mode", _i32)]


class cowa_plan_info(ctypes.Structure):
    _fields_ = [("Lq", _i32), ("Lk", _i32), ("Hkv", _i32), ("Bq", _i32), ("Bk", _i32),
                ("nqb", _i32), ("nkb", _i32), ("nnz", _i64), ("n_partial", _i64),
                ("visited", _i64), ("edges", _i64)]


class cowa_plan_dev(ctypes.Structure):
    _fields_ = [("info", cowa_plan_info), ("win", cowa_window),
                ("row_ptr", _p), ("row_ent", _p), ("col_ptr", _p), ("col_ent", _p),
                ("row_order", _p), ("col_order", _p)]


class cowa_problem(ctypes.Structure):
    _fields_ = [("B", _i32), ("Lq", _i32), ("Lk", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32),
                ("dtype", _i32), ("scale", ctypes.c_float), ("win", cowa_window)]


class cowa_wcache(ctypes.Structure):
    _fields_ = [("B", _i32), ("Hkv", _i32), ("D", _i32), ("Lmax", _i32), ("win", cowa_window),
                ("k", _p), ("v", _p)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libcowa.so is not built ({_LIB_PATH}); run "
                          "`python -m structured_sparse_attention_plan_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.cowa_status_string.argtypes = [ctypes.c_int]
    lib.cowa_status_string.restype = ctypes.c_char_p
    lib.cowa_window_make.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(cowa_window)]
    lib.cowa_window_make.restype = ctypes.c_int
    lib.cowa_plan_blocks.argtypes = [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(cowa_window),
                                     ctypes.POINTER(cowa_plan_info), _pi32, _pi32, _pi32, _pi32,
                                     _pi32, _pi32]
    lib.cowa_plan_blocks.restype = ctypes.c_int
    lib.cowa_tile_sizes.argtypes = [ctypes.c_int, ctypes.POINTER(cowa_problem), _pi32, _pi32]
    lib.cowa_tile_sizes.restype = ctypes.c_int
    lib.cowa_workspace_size.argtypes = [ctypes.c_int, ctypes.POINTER(cowa_problem),
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.cowa_workspace_size.restype = ctypes.c_int
    lib.cowa_fwd.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                             _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
    lib.cowa_fwd.restype = ctypes.c_int
    lib.cowa_mala_fwd.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                                  ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
    lib.cowa_mala_fwd.restype = ctypes.c_int
    lib.cowa_bwd.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                             _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _p, ctypes.c_size_t,
                             _p]
    lib.cowa_bwd.restype = ctypes.c_int
    lib.cowa_mala_bwd.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                                  ctypes.POINTER(cowa_plan_dev), _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _p, _p, _p, ctypes.c_size_t, _p]
    lib.cowa_mala_bwd.restype = ctypes.c_int
    lib.cowa_decode.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                                _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
    lib.cowa_decode.restype = ctypes.c_int
    lib.cowa_decode_varlen.argtypes = [ctypes.POINTER(cowa_problem), _p, _p, _p, _p, _p, _p, _p,
                                       ctypes.c_size_t, _p]
    lib.cowa_decode_varlen.restype = ctypes.c_int
    lib.cowa_wcache_layout.argtypes = [ctypes.POINTER(cowa_window), _i32, _i32, ctypes.POINTER(_i64),
                                       ctypes.POINTER(_i64)]
    lib.cowa_wcache_layout.restype = ctypes.c_int
    lib.cowa_wcache_append.argtypes = [ctypes.POINTER(cowa_wcache), _p, _p, _i32, _p, _p]
    lib.cowa_wcache_append.restype = ctypes.c_int
    lib.cowa_wcache_decode.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_wcache), _p, _p,
                                       _p, _p, _p, ctypes.c_size_t, _p]
    lib.cowa_wcache_decode.restype = ctypes.c_int
    lib.cowa_decode_noalloc.argtypes = [ctypes.POINTER(cowa_problem), ctypes.POINTER(cowa_plan_dev),
                                        _p, _p, _p, _p, _p, _p]
    lib.cowa_decode_noalloc.restype = ctypes.c_int
    return lib


lib = _load()


def status_string(status):
    return lib.cowa_status_string(int(status)).decode()


class CowaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def check(fn, status):
    if status != COWA_OK:
        raise CowaError(fn, status)
