"""ctypes declarations of the C ABI in ``include/pa.h`` (libpa_mi355x.so).

Loading fails loudly when the shared library has not been built: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libpa_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

PA_OK = 0
PA_ERR_INVAL = -1
PA_ERR_NOMEM = -2
PA_ERR_STATE = -3
PA_ERR_HIP = -4
PA_ERR_UNSUPPORTED = -5

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PA_FP8_E5M2 = 0, 1, 2, 3, 4


class PaPoolStats(ctypes.Structure):
    _fields_ = [("total", ctypes.c_int32), ("used", ctypes.c_int32),
                ("shared", ctypes.c_int32), ("free", ctypes.c_int32)]


class PaPrefixStats(ctypes.Structure):
    _fields_ = [("entries", ctypes.c_int32), ("tail_entries", ctypes.c_int32),
                ("resident", ctypes.c_int32), ("index_only", ctypes.c_int32)]


# kernel-configuration overrides (pa_set_option), for tests and measurements
PA_OPTIONS = {"PA_FORCE_VALU": 0, "PA_PARTITION_TOKENS": 1, "PA_MULTI_WAVES": 2, "PA_MULTI_ROW_TILES": 3,
              "PA_MULTI_PASS_GROUP": 4, "PA_MULTI_MIN_RANGE": 5, "PA_DECODE_SEQ_COST": 6,
              "PA_MULTI_SEQ_COST": 7, "PA_YOUNG_SHARE": 8}

PA_PREFIX_TAIL = 1
PA_PREFIX_RESIDENT = 2


class PaBatchInfo(ctypes.Structure):
    _fields_ = [("scheduled", ctypes.c_int32), ("prefill", ctypes.c_int32), ("preempted", ctypes.c_int32),
                ("freed_requests", ctypes.c_int32), ("freed_blocks", ctypes.c_int32),
                ("waiting", ctypes.c_int32), ("active", ctypes.c_int32)]


class PaRing(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("rope_style", ctypes.c_int32),
                ("rope_table", ctypes.c_void_p), ("rope_capacity", ctypes.c_int32),
                ("rope_head_dim", ctypes.c_int32)]


_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

# name -> (restype, argtypes); every symbol include/pa.h declares
SIGNATURES = {
    "pa_create_pool": (ctypes.c_int, [ctypes.POINTER(_p), _i32, _i32, _i32, _i32, ctypes.c_int, _p, _p]),
    "pa_create_pool_fp8": (ctypes.c_int, [ctypes.POINTER(_p), _i32, _i32, _i32, _i32, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                          _p, _p]),
    "pa_create_pool_kv8": (ctypes.c_int, [ctypes.POINTER(_p), _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                          _p, _p]),
    "pa_destroy_pool": (None, [_p]),
    "pa_alloc_block": (_i32, [_p]),
    "pa_incref_block": (ctypes.c_int, [_p, _i32]),
    "pa_decref_block": (ctypes.c_int, [_p, _i32]),
    "pa_get_refcount": (_i32, [_p, _i32]),
    "pa_get_stats": (ctypes.c_int, [_p, ctypes.POINTER(PaPoolStats)]),
    "pa_block_hashes": (ctypes.c_int, [_p, _i64, _i32, _p]),
    "pa_prefix_match": (ctypes.c_int, [_p, _p, _i64, _p, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i64)]),
    "pa_prefix_insert": (ctypes.c_int, [_p, _p, _i64, _p, _i32, ctypes.c_uint32, ctypes.POINTER(_i32)]),
    "pa_prefix_evict": (ctypes.c_int, [_p, _i32, _p, ctypes.POINTER(_i32)]),
    "pa_prefix_clear": (ctypes.c_int, [_p]),
    "pa_prefix_get_stats": (ctypes.c_int, [_p, ctypes.POINTER(PaPrefixStats)]),
    "pa_cow_block": (ctypes.c_int, [_p, _i32, ctypes.POINTER(_i32)]),
    "pa_copy_blocks": (ctypes.c_int, [_p, _p, _p, _i32, _p]),
    "pa_batcher_create": (ctypes.c_int, [_p, _i32, _i32, ctypes.POINTER(_p)]),
    "pa_batcher_destroy": (None, [_p]),
    "pa_batcher_add": (ctypes.c_int, [_p, ctypes.c_uint64, _i32, _i32]),
    "pa_batcher_schedule": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, ctypes.POINTER(PaBatchInfo)]),
    "pa_batcher_step": (ctypes.c_int, [_p, ctypes.c_uint64]),
    "pa_ring_slot": (_i32, [_i64, _i32, _i32]),
    "pa_compute_slot_mapping": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i32,
                                               ctypes.POINTER(PaRing), _p]),
    "pa_reshape_and_cache": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p]),
    "pa_decode_workspace_bytes": (_sz, [_p, _i32, _i32, _i32, ctypes.POINTER(PaRing)]),
    "pa_rope_table_bytes": (_sz, [_i32, _i32]),
    "pa_rope_table_init": (ctypes.c_int, [_p, _i32, _i32, ctypes.c_float, _p]),
    "pa_decode": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, ctypes.c_float,
                                 ctypes.POINTER(PaRing), _p, _sz, _p]),
    "pa_decode_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32,
                                        ctypes.c_float, ctypes.POINTER(PaRing), _p, _sz, _p]),
    "pa_decode_multi_workspace_bytes": (_sz, [_p, _i32, _i32, _i32, _i32]),
    "pa_decode_multi": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, ctypes.c_float,
                                       _p, _sz, _p]),
    "pa_check_decode_inputs": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _i32, ctypes.POINTER(PaRing), _p, _i32,
                                              _p, _p]),
    "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_hip_error": (ctypes.c_char_p, []),
    "pa_decode_append_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32,
                                                ctypes.c_float, ctypes.POINTER(PaRing), _p]),
    "pa_decode_noalloc_scratch_bytes": (_sz, []),
    "pa_decode_verify_ring": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                             ctypes.c_float, ctypes.POINTER(PaRing), _p, _sz, _p]),
    "pa_decode_verify_ring_workspace_bytes": (_sz, [_p, _i32, _i32, _i32]),
    "pa_read_probe": (ctypes.c_int, [_p, _sz, _p, _p]),
    "pa_set_option": (ctypes.c_int, [ctypes.c_int, _i32]),
    "pa_get_option": (_i32, [ctypes.c_int]),
}

_LIB = None


def use_timeline_build() -> None:
    """Load the measurement build (``libpa_mi355x_timeline.so``: the same
    library with per-wave timeline stamps in the stream-K decode) instead of
    the product library.  Must precede the first load."""
    global LIB_NAME, LIB_PATH
    if _LIB is not None:
        raise RuntimeError("the library is already loaded")
    LIB_NAME = "libpa_mi355x_timeline.so"
    LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)


def load() -> ctypes.CDLL:
    """Load libpa_mi355x.so (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_NAME} is not built at {LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
