"""ctypes declarations for librcattn.so (the C ABI in include/rc.h).

The library is built in-tree by ``python prefix_shared_kv_amd/build.py`` (run by path:
importing the package would load the library being rebuilt).  There
is no fallback: if it is missing or does not load, importing raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# RC_SANITIZED=1: the build with AddressSanitizer / UndefinedBehaviorSanitizer on
# its host code (prefix_shared_kv_amd/build_host_sanitized.py), for CPU test runs
LIB_PATH = os.path.join(_HERE, "librcattn_san.so" if os.environ.get("RC_SANITIZED") == "1" else "librcattn.so")

RC_OK, RC_ERR_ARG, RC_ERR_SHAPE, RC_ERR_DTYPE, RC_ERR_RANGE, RC_ERR_NOMEM, RC_ERR_HIP, RC_ERR_INTERNAL = range(8)
RC_F32, RC_BF16 = 0, 1
RC_DEVERR_SLOT, RC_DEVERR_TABLE, RC_DEVERR_LENGTH, RC_DEVERR_PLAN = 1, 2, 4, 8
RC_PLAN_MAGIC, RC_PLAN_HEADER, RC_PLAN_ITEM, RC_PLAN_ITEM_OWN = 0x52435031, 8, 8, 1
RC_DECODE_COLS, RC_EXTEND_SHARED_COLS = 128, 256
RC_DECODE_STATIC_WORKSPACE_BYTES = 64 << 20
RC_EMIT_EVICT, RC_EMIT_FULL_MATCH = 1, 2

STATUS_NAMES = {0: "RC_OK", 1: "RC_ERR_ARG", 2: "RC_ERR_SHAPE", 3: "RC_ERR_DTYPE", 4: "RC_ERR_RANGE",
                5: "RC_ERR_NOMEM", 6: "RC_ERR_HIP", 7: "RC_ERR_INTERNAL"}


class RcShape(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("pool_slots", C.c_int64), ("page_size", C.c_int32),
                ("reserved", C.c_int32)]


class RcPlanInfo(C.Structure):
    _fields_ = [("n_items", C.c_int32), ("n_members", C.c_int32), ("max_splits", C.c_int32), ("batch", C.c_int32),
                ("group", C.c_int32), ("chunk", C.c_int32), ("max_cols", C.c_int32), ("shared_items", C.c_int32),
                ("narrow_begin", C.c_int32), ("narrow_first", C.c_int32), ("plan_ints", C.c_int64), ("unique_positions", C.c_int64), ("logical_positions", C.c_int64)]


class RcRadixStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("nodes", "cached_tokens", "free_slots", "pool_slots", "splits", "matches",
                                         "matched_tokens", "inserted_tokens", "duplicate_slots", "evicted_tokens",
                                         "evicted_nodes", "locked_tokens", "page_symbols")]


class RcProfEntry(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int64), ("total_ms", C.c_double)]


class RcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


P = C.c_void_p
I32P = C.POINTER(C.c_int32)
I64P = C.POINTER(C.c_int64)
i32, i64, f32 = C.c_int32, C.c_int64, C.c_float

_SIGS = {
    "rc_last_error": (C.c_char_p, []),
    "rc_version": (C.c_char_p, []),
    "rc_set_error_word": (i32, [P]),
    "rc_upload_table_rows": (i32, [P, i64, P, i64, i64, i64, i64, i64, P]),
    "rc_kv_store": (i32, [C.POINTER(RcShape), P, P, P, P, P, i64, P]),
    "rc_label_distribution": (i32, [P, i32, i64, i64, i32, P, i32, P, P, P, P, P, P]),
    "rc_extend_attention": (i32, [C.POINTER(RcShape), P, P, P, P, P, P, P, i32, i64, P, P, P, P, i32, i64, i32, f32, P]),
    "rc_plan_decode_unshared": (i32, [i32, P, P, i32, i32, P, i64, C.POINTER(RcPlanInfo)]),
    "rc_decode_workspace_bytes": (i64, [C.POINTER(RcShape), C.POINTER(RcPlanInfo)]),
    "rc_decode_attention": (i32, [C.POINTER(RcShape), P, P, P, P, P, P, P, P, i32, i64, P, i32, P,
                                  C.POINTER(RcPlanInfo), f32, P, i64, P]),
    "rc_decode_attention_static": (i32, [C.POINTER(RcShape), P, P, P, P, P, P, P, P, i32, i64, P, i32, P,
                                         C.POINTER(RcPlanInfo), f32, P]),
    "rc_extend_attention_shared": (i32, [C.POINTER(RcShape), P, P, P, P, P, i32, i64, P, i32, P,
                                         C.POINTER(RcPlanInfo), f32, P, i64, P]),
    "rc_radix_create": (i32, [i64, P, C.POINTER(P)]),
    "rc_radix_create_paged": (i32, [i64, i32, P, C.POINTER(P)]),
    "rc_radix_destroy": (None, [P]),
    "rc_radix_match": (i32, [P, P, i64, P, I64P]),
    "rc_radix_alloc": (i32, [P, i64, P]),
    "rc_radix_free": (i32, [P, P, i64]),
    "rc_radix_insert": (i32, [P, P, P, i64, I64P]),
    "rc_radix_emit_rows": (i32, [P, i32, P, P, i32, P, P, i32, i64, P, P, i32, P, P, P, P]),
    "rc_radix_free_rows": (i32, [P, i32, P, P, i32, i64, P, P]),
    "rc_decode_steps": (i32, [P, i32, i64, i32, i32, P, P, P, i32, P, P]),
    "rc_radix_lock": (i32, [P, i32, P, P, P, P, P]),
    "rc_radix_unlock": (i32, [P, P, i32]),
    "rc_radix_evict": (i32, [P, i64, I64P]),
    "rc_radix_insert_rows": (i32, [P, i32, P, P, P, P, P, i32, i64, P]),
    "rc_radix_fork": (i32, [P, P, P, i64, i32, P, P, i32, i64]),
    "rc_radix_plan_decode": (i32, [P, i32, P, P, P, P, P, i32, i32, P, i64, C.POINTER(RcPlanInfo)]),
    "rc_radix_plan_extend": (i32, [P, i32, P, P, P, P, P, i32, i32, P, i64, C.POINTER(RcPlanInfo), P]),
    "rc_radix_stats_get": (i32, [P, C.POINTER(RcRadixStats)]),
    "rc_prof_enable": (i32, [i32]),
    "rc_prof_tag": (i32, [C.c_char_p]),
    "rc_prof_collect": (i32, [C.POINTER(RcProfEntry), i32, I32P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python prefix_shared_kv_amd/build.py` "
                          "(there is no fallback implementation)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.rc_last_error().decode()


def check(status: int) -> None:
    if status != RC_OK:
        raise RcError(status, last_error())
