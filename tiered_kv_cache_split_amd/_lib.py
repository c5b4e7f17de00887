"""ctypes declarations of librkv's C ABI (include/rkv.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librkv.so")

RKV_TYPE_F32, RKV_TYPE_F16, RKV_TYPE_Q4_0, RKV_TYPE_Q8_0 = 0, 1, 2, 8
RKV_OK, RKV_ERR_ARG, RKV_ERR_UNSUPPORTED, RKV_ERR_HIP, RKV_ERR_NOMEM, RKV_ERR_CAPTURE = 0, -1, -2, -3, -4, -5
RKV_LIFT_BULK, RKV_LIFT_UVA, RKV_LIFT_KERNEL, RKV_LIFT_AUTO, RKV_LIFT_DIRECT = 0, 1, 2, 3, 4
RKV_RESIDENCY_AUTO, RKV_RESIDENCY_RESIDENT, RKV_RESIDENCY_WINDOW = 0, 1, 2
RKV_TAIL_LIFT, RKV_TAIL_HOST = 0, 1
RKV_DQ_DECODE_MMA, RKV_DQ_PREFILL, RKV_DQ_VECTOR, RKV_DQ_HEAD_DIM = 0, 1, 2, 3

i64 = ctypes.c_int64
vp = ctypes.c_void_p


class RkvTensor(ctypes.Structure):
    _fields_ = [("data", vp), ("type", ctypes.c_int32), ("ne", i64 * 4), ("nb", i64 * 4)]


class RkvStats(ctypes.Structure):
    _fields_ = [("n_segments", ctypes.c_int32), ("n_partials", ctypes.c_int32),
                ("n_tail_tiles", ctypes.c_int32), ("lift_mode", ctypes.c_int32),
                ("lift_bytes", i64), ("splits_window", ctypes.c_int32),
                ("kernel_variant", ctypes.c_int32), ("tail_host", ctypes.c_int32),
                ("host_tail_ms", ctypes.c_float)]


class RkvBcacheCounters(ctypes.Structure):
    _fields_ = [("misses", ctypes.c_uint64), ("lookups", ctypes.c_uint64), ("calls", ctypes.c_uint64),
                ("epoch", ctypes.c_int32), ("hand", ctypes.c_int32), ("last_misses", ctypes.c_int32),
                ("overflow", ctypes.c_int32)]


TP = ctypes.POINTER(RkvTensor)

# name -> (restype, argtypes); every name is exported by librkv.so and declared in rkv.h
SIGNATURES = {
    "rkv_version": (ctypes.c_char_p, []),
    "rkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "rkv_last_error": (ctypes.c_char_p, []),
    "rkv_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(vp)]),
    "rkv_reserve": (ctypes.c_int, [vp, i64, i64, ctypes.c_int, i64]),
    "rkv_destroy": (None, [vp]),
    "rkv_get_stats": (ctypes.c_int, [vp, ctypes.POINTER(RkvStats)]),
    "rkv_set_lift_mode": (ctypes.c_int, [vp, ctypes.c_int]),
    "rkv_set_direct_tail_max": (ctypes.c_int, [vp, ctypes.c_int64]),
    "rkv_set_splits": (ctypes.c_int, [vp, ctypes.c_int]),
    "rkv_set_lift_timing": (ctypes.c_int, [vp, ctypes.c_int]),
    "rkv_lift_timing_ms": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
    "rkv_set_kernel_timing": (ctypes.c_int, [vp, ctypes.c_int]),
    "rkv_kernel_timing_ms": (ctypes.c_int, [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
    "rkv_attn_decode": (ctypes.c_int, [vp, TP, TP, TP, TP, TP, TP, i64, i64, ctypes.c_float, vp, vp, vp]),
    "rkv_attn_prefill": (ctypes.c_int, [vp, TP, TP, TP, TP, TP, TP, i64, i64, ctypes.c_float, i64, vp, vp, vp]),
    "rkv_attn_rows": (ctypes.c_int, [vp, TP, TP, TP, vp, i64, TP, ctypes.c_float, vp, vp, vp]),
    "rkv_attn_partial": (ctypes.c_int, [vp, TP, TP, TP, TP, i64, i64, ctypes.c_float, vp, vp]),
    "rkv_lse_merge": (ctypes.c_int, [vp, ctypes.c_int, i64, ctypes.c_int, vp, vp, vp]),
    "rkv_tail_lift": (ctypes.c_int, [vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp), vp]),
    "rkv_bcache_create": (ctypes.c_int, [TP, TP, i64, i64, ctypes.POINTER(vp)]),
    "rkv_bcache_destroy": (None, [vp]),
    "rkv_bcache_reset": (ctypes.c_int, [vp, vp]),
    "rkv_bcache_resolve": (ctypes.c_int, [vp, vp, i64, ctypes.c_int, vp, vp]),
    "rkv_bcache_pools": (ctypes.c_int, [vp, TP, TP]),
    "rkv_bcache_append": (ctypes.c_int, [vp, vp, vp, i64, vp]),
    "rkv_bcache_counters": (ctypes.c_int, [vp, ctypes.POINTER(RkvBcacheCounters)]),
    "rkv_bcache_map": (ctypes.c_int, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)]),
    "rkv_attn_decode_noalloc": (ctypes.c_int, [TP, TP, TP, TP, ctypes.c_float, vp, vp, vp]),
    "rkv_dequant_rows": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, vp]),
    "rkv_set_softcap": (ctypes.c_int, [vp, ctypes.c_float]),
    "rkv_set_tail_mode": (ctypes.c_int, [vp, ctypes.c_int, ctypes.c_int]),
    "rkv_choose_tail_mode": (ctypes.c_int, [i64, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_int)]),
    "rkv_tail_partial_host": (ctypes.c_int, [TP, TP, TP, TP, i64, i64, ctypes.c_float, ctypes.c_float, vp,
                                             ctypes.c_int]),
    "rkv_plan_window": (ctypes.c_int, [vp, i64, i64, i64, i64, i64, i64, ctypes.POINTER(i64)]),
    "rkv_window_mode": (ctypes.c_int, [ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load librkv.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"librkv.so not found at {LIB_PATH}: build it first "
                           "(python -m tiered_kv_cache_split_amd.build)")
    # torch ships its own HIP runtime; loaded first, it also satisfies librkv's dependency, so
    # the process holds one runtime (device pointers and streams are shared between the two).
    # Loaded after librkv, a second copy would come up beside the system one and fail to start.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class RkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.rkv_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.rkv_strerror(status).decode()} ({status}): {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != RKV_OK:
        raise RkvError(status, where)
