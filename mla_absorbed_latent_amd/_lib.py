"""ctypes view of the C ABI in include/mla.h (and the measurement helpers of
include/mla_bench.h).  Argument marshalling only.

Loading never falls back to anything: if the shared library is missing the
import fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libmla_absorbed_latent.so")

MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_VALUE, MLA_ERR_ALIGN, MLA_ERR_WORKSPACE, \
    MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = range(8)
CACHE_BF16, CACHE_INT8, CACHE_INT4, CACHE_INT4_SYM, CACHE_INT8_TOK, CACHE_FP8_TOK, CACHE_INT4_SYM_K4, \
    CACHE_INT8_CHAN = range(8)


class MlaConfig(C.Structure):
    _fields_ = [("num_heads", C.c_int32), ("qk_nope_dim", C.c_int32), ("kv_lora_rank", C.c_int32),
                ("rope_dim", C.c_int32), ("v_head_dim", C.c_int32), ("block_size", C.c_int32),
                ("cache_dtype", C.c_int32), ("softmax_scale", C.c_float)]


class WorkItem(C.Structure):
    _fields_ = [("seq", C.c_int32), ("first_page", C.c_int32), ("n_pages", C.c_int32), ("out_row", C.c_int32)]


# Every symbol include/*.h declares, with its C signature.
_P = C.c_void_p
_CFG = C.POINTER(MlaConfig)
SIGNATURES = {
    "mla_config_check": (C.c_int, [_CFG]),
    "mla_cache_bytes_per_token": (C.c_size_t, [_CFG]),
    "mla_cache_page_bytes": (C.c_size_t, [_CFG]),
    "mla_decode_workspace_bytes": (C.c_size_t, [_CFG, C.c_int32]),
    "mla_cache_append": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, _P, C.c_int32, _P]),
    "mla_absorb_q": (C.c_int, [_CFG, _P, _P, _P, _P, C.c_int32, _P]),
    "mla_plan_splits": (C.c_int, [_CFG, C.POINTER(C.c_int32), C.c_int32, C.c_int32, C.c_int32,
                                  C.POINTER(WorkItem), C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "mla_decode_attn": (C.c_int, [_CFG, _P, _P, C.c_int64, _P, C.c_int32, _P, _P, C.c_int32, _P, _P,
                                  C.c_int32, _P]),
    "mla_decode_combine": (C.c_int, [_CFG, _P, _P, _P, _P, _P, C.c_int32, _P]),
    "mla_out_proj": (C.c_int, [_CFG, _P, _P, _P, _P, C.c_int32, _P, _P, C.c_int32, _P]),
    "mla_decode_combine_out_proj": (C.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, C.c_int32, _P, _P,
                                              C.c_int32, _P]),
    "mla_layer_front": (C.c_int, [_CFG, _P, C.c_int32, _P, _P, _P, C.c_float, C.c_float, _P, C.c_size_t,
                                  _P, _P, _P, _P, C.c_int32, _P]),
    "mla_layer_front_append": (C.c_int, [_CFG, _P, C.c_int32, _P, _P, _P, C.c_float, C.c_float, _P, C.c_size_t,
                                         _P, _P, _P, _P, _P, C.c_int64, _P, C.c_int32, _P]),
    "mla_layer_front_workspace_bytes": (C.c_size_t, [_CFG, C.c_int32]),
    "mla_layer_front_noalloc": (C.c_int, [_CFG, _P, C.c_int32, _P, _P, _P, C.c_float, C.c_float,
                                          _P, _P, _P, _P, C.c_int32, _P]),
    "mla_prefill_attn": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, _P, C.c_int32, _P, _P, _P, C.c_size_t, _P, _P,
                                   _P]),
    "mla_prefill_workspace_bytes": (C.c_size_t, [_CFG, C.c_int32]),
    "mla_out_residual": (C.c_int, [_CFG, _P, _P, C.c_int32, _P, _P, _P, C.c_size_t, C.c_int32, _P]),
    "mla_append_absorb_q": (C.c_int, [_CFG, _P, C.c_int64, _P, _P, _P, C.c_int32, _P, _P, _P, _P, C.c_int32, _P]),
    "mla_status_string": (C.c_char_p, [C.c_int]),
    # include/mla_bench.h (measurement helpers)
    "mla_bench_stream_read": (C.c_int32, [_P, C.c_int64, _P, C.c_int32, _P]),
    "mla_bench_mfma_loop": (C.c_int32, [C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "mla_bench_clock_probe": (C.c_int32, [C.c_int32, _P, _P]),
    "mla_bench_cu_read": (C.c_int32, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P, _P]),
    "mla_last_hip_error": (C.c_int32, []),
}

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("%s is missing: build it with `python -m mla_absorbed_latent_amd.build` "
                          "(hipcc, gfx950); there is no fallback implementation" % LIB_PATH)
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
