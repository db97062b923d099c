"""ctypes view of libpa.so (the C ABI declared in include/pa.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_SCRATCH = -5

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_MASK_NONE = 0
PA_MASK_CAUSAL = 1
PA_KV_SAME = 0
PA_KV_FP8_E4M3 = 1
PA_DEBUG_BAD_PAGE = 1
PA_DEBUG_BAD_CONTEXT = 2
PA_DEBUG_BAD_ROWS = 4
PA_DEBUG_BAD_GROUPS = 8

EXPORTED = ("pa_decode_plan", "pa_decode", "pa_split_reduce", "pa_prefill_plan", "pa_prefill",
            "pa_attention_plan", "pa_attention", "pa_append", "pa_decode_noalloc",
            "pa_decode_shared_plan", "pa_decode_shared", "pa_status_string",
            "pa_abi_version")


class PaArgs(ctypes.Structure):
    _fields_ = [
        ("query", ctypes.c_void_p),
        ("key_pages", ctypes.c_void_p),
        ("value_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("context_lens", ctypes.c_void_p),
        ("query_lens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("debug_trace", ctypes.c_void_p),
        ("debug_visits", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("query_start_loc", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32),
        ("debug_errors", ctypes.c_void_p),
    ]


class PaWorkspace(ctypes.Structure):
    _fields_ = [
        ("partial_out", ctypes.c_void_p),
        ("partial_lse", ctypes.c_void_p),
        ("num_splits", ctypes.c_int32),
        ("partition_tokens", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("num_counters", ctypes.c_int32),
        ("counters", ctypes.c_void_p),
        ("prefill_splits", ctypes.c_int32),
    ]


class PaAppendArgs(ctypes.Structure):
    _fields_ = [
        ("key", ctypes.c_void_p),
        ("value", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p),
        ("key_pages", ctypes.c_void_p),
        ("value_pages", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class PaPrefixGroups(ctypes.Structure):
    _fields_ = [
        ("group_start", ctypes.c_void_p),
        ("prefix_lens", ctypes.c_void_p),
        ("num_groups", ctypes.c_int32),
        ("max_group_size", ctypes.c_int32),
    ]


ABI_VERSION = 12  # PA_ABI_VERSION of the structs below

ROUTE_DECODE = 0
ROUTE_PREFILL = 1
ROUTE_RAGGED = 2

SCHEDULE_PARTITIONS = 0
SCHEDULE_BALANCED = 1
SCHEDULE_KEY_SPLIT = 2


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_96_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    A = ctypes.POINTER(PaArgs)
    W = ctypes.POINTER(PaWorkspace)
    L.pa_decode_plan.argtypes = [A, ctypes.c_int32, W, ctypes.POINTER(ctypes.c_size_t)]
    L.pa_decode_plan.restype = ctypes.c_int
    L.pa_decode.argtypes = [A, W, ctypes.c_void_p]
    L.pa_decode.restype = ctypes.c_int
    L.pa_split_reduce.argtypes = [A, W, ctypes.c_void_p]
    L.pa_split_reduce.restype = ctypes.c_int
    L.pa_prefill_plan.argtypes = [A, ctypes.c_int32, W, ctypes.POINTER(ctypes.c_size_t)]
    L.pa_prefill_plan.restype = ctypes.c_int
    L.pa_prefill.argtypes = [A, W, ctypes.c_void_p]
    L.pa_prefill.restype = ctypes.c_int
    L.pa_attention_plan.argtypes = [A, ctypes.c_int32, W, ctypes.POINTER(ctypes.c_size_t),
                                    ctypes.POINTER(ctypes.c_int32)]
    L.pa_attention_plan.restype = ctypes.c_int
    L.pa_attention.argtypes = [A, W, ctypes.c_void_p]
    L.pa_attention.restype = ctypes.c_int
    L.pa_append.argtypes = [ctypes.POINTER(PaAppendArgs), ctypes.c_void_p]
    L.pa_append.restype = ctypes.c_int
    L.pa_decode_noalloc.argtypes = [A, ctypes.c_void_p]
    L.pa_decode_noalloc.restype = ctypes.c_int
    G = ctypes.POINTER(PaPrefixGroups)
    L.pa_decode_shared_plan.argtypes = [A, G, ctypes.c_int32, W, ctypes.POINTER(ctypes.c_size_t)]
    L.pa_decode_shared_plan.restype = ctypes.c_int
    L.pa_decode_shared.argtypes = [A, G, W, ctypes.c_void_p]
    L.pa_decode_shared.restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int32]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_abi_version.argtypes = []
    L.pa_abi_version.restype = ctypes.c_int32
    if L.pa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {L.pa_abi_version()}, this binding "
                          f"expects {ABI_VERSION}; rebuild it")
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().pa_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PaError(fn, status, status_string(status))
