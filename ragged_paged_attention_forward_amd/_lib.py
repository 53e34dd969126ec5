"""ctypes view of the C ABI declared in include/rpa.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librpa.so")

RPA_OK = 0
RPA_ERR_INVALID_ARG = -1
RPA_ERR_UNSUPPORTED = -2
RPA_ERR_OOM = -3
RPA_ERR_HIP = -4

RPA_OPT_DECODE_SPLIT_KEYS = 1
RPA_OPT_PATH = 2
RPA_OPT_DECODE_MAX_ROWS = 4
RPA_OPT_DECODE_WAVES = 5
RPA_OPT_KERNEL_TIMING = 6
RPA_OPT_XCD_GROUPS = 7
RPA_OPT_FUSED_MERGE = 8
RPA_OPT_PREFILL_SPLIT_KEYS = 9
RPA_OPT_CONCURRENT = 10
RPA_OPT_FP8_STAGE = 11

RPA_KERNEL_PREFILL = 0
RPA_KERNEL_DECODE = 1
RPA_KERNEL_MERGE = 2
RPA_KERNEL_APPEND = 3
RPA_KERNEL_STAGE = 4
RPA_KERNEL_DECODE2 = 5

EXPORTED = ("rpa_create", "rpa_forward", "rpa_forward_append", "rpa_forward_fp8", "rpa_forward_fp8_append", "rpa_destroy", "rpa_release_captured", "rpa_forward_noalloc", "rpa_status_string",
            "rpa_last_error", "rpa_set_option", "rpa_plan", "rpa_kernel_times", "rpa_probe_read", "rpa_probe_mfma",
            "rpa_probe_e4m3")


class Config(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_num_seqs", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("max_q_tokens", ctypes.c_int64)]


class WorkItem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "seq", "kv_head", "q_start", "q_count", "q_pos0", "kv_begin", "kv_end", "split_group",
        "split_index", "num_splits", "partial_base", "kind", "self_append", "new_pos0")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_prefill_items", ctypes.c_int32), ("num_decode_items", ctypes.c_int32),
                ("num_split_groups", ctypes.c_int32), ("num_partials", ctypes.c_int32),
                ("prefill_rows", ctypes.c_int32), ("decode_split_keys", ctypes.c_int32),
                ("visible_pairs", ctypes.c_int64), ("prefill_split_keys", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class RpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load librpa.so; fail loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m ragged_paged_attention_forward_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    lib.rpa_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
    lib.rpa_create.restype = ctypes.c_int
    # host metadata arrays are passed as plain addresses (numpy .ctypes.data)
    lib.rpa_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_float, vp, vp]
    lib.rpa_forward.restype = ctypes.c_int
    lib.rpa_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, vp, vp]
    lib.rpa_forward_noalloc.restype = ctypes.c_int
    lib.rpa_forward_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_float, vp, vp]
    lib.rpa_forward_append.restype = ctypes.c_int
    lib.rpa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_float, vp, vp]
    lib.rpa_forward_fp8.restype = ctypes.c_int
    lib.rpa_forward_fp8_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_float, vp, vp]
    lib.rpa_forward_fp8_append.restype = ctypes.c_int
    lib.rpa_destroy.argtypes = [vp]
    lib.rpa_destroy.restype = None
    lib.rpa_release_captured.argtypes = [vp]
    lib.rpa_release_captured.restype = ctypes.c_int
    lib.rpa_status_string.argtypes = [ctypes.c_int]
    lib.rpa_status_string.restype = ctypes.c_char_p
    lib.rpa_last_error.argtypes = [vp]
    lib.rpa_last_error.restype = ctypes.c_char_p
    lib.rpa_set_option.argtypes = [vp, ctypes.c_int32, ctypes.c_int64]
    lib.rpa_set_option.restype = ctypes.c_int
    lib.rpa_plan.argtypes = [vp, i32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(PlanInfo),
                             ctypes.POINTER(WorkItem), ctypes.c_int32]
    lib.rpa_plan.restype = ctypes.c_int
    lib.rpa_kernel_times.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                     i32p]
    lib.rpa_kernel_times.restype = ctypes.c_int
    lib.rpa_probe_read.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.rpa_probe_read.restype = ctypes.c_int
    lib.rpa_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.rpa_probe_e4m3.argtypes = [vp, vp, ctypes.c_int64, vp]
    lib.rpa_probe_e4m3.restype = ctypes.c_int
    lib.rpa_probe_mfma.restype = ctypes.c_int
    _lib = lib
    return lib
