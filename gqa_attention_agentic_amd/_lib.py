"""ctypes binding of libgqa_attn.so (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module
converts torch tensors to device pointers, Python lists to host int32
arrays, and status codes to exceptions. There is no fallback: if the
library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgqa_attn.so")

GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_UNSUPPORTED = -2
GQA_ERR_NO_MEMORY = -3
GQA_ERR_HIP = -4
GQA_BF16 = 0
GQA_FP32 = 1

# Every symbol include/gqa_attn.h declares.
EXPORTED = (
    "gqa_attn_create", "gqa_attn_forward", "gqa_attn_destroy", "gqa_attn_last_error",
    "gqa_attn_plan_stats", "gqa_attn_plan_splits", "gqa_attn_enable_timing",
    "gqa_attn_kernel_times", "gqa_attn_plan_host", "gqa_attn_append_kv", "gqa_attn_append_times",
    "gqa_attn_forward_noalloc", "gqa_attn_kernel_times_list",
)
# Every symbol include/gqa_probe.h declares (measurement only).
PROBES = ("gqa_probe_mfma_bf16", "gqa_probe_read")


class Params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("workspace_bytes_cap", ctypes.c_int64)]


class PlanStats(ctypes.Structure):
    _fields_ = [("n_items_wide", ctypes.c_int64), ("n_items_narrow", ctypes.c_int64),
                ("n_kv_tiles", ctypes.c_int64), ("n_merge_rows", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("n_units", ctypes.c_int64),
                ("max_splits", ctypes.c_int32), ("merge_launch", ctypes.c_int32),
                ("wide_cus", ctypes.c_int32), ("narrow_cus", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gqa_attn status {status}: {message}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("GQA_ATTN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m gqa_attention_agentic_amd.build`")
    lib = ctypes.CDLL(p)
    P, I32, I64, VP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    I32P = ctypes.POINTER(ctypes.c_int32)
    lib.gqa_attn_create.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(P)]
    lib.gqa_attn_forward.argtypes = [P, VP, VP, VP, I32, VP, VP, VP, I32, I32, I32P, I32P, I32, I32P, I32P,
                                     I32P, I32P, I32, VP, VP, VP]
    lib.gqa_attn_forward_noalloc.argtypes = lib.gqa_attn_forward.argtypes
    DP = ctypes.POINTER(ctypes.c_double)
    lib.gqa_attn_kernel_times_list.argtypes = [P, DP, DP, I64, ctypes.POINTER(I64)]
    lib.gqa_probe_mfma_bf16.argtypes = [I32, I32, I32, DP, DP]
    lib.gqa_probe_read.argtypes = [VP, I64, I32, I32, DP, DP]
    lib.gqa_attn_destroy.argtypes = [P]
    lib.gqa_attn_last_error.restype = ctypes.c_char_p
    lib.gqa_attn_plan_stats.argtypes = [P, ctypes.POINTER(PlanStats)]
    lib.gqa_attn_plan_splits.argtypes = [P, I32P, I32]
    lib.gqa_attn_enable_timing.argtypes = [P, I32]
    lib.gqa_attn_kernel_times.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]
    lib.gqa_attn_plan_host.argtypes = [ctypes.POINTER(Params), I32, I32P, I32P, I32, I32P, I32P, I32P,
                                       I32P, I32, I32P, I64, ctypes.POINTER(I64), I32P,
                                       ctypes.POINTER(PlanStats)]
    lib.gqa_attn_append_kv.argtypes = [P, VP, VP, VP, VP, I32, VP, I32, I32, I32P, I32P, VP]
    lib.gqa_attn_append_times.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]
    for name in ("gqa_attn_create", "gqa_attn_forward", "gqa_attn_destroy", "gqa_attn_plan_stats",
                 "gqa_attn_plan_splits", "gqa_attn_enable_timing", "gqa_attn_kernel_times",
                 "gqa_attn_plan_host", "gqa_attn_append_kv", "gqa_attn_append_times",
                 "gqa_attn_forward_noalloc", "gqa_attn_kernel_times_list", "gqa_probe_mfma_bf16",
                 "gqa_probe_read"):
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def check(status: int) -> None:
    if status != GQA_OK:
        msg = load().gqa_attn_last_error().decode(errors="replace")
        raise GqaError(status, msg)


def int_array(values: Optional[Sequence[int]]):
    if values is None:
        return None
    arr = (ctypes.c_int32 * max(1, len(values)))(*[int(v) for v in values])
    return arr


def params(num_q_heads, num_kv_heads, head_dim, page_size, dtype, softmax_scale=0.0,
           workspace_bytes_cap=0) -> Params:
    return Params(num_q_heads, num_kv_heads, head_dim, page_size, dtype, float(softmax_scale),
                  int(workspace_bytes_cap))
