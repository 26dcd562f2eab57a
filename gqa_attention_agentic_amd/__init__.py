"""MI355X (gfx950) shared-prefix GQA flash attention.

Python face of ``libgqa_attn.so`` (C ABI in ``include/gqa_attn.h``). The
functions here marshal torch tensors and Python lists into the C calls;
PyTorch only provides device memory and the stream. Every step of the
attention -- the Q fold, paged K/V reads, QK^T and PV on MFMA, the online
softmax, causal tile skipping and the log-sum-exp merge -- runs in the
library's HIP kernels. If the library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

from . import _lib
from ._lib import GqaError, load  # noqa: F401

__all__ = ["GqaAttention", "plan_host", "probe_mfma_bf16", "probe_read", "load", "GqaError"]

_DTYPES = {"bf16": _lib.GQA_BF16, "fp32": _lib.GQA_FP32}


def _dtype_code(dtype) -> int:
    import torch
    if dtype in (torch.bfloat16, "bf16"):
        return _lib.GQA_BF16
    if dtype in (torch.float32, "fp32"):
        return _lib.GQA_FP32
    raise ValueError(f"unsupported dtype {dtype!r}")


def _check_lengths(ng, nb, group_shared_len, branch_q_len, branch_private_len, splits):
    """The C ABI takes bare host pointers; their lengths are checked here."""
    if len(group_shared_len) != ng:
        raise ValueError("group_shared_len must have one entry per group")
    if len(branch_q_len) != nb or len(branch_private_len) != nb:
        raise ValueError("branch arrays must have one entry per branch")
    if splits is not None and len(splits) != ng + nb:
        raise ValueError("splits_override must have n_groups + n_branches entries")


class GqaAttention:
    """One handle: fixed head geometry, page size and dtype; reusable across
    forwards (the plan is rebuilt only when the metadata changes)."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 dtype="bf16", softmax_scale: float = 0.0, workspace_bytes_cap: int = 0):
        self.lib = load()
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.page_size = page_size
        self.dtype_code = _dtype_code(dtype)
        p = _lib.params(num_q_heads, num_kv_heads, head_dim, page_size, self.dtype_code,
                        softmax_scale, workspace_bytes_cap)
        h = ctypes.c_void_p()
        _lib.check(self.lib.gqa_attn_create(ctypes.byref(p), ctypes.byref(h)))
        self._h = h
        self._n_units = 0
        self._meta_key = None
        self._meta_arrays = None

    # ------------------------------------------------------------ forward --
    def forward(self, q, k_shared, v_shared, k_pages, v_pages, page_table,
                group_shared_start: Sequence[int], group_shared_len: Sequence[int],
                branch_group: Sequence[int], branch_q_len: Sequence[int],
                branch_private_len: Sequence[int], causal: bool,
                splits: Optional[Sequence[int]] = None, out=None, lse=None, stream=None):
        import torch
        want = torch.bfloat16 if self.dtype_code == _lib.GQA_BF16 else torch.float32
        dev = q.get_device()
        for name, t in (("q", q), ("k_shared", k_shared), ("v_shared", v_shared),
                        ("k_pages", k_pages), ("v_pages", v_pages)):
            if t.dtype != want or t.get_device() != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor on {q.device}")
        if page_table.dtype != torch.int32 or page_table.get_device() != dev or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 tensor on the same device")
        n_tok = q.shape[0]
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(n_tok, self.num_q_heads, dtype=torch.float32, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        # Metadata arrays are converted once per distinct metadata (compared by value).
        meta = (tuple(group_shared_start), tuple(group_shared_len), tuple(branch_group), tuple(branch_q_len),
                tuple(branch_private_len), None if splits is None else tuple(splits))
        if meta != self._meta_key:
            ng, nb = len(meta[0]), len(meta[2])
            _check_lengths(ng, nb, meta[1], meta[3], meta[4], meta[5])
            self._meta_arrays = tuple(_lib.int_array(x) for x in meta)
            self._meta_key = meta
        gs, gl, bg, bq, bp, sp = self._meta_arrays
        ng, nb = len(meta[0]), len(meta[2])
        ptr = lambda t: t.data_ptr() if t.numel() > 0 else None
        st = self.lib.gqa_attn_forward(
            self._h, ptr(q), ptr(k_shared), ptr(v_shared), k_shared.shape[1], ptr(k_pages), ptr(v_pages),
            ptr(page_table), page_table.shape[1] if page_table.dim() == 2 else 0,
            ng, gs, gl, nb, bg, bq, bp, sp, int(bool(causal)), ptr(out), ptr(lse), stream)
        _lib.check(st)
        self._n_units = ng + nb
        return out, lse

    def forward_inputs(self, inp, causal: bool, splits=None, out=None, lse=None, stream=None):
        """forward() on a ``workload.Inputs`` record."""
        return self.forward(inp.q, inp.k_shared, inp.v_shared, inp.k_pages, inp.v_pages, inp.page_table,
                            inp.group_shared_start, inp.group_shared_len, inp.branch_group,
                            inp.branch_q_len, inp.branch_private_len, causal, splits=splits,
                            out=out, lse=lse, stream=stream)

    def append_kv(self, k_new, v_new, k_pages, v_pages, page_table, branch_private_len: Sequence[int],
                  branch_n_new: Sequence[int], stream=None) -> None:
        """Appends k_new / v_new ([rows, H_kv, d], branch b's branch_n_new[b]
        rows contiguous, branches in order) to the branches' private pages,
        after their branch_private_len[b] existing tokens (gqa_attn_append_kv)."""
        import torch
        want = torch.bfloat16 if self.dtype_code == _lib.GQA_BF16 else torch.float32
        dev = k_pages.get_device()
        for name, t in (("k_new", k_new), ("v_new", v_new), ("k_pages", k_pages), ("v_pages", v_pages)):
            if t.dtype != want or t.get_device() != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {want} tensor on {k_pages.device}")
        if page_table.dtype != torch.int32 or page_table.get_device() != dev or not page_table.is_contiguous():
            raise ValueError("page_table must be a contiguous int32 tensor on the same device")
        nb = len(branch_n_new)
        if len(branch_private_len) != nb or (page_table.dim() == 2 and page_table.shape[0] < nb):
            raise ValueError("branch_private_len, branch_n_new and page_table rows must cover the same branches")
        if tuple(k_new.shape) != (sum(branch_n_new), self.num_kv_heads, self.head_dim) or v_new.shape != k_new.shape:
            raise ValueError("k_new / v_new must be [sum(branch_n_new), num_kv_heads, head_dim]")
        if (k_pages.dim() != 4 or tuple(k_pages.shape[1:]) != (self.num_kv_heads, self.page_size, self.head_dim)
                or v_pages.shape != k_pages.shape):
            raise ValueError("k_pages / v_pages must be [n_pages, num_kv_heads, page_size, head_dim]")
        if stream is None:
            stream = torch.cuda.current_stream(k_pages.device).cuda_stream
        ptr = lambda t: t.data_ptr() if t.numel() > 0 else None
        _lib.check(self.lib.gqa_attn_append_kv(
            self._h, ptr(k_new), ptr(v_new), ptr(k_pages), ptr(v_pages), k_pages.shape[0], ptr(page_table),
            page_table.shape[1] if page_table.dim() == 2 else 0, nb, _lib.int_array(branch_private_len),
            _lib.int_array(branch_n_new), stream))

    # ------------------------------------------------------- introspection --
    def plan_stats(self) -> dict:
        s = _lib.PlanStats()
        _lib.check(self.lib.gqa_attn_plan_stats(self._h, ctypes.byref(s)))
        return s.as_dict()

    def plan_splits(self):
        arr = (ctypes.c_int32 * max(1, self._n_units))()
        _lib.check(self.lib.gqa_attn_plan_splits(self._h, arr, self._n_units))
        return list(arr)[: self._n_units]

    def enable_timing(self, on: bool = True) -> None:
        _lib.check(self.lib.gqa_attn_enable_timing(self._h, int(bool(on))))

    def kernel_times(self):
        """(attention ms, merge ms, forwards) summed since timing was enabled."""
        a, m, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
        _lib.check(self.lib.gqa_attn_kernel_times(self._h, ctypes.byref(a), ctypes.byref(m), ctypes.byref(n)))
        return a.value, m.value, n.value

    def kernel_times_list(self):
        """Per timed forward since timing was enabled: a list of (attention
        ms, merge ms), in issue order; clears the records."""
        n = ctypes.c_int64()
        st = self.lib.gqa_attn_kernel_times_list(self._h, None, None, 0, ctypes.byref(n))
        if st != _lib.GQA_OK and n.value == 0:
            _lib.check(st)
        cap = max(1, n.value)
        a, m = (ctypes.c_double * cap)(), (ctypes.c_double * cap)()
        _lib.check(self.lib.gqa_attn_kernel_times_list(self._h, a, m, cap, ctypes.byref(n)))
        return [(a[k], m[k]) for k in range(n.value)]

    def append_times(self):
        """(append kernel ms, appends) summed since timing was enabled."""
        m, n = ctypes.c_double(), ctypes.c_int64()
        _lib.check(self.lib.gqa_attn_append_times(self._h, ctypes.byref(m), ctypes.byref(n)))
        return m.value, n.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            self.lib.gqa_attn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_host(num_q_heads, num_kv_heads, head_dim, page_size, group_shared_start, group_shared_len,
              branch_group, branch_q_len, branch_private_len, causal, splits=None, dtype="bf16"):
    """Host-only planner (no device use): returns (items, splits, stats) where
    items is a list of (unit_slot, kv, row_begin, n_rows, key_begin, key_end,
    split, kernel, bin, chain) tuples; kernel 0 = 128/256-row, 1 = 32-row;
    bin is the workgroup of that kernel that runs the item; chain bit 0: the
    item continues the previous item's state, bit 1: it hands its state on."""
    lib = load()
    p = _lib.params(num_q_heads, num_kv_heads, head_dim, page_size, _dtype_code(dtype))
    ng, nb = len(group_shared_start), len(branch_group)
    _check_lengths(ng, nb, group_shared_len, branch_q_len, branch_private_len, splits)
    args = (ctypes.byref(p), ng, _lib.int_array(group_shared_start), _lib.int_array(group_shared_len),
            nb, _lib.int_array(branch_group), _lib.int_array(branch_q_len),
            _lib.int_array(branch_private_len), _lib.int_array(splits), int(bool(causal)))
    n = ctypes.c_int64()
    _lib.check(lib.gqa_attn_plan_host(*args, None, 0, ctypes.byref(n), None, None))
    items = (ctypes.c_int32 * max(10, 10 * n.value))()
    spl = (ctypes.c_int32 * max(1, ng + nb))()
    stats = _lib.PlanStats()
    _lib.check(lib.gqa_attn_plan_host(*args, items, n.value, ctypes.byref(n), spl, ctypes.byref(stats)))
    flat = list(items)
    return ([tuple(flat[10 * i:10 * i + 10]) for i in range(n.value)], list(spl)[: ng + nb], stats.as_dict())


def probe_mfma_bf16(waves_per_simd: int = 2, iters: int = 2048, reps: int = 20):
    """Achievable bf16 MFMA rate (include/gqa_probe.h): (median TFLOP/s,
    median ms per launch)."""
    lib = load()
    t, ms = ctypes.c_double(), ctypes.c_double()
    _lib.check(lib.gqa_probe_mfma_bf16(int(waves_per_simd), int(iters), int(reps), ctypes.byref(t), ctypes.byref(ms)))
    return t.value, ms.value


def probe_read(buf, bytes_per_copy: int, n_copies: int, reps: int = 20):
    """Achievable streaming-read rate over copy k % n_copies of the device
    tensor `buf` (include/gqa_probe.h): (median GB/s, median us per launch)."""
    lib = load()
    if buf.numel() * buf.element_size() < bytes_per_copy * n_copies:
        raise ValueError("buf is smaller than n_copies x bytes_per_copy")
    g, us = ctypes.c_double(), ctypes.c_double()
    _lib.check(lib.gqa_probe_read(buf.data_ptr(), int(bytes_per_copy), int(n_copies), int(reps), ctypes.byref(g),
                                  ctypes.byref(us)))
    return g.value, us.value
