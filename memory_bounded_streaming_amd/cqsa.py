"""ctypes binding of libcqsa.so (argument marshalling only).

Each function has the name of the C entry point it calls (see ``include/cqsa.h``);
every step of the computation runs in the library.  Pointer arguments accept a
plain integer address, ``None`` (NULL), or any object with ``data_ptr()`` (a torch
tensor) or a numpy array.  Streams accept an integer handle, ``None`` or an object
with a ``cuda_stream`` attribute (a torch stream).  Failures raise ``CqsaError``.

The library must have been built (``python -m memory_bounded_streaming_amd.build``);
``load()`` raises if it is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "CqsaError", "load", "CQSA_BF16", "CQSA_F32", "CQSA_RES_DEVICE", "CQSA_RES_HOST_PINNED",
    "CQSA_FLAG_HOST_ACC", "CQSA_FLAG_KV_SINGLE", "CQSA_FLAG_PAD", "CQSA_FLAG_CAUSAL", "CQSA_FLAG_FREE_BUDGET",
    "CQSA_OK", "CQSA_EINVAL", "CQSA_ENOSET", "CQSA_EDIVIDE", "CQSA_EBUDGET", "CQSA_EHIP", "CQSA_ENOMEM",
    "CQSA_ESMALL", "MODE_NAMES", "cqsa_plan_fallback", "cqsa_debug_fail_allocations",
    "cqsa_version", "cqsa_difference_set", "cqsa_plan_create", "cqsa_plan_info_get", "cqsa_plan_schedule",
    "cqsa_plan_coverage", "cqsa_plan_destroy", "cqsa_workspace_size", "cqsa_partials", "cqsa_merge",
    "cqsa_forward", "cqsa_forward_noalloc", "cqsa_backward_workspace_size", "cqsa_backward", "cqsa_plan_estimate", "cqsa_status_string", "cqsa_last_error", "Plan",
]

CQSA_BF16, CQSA_F32 = 0, 1
CQSA_RES_DEVICE, CQSA_RES_HOST_PINNED = 0, 1
CQSA_FLAG_HOST_ACC, CQSA_FLAG_KV_SINGLE, CQSA_FLAG_PAD, CQSA_FLAG_CAUSAL = 0x1, 0x2, 0x4, 0x8
CQSA_FLAG_FREE_BUDGET = 0x10
(CQSA_OK, CQSA_EINVAL, CQSA_ENOSET, CQSA_EDIVIDE, CQSA_EBUDGET, CQSA_EHIP, CQSA_ENOMEM,
 CQSA_ESMALL) = 0, -1, -2, -3, -4, -5, -6, -7
MODE_NAMES = {1: "device_acc_kv2", 2: "host_acc_kv2", 3: "device_acc_kv1", 4: "host_acc_kv1"}
MAX_LEVELS = 12

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcqsa.so")
_lib = None


class CqsaError(RuntimeError):
    def __init__(self, status: int, text: str, detail: str):
        super().__init__(f"{text} ({detail})" if detail else text)
        self.status = status
        self.detail = detail


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("levels", ctypes.c_int32),
        ("c", ctypes.c_int32 * MAX_LEVELS), ("l", ctypes.c_int32 * MAX_LEVELS),
        ("n_tasks", ctypes.c_int64), ("unit_tokens", ctypes.c_int64), ("n_units", ctypes.c_int64),
        ("visits", ctypes.c_int64), ("task_tokens", ctypes.c_int64), ("budget_bytes", ctypes.c_int64),
        ("stream_mode", ctypes.c_int32), ("kv_buffers", ctypes.c_int32),
        ("stream_workspace_bytes", ctypes.c_int64), ("device_workspace_bytes", ctypes.c_int64),
        ("host_acc_bytes", ctypes.c_int64), ("useful_flop", ctypes.c_double),
        ("padded_tokens", ctypes.c_int64), ("bwd_stream_mode", ctypes.c_int32), ("bwd_host_stats", ctypes.c_int32),
        ("bwd_stream_workspace_bytes", ctypes.c_int64),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("t_total_ms", ctypes.c_double), ("t_h2d_ms", ctypes.c_double), ("t_attn_ms", ctypes.c_double),
        ("t_merge_ms", ctypes.c_double), ("t_d2h_ms", ctypes.c_double),
        ("bytes_h2d", ctypes.c_int64), ("bytes_d2h", ctypes.c_int64), ("peak_device_bytes", ctypes.c_int64),
        ("n_attn_launches", ctypes.c_int64), ("n_merge_launches", ctypes.c_int64),
        ("n_h2d_copies", ctypes.c_int64), ("n_d2h_copies", ctypes.c_int64), ("useful_flop", ctypes.c_double),
        ("bytes_d2d", ctypes.c_int64), ("observed_peak_bytes", ctypes.c_int64),
        ("device_free_at_entry", ctypes.c_int64), ("levels_used", ctypes.c_int32), ("replans", ctypes.c_int32),
    ]


class Rates(ctypes.Structure):
    _fields_ = [("attn_tflops", ctypes.c_double), ("merge_gbs", ctypes.c_double), ("h2d_gbs", ctypes.c_double),
                ("d2h_gbs", ctypes.c_double)]


class Estimate(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64), ("padded_tokens", ctypes.c_int64),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("levels", ctypes.c_int32),
        ("c", ctypes.c_int32 * MAX_LEVELS), ("l", ctypes.c_int32 * MAX_LEVELS),
        ("n_tasks", ctypes.c_int64), ("unit_tokens", ctypes.c_int64), ("visits", ctypes.c_int64),
        ("task_tokens", ctypes.c_int64), ("stream_mode", ctypes.c_int32), ("kv_buffers", ctypes.c_int32),
        ("stream_workspace_bytes", ctypes.c_int64), ("per_task_descriptor_bytes", ctypes.c_int64),
        ("host_pinned_bytes", ctypes.c_int64), ("bytes_h2d", ctypes.c_int64), ("bytes_d2h", ctypes.c_int64),
        ("bytes_d2d", ctypes.c_int64),
        ("merge_bytes", ctypes.c_int64), ("useful_flop", ctypes.c_double),
        ("t_attn_s", ctypes.c_double), ("t_merge_s", ctypes.c_double), ("t_h2d_s", ctypes.c_double),
        ("t_d2h_s", ctypes.c_double), ("t_est_s", ctypes.c_double), ("materializable", ctypes.c_int32),
        ("bwd_levels", ctypes.c_int32), ("bwd_stream_mode", ctypes.c_int32), ("bwd_host_stats", ctypes.c_int32),
        ("bwd_reserved", ctypes.c_int32), ("bwd_task_tokens", ctypes.c_int64),
        ("bwd_stream_workspace_bytes", ctypes.c_int64),
    ]


EXPORTS = {
    "cqsa_version": (ctypes.c_char_p, []),
    "cqsa_difference_set": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]),
    "cqsa_plan_create": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p)]),
    "cqsa_plan_info_get": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]),
    "cqsa_plan_schedule": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]),
    "cqsa_plan_coverage": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]),
    "cqsa_plan_destroy": (None, [ctypes.c_void_p]),
    "cqsa_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]),
    "cqsa_partials": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 6),
    "cqsa_merge": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5),
    "cqsa_forward": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 5 +
                     [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(Stats)]),
    "cqsa_forward_noalloc": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 6),
    "cqsa_backward_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)]),
    "cqsa_backward": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_void_p] * 9 +
                      [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(Stats)]),
    "cqsa_plan_estimate": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int64,
                                          ctypes.c_uint32, ctypes.POINTER(Rates), ctypes.POINTER(Estimate)]),
    "cqsa_plan_fallback": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_void_p)]),
    "cqsa_debug_fail_allocations": (ctypes.c_int, [ctypes.c_int32]),
    "cqsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cqsa_last_error": (ctypes.c_char_p, []),
}


def load(path: str | None = None):
    """Load libcqsa.so once and declare its signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m memory_bounded_streaming_amd.build` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    if isinstance(x, np.ndarray):
        return int(x.ctypes.data)
    raise TypeError(f"cannot pass {type(x).__name__} as a pointer")


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"cannot pass {type(s).__name__} as a stream")


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        raise CqsaError(status, lib.cqsa_status_string(status).decode(), lib.cqsa_last_error().decode())


def cqsa_version() -> str:
    return load().cqsa_version().decode()


def cqsa_status_string(status: int) -> str:
    return load().cqsa_status_string(status).decode()


def cqsa_last_error() -> str:
    return load().cqsa_last_error().decode()


def cqsa_difference_set(l: int) -> list[int]:
    buf = (ctypes.c_int32 * max(l, 1))()
    _check(load().cqsa_difference_set(l, buf, max(l, 1)))
    return list(buf[:l])


def cqsa_plan_create(n: int, heads: int, head_dim: int, dtype: int, l_levels, n_levels: int | None = None,
                     budget_bytes: int = 0, flags: int = 0) -> int:
    """Returns an opaque plan handle; free it with cqsa_plan_destroy."""
    levels = list(l_levels)
    if n_levels is None:
        n_levels = len(levels)
    arr = (ctypes.c_int32 * max(1, len(levels)))(*levels)
    out = ctypes.c_void_p()
    _check(load().cqsa_plan_create(n, heads, head_dim, dtype, arr, n_levels, budget_bytes, flags,
                                   ctypes.byref(out)))
    return out.value


def cqsa_plan_info_get(plan: int) -> dict:
    info = PlanInfo()
    _check(load().cqsa_plan_info_get(plan, ctypes.byref(info)))
    d = {name: getattr(info, name) for name, _ in PlanInfo._fields_}
    d["c"] = list(info.c[:info.levels])
    d["l"] = list(info.l[:info.levels])
    return d


def cqsa_plan_schedule(plan: int) -> np.ndarray:
    needed = ctypes.c_int64()
    lib = load()
    _check(lib.cqsa_plan_schedule(plan, None, 0, ctypes.byref(needed)))
    buf = np.zeros(needed.value, dtype=np.int64)
    _check(lib.cqsa_plan_schedule(plan, buf.ctypes.data, buf.size, ctypes.byref(needed)))
    return buf


def cqsa_plan_coverage(plan: int) -> np.ndarray:
    needed = ctypes.c_int64()
    lib = load()
    _check(lib.cqsa_plan_coverage(plan, None, 0, ctypes.byref(needed)))
    u = int(round(needed.value ** 0.5))
    buf = np.zeros((u, u), dtype=np.int32)
    _check(lib.cqsa_plan_coverage(plan, buf.ctypes.data, buf.size, ctypes.byref(needed)))
    return buf


def cqsa_plan_destroy(plan: int) -> None:
    if plan:
        load().cqsa_plan_destroy(plan)


def cqsa_workspace_size(plan: int, residency: int) -> int:
    out = ctypes.c_int64()
    _check(load().cqsa_workspace_size(plan, residency, ctypes.byref(out)))
    return out.value


def cqsa_partials(plan: int, q, k, v, n_out, ml_out, stream=None) -> None:
    _check(load().cqsa_partials(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(n_out), _ptr(ml_out), _stream(stream)))


def cqsa_merge(plan: int, n_in, ml_in, o, lse=None, stream=None) -> None:
    _check(load().cqsa_merge(plan, _ptr(n_in), _ptr(ml_in), _ptr(o), _ptr(lse), _stream(stream)))


def cqsa_forward(plan: int, q, k, v, o, lse=None, residency: int = CQSA_RES_DEVICE, workspace=None,
                 workspace_bytes: int = 0, stream=None, stats: bool = False) -> dict | None:
    st = Stats() if stats else None
    if workspace is not None and workspace_bytes == 0 and hasattr(workspace, "numel"):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load().cqsa_forward(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), residency, _ptr(workspace),
                               workspace_bytes, _stream(stream), ctypes.byref(st) if st is not None else None))
    if st is None:
        return None
    return {name: getattr(st, name) for name, _ in Stats._fields_}


def cqsa_forward_noalloc(plan: int, q, k, v, o, lse=None, stream=None) -> None:
    """Device-resident forward with the library's static scratch array (no allocation)."""
    _check(load().cqsa_forward_noalloc(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)))


def cqsa_backward_workspace_size(plan: int, residency: int = CQSA_RES_DEVICE) -> int:
    out = ctypes.c_int64()
    _check(load().cqsa_backward_workspace_size(plan, residency, ctypes.byref(out)))
    return out.value


def cqsa_backward(plan: int, q, k, v, o, lse, d_o, dq, dk, dv, residency: int = CQSA_RES_DEVICE, workspace=None,
                  workspace_bytes: int = 0, stream=None, stats: bool = False) -> dict | None:
    st = Stats() if stats else None
    if workspace is not None and workspace_bytes == 0 and hasattr(workspace, "numel"):
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load().cqsa_backward(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk),
                                _ptr(dv), residency, _ptr(workspace), workspace_bytes, _stream(stream),
                                ctypes.byref(st) if st is not None else None))
    if st is None:
        return None
    return {name: getattr(st, name) for name, _ in Stats._fields_}


def cqsa_plan_estimate(n: int, heads: int, head_dim: int, dtype: int, l_levels, n_levels: int | None = None,
                       budget_bytes: int = 0, flags: int = 0, rates=None) -> dict:
    """Closed-form dry run; rates: dict with attn_tflops, merge_gbs, h2d_gbs, d2h_gbs."""
    levels = list(l_levels)
    if n_levels is None:
        n_levels = len(levels)
    arr = (ctypes.c_int32 * max(1, len(levels)))(*levels)
    r = Rates(**(rates or {}))
    out = Estimate()
    _check(load().cqsa_plan_estimate(n, heads, head_dim, dtype, arr, n_levels, budget_bytes, flags,
                                     ctypes.byref(r), ctypes.byref(out)))
    d = {name: getattr(out, name) for name, _ in Estimate._fields_}
    d["c"] = list(out.c[:out.levels])
    d["l"] = list(out.l[:out.levels])
    return d


def cqsa_plan_fallback(plan: int, budget_bytes: int) -> int:
    """Handle of the plan one level deeper under budget_bytes; free it with cqsa_plan_destroy."""
    out = ctypes.c_void_p()
    _check(load().cqsa_plan_fallback(plan, budget_bytes, ctypes.byref(out)))
    return out.value


def cqsa_debug_fail_allocations(count: int) -> None:
    _check(load().cqsa_debug_fail_allocations(count))


class Plan:
    """Owning wrapper of a plan handle (the same calls, with the handle bound)."""

    def __init__(self, n, heads, head_dim, dtype, l_levels, n_levels=None, budget_bytes=0, flags=0, handle=None):
        if handle is None:
            handle = cqsa_plan_create(n, heads, head_dim, dtype, l_levels, n_levels, budget_bytes, flags)
        self.handle = handle
        self.info = cqsa_plan_info_get(self.handle)

    def fallback(self, budget_bytes):
        """The out-of-memory fallback plan (one level deeper) as an owning Plan."""
        return Plan(None, None, None, None, None, handle=cqsa_plan_fallback(self.handle, budget_bytes))

    def schedule(self):
        return cqsa_plan_schedule(self.handle)

    def coverage(self):
        return cqsa_plan_coverage(self.handle)

    def workspace_size(self, residency):
        return cqsa_workspace_size(self.handle, residency)

    def partials(self, *a, **kw):
        return cqsa_partials(self.handle, *a, **kw)

    def merge(self, *a, **kw):
        return cqsa_merge(self.handle, *a, **kw)

    def forward(self, *a, **kw):
        return cqsa_forward(self.handle, *a, **kw)

    def forward_noalloc(self, *a, **kw):
        return cqsa_forward_noalloc(self.handle, *a, **kw)

    def backward_workspace_size(self, residency=CQSA_RES_DEVICE):
        return cqsa_backward_workspace_size(self.handle, residency)

    def backward(self, *a, **kw):
        return cqsa_backward(self.handle, *a, **kw)

    def close(self):
        if self.handle:
            cqsa_plan_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
