"""ctypes binding of libkvpage.so: same names as the C ABI in include/kvpage.h.

Argument marshalling only.  Every step of the decode path runs in the HIP
library; torch supplies device memory and the stream.  If the shared library
is missing this module raises at first use -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvpage.so")

KVPAGE_OK = 0
KVPAGE_ERR_INVALID_ARG = -1
KVPAGE_ERR_UNSUPPORTED = -2
KVPAGE_ERR_CAPACITY = -3
KVPAGE_ERR_HIP = -4
KVPAGE_ERR_SCRATCH = -5
KVPAGE_NOALLOC_WORKSPACE_BYTES = 64 << 20
KVPAGE_F16 = 0
KVPAGE_BF16 = 1


class kvpage_task(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("kv_head", ctypes.c_int32),
                ("tok_begin", ctypes.c_int32), ("tok_end", ctypes.c_int32)]


class kvpage_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("split_tokens", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class kvpage_budget(ctypes.Structure):
    _fields_ = [("page_mass", ctypes.c_void_p), ("s_prev", ctypes.c_void_p),
                ("s_next", ctypes.c_void_p), ("alpha_fast", ctypes.c_float),
                ("alpha_slow", ctypes.c_float), ("page_max", ctypes.c_void_p)]


class kvpage_launch_opts(ctypes.Structure):
    _fields_ = [("attn_start", ctypes.c_void_p), ("attn_stop", ctypes.c_void_p),
                ("max_workgroups", ctypes.c_int32), ("shared_pages", ctypes.c_void_p)]


class KvpageError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {status} ({text})")
        self.status = status


_P = ctypes.c_void_p
_S = ctypes.POINTER(kvpage_shape)
_B = ctypes.POINTER(kvpage_budget)
_SIGS = {
    "kvpage_queue_capacity": (ctypes.c_int32, [_S]),
    "kvpage_workspace_bytes": (ctypes.c_int64, [_S, ctypes.c_int32]),
    "kvpage_build_queue": (ctypes.c_int, [_S, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "kvpage_split_attn": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _B, _P]),
    "kvpage_merge_splits": (ctypes.c_int, [_S, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "kvpage_decode_attn": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                          _B, _P, _P, _P]),
    "kvpage_page_mass": (ctypes.c_int, [_S, _B, _P, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "kvpage_decode_step": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                          _B, _P, _P, ctypes.POINTER(kvpage_launch_opts), _P]),
    "kvpage_decode_step_noalloc": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P,
                                                  ctypes.c_int32, _B, _P, _P,
                                                  ctypes.POINTER(kvpage_launch_opts), _P]),
    "kvpage_debug_gather_offsets": (ctypes.c_int, [_S, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "kvpage_choose_split": (ctypes.c_int32, [_S, _P, ctypes.c_int32]),
    "kvpage_append_kv": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kvpage_check_inputs": (ctypes.c_int, [_S, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P]),
    "kvpage_budget_decide": (ctypes.c_int, [_S, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P]),
    "kvpage_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvpage.so (built in-tree by ``build()``); raise if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_07_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().kvpage_status_string(status).decode()


def _check(fn: str, status: int) -> int:
    if status != KVPAGE_OK:
        raise KvpageError(fn, status, status_string(status))
    return status


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


# kvpage_shape.flags: no K/V page is referenced by two sequences in the call;
# the attention kernel's tile loads are then non-temporal.
KVPAGE_FLAG_STREAM_KV = 1


def make_shape(B, Hq, Hkv, d, page_size, split_tokens, max_pages, num_pages, dtype, scale,
               flags=0) -> kvpage_shape:
    code = {"f16": KVPAGE_F16, "bf16": KVPAGE_BF16}.get(dtype, dtype)
    return kvpage_shape(B, Hq, Hkv, d, page_size, split_tokens, max_pages, num_pages, code,
                        scale, flags)


def make_budget(page_mass, s_prev, s_next, page_max, alpha_fast=0.5, alpha_slow=0.05):
    return kvpage_budget(_ptr(page_mass), _ptr(s_prev), _ptr(s_next), alpha_fast, alpha_slow,
                         _ptr(page_max))


# ------------------------------------------------------------ raw entry points

def kvpage_queue_capacity(shape: kvpage_shape) -> int:
    cap = lib().kvpage_queue_capacity(ctypes.byref(shape))
    if cap < 0:
        raise KvpageError("kvpage_queue_capacity", cap, status_string(cap))
    return cap


def kvpage_choose_split(shape: kvpage_shape, ctx_lens, wavefronts: int = 0) -> int:
    """Split size for ``ctx_lens`` (host integers); ``wavefronts`` <= 0 asks the device."""
    arr = (ctypes.c_int32 * max(1, len(ctx_lens)))(*[int(c) for c in ctx_lens])
    split = lib().kvpage_choose_split(ctypes.byref(shape), arr if len(ctx_lens) else None,
                                      int(wavefronts))
    if split < 0:
        raise KvpageError("kvpage_choose_split", split, status_string(split))
    return split


KVPAGE_APPEND_FULL, KVPAGE_APPEND_NO_PAGE, KVPAGE_APPEND_BAD_PAGE = 1, 2, 4


def kvpage_append_kv(shape, k_new, v_new, k_pool, v_pool, block_tables, ctx_lens, ctx_lens_out,
                     free_pages, free_count, free_count_out, status, stream=None):
    return _check("kvpage_append_kv", lib().kvpage_append_kv(
        ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), _ptr(ctx_lens), _ptr(ctx_lens_out), _ptr(free_pages),
        _ptr(free_count), _ptr(free_count_out), _ptr(status), _stream(stream)))


KVPAGE_CHECK_LENGTH, KVPAGE_CHECK_PAGE, KVPAGE_CHECK_QUEUE = 1, 2, 4


def kvpage_check_inputs(shape, ctx_lens, block_tables, tasks, group_offsets, n_tasks, capacity,
                        status, stream=None):
    """Debug checks of the decode preconditions; ``tasks``, ``group_offsets`` and
    ``n_tasks`` may all be None.  Writes the KVPAGE_CHECK_* bits to ``status``."""
    return _check("kvpage_check_inputs", lib().kvpage_check_inputs(
        ctypes.byref(shape), _ptr(ctx_lens), _ptr(block_tables), _ptr(tasks),
        _ptr(group_offsets), _ptr(n_tasks), int(capacity), _ptr(status), _stream(stream)))


KVPAGE_DECIDE_NONE = 0
KVPAGE_DECIDE_ACQUIRE = 1
KVPAGE_DECIDE_COMPRESS = 2


def kvpage_budget_decide(shape, page_max, ctx_lens, tau, ws_size, ws_level, ws_union, decision,
                         victim, stream=None):
    return _check("kvpage_budget_decide", lib().kvpage_budget_decide(
        ctypes.byref(shape), _ptr(page_max), _ptr(ctx_lens), ctypes.c_float(tau), _ptr(ws_size),
        _ptr(ws_level), _ptr(ws_union), _ptr(decision), _ptr(victim), _stream(stream)))


def kvpage_workspace_bytes(shape: kvpage_shape, capacity: int) -> int:
    n = lib().kvpage_workspace_bytes(ctypes.byref(shape), capacity)
    if n < 0:
        raise KvpageError("kvpage_workspace_bytes", int(n), status_string(int(n)))
    return int(n)


def kvpage_build_queue(shape, ctx_lens, tasks, capacity, group_offsets, n_tasks, stream=None):
    return _check("kvpage_build_queue", lib().kvpage_build_queue(
        ctypes.byref(shape), _ptr(ctx_lens), _ptr(tasks), capacity, _ptr(group_offsets),
        _ptr(n_tasks), _stream(stream)))


def kvpage_split_attn(shape, q, k_pool, v_pool, block_tables, ctx_lens, tasks, n_tasks, capacity,
                      workspace, budget=None, stream=None):
    return _check("kvpage_split_attn", lib().kvpage_split_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(ctx_lens), _ptr(tasks), _ptr(n_tasks), capacity, _ptr(workspace),
        None if budget is None else ctypes.byref(budget), _stream(stream)))


def kvpage_merge_splits(shape, group_offsets, capacity, workspace, out, lse, stream=None):
    return _check("kvpage_merge_splits", lib().kvpage_merge_splits(
        ctypes.byref(shape), _ptr(group_offsets), capacity, _ptr(workspace), _ptr(out),
        _ptr(lse), _stream(stream)))


def kvpage_decode_attn(shape, q, k_pool, v_pool, block_tables, ctx_lens, tasks, group_offsets,
                       n_tasks, capacity, workspace, budget, out, lse, stream=None):
    return _check("kvpage_decode_attn", lib().kvpage_decode_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(ctx_lens), _ptr(tasks), _ptr(group_offsets), _ptr(n_tasks), capacity,
        _ptr(workspace), None if budget is None else ctypes.byref(budget), _ptr(out), _ptr(lse),
        _stream(stream)))


def kvpage_page_mass(shape, budget, q, lse, ctx_lens, group_offsets, capacity, workspace,
                     stream=None):
    return _check("kvpage_page_mass", lib().kvpage_page_mass(
        ctypes.byref(shape), None if budget is None else ctypes.byref(budget), _ptr(q), _ptr(lse),
        _ptr(ctx_lens), _ptr(group_offsets), capacity, _ptr(workspace), _stream(stream)))


def kvpage_decode_step(shape, q, k_pool, v_pool, block_tables, ctx_lens, tasks, group_offsets,
                       n_tasks, capacity, workspace, budget, out, lse, opts=None, stream=None):
    return _check("kvpage_decode_step", lib().kvpage_decode_step(
        ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(ctx_lens), _ptr(tasks), _ptr(group_offsets), _ptr(n_tasks), capacity,
        _ptr(workspace), None if budget is None else ctypes.byref(budget), _ptr(out), _ptr(lse),
        None if opts is None else ctypes.byref(opts), _stream(stream)))


def kvpage_decode_step_noalloc(shape, q, k_pool, v_pool, block_tables, ctx_lens, tasks,
                               group_offsets, n_tasks, capacity, budget, out, lse, opts=None,
                               stream=None):
    return _check("kvpage_decode_step_noalloc", lib().kvpage_decode_step_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        _ptr(ctx_lens), _ptr(tasks), _ptr(group_offsets), _ptr(n_tasks), capacity,
        None if budget is None else ctypes.byref(budget), _ptr(out), _ptr(lse),
        None if opts is None else ctypes.byref(opts), _stream(stream)))


def kvpage_debug_gather_offsets(shape, block_tables, tasks, n_tasks, capacity, offsets,
                                stream=None):
    return _check("kvpage_debug_gather_offsets", lib().kvpage_debug_gather_offsets(
        ctypes.byref(shape), _ptr(block_tables), _ptr(tasks), _ptr(n_tasks), capacity,
        _ptr(offsets), _stream(stream)))


# ----------------------------------------------------------- HIP events
# Resolved through libkvpage.so's own dependency scope, so they belong to the
# same HIP runtime instance as the kernels they time.

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


class HipEvent:
    """A HIP event for timestamps.  By default created with
    hipEventDisableSystemFence: timing-only, so recording it does not write
    back and invalidate caches around the work it brackets."""

    def __init__(self, flags: int = HIP_EVENT_DISABLE_SYSTEM_FENCE):
        h = lib()
        self.handle = ctypes.c_void_p()
        if h.hipEventCreateWithFlags(ctypes.byref(self.handle), ctypes.c_uint(flags)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None):
        if lib().hipEventRecord(self.handle, _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if lib().hipEventSynchronize(self.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_ms(self, stop: "HipEvent") -> float:
        ms = ctypes.c_float()
        if lib().hipEventElapsedTime(ctypes.byref(ms), self.handle, stop.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle:
                lib().hipEventDestroy(self.handle)
        except Exception:
            pass


def make_opts(start: HipEvent | None = None, stop: HipEvent | None = None,
              max_workgroups: int = 0, shared_pages=None) -> kvpage_launch_opts:
    """shared_pages: None or a device int32 [B] tensor (or address)."""
    return kvpage_launch_opts(start.handle if start else None, stop.handle if stop else None,
                              max_workgroups,
                              shared_pages if isinstance(shared_pages, (int, type(None)))
                              else shared_pages.data_ptr())
