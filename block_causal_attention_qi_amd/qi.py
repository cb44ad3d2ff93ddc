"""Thin ctypes binding of libqi (C ABI in include/qi.h), same names as the C calls.

Argument marshalling only: torch tensors are passed as device pointers and the current
torch stream as the HIP stream; every step of the computation runs in libqi's HIP
kernels.  Importing this module loads libqi.so and raises ImportError if it has not been
built (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqi.so")

QI_OK, QI_ERR_INVALID_ARG, QI_ERR_UNSUPPORTED, QI_ERR_STATE, QI_ERR_BUFFER_TOO_SMALL, \
    QI_ERR_HIP = range(6)
QI_KV_BF16, QI_KV_FP8_E4M3, QI_KV_FP8_V = 0, 1, 2
QI_CALL_PREFIX, QI_CALL_DENOISE, QI_CALL_FULL = 0, 1, 2
QI_MAX_REQUESTS, QI_MAX_REFS, QI_MAX_HEADS = 64, 10, 128
QI_NOALLOC_MAX_PARTIALS = 262144
QI_LAUNCH_ITEM_FIELDS = 6

EXPORTS = ("qi_plan_create", "qi_plan_destroy", "qi_plan_sizes", "qi_plan_upload",
           "qi_prefix_kv_build", "qi_prefix_kv_build_noalloc", "qi_denoise_attn_step", "qi_attn_full_reference_step",
           "qi_plan_tile_map", "qi_plan_kernel_tile", "qi_plan_launch_items", "qi_plan_cache_offset",
           "qi_plan_pairs", "qi_plan_tokens", "qi_status_string")


class QiError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, _string(status), status))


class _WaveDesc(ctypes.Structure):
    _fields_ = [("n_requests", ctypes.c_int32), ("n_refs", ctypes.POINTER(ctypes.c_int32)),
                ("block_len", ctypes.POINTER(ctypes.c_int32)), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


def _load():
    # torch ships its own libamdhip64 with the same soname as the system one; loading
    # torch first makes libqi bind to that runtime, so the process holds exactly one HIP
    # runtime and torch's device pointers and streams are valid in libqi.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqi.so is not built (run __graft_entry__.build() or "
                          "python -m block_causal_attention_qi_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, VP, SZ, I32, I64 = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, \
        ctypes.c_int64
    sig = {
        "qi_plan_create": ([ctypes.POINTER(_WaveDesc), ctypes.POINTER(P)], I32),
        "qi_plan_destroy": ([P], None),
        "qi_plan_sizes": ([P, ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I32),
        "qi_plan_upload": ([P, VP, SZ, VP], I32),
        "qi_prefix_kv_build": ([P, VP, VP, VP, VP, VP, SZ, VP], I32),
        "qi_prefix_kv_build_noalloc": ([P, VP, VP, VP, VP, VP, SZ, VP], I32),
        "qi_denoise_attn_step": ([P, VP, SZ, VP, VP, VP, VP, VP], I32),
        "qi_attn_full_reference_step": ([P, VP, VP, VP, VP, VP], I32),
        "qi_plan_tile_map": ([P, I32, I32, I32, VP, SZ, ctypes.POINTER(SZ)], I32),
        "qi_plan_kernel_tile": ([P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)], I32),
        "qi_plan_launch_items": ([P, I32, VP, SZ, ctypes.POINTER(SZ)], I32),
        "qi_plan_cache_offset": ([P, I32, I32, I32, I32, ctypes.POINTER(SZ)], I32),
        "qi_plan_pairs": ([P, I32, ctypes.POINTER(I64)], I32),
        "qi_plan_tokens": ([P, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)], I32),
        "qi_status_string": ([I32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _string(status):
    return lib.qi_status_string(status).decode()


def qi_status_string(status):
    return _string(status)


def _check(status, where):
    if status != QI_OK:
        raise QiError(status, where)


class Plan:
    """Host-side plan of one wave (owns a qi_plan*)."""

    def __init__(self, requests, n_heads, head_dim, kv_dtype="bf16"):
        self.requests = [list(map(int, b)) for b in requests]
        self.n_heads, self.head_dim = int(n_heads), int(head_dim)
        self.kv_dtype = kv_dtype
        kv = {"bf16": QI_KV_BF16, "fp8": QI_KV_FP8_E4M3, "fp8_v": QI_KV_FP8_V}.get(kv_dtype, kv_dtype)
        n_refs = [len(b) - 2 for b in self.requests]
        flat = [x for b in self.requests for x in b]
        self._refs = (ctypes.c_int32 * max(1, len(n_refs)))(*n_refs)
        self._bl = (ctypes.c_int32 * max(1, len(flat)))(*flat)
        desc = _WaveDesc(len(self.requests), self._refs, self._bl, self.n_heads,
                         self.head_dim, int(kv) if isinstance(kv, int) else -1)
        self._h = ctypes.c_void_p()
        _check(lib.qi_plan_create(ctypes.byref(desc), ctypes.byref(self._h)), "qi_plan_create")
        self.workspace = None   # keeps the uploaded workspace tensor alive

    @property
    def handle(self):
        if not self._h:
            raise QiError(QI_ERR_INVALID_ARG, "plan already destroyed")
        return self._h

    def close(self):
        if self._h:
            lib.qi_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def cache_bytes(self):
        return qi_plan_sizes(self)[0]

    @property
    def workspace_bytes(self):
        return qi_plan_sizes(self)[1]


def _ptr(t, name, dtype=None, numel=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def qi_plan_create(requests, n_heads, head_dim, kv_dtype="bf16"):
    return Plan(requests, n_heads, head_dim, kv_dtype)


def qi_plan_destroy(plan):
    plan.close()


def qi_plan_sizes(plan):
    c, w = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.qi_plan_sizes(plan.handle, ctypes.byref(c), ctypes.byref(w)), "qi_plan_sizes")
    return c.value, w.value


def qi_plan_upload(plan, workspace, stream=None):
    import torch
    _check(lib.qi_plan_upload(plan.handle, _ptr(workspace, "workspace", torch.uint8),
                              workspace.numel(), _stream(stream)), "qi_plan_upload")
    plan.workspace = workspace


def qi_plan_tokens(plan):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.qi_plan_tokens(plan.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "qi_plan_tokens")
    return a.value, b.value, c.value


def _live_numel(plan, call):
    pre, img, tot = qi_plan_tokens(plan)
    n = {QI_CALL_PREFIX: pre, QI_CALL_DENOISE: img, QI_CALL_FULL: tot}[call]
    return n * plan.n_heads * plan.head_dim


def qi_prefix_kv_build(plan, q_pre, k_pre, v_pre, o_pre, cache, stream=None):
    import torch
    n = _live_numel(plan, QI_CALL_PREFIX)
    bf = torch.bfloat16
    _check(lib.qi_prefix_kv_build(plan.handle, _ptr(q_pre, "q_pre", bf, n),
                                  _ptr(k_pre, "k_pre", bf, n), _ptr(v_pre, "v_pre", bf, n),
                                  _ptr(o_pre, "o_pre", bf, n), _ptr(cache, "cache", torch.uint8),
                                  cache.numel(), _stream(stream)), "qi_prefix_kv_build")


def qi_prefix_kv_build_noalloc(plan, q_pre, k_pre, v_pre, o_pre, cache, stream=None):
    """qi_prefix_kv_build whose fp8 absmax partials use the library's static scratch."""
    import torch
    n = _live_numel(plan, QI_CALL_PREFIX)
    bf = torch.bfloat16
    _check(lib.qi_prefix_kv_build_noalloc(plan.handle, _ptr(q_pre, "q_pre", bf, n),
                                          _ptr(k_pre, "k_pre", bf, n), _ptr(v_pre, "v_pre", bf, n),
                                          _ptr(o_pre, "o_pre", bf, n),
                                          _ptr(cache, "cache", torch.uint8), cache.numel(),
                                          _stream(stream)), "qi_prefix_kv_build_noalloc")


def qi_denoise_attn_step(plan, cache, q_img, k_img, v_img, o_img, stream=None):
    import torch
    n = _live_numel(plan, QI_CALL_DENOISE)
    bf = torch.bfloat16
    _check(lib.qi_denoise_attn_step(plan.handle, _ptr(cache, "cache", torch.uint8), cache.numel(),
                                    _ptr(q_img, "q_img", bf, n), _ptr(k_img, "k_img", bf, n),
                                    _ptr(v_img, "v_img", bf, n), _ptr(o_img, "o_img", bf, n),
                                    _stream(stream)), "qi_denoise_attn_step")


def qi_attn_full_reference_step(plan, q_all, k_all, v_all, o_all, stream=None):
    import torch
    n = _live_numel(plan, QI_CALL_FULL)
    bf = torch.bfloat16
    _check(lib.qi_attn_full_reference_step(plan.handle, _ptr(q_all, "q_all", bf, n),
                                           _ptr(k_all, "k_all", bf, n),
                                           _ptr(v_all, "v_all", bf, n),
                                           _ptr(o_all, "o_all", bf, n), _stream(stream)),
           "qi_attn_full_reference_step")


def qi_plan_tile_map(plan, call, bm, bn):
    need = ctypes.c_size_t()
    st = lib.qi_plan_tile_map(plan.handle, call, bm, bn, None, 0, ctypes.byref(need))
    if st not in (QI_OK, QI_ERR_BUFFER_TOO_SMALL):
        _check(st, "qi_plan_tile_map")
    out = np.zeros(max(1, need.value), dtype=np.uint8)
    _check(lib.qi_plan_tile_map(plan.handle, call, bm, bn, out.ctypes.data_as(ctypes.c_void_p),
                                out.size, ctypes.byref(need)), "qi_plan_tile_map")
    return out[:need.value]


def qi_plan_kernel_tile(plan, call):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.qi_plan_kernel_tile(plan.handle, call, ctypes.byref(bm), ctypes.byref(bn)),
           "qi_plan_kernel_tile")
    return bm.value, bn.value


def qi_plan_launch_items(plan, call):
    """Launch schedule of a call: int32 array [workgroups, 6] of (request, head, first
    row as a position in the request's sequence, row count, first key, end key: the key
    chunk the workgroup visits); padding rows are -1."""
    need = ctypes.c_size_t()
    st = lib.qi_plan_launch_items(plan.handle, call, None, 0, ctypes.byref(need))
    if st not in (QI_OK, QI_ERR_BUFFER_TOO_SMALL):
        _check(st, "qi_plan_launch_items")
    out = np.zeros(max(QI_LAUNCH_ITEM_FIELDS, need.value), dtype=np.int32)
    _check(lib.qi_plan_launch_items(plan.handle, call, out.ctypes.data_as(ctypes.c_void_p),
                                    out.size, ctypes.byref(need)), "qi_plan_launch_items")
    return out[:need.value].reshape(-1, QI_LAUNCH_ITEM_FIELDS)


def qi_plan_cache_offset(plan, req, kv, head, tok):
    off = ctypes.c_size_t()
    _check(lib.qi_plan_cache_offset(plan.handle, req, kv, head, tok, ctypes.byref(off)),
           "qi_plan_cache_offset")
    return off.value


def qi_plan_pairs(plan, call):
    n = ctypes.c_int64()
    _check(lib.qi_plan_pairs(plan.handle, call, ctypes.byref(n)), "qi_plan_pairs")
    return n.value


def useful_flops(plan, call):
    """4 * D * H * allowed pairs of the call over the wave."""
    return 4 * plan.head_dim * plan.n_heads * qi_plan_pairs(plan, call)


def allocate(plan, device="cuda", stream=None):
    """Allocate one cache arena and the workspace for a plan, and upload the workspace.
    Returns (cache, workspace) uint8 device tensors."""
    import torch
    cache = torch.empty(max(1, plan.cache_bytes), dtype=torch.uint8, device=device)
    ws = torch.empty(max(256, plan.workspace_bytes), dtype=torch.uint8, device=device)
    qi_plan_upload(plan, ws, stream)
    return cache, ws
