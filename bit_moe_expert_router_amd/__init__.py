"""Routed mixture-of-experts layer on MI355X (gfx950).

Thin ctypes binding over ``libmoe.so`` (declared in ``include/moe.h``): argument
marshalling only, every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory and streams.  The functions keep the C-ABI's
names (``moe_route``, ``moe_forward``, ``set_expert_table`` ...) and take torch
tensors where the C side takes device pointers.

There is no fallback: if the HIP library is missing, importing this package
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_E_ARG, MOE_E_UNSUPPORTED, MOE_E_NOMEM, MOE_E_HIP, MOE_E_STATE = range(6)
MOE_WS_ERROR_OFFSET = 4  # byte offset of the workspace's int32 error word (moe.h)
MOE_WS_COUNTER_BYTES = 167936  # the workspace's leading counter region (moe.h)
MOE_ERR_ROUTING = 1
MOE_ERR_RANGE = 4
MOE_ERR_COMBINE = 8
_STATUS = {0: "MOE_OK", 1: "MOE_E_ARG", 2: "MOE_E_UNSUPPORTED", 3: "MOE_E_NOMEM",
           4: "MOE_E_HIP", 5: "MOE_E_STATE"}


class moe_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("scale_f16", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32)]


class moe_expert_ref(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


EXPORTS = ("moe_create", "moe_destroy", "moe_workspace_bytes", "moe_workspace_init",
           "set_expert_table", "moe_expert_table_device", "moe_set_shared", "moe_route",
           "moe_forward", "moe_forward_noalloc", "moe_rmsnorm_bf16", "moe_last_error",
           "moe_profile_enable", "moe_profile_read", "moe_host_arena_create",
           "moe_host_arena_destroy", "moe_cache_state_bytes", "moe_cache_init", "moe_cache_step",
           "moe_stack_layer", "moe_layer_forward", "moe_stream_read", "moe_profile_read_stats")
MOE_CACHE_LFU, MOE_CACHE_CLOCK = 0, 1


def _load():
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    # PyTorch first: libmoe.so and torch resolve the same HIP runtime soname, and
    # the process must use the runtime torch was built with, whichever module a
    # caller imports first
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.moe_create.argtypes = [ctypes.POINTER(moe_cfg), i32, ctypes.POINTER(vp)]
    lib.moe_destroy.argtypes = [vp]
    lib.moe_workspace_bytes.argtypes = [vp, i32]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_init.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.set_expert_table.argtypes = [vp, i32, ctypes.POINTER(moe_expert_ref), vp]
    lib.moe_expert_table_device.argtypes = [vp, i32]
    lib.moe_expert_table_device.restype = vp
    lib.moe_set_shared.argtypes = [vp, i32, vp, vp, vp]
    lib.moe_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_forward.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                ctypes.c_size_t, vp]
    lib.moe_forward_noalloc.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_rmsnorm_bf16.argtypes = [vp, vp, vp, i32, ctypes.c_float, vp, vp]
    lib.moe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.moe_stack_layer.argtypes = [vp, i32, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_layer_forward.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.moe_host_arena_create.argtypes = [ctypes.c_size_t, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.moe_host_arena_destroy.argtypes = [vp]
    lib.moe_cache_state_bytes.argtypes = [vp, i32]
    lib.moe_cache_state_bytes.restype = ctypes.c_size_t
    lib.moe_cache_init.argtypes = [vp, i32, i32, i32, ctypes.c_double,
                                   ctypes.POINTER(moe_expert_ref), vp, ctypes.c_size_t, vp,
                                   ctypes.c_size_t, vp]
    lib.moe_cache_step.argtypes = [vp, i32, vp, vp, vp]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_profile_enable.argtypes = [i32]
    lib.moe_profile_enable.restype = st
    lib.moe_profile_read.argtypes = [i32, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.moe_profile_read.restype = i32
    lib.moe_profile_read_stats.argtypes = [i32, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int64)]
    lib.moe_profile_read_stats.restype = i32
    for f in ("moe_create", "moe_destroy", "moe_workspace_init", "set_expert_table",
              "moe_set_shared", "moe_route", "moe_forward", "moe_forward_noalloc",
              "moe_rmsnorm_bf16", "moe_host_arena_create", "moe_host_arena_destroy",
              "moe_cache_init", "moe_cache_step", "moe_stack_layer", "moe_layer_forward",
              "moe_stream_read"):
        getattr(lib, f).restype = st
    return lib


lib = _load()


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.moe_last_error().decode()
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ C-ABI wrappers
def moe_create(hidden, inter, n_experts, top_k, bits, group, scale_f16, shared_inter,
               max_tokens, n_layers=1) -> int:
    cfg = moe_cfg(hidden, inter, n_experts, top_k, bits, group, int(scale_f16), shared_inter,
                  max_tokens)
    out = ctypes.c_void_p()
    _check(lib.moe_create(ctypes.byref(cfg), n_layers, ctypes.byref(out)), "moe_create")
    return out.value


def moe_destroy(ctx: int):
    _check(lib.moe_destroy(ctx), "moe_destroy")


def moe_workspace_bytes(ctx: int, n_tokens: int) -> int:
    return lib.moe_workspace_bytes(ctx, n_tokens)


def moe_workspace_init(ctx: int, ws, stream=None):
    _check(lib.moe_workspace_init(ctx, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_workspace_init")


def set_expert_table(ctx: int, layer: int, refs: Sequence[tuple], stream=None):
    """refs[e] = (gate_ptr, up_ptr, down_ptr) device addresses, logical order."""
    arr = (moe_expert_ref * len(refs))(*[moe_expert_ref(g, u, d) for g, u, d in refs])
    _check(lib.set_expert_table(ctx, layer, arr, _stream(stream)), "set_expert_table")


def moe_expert_table_device(ctx: int, layer: int) -> int:
    return lib.moe_expert_table_device(ctx, layer) or 0


def moe_set_shared(ctx: int, layer: int, gate, up, down):
    _check(lib.moe_set_shared(ctx, layer, _ptr(gate), _ptr(up), _ptr(down)), "moe_set_shared")


def moe_route(ctx: int, x_bf16, T: int, w_router, bias, topk_ids, topk_w, expert_offsets,
              sorted_pairs, pair_pos, ws, stream=None):
    _check(lib.moe_route(ctx, _ptr(x_bf16), T, _ptr(w_router), _ptr(bias), _ptr(topk_ids),
                         _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_pos),
                         _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_route")


def moe_forward(ctx: int, layer: int, x_bf16, T: int, topk_ids, topk_w, expert_offsets,
                sorted_pairs, out, pair_out, ws, stream=None):
    _check(lib.moe_forward(ctx, layer, _ptr(x_bf16), T, _ptr(topk_ids), _ptr(topk_w),
                           _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(out),
                           _ptr(pair_out), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)),
           "moe_forward")


def moe_layer_forward(ctx: int, layer: int, x_bf16, T: int, w_router, bias, topk_ids, topk_w,
                      expert_offsets, sorted_pairs, pair_pos, out, pair_out, ws, stream=None):
    _check(lib.moe_layer_forward(ctx, layer, _ptr(x_bf16), T, _ptr(w_router), _ptr(bias),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                                 _ptr(sorted_pairs), _ptr(pair_pos), _ptr(out), _ptr(pair_out),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_layer_forward")


def moe_forward_noalloc(ctx: int, layer: int, x_bf16, T: int, topk_ids, topk_w,
                        expert_offsets, sorted_pairs, out, pair_out, stream=None):
    _check(lib.moe_forward_noalloc(ctx, layer, _ptr(x_bf16), T, _ptr(topk_ids), _ptr(topk_w),
                                   _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(out),
                                   _ptr(pair_out), _stream(stream)),
           "moe_forward_noalloc")


def moe_host_arena_create(nbytes: int):
    """pinned host memory mapped for the device -> (host address, device address)"""
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib.moe_host_arena_create(nbytes, ctypes.byref(h), ctypes.byref(d)),
           "moe_host_arena_create")
    return h.value, d.value


def moe_host_arena_destroy(host: int):
    _check(lib.moe_host_arena_destroy(host), "moe_host_arena_destroy")


def moe_cache_state_bytes(ctx: int, slots: int) -> int:
    return lib.moe_cache_state_bytes(ctx, slots)


def moe_cache_init(ctx: int, layer: int, slots: int, policy: int, decay: float,
                   home: Sequence[tuple], slot_arena, slot_bytes: int, state, stream=None):
    """home[e] = (gate, up, down) addresses of expert e's home copy"""
    arr = (moe_expert_ref * len(home))(*[moe_expert_ref(g, u, d) for g, u, d in home])
    _check(lib.moe_cache_init(ctx, layer, slots, policy, decay, arr, _ptr(slot_arena), slot_bytes,
                              _ptr(state), state.numel() * state.element_size(),
                              _stream(stream)),
           "moe_cache_init")


def moe_cache_step(ctx: int, layer: int, expert_offsets, state, stream=None):
    _check(lib.moe_cache_step(ctx, layer, _ptr(expert_offsets), _ptr(state), _stream(stream)),
           "moe_cache_step")


def moe_last_error() -> str:
    return lib.moe_last_error().decode()


def moe_profile_enable(on: bool):
    _check(lib.moe_profile_enable(int(bool(on))), "moe_profile_enable")


def moe_profile_read(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} since the last read (waits for the events)"""
    names = ctypes.create_string_buffer(32 * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    n = (ctypes.c_int64 * max_kernels)()
    k = lib.moe_profile_read(max_kernels, names, ms, n)
    raw = names.raw
    return {raw[32 * i:32 * i + 32].split(b"\0")[0].decode(): (ms[i], n[i]) for i in range(k)}


def moe_profile_read_stats(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, median ms, typical mean ms, launches)} since the last
    read; the typical mean is the mean of the launches within twice the median"""
    names = ctypes.create_string_buffer(32 * max_kernels)
    ms = (ctypes.c_double * max_kernels)()
    med = (ctypes.c_double * max_kernels)()
    tm = (ctypes.c_double * max_kernels)()
    n = (ctypes.c_int64 * max_kernels)()
    k = lib.moe_profile_read_stats(max_kernels, names, ms, med, tm, n)
    raw = names.raw
    return {raw[32 * i:32 * i + 32].split(b"\0")[0].decode(): (ms[i], med[i], tm[i], n[i])
            for i in range(k)}


def moe_rmsnorm_bf16(ctx: int, resid, add, T: int, eps: float, y_bf16, stream=None):
    _check(lib.moe_rmsnorm_bf16(ctx, _ptr(resid), _ptr(add), T, eps, _ptr(y_bf16),
                                _stream(stream)),
           "moe_rmsnorm_bf16")


def moe_stack_layer(ctx: int, layer: int, resid, T: int, eps: float, w_router, bias, topk_ids,
                    topk_w, expert_offsets, sorted_pairs, pair_pos, xn_bf16, out, ws,
                    stream=None):
    _check(lib.moe_stack_layer(ctx, layer, _ptr(resid), T, eps, _ptr(w_router), _ptr(bias),
                               _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                               _ptr(sorted_pairs), _ptr(pair_pos), _ptr(xn_bf16), _ptr(out),
                               _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_stack_layer")


def moe_stream_read(src, nbytes: int, sink, stream=None):
    _check(lib.moe_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "moe_stream_read")


from .layer import MoELayer, RoutingBuffers  # noqa: E402,F401
