"""Thin ctypes binding of ``libmoe_w4a16.so`` (see ``include/moe_w4a16.h``).

Argument marshalling only: every step of the MoE path runs in the library's
HIP kernels.  Functions carry the C names; tensors are torch tensors on the
GPU (any object with ``data_ptr()`` works), ``None`` becomes NULL.  A nonzero
return code raises :class:`MoeError` with the library's message.  The
library must have been built (``python -m packed_bit_expert_amd.build``);
there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_w4a16.so")

ABI_VERSION = 1
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_SHAPE = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_ABI_MISMATCH = -5
ERR_HIP = -6
ERR_DEVICE_CHECK = -7

SCALE_E8M0_G32 = 0
SCALE_E4M3_G16 = 1

FLAG_PRENORM = 1 << 0
FLAG_FORCE_DECODE = 1 << 1
FLAG_FORCE_BATCHED = 1 << 2
FLAG_CHECK_IDS = 1 << 3
FLAG_SERIAL = 1 << 4
FLAG_W4A4 = 1 << 5

EXPORTS = [
    "moe_w4a16_abi_version", "moe_w4a16_last_error", "moe_w4a16_shape_supported",
    "moe_w4a16_workspace_bytes", "moe_w4a16_workspace_init", "moe_w4a16_forward",
    "moe_w4a16_forward_debug", "moe_w4a16_stack_forward", "moe_w4a16_dequant",
    "moe_w4a16_combine", "moe_w4a16_sort_pairs", "moe_w4a16_device_status",
    "moe_w4a16_stream_read", "moe_w4a16_delay", "moe_w4a16_timing_begin",
    "moe_w4a16_timing_end", "moe_w4a16_route", "moe_w4a16_forward_routed",
    "moe_w4a16_stack_forward_routed", "moe_w4a16_hybrid_create", "moe_w4a16_hybrid_destroy",
    "moe_w4a16_hybrid_forward", "moe_w4a16_hybrid_stats", "moe_w4a16_hybrid_last_requests",
    "moe_w4a16_decode_floor", "moe_w4a16_empty_launch", "moe_w4a16_read_burst",
    "moe_w4a16_forward_noalloc", "moe_w4a16_grid_barrier",
]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Cfg(C.Structure):
    _fields_ = [
        ("abi_version", C.c_int32), ("num_tokens", C.c_int32), ("hidden", C.c_int32),
        ("inter", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
        ("scale_fmt", C.c_int32), ("flags", C.c_uint32), ("tensor_scales", C.c_void_p),
        ("residual", C.c_void_p), ("prenorm_eps", C.c_float), ("reserved0", C.c_int32),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("stream", C.c_void_p),
    ]


KERNEL_KINDS = {1: "decode gate/up", 2: "decode down + combine", 3: "slot resolve",
                4: "batched gate/up GEMM", 5: "batched down GEMM", 6: "combine", 7: "sort",
                8: "dequant", 9: "stream read", 10: "workspace fill", 11: "delay",
                12: "router", 13: "pre-norm",
                14: "x to MXFP4", 15: "decode gate/up floor (loads only)",
                16: "decode down floor (loads only)", 17: "empty kernel", 18: "burst read",
                19: "grid barriers"}


class Dump(C.Structure):
    _fields_ = [("u", C.c_void_p), ("g", C.c_void_p), ("v", C.c_void_p), ("h", C.c_void_p),
                ("y", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m packed_bit_expert_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
        sig = {
            "moe_w4a16_abi_version": (C.c_int, []),
            "moe_w4a16_last_error": (C.c_char_p, []),
            "moe_w4a16_shape_supported": (C.c_int, [I32, I32]),
            "moe_w4a16_workspace_bytes": (SZ, [C.POINTER(Cfg)]),
            "moe_w4a16_workspace_init": (C.c_int, [P, SZ, P]),
            "moe_w4a16_forward": (C.c_int, [P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_forward_debug": (C.c_int, [P, P, P, P, P, P, C.POINTER(Cfg), C.POINTER(Dump)]),
            "moe_w4a16_forward_noalloc": (C.c_int, [P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_stack_forward": (C.c_int, [I32, P, P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_dequant": (C.c_int, [P, P, I32, I32, I32, P, P]),
            "moe_w4a16_combine": (C.c_int, [P, P, P, P, I32, I32, I32, P]),
            "moe_w4a16_sort_pairs": (C.c_int, [P, I32, I32, I32, P, P, P, P]),
            "moe_w4a16_device_status": (C.c_int, [P, C.POINTER(C.c_int32), P]),
            "moe_w4a16_stream_read": (C.c_int, [P, SZ, P, P]),
            "moe_w4a16_delay": (C.c_int, [C.c_uint32, P]),
            "moe_w4a16_decode_floor": (C.c_int, [I32, P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_empty_launch": (C.c_int, [I32, I32, P, P]),
            "moe_w4a16_read_burst": (C.c_int, [P, SZ, I32, P, P]),
            "moe_w4a16_grid_barrier": (C.c_int, [I32, I32, P, P]),
            "moe_w4a16_route": (C.c_int, [P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_forward_routed": (C.c_int, [P, P, P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_stack_forward_routed": (C.c_int, [I32, P, P, P, P, P, P, P, P, P,
                                                         C.POINTER(Cfg)]),
            "moe_w4a16_timing_begin": (C.c_int, [I32]),
            "moe_w4a16_timing_end": (C.c_int, [C.POINTER(C.c_float), C.POINTER(C.c_int32), I32]),
            "moe_w4a16_hybrid_create": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, I32, P, I32, I32,
                                                  C.POINTER(P)]),
            "moe_w4a16_hybrid_destroy": (C.c_int, [P]),
            "moe_w4a16_hybrid_forward": (C.c_int, [P, P, P, P, P, P, P, P, C.POINTER(Cfg)]),
            "moe_w4a16_hybrid_stats": (C.c_int, [P, C.POINTER(C.c_int64)]),
            "moe_w4a16_hybrid_last_requests": (C.c_int, [P, C.POINTER(C.c_int32),
                                                         C.POINTER(C.c_uint8), I32,
                                                         C.POINTER(C.c_int32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.moe_w4a16_abi_version() != ABI_VERSION:
            raise RuntimeError("libmoe_w4a16.so ABI version mismatch")
        _lib = L
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != OK:
        raise MoeError(rc, lib().moe_w4a16_last_error().decode())


def make_cfg(num_tokens, hidden=2048, inter=1536, num_experts=64, top_k=4,
             scale_fmt=SCALE_E8M0_G32, flags=0, tensor_scales=None, residual=None,
             prenorm_eps=1e-5, workspace=None, workspace_bytes=None, stream=0) -> Cfg:
    """Fill a cfg struct; ``stream`` 0 means the default stream, None means
    torch's current stream."""
    c = Cfg()
    c.abi_version = ABI_VERSION
    c.num_tokens = num_tokens
    c.hidden, c.inter = hidden, inter
    c.num_experts, c.top_k = num_experts, top_k
    c.scale_fmt = scale_fmt
    c.flags = flags
    c.tensor_scales = _p(tensor_scales)
    c.residual = _p(residual)
    c.prenorm_eps = prenorm_eps
    c.workspace = _p(workspace)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    c.workspace_bytes = workspace_bytes
    c.stream = _stream(stream) if stream != 0 else None
    return c


# -- the C entry points ------------------------------------------------------------------

def moe_w4a16_abi_version() -> int:
    return lib().moe_w4a16_abi_version()


def moe_w4a16_last_error() -> str:
    return lib().moe_w4a16_last_error().decode()


def moe_w4a16_shape_supported(hidden: int, inter: int) -> bool:
    return bool(lib().moe_w4a16_shape_supported(hidden, inter))


def moe_w4a16_workspace_bytes(cfg: Cfg) -> int:
    return lib().moe_w4a16_workspace_bytes(C.byref(cfg))


def moe_w4a16_workspace_init(workspace, nbytes: int, stream=0):
    _check(lib().moe_w4a16_workspace_init(_p(workspace), nbytes, None if stream == 0 else _stream(stream)))


def moe_w4a16_forward(x, expert_ids, route_w, packed_weights, scales, out, cfg: Cfg):
    _check(lib().moe_w4a16_forward(_p(x), _p(expert_ids), _p(route_w), _p(packed_weights),
                                   _p(scales), _p(out), C.byref(cfg)))


def moe_w4a16_forward_noalloc(x, expert_ids, route_w, packed_weights, scales, out, cfg: Cfg):
    _check(lib().moe_w4a16_forward_noalloc(_p(x), _p(expert_ids), _p(route_w),
                                           _p(packed_weights), _p(scales), _p(out), C.byref(cfg)))


def moe_w4a16_forward_debug(x, expert_ids, route_w, packed_weights, scales, out, cfg: Cfg,
                            u=None, g=None, v=None, h=None, y=None):
    d = Dump(_p(u), _p(g), _p(v), _p(h), _p(y))
    _check(lib().moe_w4a16_forward_debug(_p(x), _p(expert_ids), _p(route_w), _p(packed_weights),
                                         _p(scales), _p(out), C.byref(cfg), C.byref(d)))


def moe_w4a16_stack_forward(num_layers, x, expert_ids, route_w, packed_weights, scales,
                            tensor_scales, out, cfg: Cfg):
    _check(lib().moe_w4a16_stack_forward(num_layers, _p(x), _p(expert_ids), _p(route_w),
                                         _p(packed_weights), _p(scales), _p(tensor_scales),
                                         _p(out), C.byref(cfg)))


def moe_w4a16_dequant(nibbles, scales, rows, cols, scale_fmt, out, stream=0):
    _check(lib().moe_w4a16_dequant(_p(nibbles), _p(scales), rows, cols, scale_fmt, _p(out),
                                   None if stream == 0 else _stream(stream)))


def moe_w4a16_combine(y, route_w, residual, out, num_tokens, top_k, hidden, stream=0):
    _check(lib().moe_w4a16_combine(_p(y), _p(route_w), _p(residual), _p(out), num_tokens, top_k,
                                   hidden, None if stream == 0 else _stream(stream)))


def moe_w4a16_sort_pairs(expert_ids, num_tokens, top_k, num_experts, counts, offsets, perm,
                         stream=0):
    _check(lib().moe_w4a16_sort_pairs(_p(expert_ids), num_tokens, top_k, num_experts, _p(counts),
                                      _p(offsets), _p(perm), None if stream == 0 else _stream(stream)))


def moe_w4a16_device_status(workspace, stream=0) -> int:
    code = C.c_int32(0)
    rc = lib().moe_w4a16_device_status(_p(workspace), C.byref(code),
                                       None if stream == 0 else _stream(stream))
    if rc not in (OK, ERR_DEVICE_CHECK):
        _check(rc)
    return code.value


def moe_w4a16_stream_read(src, nbytes, sink, stream=0):
    _check(lib().moe_w4a16_stream_read(_p(src), nbytes, _p(sink),
                                       None if stream == 0 else _stream(stream)))


def moe_w4a16_delay(microseconds: int, stream=0):
    _check(lib().moe_w4a16_delay(microseconds, None if stream == 0 else _stream(stream)))


def moe_w4a16_decode_floor(num_layers, x, expert_ids, route_w, packed_weights, scales, sink,
                           cfg: Cfg):
    _check(lib().moe_w4a16_decode_floor(num_layers, _p(x), _p(expert_ids), _p(route_w),
                                        _p(packed_weights), _p(scales), _p(sink), C.byref(cfg)))


def moe_w4a16_empty_launch(workgroups, threads, sink, stream=0):
    _check(lib().moe_w4a16_empty_launch(workgroups, threads, _p(sink),
                                        None if stream == 0 else _stream(stream)))


def moe_w4a16_read_burst(src, nbytes, loads_per_lane, sink, stream=0):
    _check(lib().moe_w4a16_read_burst(_p(src), nbytes, loads_per_lane, _p(sink),
                                      None if stream == 0 else _stream(stream)))


def moe_w4a16_grid_barrier(workgroups, barriers, counter, stream=0):
    _check(lib().moe_w4a16_grid_barrier(workgroups, barriers, _p(counter),
                                        None if stream == 0 else _stream(stream)))


def moe_w4a16_timing_begin(capacity: int):
    _check(lib().moe_w4a16_timing_begin(capacity))


def moe_w4a16_timing_end(capacity: int):
    """Per-launch (milliseconds, MOE_KERNEL_* kind) lists, in launch order."""
    ms = (C.c_float * capacity)()
    kinds = (C.c_int32 * capacity)()
    n = lib().moe_w4a16_timing_end(ms, kinds, capacity)
    if n < 0:
        _check(n)
    return list(ms[:n]), list(kinds[:n])


def moe_w4a16_route(x, router_w, expert_bias, expert_ids, route_w, cfg: Cfg):
    _check(lib().moe_w4a16_route(_p(x), _p(router_w), _p(expert_bias), _p(expert_ids),
                                 _p(route_w), C.byref(cfg)))


def moe_w4a16_forward_routed(x, router_w, expert_bias, packed_weights, scales, out, expert_ids,
                             route_w, cfg: Cfg):
    _check(lib().moe_w4a16_forward_routed(_p(x), _p(router_w), _p(expert_bias),
                                          _p(packed_weights), _p(scales), _p(out),
                                          _p(expert_ids), _p(route_w), C.byref(cfg)))


def moe_w4a16_stack_forward_routed(num_layers, x, router_w, expert_bias, packed_weights, scales,
                                   tensor_scales, out, expert_ids, route_w, cfg: Cfg):
    _check(lib().moe_w4a16_stack_forward_routed(num_layers, _p(x), _p(router_w),
                                                _p(expert_bias), _p(packed_weights), _p(scales),
                                                _p(tensor_scales), _p(out), _p(expert_ids),
                                                _p(route_w), C.byref(cfg)))


# -- hybrid (partially resident) layers ---------------------------------------------

def moe_w4a16_hybrid_create(triplet_bytes, nibble_bytes, cache_bytes, staging_slots,
                            device_staging, max_experts, max_pairs) -> int:
    """Returns the opaque handle (an int)."""
    h = C.c_void_p()
    _check(lib().moe_w4a16_hybrid_create(int(triplet_bytes), int(nibble_bytes), int(cache_bytes),
                                         int(staging_slots), _p(device_staging), int(max_experts),
                                         int(max_pairs), C.byref(h)))
    return h.value


def moe_w4a16_hybrid_destroy(handle):
    _check(lib().moe_w4a16_hybrid_destroy(handle))


def _ptr_array(values):
    arr = (C.c_void_p * len(values))()
    for i, v in enumerate(values):
        arr[i] = v if v else None
    return arr


def moe_w4a16_hybrid_forward(handle, x, expert_ids, route_w, resident_w, resident_s, host_src,
                             out, cfg: Cfg):
    """resident_w / resident_s / host_src: sequences of E ints (device or
    host addresses, 0 for none)."""
    rw, rs, hs = _ptr_array(resident_w), _ptr_array(resident_s), _ptr_array(host_src)
    _check(lib().moe_w4a16_hybrid_forward(handle, _p(x), _p(expert_ids), _p(route_w),
                                          C.cast(rw, C.c_void_p), C.cast(rs, C.c_void_p),
                                          C.cast(hs, C.c_void_p), _p(out), C.byref(cfg)))


def moe_w4a16_hybrid_stats(handle):
    """{calls, hits, misses, h2d_bytes}"""
    st = (C.c_int64 * 4)()
    _check(lib().moe_w4a16_hybrid_stats(handle, st))
    return {"calls": st[0], "hits": st[1], "misses": st[2], "h2d_bytes": st[3]}


def moe_w4a16_hybrid_last_requests(handle, capacity=1024):
    ex = (C.c_int32 * capacity)()
    hit = (C.c_uint8 * capacity)()
    n = C.c_int32()
    _check(lib().moe_w4a16_hybrid_last_requests(handle, ex, hit, capacity, C.byref(n)))
    return list(ex[:n.value]), list(hit[:n.value])
