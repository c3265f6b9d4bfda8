"""ctypes binding of the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  Arrays are
numpy host arrays; BF16 values travel as their uint16 bit patterns.

Everything the oracle computes is defined in ``moe_oracle.c`` (fp64,
sequential sums, one round-to-nearest-even to BF16 at each point where the
MXFP4 model card "LFM2.5-24B-A2B -- Packed MXFP4 Inference" ("Model and
quantization", "Grouped top-4 expert execution") puts a BF16 output).
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

FMT_E8M0_G32 = 0
FMT_E4M3_G16 = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def _declare(L):
    P = C.c_void_p
    L.oracle_e2m1.restype = C.c_double
    L.oracle_e2m1.argtypes = [C.c_int]
    L.oracle_e8m0.restype = C.c_double
    L.oracle_e8m0.argtypes = [C.c_int]
    L.oracle_e4m3fn.restype = C.c_double
    L.oracle_e4m3fn.argtypes = [C.c_int]
    L.oracle_bf16_from_f64.restype = C.c_uint16
    L.oracle_bf16_from_f64.argtypes = [C.c_double]
    L.oracle_f64_from_bf16.restype = C.c_double
    L.oracle_f64_from_bf16.argtypes = [C.c_uint16]
    L.oracle_bf16_round_array.restype = None
    L.oracle_bf16_round_array.argtypes = [P, P, C.c_int64]
    L.oracle_dequant.restype = C.c_int
    L.oracle_dequant.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P]
    L.oracle_combine.restype = None
    L.oracle_combine.argtypes = [P, P, P, P, C.c_int, C.c_int, C.c_int]
    L.oracle_prenorm.restype = None
    L.oracle_prenorm.argtypes = [P, P, C.c_int, C.c_double]
    L.oracle_sort_pairs.restype = C.c_int
    L.oracle_sort_pairs.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P, P]
    L.oracle_moe_forward.restype = C.c_int
    L.oracle_moe_forward.argtypes = [
        C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
        P, P, P, P, P, P, P, C.c_int, C.c_double, P, P, P, P, P, P, C.c_int]
    L.oracle_moe_forward_w4a4.restype = C.c_int
    L.oracle_moe_forward_w4a4.argtypes = L.oracle_moe_forward.argtypes
    L.oracle_quant_mxfp4.restype = C.c_int
    L.oracle_quant_mxfp4.argtypes = [P, C.c_int, C.c_int, P, P]
    L.oracle_lru.restype = C.c_int
    L.oracle_lru.argtypes = [P, C.c_int, C.c_int, P]
    L.oracle_threads_available.restype = C.c_int
    L.oracle_threads_available.argtypes = []
    L.oracle_route.restype = C.c_int
    L.oracle_route.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, C.c_int, C.c_double,
                               P, P, P]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# -- formats -----------------------------------------------------------------

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(int(code))


def e8m0(e: int) -> float:
    return lib().oracle_e8m0(int(e))


def e4m3fn(c: int) -> float:
    return lib().oracle_e4m3fn(int(c))


def bf16_from_f64(values) -> np.ndarray:
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_round_array(_ptr(v), _ptr(out), v.size)
    return out


def f64_from_bf16(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(nibbles, scales, rows: int, cols: int, fmt: int) -> np.ndarray:
    nib = _c(nibbles, np.uint8)
    sc = _c(scales, np.uint8)
    out = np.empty((rows, cols), np.float64)
    rc = lib().oracle_dequant(_ptr(nib), _ptr(sc), rows, cols, fmt, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant rejected the arguments")
    return out


def combine(y, route_w, residual=None) -> np.ndarray:
    """y [T][K][H] bf16 bits, route_w [T][K] bf16 bits -> out [T][H] bf16 bits."""
    y = _c(y, np.uint16)
    w = _c(route_w, np.uint16)
    T, K, H = y.shape
    r = None if residual is None else _c(residual, np.uint16)
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine(_ptr(y), _ptr(w), _ptr(r), _ptr(out), T, K, H)
    return out


def prenorm(x, eps: float) -> np.ndarray:
    """Weightless RMS pre-norm of every row of x (BF16 bits [..., H])."""
    x = _c(x, np.uint16)
    out = np.empty_like(x)
    H = x.shape[-1]
    xr, orr = x.reshape(-1, H), out.reshape(-1, H)
    for r in range(xr.shape[0]):
        lib().oracle_prenorm(_ptr(xr[r]), _ptr(orr[r]), H, float(eps))
    return out


def sort_pairs(ids, num_experts: int):
    ids = _c(ids, np.int32)
    T, K = ids.shape
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    rc = lib().oracle_sort_pairs(_ptr(ids), T, K, num_experts, _ptr(counts), _ptr(offsets),
                                 _ptr(perm))
    if rc != 0:
        raise ValueError("oracle_sort_pairs rejected the ids")
    return counts, offsets, perm


def quant_mxfp4(v):
    """MXFP4 quantisation of BF16 rows (see oracle_quant_mxfp4): v [rows][cols]
    BF16 bits -> (codes [rows][cols/2] uint8, low nibble = even k;
    scales [rows][cols/32] E8M0 uint8)."""
    v = _c(v, np.uint16)
    if v.ndim == 1:
        v = v[None, :]
    rows, cols = v.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    if lib().oracle_quant_mxfp4(_ptr(v), rows, cols, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("oracle_quant_mxfp4: cols must be a multiple of 32")
    return codes, scales


def lru(keys, capacity: int) -> np.ndarray:
    """Hit (1) or miss (0) of each request of an LRU cache of `capacity`
    entries (see oracle_lru)."""
    k = _c(keys, np.int64)
    hit = np.zeros(k.size, np.uint8)
    if lib().oracle_lru(_ptr(k), k.size, int(capacity), _ptr(hit)) < 0:
        raise ValueError("oracle_lru: capacity must be >= 1")
    return hit


def lru_requests(ids, cpu_backed) -> list:
    """The cache requests of one call: the distinct CPU-backed experts of
    ids [T][K] in order of first appearance (token-major, slot order)."""
    seen, out = set(), []
    for e in np.asarray(ids).ravel().tolist():
        if cpu_backed[e] and e not in seen:
            seen.add(e)
            out.append(e)
    return out


def threads_available() -> int:
    return lib().oracle_threads_available()


def moe_forward(x, ids, route_w, nibbles, scales, *, hidden, inter, num_experts, fmt,
                tensor_scales=None, residual=None, prenorm=False, eps=1e-5,
                dumps=False, nthreads=0, w4a4=False):
    """One MoE layer on the CPU (the W4A4 layer when ``w4a4``: activations
    quantised to MXFP4 before each GEMV, MXFP4 weights only).

    x [T][H] bf16 bits; ids [T][K] int32; route_w [T][K] bf16 bits;
    nibbles / scales: sequences (length E) of per-expert uint8 arrays, or None
    for experts that are never selected; tensor_scales [E][2] float32 or None.
    Returns out [T][H] (bf16 bits), plus a dict of intermediate BF16 tensors
    (u, g, v, h, y) when ``dumps`` is true.
    """
    x = _c(x, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(route_w, np.uint16)
    T, H = x.shape
    K = ids.shape[1]
    assert H == hidden and ids.shape[0] == T and w.shape == ids.shape
    E, I = num_experts, inter
    keep = []
    nib_tab = (C.c_void_p * E)()
    sc_tab = (C.c_void_p * E)()
    for e in range(E):
        if nibbles[e] is None:
            continue
        a = _c(nibbles[e], np.uint8)
        s = _c(scales[e], np.uint8)
        keep += [a, s]
        nib_tab[e] = a.ctypes.data
        sc_tab[e] = s.ctypes.data
    for e in np.unique(ids):
        if nibbles[int(e)] is None:
            raise ValueError(f"expert {int(e)} selected but no weights given")
    ts = None if tensor_scales is None else _c(tensor_scales, np.float32)
    r = None if residual is None else _c(residual, np.uint16)
    out = np.empty((T, H), np.uint16)
    d = None
    if dumps:
        d = {"u": np.empty((T, H), np.uint16), "g": np.empty((T, K, I), np.uint16),
             "v": np.empty((T, K, I), np.uint16), "h": np.empty((T, K, I), np.uint16),
             "y": np.empty((T, K, H), np.uint16)}
    fn = lib().oracle_moe_forward_w4a4 if w4a4 else lib().oracle_moe_forward
    rc = fn(
        T, H, I, E, K, fmt, _ptr(x), _ptr(ids), _ptr(w),
        C.cast(nib_tab, C.c_void_p), C.cast(sc_tab, C.c_void_p), _ptr(ts), _ptr(r),
        1 if prenorm else 0, float(eps), _ptr(out),
        _ptr(d["u"]) if d else None, _ptr(d["g"]) if d else None, _ptr(d["v"]) if d else None,
        _ptr(d["h"]) if d else None, _ptr(d["y"]) if d else None, int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"oracle_moe_forward rejected the arguments (rc={rc})")
    return (out, d) if dumps else out


def route(x, router_w, bias=None, *, top_k, prenorm=False, eps=1e-5, logits=False):
    """Router of one layer (see oracle_route): x BF16 bits [T][H], router_w
    BF16 bits [E][H], bias float32 [E] or None.  Returns ids int32 [T][k] and
    route_w BF16 bits [T][k] (and the fp64 logits [T][E] if asked)."""
    x = np.ascontiguousarray(x, np.uint16)
    router_w = np.ascontiguousarray(router_w, np.uint16)
    T, H = x.shape
    E = router_w.shape[0]
    assert router_w.shape == (E, H)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    ids = np.zeros((T, top_k), np.int32)
    rw = np.zeros((T, top_k), np.uint16)
    lg = np.zeros((T, E), np.float64)
    rc = lib().oracle_route(T, H, E, top_k, _ptr(x), _ptr(router_w), _ptr(b), int(prenorm),
                            float(eps), _ptr(ids), _ptr(rw), _ptr(lg))
    if rc != 0:
        raise ValueError(f"oracle_route: bad arguments (k={top_k}, E={E})")
    return (ids, rw, lg) if logits else (ids, rw)
