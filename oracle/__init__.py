"""Reference oracle for the routed-MoE layer and its LRU expert cache.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (``expert_ffn_cache_amd``) and never imports it.  The C part
(``moe_oracle.c``) is the plain, double-precision definition of the layer; the
LRU simulator (``lru_sim.py``) is a sequential loop.
"""
import ctypes
import os

import numpy as np

from . import _build
from .lru_sim import LruSim, CapacityError, StaticPlacement, qstar  # noqa: F401

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.lib_path()
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.oracle_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_router_logits.restype = None
        L.oracle_route.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_route.restype = None
        L.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_permute.restype = i32
        L.oracle_expert_ffn.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32, vp, vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_moe_layer.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, i32,
                                       vp, vp, vp, vp]
        L.oracle_moe_layer.restype = None
        L.oracle_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.oracle_combine.restype = None
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = None
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("oracle takes fp32 arrays or bf16 bit patterns (uint16)")


def router_logits(x, wr):
    x = np.ascontiguousarray(x, dtype=np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, d = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_router_logits(_p(x), _p(wr), T, d, E, _p(out))
    return out


def route(logits, k):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_route(_p(lg), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids, E):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    if lib().oracle_permute(_p(ids), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv)) != 0:
        raise ValueError("expert id out of range")
    return counts, offsets, perm, inv


# FP4 E2M1 magnitudes by the low three code bits (OCP Microscaling Formats (MX) v1.0, the
# FP4 element table): exponent bits 2:1 with bias 1, mantissa bit 0, no infinities or NaN.
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_dequant(codes, scales):
    """Exact values of MXFP4 rows (float64 [R, K]) from codes [R, K/2] and scales [R, K/32].

    OCP MX v1.0: a block of 32 elements shares the scale 2^(s - 127) (E8M0, s = 255 is NaN
    and not used here); element = (-1)^(code bit 3) * E2M1 magnitude * scale.  Element 2j
    of a row is the low nibble of code byte j, element 2j + 1 the high nibble (the layout
    the library documents for MXFP4 entries)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, half = codes.shape
    q = np.empty((R, 2 * half), dtype=np.uint8)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    if np.any(scales == 255):
        raise ValueError("E8M0 NaN scale")
    # value of each of the 16 codes: sign bit 3, E2M1 magnitude from bits 2:0
    code_value = np.array([(-1.0 if c & 8 else 1.0) * _E2M1[c & 7] for c in range(16)])
    block = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return (code_value[q].reshape(R, -1, 32) * block[:, :, None]).reshape(R, 2 * half)


class ExpertTable:
    """Per-expert weight pointers (keeps the arrays alive).  experts: {e: (wg, wu, wd)}."""

    def __init__(self, E, experts):
        self.E = E
        self.keep = []
        self.wg = (ctypes.c_void_p * E)()
        self.wu = (ctypes.c_void_p * E)()
        self.wd = (ctypes.c_void_p * E)()
        self.dtype = None
        for e, (g, u, dn) in experts.items():
            g, u, dn = (np.ascontiguousarray(a) for a in (g, u, dn))
            self.keep += [g, u, dn]
            self.wg[e] = g.ctypes.data
            self.wu[e] = u.ctypes.data
            self.wd[e] = dn.ctypes.data
            self.dtype = _dtype_code(g)
            self.f, self.d = g.shape


def expert_ffn(x, ids, table, assign):
    """y[q] = FFN_{ids.flat[a]}(x[a // k]) for a in assign; float64 [len(assign), d]."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    assign = np.ascontiguousarray(assign, dtype=np.int32)
    d, f = table.d, table.f
    y = np.empty((len(assign), d), dtype=np.float64)
    lib().oracle_expert_ffn(_p(x), _dtype_code(x), d, f, k, _p(ids), table.wg, table.wu, table.wd,
                            table.dtype, len(assign), _p(assign), _p(y))
    return y


def moe_layer(x, logits, k, table, tokens=None):
    """Route all tokens and compute out[q] for q over `tokens` (default: all).

    Returns (ids [T,k] int32, w [T,k] float64, out [len(tokens), d] float64)."""
    x = np.ascontiguousarray(x)
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    d, f = table.d, table.f
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    out = np.empty((len(tokens), d), dtype=np.float64)
    lib().oracle_moe_layer(_p(x), _dtype_code(x), _p(lg), T, d, E, k, f, table.wg, table.wu,
                           table.wd, table.dtype, len(tokens), _p(tokens), _p(ids), _p(w), _p(out))
    return ids, w, out


def combine(yperm, inv, w):
    yperm = np.ascontiguousarray(yperm, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    inv = np.ascontiguousarray(inv, dtype=np.int32)
    T, k = w.shape
    d = yperm.shape[1]
    out = np.empty((T, d), dtype=np.float64)
    lib().oracle_combine(_p(yperm), _p(inv), _p(w), T, k, d, _p(out))
    return out


def set_threads(n):
    """Threads the oracle's parallel loops use from now on (1 = single core)."""
    lib().oracle_set_threads(int(n))


def max_threads():
    return int(lib().oracle_max_threads())
