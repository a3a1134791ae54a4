"""Seeded synthetic inputs for the routed-MoE layer (test and benchmark infrastructure).

Shared by the oracle and by the GPU path's tests and benchmark.  Holds none of
the layer's arithmetic: every value is a function of (seed, tensor tag, logical
index) only, so the oracle can regenerate any single expert matrix by index.
The C implementation is ``gen/gen.c`` (SplitMix64 bits, twelve-uniform
Irwin-Hall normals); this module is a ctypes wrapper around it.
"""
import ctypes
import os

import numpy as np

from . import _build

# Tensor tags: every logical tensor of a workload gets its own stream.
TAG_X = 1
TAG_WR = 2
TAG_WG = 3
TAG_WU = 4
TAG_WD = 5
TAG_LOGIT = 6
TAG_RANK = 7
TAG_MSTAY = 8
TAG_MZIPF = 9
TAG_MCHOSEN = 10
TAG_MNOISE = 11
TAG_MRANK = 12
TAG_MISC = 13

F32 = 0
BF16 = 1
MXFP4 = 2  # weights only: OCP MX FP4 (E2M1 codes, one E8M0 scale per 32 elements)

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.lib_path()
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp, fl, db = ctypes.c_void_p, ctypes.c_float, ctypes.c_double
        L.gen_u64.argtypes = [u64, u64, u64]
        L.gen_u64.restype = u64
        L.gen_uniform.argtypes = [u64, u64, u64]
        L.gen_uniform.restype = db
        L.gen_normal.argtypes = [u64, u64, u64, fl]
        L.gen_normal.restype = fl
        L.gen_fill_normal.argtypes = [u64, u64, u64, i64, fl, i32, vp]
        L.gen_fill_normal.restype = None
        L.gen_fill_normal_segments.argtypes = [u64, u64, i64, vp, i64, fl, i32, vp, vp]
        L.gen_fill_normal_segments.restype = None
        L.gen_mxfp4_block.argtypes = [vp, vp, vp]
        L.gen_mxfp4_block.restype = None
        L.gen_fill_mxfp4_rows.argtypes = [u64, u64, i64, vp, i64, fl, vp, vp, vp, vp]
        L.gen_fill_mxfp4_rows.restype = None
        L.gen_fill_mxfp4_tiled.argtypes = [u64, u64, i64, vp, i64, i64, fl, vp, vp, vp, vp]
        L.gen_fill_mxfp4_tiled.restype = None
        L.gen_rank_perm.argtypes = [u64, u64, i32, vp]
        L.gen_rank_perm.restype = None
        L.gen_zipf_bias.argtypes = [u64, u64, i32, db, db, vp]
        L.gen_zipf_bias.restype = None
        L.gen_routing_logits.argtypes = [u64, u64, i32, i32, i32, vp, db, i32, vp]
        L.gen_routing_logits.restype = i64
        L.gen_markov_routing.argtypes = [u64, i32, i32, i32, i32, i32, db, db,
                                         u64, u64, u64, u64, u64, vp, vp]
        L.gen_markov_routing.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(seed, tag, i0, shape, sd=1.0, dtype=F32):
    """Elements i0 .. i0+prod(shape)-1 of stream (seed, tag); bf16 is returned as uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    lib().gen_fill_normal(seed, tag, i0, n, float(sd), dtype, _ptr(out))
    return out.reshape(shape)


def fill_normal_ptr(seed, tag, i0, n, sd, dtype, dst_ptr):
    """Fill n elements at raw host address dst_ptr (for pinned buffers)."""
    lib().gen_fill_normal(seed, tag, i0, int(n), float(sd), dtype, ctypes.c_void_p(dst_ptr))


def fill_segments_ptr(seed, tag, src_i0, seg_len, sd, dtype, dst_ptr, dst_off):
    """Fill len(src_i0) segments of seg_len elements into raw host address dst_ptr."""
    src = np.ascontiguousarray(src_i0, dtype=np.uint64)
    off = np.ascontiguousarray(dst_off, dtype=np.int64)
    lib().gen_fill_normal_segments(seed, tag, len(src), _ptr(src), int(seg_len), float(sd), dtype,
                                   ctypes.c_void_p(dst_ptr), _ptr(off))


def bf16_bits_to_f32(u16):
    """Exact upcast of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rank_perm(seed, tag, E):
    out = np.empty(E, dtype=np.int32)
    lib().gen_rank_perm(seed, tag, E, _ptr(out))
    return out


def zipf_bias(seed, tag, E, alpha, s=1.1):
    out = np.empty(E, dtype=np.float32)
    lib().gen_zipf_bias(seed, tag, E, float(alpha), float(s), _ptr(out))
    return out


def routing_logits(seed, tag, T, E, k, bias=None, min_gap=1e-3, max_attempts=64):
    """[T, E] fp32 router logits, N(0,1) (+ bias), with the top-k margin guard."""
    out = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r = lib().gen_routing_logits(seed, tag, T, E, k, None if b is None else _ptr(b),
                                 float(min_gap), max_attempts, _ptr(out))
    if r < 0:
        raise RuntimeError("routing_logits: a row kept a top-k gap below min_gap")
    return out


def markov_routing(seed, steps, L, B, E, k, p_stay=0.7, zipf_s=1.1):
    """Multi-step decode routing trace: (ids [steps,L,B,k] int32, logits [steps,L,B,E] fp32)."""
    ids = np.empty((steps, L, B, k), dtype=np.int32)
    logits = np.empty((steps, L, B, E), dtype=np.float32)
    lib().gen_markov_routing(seed, steps, L, B, E, k, float(p_stay), float(zipf_s),
                             TAG_MRANK, TAG_MSTAY, TAG_MZIPF, TAG_MCHOSEN, TAG_MNOISE,
                             _ptr(ids), _ptr(logits))
    return ids, logits


def mxfp4_block(values):
    """Quantise 32 fp32 values to MXFP4: (16 code bytes, scale byte) (see gen/gen.c)."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    assert v.shape == (32,)
    codes = np.zeros(16, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.uint8)
    lib().gen_mxfp4_block(v.ctypes.data, codes.ctypes.data, scale.ctypes.data)
    return codes, int(scale[0])


def fill_mxfp4_rows_ptr(seed, tag, row_i0, K, sd, codes_ptr, code_off, scales_ptr, scale_off):
    """Rows of K normals quantised to MXFP4 into raw buffers (byte offsets per row)."""
    row_i0 = np.ascontiguousarray(row_i0, dtype=np.uint64)
    code_off = np.ascontiguousarray(code_off, dtype=np.int64)
    scale_off = np.ascontiguousarray(scale_off, dtype=np.int64)
    lib().gen_fill_mxfp4_rows(seed, tag, len(row_i0), row_i0.ctypes.data, K, sd, codes_ptr,
                              code_off.ctypes.data, scales_ptr, scale_off.ctypes.data)


def fill_mxfp4_tiled_ptr(seed, tag, i0, R, K, sd, codes_ptr, code_base, scales_ptr, scale_base):
    """Matrices q of R x K normals (logical start i0[q]) quantised to MXFP4 in the library's
    tiled entry layout (see gen/gen.c), at byte offsets code_base[q] / scale_base[q]."""
    i0 = np.ascontiguousarray(i0, dtype=np.uint64)
    code_base = np.ascontiguousarray(code_base, dtype=np.int64)
    scale_base = np.ascontiguousarray(scale_base, dtype=np.int64)
    assert R % 16 == 0 and K % 32 == 0
    lib().gen_fill_mxfp4_tiled(seed, tag, len(i0), i0.ctypes.data, R, K, sd, codes_ptr,
                               code_base.ctypes.data, scales_ptr, scale_base.ctypes.data)


def mxfp4_rows(seed, tag, i0, R, K, sd):
    """R consecutive rows of K normals starting at logical index i0, quantised to MXFP4:
    (codes [R, K/2] uint8, scales [R, K/32] uint8)."""
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 32), dtype=np.uint8)
    rows = np.arange(R, dtype=np.uint64) * np.uint64(K) + np.uint64(i0)
    fill_mxfp4_rows_ptr(seed, tag, rows, K, sd, codes.ctypes.data,
                        np.arange(R, dtype=np.int64) * (K // 2), scales.ctypes.data,
                        np.arange(R, dtype=np.int64) * (K // 32))
    return codes, scales
