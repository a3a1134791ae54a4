"""Writes generated expert weights into host or device buffers in the cache-entry layout.

The entry layout is the library's documented one (include/moe_cache.h):
[W_gate f x d][W_up f x d][W_down d x f], each row-major, one entry per
(layer, expert); for MXFP4 weights, [codes of W_gate][codes of W_up][codes of
W_down][scales of W_gate][scales of W_up][scales of W_down], each matrix in tiles
of 16 rows x 128 elements (gen/gen.c gives the byte offsets).  This module only
places generated values; it computes nothing of the layer.
"""
import ctypes

import numpy as np

from . import TAG_WG, TAG_WU, TAG_WD, MXFP4, fill_segments_ptr, fill_mxfp4_tiled_ptr
from .configs import wg_index, wd_index


def _fill_mxfp4_entries(w, pairs, dst_ptr, stride_bytes):
    d, f = w.d, w.f
    fd = f * d
    code_base = {"g": 0, "u": fd // 2, "d": fd}
    scale_base = {"g": 3 * fd // 2, "u": 3 * fd // 2 + fd // 32, "d": 3 * fd // 2 + 2 * fd // 32}
    base = np.arange(len(pairs), dtype=np.int64) * stride_bytes
    for tag, key, rows, K, index in ((TAG_WG, "g", f, d, wg_index), (TAG_WU, "u", f, d, wg_index),
                                     (TAG_WD, "d", d, f, wd_index)):
        i0 = np.array([index(w, l, e) for l, e in pairs], dtype=np.uint64)
        fill_mxfp4_tiled_ptr(w.seed, tag, i0, rows, K, w.w_sd, dst_ptr, base + code_base[key],
                             dst_ptr, base + scale_base[key])


def fill_entries_ptr(w, pairs, dst_ptr, entry_stride_elems):
    """Entry q of dst (host address) <- weights of pairs[q] = (layer, expert)."""
    pairs = list(pairs)
    if not pairs:
        return
    if w.dtype == MXFP4:
        _fill_mxfp4_entries(w, pairs, dst_ptr, entry_stride_elems * w.elem)
        return
    fd = w.f * w.d
    base = np.arange(len(pairs), dtype=np.int64) * entry_stride_elems
    gidx = np.array([wg_index(w, l, e) for l, e in pairs], dtype=np.uint64)
    didx = np.array([wd_index(w, l, e) for l, e in pairs], dtype=np.uint64)
    fill_segments_ptr(w.seed, TAG_WG, gidx, fd, w.w_sd, w.dtype, dst_ptr, base)
    fill_segments_ptr(w.seed, TAG_WU, gidx, fd, w.w_sd, w.dtype, dst_ptr, base + fd)
    fill_segments_ptr(w.seed, TAG_WD, didx, fd, w.w_sd, w.dtype, dst_ptr, base + 2 * fd)


def torch_dtype(w):
    import torch
    return torch.float32 if w.elem == 4 else torch.uint8 if w.dtype == MXFP4 else torch.bfloat16


def fill_device_entries(w, pairs, arena, slots, chunk=16, staging=None):
    """arena[slots[q]] <- entry of pairs[q]; arena is a device tensor [S, entry_elems].

    Generation happens on the host into a pinned staging buffer, chunk entries at a time."""
    import torch
    pairs, slots = list(pairs), list(slots)
    n_el = w.entry_elems
    if staging is None:
        staging = torch.empty((chunk, n_el), dtype=arena.dtype, pin_memory=True)
    for c0 in range(0, len(pairs), chunk):
        sub = pairs[c0:c0 + chunk]
        fill_entries_ptr(w, sub, staging.data_ptr(), n_el)
        torch.cuda.synchronize()
        for q, s in enumerate(slots[c0:c0 + chunk]):
            arena[s].copy_(staging[q], non_blocking=True)
        torch.cuda.synchronize()


def device_arena_all_experts(w, layer=0):
    """Device arena with all E experts of `layer` resident at slot e (identity slots)."""
    import torch
    arena = torch.empty((w.E, w.entry_elems), dtype=torch_dtype(w), device="cuda")
    fill_device_entries(w, [(layer, e) for e in range(w.E)], arena, range(w.E))
    return arena


class PinnedHostBuffer:
    """Page-locked host memory of an exact size (hipHostMalloc; torch's pinned allocator
    rounds large requests up to a power of two).  Freed with hipHostFree on close/GC."""

    def __init__(self, nbytes):
        import torch  # noqa: F401  (the HIP runtime is the one torch loaded)
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                            ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [ctypes.c_void_p]
        ptr = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(ptr), int(nbytes), 0)
        if rc != 0 or not ptr.value:
            raise MemoryError(f"hipHostMalloc({nbytes}) failed with status {rc}")
        self.ptr, self.nbytes = ptr.value, int(nbytes)

    def data_ptr(self):
        return self.ptr

    def close(self):
        if self.ptr:
            self._hip.hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HostPool(PinnedHostBuffer):
    """Pinned host pool of L*E entries, layer-major: entry (l, e) at l*E + e."""

    def __init__(self, w):
        super().__init__(w.L * w.E * w.entry_bytes)
        self.w = w

    def entry_ptr(self, i):
        return self.ptr + i * self.w.entry_bytes


def host_pool(w):
    """Pinned host pool holding every (layer, expert) entry of workload w."""
    pool = HostPool(w)
    step = 64
    pairs = [(l, e) for l in range(w.L) for e in range(w.E)]
    for c0 in range(0, len(pairs), step):
        fill_entries_ptr(w, pairs[c0:c0 + step], pool.entry_ptr(c0), w.entry_elems)
    return pool
