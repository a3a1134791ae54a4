"""Python binding of libmoecache.so (MI355X routed-MoE layer with a device LRU expert cache).

Argument marshalling only: every function here forwards to the C entry point
of the same name in ``include/moe_cache.h``; every step of the layer runs in
the library's HIP kernels.  Pointer arguments accept a ``torch.Tensor`` (its
``data_ptr()``), a raw integer address, or ``None`` (NULL).  Stream arguments
accept a ``torch.cuda.Stream``, a raw ``hipStream_t`` integer, or ``None``
(torch's current stream).  A non-zero status raises :class:`MoeError`.

There is no fallback: if the library cannot be loaded or built, importing a
function fails.
"""
import ctypes
import os

from . import _build

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_ECAPACITY = -4
MOE_ERANGE = -5
MOE_ETOOBIG = -6
MOE_ETIMEOUT = -7

MOE_F32 = 0
MOE_BF16 = 1
MOE_MXFP4 = 2

MOE_PATH_AUTO = 0
MOE_PATH_GEMV = 1
MOE_PATH_GEMM = 2

EXPORTS = [
    "moe_strerror", "moe_abi_version", "moe_router_logits", "moe_route",
    "moe_permute_workspace_bytes", "moe_permute", "moe_route_permute", "moe_entry_bytes",
    "moe_expert_ffn_workspace_bytes",
    "moe_expert_ffn", "moe_expert_ffn_noalloc", "moe_expert_ffn_noalloc_max_bytes",
    "moe_combine", "moe_decode_token_workspace_bytes", "moe_decode_token", "cache_init", "cache_lookup_update",
    "cache_lookup_update_split", "cache_fill",
    "cache_fill_device", "cache_fill_masks", "cache_resize", "layer_stream_prefetch", "moe_hbm_read_probe", "moe_copy_probe",
]


class MoeError(RuntimeError):
    def __init__(self, name, status):
        super().__init__(f"{name}: {strerror(status)} (status {status})")
        self.status = status


class moe_cache_t(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("E", ctypes.c_int32), ("S", ctypes.c_int32),
        ("pool_entries", ctypes.c_int32), ("entry_bytes", ctypes.c_size_t),
        ("slot_of", ctypes.c_void_p), ("key_of", ctypes.c_void_p), ("stamp", ctypes.c_void_p),
        ("clock", ctypes.c_void_p), ("stats", ctypes.c_void_p), ("status", ctypes.c_void_p),
        ("arena", ctypes.c_void_p), ("host_pool", ctypes.c_void_p),
    ]


class moe_fill_t(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("expert", ctypes.c_int32), ("evicted_key", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libmoecache.so (built in-tree with hipcc if it is not there yet)."""
    global _lib
    if _lib is None:
        path = _build.lib_path()
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        i32, vp, sz, cp = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_char_p
        sig = {
            "moe_strerror": ([i32], cp),
            "moe_abi_version": ([], i32),
            "moe_router_logits": ([vp, vp, i32, i32, i32, i32, vp, vp], i32),
            "moe_route": ([vp, i32, i32, i32, vp, vp, vp], i32),
            "moe_permute_workspace_bytes": ([i32, i32, i32], sz),
            "moe_permute": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp, vp], i32),
            "moe_route_permute": ([vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp], i32),
            "moe_entry_bytes": ([i32, i32, i32], sz),
            "moe_expert_ffn_workspace_bytes": ([i32, i32, i32, i32], sz),
            "moe_expert_ffn": ([vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, i32, vp, vp,
                                i32, vp, sz, vp, i32, i32, vp, vp], i32),
            "moe_expert_ffn_noalloc": ([vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, i32,
                                        vp, vp, i32, vp, i32, i32, vp, vp], i32),
            "moe_expert_ffn_noalloc_max_bytes": ([], sz),
            "moe_combine": ([vp, i32, vp, vp, i32, i32, i32, vp, vp], i32),
            "moe_decode_token_workspace_bytes": ([i32, i32], sz),
            "moe_decode_token": ([vp, vp, i32, i32, i32, i32, vp, vp, sz, i32, vp, i32, vp, vp, vp,
                                  sz, vp, vp, vp], i32),
            "cache_init": ([ctypes.POINTER(moe_cache_t), vp], i32),
            "cache_lookup_update": ([ctypes.POINTER(moe_cache_t), i32, vp, i32, i32, vp, vp, vp,
                                     vp], i32),
            "cache_lookup_update_split": ([ctypes.POINTER(moe_cache_t), i32, vp, i32, i32, i32, i32,
                                           vp, vp, vp, vp, vp], i32),
            "cache_fill": ([ctypes.POINTER(moe_cache_t), vp, i32, vp], i32),
            "cache_fill_device": ([ctypes.POINTER(moe_cache_t), vp, vp, i32, vp], i32),
            "cache_fill_masks": ([vp, vp, vp, i32, vp, vp, vp, vp], i32),
            "cache_resize": ([ctypes.POINTER(moe_cache_t), ctypes.POINTER(moe_cache_t), vp], i32),
            "layer_stream_prefetch": ([vp, vp, sz, i32, vp, vp, vp], i32),
            "moe_hbm_read_probe": ([vp, sz, vp, vp], i32),
            "moe_copy_probe": ([vp, vp, sz, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ev(ev):
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    return ev.cuda_event


def _check(name, rc):
    if rc != MOE_OK:
        raise MoeError(name, rc)


def strerror(status):
    return lib().moe_strerror(status).decode()


def abi_version():
    return lib().moe_abi_version()


def moe_router_logits(x, w_router, dtype, T, d, E, logits, stream=None):
    _check("moe_router_logits",
           lib().moe_router_logits(_p(x), _p(w_router), dtype, T, d, E, _p(logits), _s(stream)))


def moe_route(logits, T, E, k, topk_ids, topk_w, stream=None):
    _check("moe_route", lib().moe_route(_p(logits), T, E, k, _p(topk_ids), _p(topk_w), _s(stream)))


def moe_permute_workspace_bytes(T, k, E):
    return lib().moe_permute_workspace_bytes(T, k, E)


def moe_permute(topk_ids, T, k, E, counts, offsets, perm, inv, ws, ws_bytes, status=None,
                stream=None):
    _check("moe_permute", lib().moe_permute(_p(topk_ids), T, k, E, _p(counts), _p(offsets),
                                            _p(perm), _p(inv), _p(ws), ws_bytes, _p(status),
                                            _s(stream)))


def moe_route_permute(logits, T, E, k, topk_ids, topk_w, counts, offsets, perm, inv, ws, ws_bytes,
                      status=None, stream=None):
    _check("moe_route_permute", lib().moe_route_permute(
        _p(logits), T, E, k, _p(topk_ids), _p(topk_w), _p(counts), _p(offsets), _p(perm), _p(inv),
        _p(ws), ws_bytes, _p(status), _s(stream)))


def moe_entry_bytes(d, f, w_dtype):
    return lib().moe_entry_bytes(d, f, w_dtype)


def moe_expert_ffn_workspace_bytes(T, k, f, act_dtype):
    return lib().moe_expert_ffn_workspace_bytes(T, k, f, act_dtype)


def moe_expert_ffn(x, act_dtype, perm, offsets, T, k, E, d, f, expert_slot, arena, entry_stride,
                   w_dtype, expert_mask, slot_key, key_base, ws, ws_bytes, y_perm, y_dtype,
                   path=MOE_PATH_AUTO, status=None, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _p(x), act_dtype, _p(perm), _p(offsets), T, k, E, d, f, _p(expert_slot), _p(arena),
        entry_stride, w_dtype, _p(expert_mask), _p(slot_key), key_base, _p(ws), ws_bytes,
        _p(y_perm), y_dtype, path, _p(status), _s(stream)))


def moe_expert_ffn_noalloc(x, act_dtype, perm, offsets, T, k, E, d, f, expert_slot, arena,
                           entry_stride, w_dtype, expert_mask, slot_key, key_base, y_perm, y_dtype,
                           path=MOE_PATH_AUTO, status=None, stream=None):
    _check("moe_expert_ffn_noalloc", lib().moe_expert_ffn_noalloc(
        _p(x), act_dtype, _p(perm), _p(offsets), T, k, E, d, f, _p(expert_slot), _p(arena),
        entry_stride, w_dtype, _p(expert_mask), _p(slot_key), key_base, _p(y_perm), y_dtype, path,
        _p(status), _s(stream)))


def moe_expert_ffn_noalloc_max_bytes():
    return lib().moe_expert_ffn_noalloc_max_bytes()


def moe_combine(y_perm, y_dtype, inv, topk_w, T, k, d, out, stream=None):
    _check("moe_combine", lib().moe_combine(_p(y_perm), y_dtype, _p(inv), _p(topk_w), T, k, d,
                                            _p(out), _s(stream)))


def moe_decode_token_workspace_bytes(k, f):
    return lib().moe_decode_token_workspace_bytes(k, f)


def moe_decode_token(logits, x, E, k, d, f, expert_slot, arena, entry_stride, w_dtype, slot_key,
                     key_base, topk_ids, topk_w, ws, ws_bytes, out, status=None, stream=None):
    _check("moe_decode_token", lib().moe_decode_token(
        _p(logits), _p(x), E, k, d, f, _p(expert_slot), _p(arena), entry_stride, w_dtype,
        _p(slot_key), key_base, _p(topk_ids), _p(topk_w), _p(ws), ws_bytes, _p(out), _p(status),
        _s(stream)))


def cache_init(cache, stream=None):
    _check("cache_init", lib().cache_init(ctypes.byref(cache), _s(stream)))


def cache_lookup_update(cache, layer, topk_ids, T, k, expert_slot, fills, n_fills, stream=None):
    _check("cache_lookup_update", lib().cache_lookup_update(
        ctypes.byref(cache), layer, _p(topk_ids), T, k, _p(expert_slot), _p(fills), _p(n_fills),
        _s(stream)))


def cache_lookup_update_split(cache, layer, topk_ids, T, k, pcie_mbps, host_mbps, expert_slot,
                              fills, n_fills, host_mask, stream=None):
    _check("cache_lookup_update_split", lib().cache_lookup_update_split(
        ctypes.byref(cache), layer, _p(topk_ids), T, k, pcie_mbps, host_mbps, _p(expert_slot),
        _p(fills), _p(n_fills), _p(host_mask), _s(stream)))


def cache_fill(cache, fills_host, n_fills, copy_stream=None):
    _check("cache_fill", lib().cache_fill(ctypes.byref(cache), _p(fills_host), n_fills,
                                          _s(copy_stream)))


def cache_fill_device(cache, fills, n_fills, max_fills, stream=None):
    _check("cache_fill_device", lib().cache_fill_device(ctypes.byref(cache), _p(fills),
                                                        _p(n_fills), max_fills, _s(stream)))


def cache_fill_masks(expert_slot, fills, n_fills, E, hit_mask, miss_mask, status=None,
                     stream=None):
    _check("cache_fill_masks", lib().cache_fill_masks(
        _p(expert_slot), _p(fills), _p(n_fills), E, _p(hit_mask), _p(miss_mask), _p(status),
        _s(stream)))


def cache_resize(old_cache, new_cache, stream=None):
    _check("cache_resize", lib().cache_resize(ctypes.byref(old_cache), ctypes.byref(new_cache),
                                              _s(stream)))


def layer_stream_prefetch(host_src, dst, nbytes, n_chunks, copy_stream=None, wait_before=None,
                          done=None):
    _check("layer_stream_prefetch", lib().layer_stream_prefetch(
        _p(host_src), _p(dst), nbytes, n_chunks, _s(copy_stream), _ev(wait_before), _ev(done)))


def moe_hbm_read_probe(src, nbytes, sink, stream=None):
    _check("moe_hbm_read_probe", lib().moe_hbm_read_probe(_p(src), nbytes, _p(sink), _s(stream)))


def moe_copy_probe(src, dst, nbytes, stream=None):
    _check("moe_copy_probe", lib().moe_copy_probe(_p(src), _p(dst), nbytes, _s(stream)))
