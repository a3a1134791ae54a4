"""CPU-side checks of the C ABI: the library loads, exports every declared entry point, and
host-side argument validation returns the documented codes before touching the GPU."""
import ctypes
import os
import re

import pytest

import expert_ffn_cache_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_cache.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 15, names
    lib = moe.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe_cache.h but not exported"
    assert sorted(moe.EXPORTS) == names


def test_strerror_and_version():
    assert moe.strerror(moe.MOE_OK) == "ok"
    for code in (moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED, moe.MOE_EHIP, moe.MOE_ECAPACITY,
                 moe.MOE_ERANGE, moe.MOE_ETOOBIG, moe.MOE_ETIMEOUT):
        assert moe.strerror(code) not in ("ok", "unknown status")
    assert moe.abi_version() == 3


def test_entry_bytes():
    assert moe.moe_entry_bytes(4096, 2048, moe.MOE_MXFP4) == 3 * 4096 * 2048 * 17 // 32
    assert moe.moe_entry_bytes(4096, 2048, moe.MOE_BF16) == 3 * 4096 * 2048 * 2
    assert moe.moe_entry_bytes(256, 512, moe.MOE_F32) == 3 * 256 * 512 * 4
    assert moe.moe_entry_bytes(64, 64, 9) == 0


def test_workspace_sizes():
    assert moe.moe_permute_workspace_bytes(8192, 6, 256) >= 48 * 256 * 4
    assert moe.moe_permute_workspace_bytes(8192, 6, 256) % 256 == 0
    assert moe.moe_expert_ffn_workspace_bytes(8192, 6, 2048, moe.MOE_BF16) == 8192 * 6 * 2048 * 2
    assert moe.moe_expert_ffn_workspace_bytes(16, 2, 512, moe.MOE_F32) == 16 * 2 * 512 * 4
    # up to 16 tokens with bf16 activations: room for h as tagged 8-byte entries (4 bytes per
    # unit), which the one-launch MXFP4 path needs; above that the plain bf16 intermediate
    assert moe.moe_expert_ffn_workspace_bytes(16, 6, 2048, moe.MOE_BF16) == 16 * 6 * 2048 * 4
    assert moe.moe_expert_ffn_workspace_bytes(1, 6, 2048, moe.MOE_BF16) == 6 * 2048 * 4
    assert moe.moe_expert_ffn_workspace_bytes(17, 6, 2048, moe.MOE_BF16) == 17 * 6 * 2048 * 2


def _rc(fn, *args):
    return getattr(moe.lib(), fn)(*args)


def test_host_validation_codes():
    L = moe.lib()
    # k > E, E > 1024, k > 16, null pointers: rejected before any launch
    assert L.moe_route(None, 4, 8, 9, None, None, None) == moe.MOE_EINVAL
    assert L.moe_route(None, 4, 2000, 2, None, None, None) == moe.MOE_EINVAL
    assert L.moe_route(None, 4, 64, 17, None, None, None) == moe.MOE_EINVAL
    assert L.moe_route(None, 4, 64, 2, None, None, None) == moe.MOE_EINVAL
    assert L.moe_router_logits(None, None, moe.MOE_BF16, 4, 64, 8, None, None) == moe.MOE_EUNSUPPORTED
    assert L.moe_combine(None, 7, None, None, 4, 2, 64, None, None) == moe.MOE_EUNSUPPORTED
    # route + permute: the checks of both, before any launch
    rp = [None, 8, 256, 6, None, None, None, None, None, None, None, 0, None, None]
    assert L.moe_route_permute(*rp) == moe.MOE_EINVAL  # null counts/offsets
    rp_k = list(rp); rp_k[3] = 300
    assert L.moe_route_permute(*rp_k) == moe.MOE_EINVAL  # k > E
    assert L.moe_combine(None, moe.MOE_F32, None, None, 4, 2, 100, None, None) == moe.MOE_EINVAL
    # d, f must be multiples of 64; dtype pairs
    args = [None, moe.MOE_BF16, None, None, 8, 6, 256, 4096, 2048, None, None, 3 * 4096 * 2048 * 2,
            moe.MOE_BF16, None, None, 0, None, 0, None, moe.MOE_F32, 0, None, None]
    bad_d = list(args); bad_d[6] = 4000
    assert L.moe_expert_ffn(*bad_d) == moe.MOE_EINVAL
    mixed = list(args); mixed[1] = moe.MOE_F32
    assert L.moe_expert_ffn(*mixed) == moe.MOE_EUNSUPPORTED
    short = list(args); short[11] = 100
    assert L.moe_expert_ffn(*short) == moe.MOE_EINVAL
    assert L.moe_expert_ffn(*args) == moe.MOE_EINVAL  # null buffers
    # a workspace smaller than the plain intermediate (T*k*f bf16) is refused before any launch,
    # whatever the weights (aligned stand-in addresses: nothing is dereferenced on this path)
    for wdt, eb in ((moe.MOE_BF16, 3 * 4096 * 2048 * 2),
                    (moe.MOE_MXFP4, moe.moe_entry_bytes(4096, 2048, moe.MOE_MXFP4))):
        small = list(args); small[11] = eb; small[12] = wdt
        small[0] = small[2] = small[3] = small[10] = small[16] = small[18] = 1 << 20
        small[17] = 8 * 6 * 2048 * 2 - 1
        assert L.moe_expert_ffn(*small) == moe.MOE_EINVAL
    # MXFP4 weights: bf16 activations only; entries at least moe_entry_bytes; both paths
    mx = list(args); mx[12] = moe.MOE_MXFP4; mx[11] = moe.moe_entry_bytes(4096, 2048, moe.MOE_MXFP4)
    mx_short = list(mx); mx_short[11] -= 16
    assert L.moe_expert_ffn(*mx_short) == moe.MOE_EINVAL
    mx_f32 = list(mx); mx_f32[1] = moe.MOE_F32
    assert L.moe_expert_ffn(*mx_f32) == moe.MOE_EUNSUPPORTED
    for path in (moe.MOE_PATH_AUTO, moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM):
        mx_p = list(mx); mx_p[20] = path
        assert L.moe_expert_ffn(*mx_p) == moe.MOE_EINVAL  # accepted up to the null buffers
    # bf16 GEMM keeps 32-bit element offsets: an explicit GEMM request past 2^32 elements of
    # h (T*k*f) or of an entry (3*d*f) is refused; AUTO is accepted (weight-streaming path)
    big_t = list(args); big_t[4] = 400_000; big_t[20] = moe.MOE_PATH_GEMM
    assert L.moe_expert_ffn(*big_t) == moe.MOE_EUNSUPPORTED
    big_t[20] = moe.MOE_PATH_AUTO
    assert L.moe_expert_ffn(*big_t) == moe.MOE_EINVAL  # accepted up to the null buffers
    fits = list(args); fits[4] = 349_525; fits[20] = moe.MOE_PATH_GEMM  # T*k*f just under 2^32
    assert L.moe_expert_ffn(*fits) == moe.MOE_EINVAL
    big_w = list(args); big_w[7] = big_w[8] = 40_000; big_w[11] = 3 * 40_000 * 40_000 * 2
    big_w[20] = moe.MOE_PATH_GEMM
    assert L.moe_expert_ffn(*big_w) == moe.MOE_EUNSUPPORTED


def test_cache_host_validation():
    c = moe.moe_cache_t(2, 4, 8, 0, 64, 1, 1, 1, 1, 1, 1, 1, 1)  # dummy non-null addresses
    assert moe.lib().cache_lookup_update(ctypes.byref(c), 2, 1, 1, 1, 1, 1, 1, None) == moe.MOE_ERANGE
    assert moe.lib().cache_lookup_update(ctypes.byref(c), -1, 1, 1, 1, 1, 1, 1, None) == moe.MOE_ERANGE
    big = moe.moe_cache_t(2, 4, 5000, 0, 64, 1, 1, 1, 1, 1, 1, 1, 1)
    assert moe.lib().cache_init(ctypes.byref(big), None) == moe.MOE_EINVAL
    bad = (moe.moe_fill_t * 2)(moe.moe_fill_t(0, 0, 1, -1), moe.moe_fill_t(8, 0, 1, -1))
    assert moe.lib().cache_fill(ctypes.byref(c), ctypes.addressof(bad), 2, None) == moe.MOE_ERANGE
    bad[1] = moe.moe_fill_t(1, 2, 1, -1)
    assert moe.lib().cache_fill(ctypes.byref(c), ctypes.addressof(bad), 2, None) == moe.MOE_ERANGE
    # a record valid for (L, E) but past a short pool is rejected before anything is enqueued
    # (the descriptor's addresses are dummies: an accepted call would have to copy from them)
    short = moe.moe_cache_t(2, 4, 8, 5, 64, 1, 1, 1, 1, 1, 1, 1, 1)  # pool holds entries 0..4
    past = (moe.moe_fill_t * 2)(moe.moe_fill_t(0, 0, 1, -1), moe.moe_fill_t(1, 1, 1, -1))
    assert moe.lib().cache_fill(ctypes.byref(short), ctypes.addressof(past), 2, None) == moe.MOE_ERANGE
    nopool = moe.moe_cache_t(2, 4, 8, 0, 64, 1, 1, 1, 1, 1, 1, 1, 1)  # pool_entries = 0
    one = (moe.moe_fill_t * 1)(moe.moe_fill_t(0, 0, 0, -1))
    assert moe.lib().cache_fill(ctypes.byref(nopool), ctypes.addressof(one), 1, None) == moe.MOE_ERANGE
    assert moe.lib().layer_stream_prefetch(None, None, 16, 1, None, None, None) == moe.MOE_EINVAL
    # device-driven fills: aligned dummy addresses; max_fills = 0 returns before any launch
    ok = moe.moe_cache_t(2, 4, 8, 0, 64, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096)
    fd = moe.lib().cache_fill_device
    assert fd(ctypes.byref(ok), 4096, 4096, 0, None) == moe.MOE_OK
    assert fd(ctypes.byref(ok), 4096, 4096, -1, None) == moe.MOE_EINVAL
    assert fd(ctypes.byref(ok), None, 4096, 0, None) == moe.MOE_EINVAL
    assert fd(ctypes.byref(c), 4096, 4096, 0, None) == moe.MOE_EINVAL  # unaligned arena
    odd = moe.moe_cache_t(2, 4, 8, 0, 72, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096)
    assert fd(ctypes.byref(odd), 4096, 4096, 0, None) == moe.MOE_EINVAL  # entry_bytes % 16
    ls = moe.lib().cache_lookup_update_split
    args = [ctypes.byref(c), 0, 1, 1, 1, 57000, 30000, 1, 1, 1, 1, None]
    for i, v in ((5, -1), (6, -1)):
        bad = list(args); bad[i] = v
        assert ls(*bad) == moe.MOE_EINVAL
    both0 = list(args); both0[5] = 0; both0[6] = 0
    assert ls(*both0) == moe.MOE_EINVAL
    nomask = list(args); nomask[10] = None
    assert ls(*nomask) == moe.MOE_EINVAL
    badlayer = list(args); badlayer[1] = 2
    assert ls(*badlayer) == moe.MOE_ERANGE
    rs = moe.lib().cache_resize
    a = moe.moe_cache_t(2, 4, 8, 0, 64, 4096, 8192, 12288, 16, 32, 48, 1 << 20, 0)
    b = moe.moe_cache_t(2, 4, 4, 0, 64, 20480, 24576, 28672, 64, 80, 96, 1 << 21, 0)
    ovl = moe.moe_cache_t.from_buffer_copy(b)
    ovl.arena = (1 << 20) + 64  # inside a's arena
    assert rs(ctypes.byref(a), ctypes.byref(ovl), None) == moe.MOE_EINVAL
    otherE = moe.moe_cache_t.from_buffer_copy(b)
    otherE.E = 5
    assert rs(ctypes.byref(a), ctypes.byref(otherE), None) == moe.MOE_EINVAL
    shared = moe.moe_cache_t.from_buffer_copy(b)
    shared.slot_of = a.slot_of
    assert rs(ctypes.byref(a), ctypes.byref(shared), None) == moe.MOE_EINVAL
    noarena = moe.moe_cache_t.from_buffer_copy(b)
    noarena.arena = 0
    assert rs(ctypes.byref(a), ctypes.byref(noarena), None) == moe.MOE_EINVAL
    fm = moe.lib().cache_fill_masks
    assert fm(4096, 4096, 4096, 0, 4096, 4096, None, None) == moe.MOE_EINVAL     # E = 0
    assert fm(4096, 4096, 4096, 1025, 4096, 4096, None, None) == moe.MOE_EINVAL  # E > 1024
    assert fm(4096, None, 4096, 8, 4096, 4096, None, None) == moe.MOE_EINVAL


def test_python_binding_raises():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(0, 4, 8, 9, 0, 0, stream=0)
    assert ei.value.status == moe.MOE_EINVAL


def test_noalloc_ffn_limit_is_checked_on_the_host():
    """The no-allocation FFN's scratch limit (8 MiB) is checked before any HIP call: a request
    whose SwiGLU intermediate exceeds it returns MOE_ETOOBIG (no GPU needed)."""
    L = moe.lib()
    assert L.moe_expert_ffn_noalloc_max_bytes() == 8 << 20
    T, k, f = 2048, 4, 1024  # 2048 * 4 * 1024 * 2 bytes = 16 MiB
    assert moe.moe_expert_ffn_workspace_bytes(T, k, f, moe.MOE_BF16) > 8 << 20
    args = [None, moe.MOE_BF16, None, None, T, k, 16, 256, f, None, None, 3 * 256 * f * 2,
            moe.MOE_BF16, None, None, 0, None, moe.MOE_F32, moe.MOE_PATH_AUTO, None, None]
    assert L.moe_expert_ffn_noalloc(*args) == moe.MOE_ETOOBIG
    bad = list(args); bad[4] = -1
    assert L.moe_expert_ffn_noalloc(*bad) == moe.MOE_EINVAL


def test_decode_token_arguments_are_checked_on_the_host():
    """moe_decode_token rejects bad arguments and shapes it does not take before any HIP call
    (fake but 16-byte aligned addresses: nothing is dereferenced on these paths)."""
    L = moe.lib()
    hdr = 256  # the launch epoch word, then an 8-byte entry per unit of h at most
    assert moe.moe_decode_token_workspace_bytes(6, 2048) == hdr + 6 * 2048 * 8
    assert moe.moe_decode_token_workspace_bytes(0, 2048) == hdr
    A = 1 << 20  # stand-in address

    def call(E=256, k=6, d=4096, f=2048, logits=A, x=A, arena=A, stride=None, wdt=moe.MOE_BF16,
             ids=A, w=A, ws=A, ws_bytes=None, out=A):
        stride = 3 * d * f * 2 if stride is None else stride
        ws_bytes = moe.moe_decode_token_workspace_bytes(k, f) if ws_bytes is None else ws_bytes
        return L.moe_decode_token(logits, x, E, k, d, f, None, arena, stride, wdt, None, 0, ids,
                                  w, ws, ws_bytes, out, None, None)

    assert call(k=0) == moe.MOE_EINVAL
    assert call(k=17, E=1024) == moe.MOE_EINVAL
    assert call(E=4, k=5) == moe.MOE_EINVAL
    assert call(E=1025) == moe.MOE_EINVAL
    assert call(d=100) == moe.MOE_EINVAL
    assert call(f=96) == moe.MOE_EINVAL
    mx = moe.moe_entry_bytes(4096, 2048, moe.MOE_MXFP4)
    assert call(wdt=moe.MOE_MXFP4, f=2560, stride=mx * 2) == moe.MOE_EUNSUPPORTED  # f > 2048
    assert call(wdt=moe.MOE_MXFP4, d=4160, f=1024, stride=mx * 2) == moe.MOE_EUNSUPPORTED
    assert call(wdt=moe.MOE_MXFP4, k=9, f=1024, stride=mx) == moe.MOE_EUNSUPPORTED  # k > 8
    assert call(wdt=moe.MOE_MXFP4, stride=mx - 16) == moe.MOE_EINVAL
    assert call(wdt=moe.MOE_F32) == moe.MOE_EUNSUPPORTED
    assert call(d=8256) == moe.MOE_EUNSUPPORTED
    assert call(f=8256, k=1) == moe.MOE_EUNSUPPORTED
    assert call(k=16, E=256, f=2048) == moe.MOE_EUNSUPPORTED   # x and h past 64 KB of LDS
    assert call(stride=3 * 4096 * 2048 * 2 - 16) == moe.MOE_EINVAL
    assert call(stride=3 * 4096 * 2048 * 2 + 8) == moe.MOE_EINVAL
    assert call(x=None) == moe.MOE_EINVAL
    assert call(out=None) == moe.MOE_EINVAL
    assert call(ws=None) == moe.MOE_EINVAL
    assert call(x=A + 8) == moe.MOE_EINVAL
    assert call(ws_bytes=hdr) == moe.MOE_EINVAL
    assert call(logits=None, ids=None) == moe.MOE_EINVAL
    assert call(logits=None, w=None) == moe.MOE_EINVAL


def test_decode_token_supported_matches_the_library():
    """The binding's shape test for the one-launch layer agrees with the library's host checks
    over a grid of shapes and weight types: a call with no output pointer returns
    MOE_EUNSUPPORTED exactly where the shape test says no, MOE_EINVAL (shape passed, missing
    output) elsewhere; nothing is launched."""
    from expert_ffn_cache_amd.layer import decode_token_supported
    L = moe.lib()
    A = 1 << 20  # stand-in address, never dereferenced
    seen = {True: 0, False: 0}
    for wdt in (moe.MOE_BF16, moe.MOE_MXFP4, moe.MOE_F32):
        for k in (1, 6, 8, 9, 16):
            for d in (64, 2048, 4096, 4160, 8192, 8256):
                for f in (64, 1024, 2048, 2560, 4096, 8192):
                    ok = decode_token_supported(1, k, d, f, moe.MOE_BF16, wdt, moe.MOE_F32)
                    stride = ((max(moe.moe_entry_bytes(d, f, wdt), 16) + 15) // 16) * 16
                    rc = L.moe_decode_token(A, A, 1024, k, d, f, None, A, stride, wdt, None, 0,
                                            A, A, A, 1 << 30, None, None, None)
                    assert rc == (moe.MOE_EINVAL if ok else moe.MOE_EUNSUPPORTED), (wdt, k, d, f)
                    seen[ok] += 1
    assert seen[True] > 20 and seen[False] > 20
    assert not decode_token_supported(2, 6, 4096, 2048, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_F32)
    assert not decode_token_supported(1, 6, 4096, 2048, moe.MOE_F32, moe.MOE_BF16, moe.MOE_F32)
    assert not decode_token_supported(1, 6, 4096, 2048, moe.MOE_BF16, moe.MOE_BF16, moe.MOE_BF16)
