"""GPU parity of double-buffered layer streaming: layer_stream_prefetch copies a layer's
expert block from the pinned host pool into one of two device buffers on a copy stream,
ordered against the compute stream by events; the copies are byte-exact and every streamed
layer's output equals the oracle on that layer's experts."""
import ctypes

import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import PinnedHostBuffer, host_pool, torch_dtype
import oracle
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, bf16_tol, dev, oracle_table, x_device

pytestmark = pytest.mark.gpu


def _recorded_event(stream):
    """A torch event whose HIP handle exists (recorded once), so it can cross the C ABI."""
    ev = torch.cuda.Event()
    ev.record(stream)
    return ev


def _host_bytes(ptr, n):
    return np.ctypeslib.as_array((ctypes.c_uint8 * n).from_address(ptr)).copy()


@pytest.mark.parametrize("nbytes,n_chunks", [(0, 3), (1, 1), (10, 16), (1000003, 7),
                                             (4 << 20, 1)])
def test_prefetch_copies_bytes_exactly(nbytes, n_chunks):
    """Empty, one-byte, more chunks than bytes, a ragged last chunk and one whole copy: the
    destination holds the source bytes and nothing past them is written; the done event
    covers the whole copy."""
    host = PinnedHostBuffer(max(nbytes, 1))
    src = np.random.default_rng(nbytes).integers(0, 256, size=max(nbytes, 1), dtype=np.uint8)
    ctypes.memmove(host.ptr, src.ctypes.data, src.size)
    dst = torch.full((max(nbytes, 1) + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    copy = torch.cuda.Stream()
    done = _recorded_event(copy)
    torch.cuda.synchronize()
    moe.layer_stream_prefetch(host.ptr, dst, nbytes, n_chunks, copy, None, done)
    done.synchronize()
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got[:nbytes], src[:nbytes])
    assert (got[nbytes:] == 0xAB).all()
    host.close()


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("T", [3, 96])
def test_streamed_layers_equal_oracle(T, dtype):
    """Four layers through two device buffers: the copy of layer l+1 (5 chunks) waits, through
    wait_before, for the compute of layer l-1 to release its buffer, and the compute of layer
    l waits for its copy's done event.  Every layer's routing equals the oracle's and its
    output is within the bf16-weight tolerance of the oracle on that layer's experts (T=3
    streams the weights, T=96 takes the grouped GEMM); the buffers end holding the last two
    layers' blocks byte for byte."""
    w = configs.Workload("stream_small", seed=71 + T, T=T, d=256, E=16, k=4, f=128,
                         dtype=dtype, L=4, alpha=0.5)
    pool = host_pool(w)
    layer_bytes = w.E * w.entry_bytes
    bufs = [torch.empty((w.E, w.entry_elems), dtype=torch_dtype(w), device="cuda")
            for _ in range(2)]
    xs = [configs.gen_x(w, l) for l in range(w.L)]
    lgs = [configs.gen_logits(w, layer=l) for l in range(w.L)]
    xs_d = [x_device(w, x) for x in xs]
    lgs_d = [dev(lg) for lg in lgs]
    layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, dtype=w.act_dtype, y_dtype=moe.MOE_F32,
                       w_dtype=w.dtype) for _ in range(w.L)]
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [_recorded_event(copy) for _ in range(w.L)]
    free = [_recorded_event(comp) for _ in range(2)]
    torch.cuda.synchronize()
    moe.layer_stream_prefetch(pool.entry_ptr(0), bufs[0], layer_bytes, 5, copy, None, ready[0])
    for l in range(w.L):
        if l + 1 < w.L:
            nb = (l + 1) % 2
            moe.layer_stream_prefetch(pool.entry_ptr((l + 1) * w.E), bufs[nb], layer_bytes, 5,
                                      copy, free[nb] if l >= 1 else None, ready[l + 1])
        comp.wait_event(ready[l])
        layers[l].forward(xs_d[l], lgs_d[l], bufs[l % 2], w.entry_bytes, stream=comp)
        free[l % 2].record(comp)
    torch.cuda.synchronize()
    for l in range(w.L):
        used = sorted(set(oracle.route(lgs[l], w.k)[0].ravel().tolist()))
        ids, _, ref = oracle.moe_layer(xs[l], lgs[l], w.k, oracle_table(w, used, layer=l))
        np.testing.assert_array_equal(layers[l].ids.cpu().numpy(), ids)
        assert_close(layers[l].out.cpu().numpy(), ref, bf16_tol(ref), f"streamed layer {l}")
        assert int(layers[l].status.item()) == 0
    for l in (w.L - 2, w.L - 1):
        got = bufs[l % 2].view(torch.uint8).reshape(-1).cpu().numpy()
        np.testing.assert_array_equal(got, _host_bytes(pool.entry_ptr(l * w.E), layer_bytes))
    pool.close()
