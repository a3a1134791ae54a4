"""Whole-layer GPU parity (route -> permute -> FFN -> combine) on the five workload shapes."""
import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import device_arena_all_experts
import oracle
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, f32_tol, bf16_tol, dev, x_device, oracle_table

pytestmark = pytest.mark.gpu


def _tiny_inputs(w):
    """x and router weight with the top-k margin guard applied to the fp64 router logits:
    a token row whose k-th/(k+1)-th gap is below 1e-3 is redrawn (next attempt index)."""
    wr = configs.gen_router_weight(w)
    x = configs.gen_x(w)
    for t in range(w.T):
        for attempt in range(1, 64):
            lg = np.sort(x[t].astype(np.float64) @ wr.astype(np.float64).T)[::-1]
            if lg[w.k - 1] - lg[w.k] >= 1e-3:
                break
            x[t] = gen.normal(w.seed, gen.TAG_X, configs.x_index(w, 0, attempt) + t * w.d, (w.d,))
    return x, wr


def test_tiny_fp32_layer_end_to_end():
    """All fp32: router logits, routing, grouping, fp32 SwiGLU experts, combine."""
    w = configs.TINY
    x, wr = _tiny_inputs(w)
    arena = device_arena_all_experts(w)
    L = MoeLayer(w.T, w.E, w.k, w.d, w.f, dtype=moe.MOE_F32, y_dtype=moe.MOE_F32)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    moe.moe_router_logits(dev(x), dev(wr), moe.MOE_F32, w.T, w.d, w.E, logits)
    out = L.forward(dev(x), logits, arena, w.entry_bytes)
    torch.cuda.synchronize()
    ref_lg = oracle.router_logits(x, wr)
    assert_close(logits.cpu().numpy(), ref_lg, 1e-5 * np.abs(ref_lg).max(), "router logits")
    ids, wt, ref = oracle.moe_layer(x, ref_lg, w.k, oracle_table(w, range(w.E)))
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    assert_close(L.w.cpu().numpy(), wt, 1e-5, "gate weights")
    assert_close(out.cpu().numpy(), ref, f32_tol(ref), "layer output")
    assert int(L.status.item()) == 0


def _run_layer(w, rotation=0, y_dtype=moe.MOE_F32, arena=None):
    x = configs.gen_x(w)
    lg = configs.gen_logits(w, rotation=rotation)
    if arena is None:
        arena = device_arena_all_experts(w)
    L = MoeLayer(w.T, w.E, w.k, w.d, w.f, dtype=w.act_dtype, y_dtype=y_dtype, w_dtype=w.dtype)
    L.forward(x_device(w, x), dev(lg), arena, w.entry_bytes)
    torch.cuda.synchronize()
    return x, lg, L, arena


@pytest.fixture(scope="module")
def decode_arena():
    w = configs.DECODE
    arena = device_arena_all_experts(w)
    yield arena
    del arena
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,alpha", [(1, 0.2), (8, 0.2), (64, 0.2), (16, 1.0), (64, 1.0)])
def test_decode_layer_full_size(T, alpha, decode_arena):
    """E=256, k=6, d=4096, f=2048, bf16, all experts resident: every output element.  Above
    8 tokens the experts are split by rows and the few-row launches loop over their items;
    alpha=1 (skewed routing) leaves most of those items without an expert."""
    w = configs.with_(configs.DECODE, T=T, alpha=alpha)
    x, lg, L, _ = _run_layer(w, arena=decode_arena)
    ids, wt, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, sorted(set(oracle.route(lg, w.k)[0].ravel().tolist()))))
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    assert_close(L.out.cpu().numpy(), ref, bf16_tol(ref), f"decode T={T} alpha={alpha}")
    assert int(L.status.item()) == 0


@pytest.mark.parametrize("alpha", [0.2, 1.0])
def test_prefill_layer_full_size_sampled(alpha, decode_arena):
    """T=8192 prefill (GEMM path): ids, counts, perm bit-exact for all tokens; outputs of
    sampled tokens (first, last, and spread over the most and least loaded experts)."""
    w = configs.with_(configs.PREFILL, alpha=alpha)
    # PREFILL uses its own seed; its weights differ from the decode arena's, so regenerate
    x, lg, L, arena = _run_layer(w)
    ids, wt = oracle.route(lg, w.k)
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    np.testing.assert_array_equal(L.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(L.perm.cpu().numpy(), perm)
    r = np.random.default_rng(int(alpha * 10))
    big = int(np.argmax(counts))
    toks = set([0, w.T - 1]) | set(r.choice(w.T, 10, replace=False).tolist())
    toks |= set((perm[offsets[big]:offsets[big + 1]][:4] // w.k).tolist())
    toks = np.array(sorted(toks), dtype=np.int32)
    need = sorted(set(ids[toks].ravel().tolist()))
    _, _, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, need), tokens=toks)
    out = L.out.cpu().numpy()[toks]
    assert_close(out, ref, bf16_tol(ref), f"prefill alpha={alpha}")
    assert int(L.status.item()) == 0
    del arena


@pytest.mark.parametrize("T,alpha", [(1, 0.2), (8, 0.2), (64, 1.0)])
def test_decode_layer_full_size_mxfp4(T, alpha):
    """The decode layer with MXFP4 experts (E=256, k=6, d=4096, f=2048, all experts
    resident; T=1 splits each strip over 4 waves, T=8 and 64 give each wave whole strips):
    every output element against the oracle on the exactly dequantised weights."""
    w = configs.with_(configs.DECODE, dtype=gen.MXFP4, T=T, alpha=alpha)
    x, lg, L, arena = _run_layer(w)
    ids, wt, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, sorted(set(oracle.route(lg, w.k)[0].ravel().tolist()))))
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    assert_close(L.out.cpu().numpy(), ref, bf16_tol(ref), f"decode mxfp4 T={T} alpha={alpha}")
    assert int(L.status.item()) == 0
    del arena


def test_prefill_layer_full_size_sampled_mxfp4():
    """T=8192 prefill with MXFP4 experts (grouped GEMM): routing and grouping bit-exact,
    outputs of sampled tokens (first, last, spread, and rows of the most loaded expert)."""
    w = configs.with_(configs.PREFILL, dtype=gen.MXFP4)
    x, lg, L, arena = _run_layer(w)
    ids, wt = oracle.route(lg, w.k)
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    np.testing.assert_array_equal(L.perm.cpu().numpy(), perm)
    r = np.random.default_rng(7)
    big = int(np.argmax(counts))
    toks = set([0, w.T - 1]) | set(r.choice(w.T, 6, replace=False).tolist())
    toks |= set((perm[offsets[big]:offsets[big + 1]][-3:] // w.k).tolist())
    toks = np.array(sorted(toks), dtype=np.int32)
    need = sorted(set(ids[toks].ravel().tolist()))
    _, _, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, need), tokens=toks)
    assert_close(L.out.cpu().numpy()[toks], ref, bf16_tol(ref), "prefill mxfp4")
    assert int(L.status.item()) == 0
    del arena


@pytest.mark.parametrize("T,E,f,dtype", [(8, 32, 256, gen.BF16), (24, 256, 256, gen.BF16),
                                         (48, 256, 256, gen.BF16), (300, 32, 256, gen.BF16),
                                         (8, 32, 256, gen.MXFP4), (8, 64, 2048, gen.MXFP4),
                                         (13, 64, 2048, gen.MXFP4), (300, 32, 256, gen.MXFP4)])
def test_layer_is_deterministic_and_graph_replayable(T, E, f, dtype):
    """Two eager runs are bit-identical; a captured graph replayed on new logits matches eager
    on every replay (one-item and looping weight-streaming launches, grouped GEMM; bf16 and
    MXFP4 experts, at f = 2048 both MXFP4 projections in one launch after its clearing
    kernel)."""
    w = configs.with_(configs.DECODE, T=T, E=E, d=512, f=f, dtype=dtype)
    x = x_device(w, configs.gen_x(w))
    arena = device_arena_all_experts(w)
    L = MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype)
    lg_in = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    outs = []
    for rot in range(3):
        lg_in.copy_(dev(configs.gen_logits(w, rotation=rot)))
        outs.append(L.forward(x, lg_in, arena, w.entry_bytes).clone())
    again = L.forward(x, lg_in, arena, w.entry_bytes).clone()
    assert torch.equal(again, outs[-1])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.forward(x, lg_in, arena, w.entry_bytes, stream=s)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            L.forward(x, lg_in, arena, w.entry_bytes, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        for rot in range(3):
            lg_in.copy_(dev(configs.gen_logits(w, rotation=rot)))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(L.out, outs[rot]), (rep, rot)


def _random_shapes(n, seed):
    """Seeded layer shapes across the dispatch boundaries: T from 1 to 200 (one-launch
    routing, weight streaming, row split, grouped GEMM), E up to 300 (not powers of two),
    k up to 8, d and f multiples of 64 (row lengths that leave short tiles and partial
    lane chunks), Zipf skews 0.2 to 1."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(r.choice([5, 16, 37, 64, 130, 300]))
        k = int(r.integers(1, min(8, E) + 1))
        T = int(r.choice([1, 3, 8, 13, 16, 17, 40, 64, 65, 200]))
        d = 64 * int(r.integers(1, 17))
        f = 64 * int(r.integers(1, 13))
        out.append((T, E, k, d, f, float(r.choice([0.2, 0.5, 1.0]))))
    return out


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("T,E,k,d,f,alpha", _random_shapes(10, 1) + _random_shapes(10, 2))
def test_layer_random_shapes(T, E, k, d, f, alpha, dtype):
    """Whole layer (routing and grouping, expert FFN on the path the host picks, combine)
    on seeded random shapes, bf16 and MXFP4 experts, against the oracle."""
    _check_layer(T, E, k, d, f, alpha, dtype)


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("T", [1, 8, 16, 100, 200, 600, 2100])
def test_layer_at_maximum_experts_and_k(T, dtype):
    """The library's limits, E = 1024 experts and k = 16, through every path: one-launch
    routing (T <= 16), weight streaming, the row split, and the grouped GEMMs (bf16 above
    2048 assignments, MXFP4 above 8192 on 64-row tiles and from 32768 on 256-row tiles,
    whose weight strips here lie partly past f = 64 and d = 128), against the oracle."""
    _check_layer(T, 1024, 16, 128, 64, 0.5, dtype)


def _check_layer(T, E, k, d, f, alpha, dtype):
    w = configs.Workload("rand", seed=T * 7 + E + d, T=T, d=d, E=E, k=k, f=f, dtype=dtype,
                         alpha=alpha)
    x, lg, L, arena = _run_layer(w)
    ids, wt, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, sorted(set(oracle.route(lg, w.k)[0].ravel().tolist()))))
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    assert_close(L.out.cpu().numpy(), ref, bf16_tol(ref), f"layer T={T} E={E} k={k} d={d} f={f}")
    assert int(L.status.item()) == 0
    del arena
