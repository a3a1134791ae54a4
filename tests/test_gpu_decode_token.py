"""The one-launch single-token layer (moe_decode_token) against the separate launches and the
oracle: bit-identical to routing + grouping + expert FFN (fp32 outputs) + combine, within the
bf16 bound of the oracle, for routed and pre-routed calls, slot indirection, stale slots,
repeated calls and graph replay."""
import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import device_arena_all_experts
import oracle
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, bf16_tol, dev, x_device, oracle_table

pytestmark = pytest.mark.gpu

# (E, k, d, f): the decode shape; rows of one and of several 512-element lane passes; rows
# that leave lanes without a chunk; d past 4096 (one unit per wave); f past 2048 (two
# experts per register group); the library's largest E and k (two groups of eight)
SHAPES = [(256, 6, 4096, 2048), (64, 6, 1024, 512), (37, 5, 320, 192), (300, 8, 8192, 1024),
          (16, 2, 64, 8192), (1024, 16, 128, 64), (8, 3, 512, 2048), (130, 1, 640, 320)]


def _workload(E, k, d, f, alpha=0.5, dtype=gen.BF16):
    return configs.Workload("tok", seed=E * 31 + k * 7 + d + f, T=1, d=d, E=E, k=k, f=f,
                            dtype=dtype, alpha=alpha)


@pytest.fixture(scope="module")
def arenas():
    cache = {}
    yield cache
    cache.clear()
    torch.cuda.empty_cache()


def _arena(arenas, w):
    key = (w.E, w.k, w.d, w.f, w.dtype)
    if key not in arenas:
        arenas.clear()
        torch.cuda.empty_cache()
        arenas[key] = device_arena_all_experts(w)
    return arenas[key]


# MXFP4 weights: the decode shape; rows shorter than a tile (K mod 128 = 64); one and eight
# experts; E past 256
SHAPES_MX = [(256, 6, 4096, 2048), (64, 6, 1024, 512), (37, 5, 320, 192), (300, 8, 2048, 1024),
             (16, 1, 64, 2048), (130, 3, 4096, 64), (64, 8, 4096, 2048)]


def _mx_split_is_four(k, d, f):
    """Whether the separate MXFP4 launches split each strip over four waves for one token (the
    split the one-launch kernel uses), which makes their results bit-identical."""
    return k * f < 32768 and k * d < 32768


def _check_one_launch(E, k, d, f, arenas, dtype):
    w = _workload(E, k, d, f, dtype=dtype)
    arena = _arena(arenas, w)
    x = configs.gen_x(w)
    xd = x_device(w, x)
    L1 = MoeLayer(1, E, k, d, f, w_dtype=w.dtype)
    L0 = MoeLayer(1, E, k, d, f, w_dtype=w.dtype)
    assert L1.fusable
    exact = dtype == gen.BF16 or _mx_split_is_four(k, d, f)
    for rot in range(3):
        lg = configs.gen_logits(w, rotation=rot)
        lgd = dev(lg)
        L0.forward(xd, lgd, arena, w.entry_bytes, fused=False)
        L1.forward(xd, lgd, arena, w.entry_bytes, fused=True)
        torch.cuda.synchronize()
        assert int(L1.status.item()) == 0 and int(L0.status.item()) == 0
        assert torch.equal(L1.ids, L0.ids) and torch.equal(L1.w, L0.w)
        if exact:
            assert torch.equal(L1.out, L0.out), f"rotation {rot}: not bit-identical"
        ids, wt = oracle.route(lg, k)
        np.testing.assert_array_equal(L1.ids.cpu().numpy(), ids)
        assert_close(L1.w.cpu().numpy(), wt, 1e-6, "gate weights")
        _, _, ref = oracle.moe_layer(x, lg, k, oracle_table(w, sorted(set(ids.ravel().tolist()))))
        assert_close(L1.out.cpu().numpy(), ref, bf16_tol(ref), f"E={E} k={k} d={d} f={f}")
    # the epoch word at the head of the workspace counts the calls made on it
    assert int(L1.tok_ws[:4].view(torch.int32).item()) == 3


@pytest.mark.parametrize("E,k,d,f", SHAPES)
def test_one_launch_equals_separate_launches_and_oracle(E, k, d, f, arenas):
    _check_one_launch(E, k, d, f, arenas, gen.BF16)


@pytest.mark.parametrize("E,k,d,f", SHAPES_MX)
def test_one_launch_mxfp4_equals_separate_launches_and_oracle(E, k, d, f, arenas):
    """MXFP4 experts: the oracle on the exactly dequantised weights; bit-identical to the
    separate launches wherever those split a strip over four waves too."""
    _check_one_launch(E, k, d, f, arenas, gen.MXFP4)


def test_pre_routed_call_and_slot_indirection(arenas):
    """logits NULL: ids and weights are inputs.  Weights reached through a slot table (a
    permuted copy of the arena) and a slot-key check give the same bits."""
    E, k, d, f = 64, 6, 1024, 512
    w = _workload(E, k, d, f)
    arena = _arena(arenas, w)
    x = x_device(w, configs.gen_x(w))
    lg = dev(configs.gen_logits(w, rotation=1))
    L = MoeLayer(1, E, k, d, f)
    ref = L.forward(x, lg, arena, w.entry_bytes, fused=True).clone()
    ids = L.ids.clone()
    # pre-routed: the caller's ids/weights (here the ones just computed), no logits
    L.out.zero_()
    L.decode_token(x, None, arena, w.entry_bytes)
    torch.cuda.synchronize()
    assert torch.equal(L.out, ref) and torch.equal(L.ids, ids)
    # slot indirection with a permuted arena and matching keys
    perm = torch.randperm(E, generator=torch.Generator().manual_seed(3)).cuda()
    arena2 = torch.empty_like(arena)
    arena2[perm] = arena                      # expert e now in slot perm[e]
    slot = perm.to(torch.int32)
    key = torch.empty(E, dtype=torch.int32, device="cuda")
    key[perm] = torch.arange(E, dtype=torch.int32, device="cuda") + 1000
    L.out.zero_()
    L.decode_token(x, lg, arena2, w.entry_bytes, expert_slot=slot, slot_key=key, key_base=1000)
    torch.cuda.synchronize()
    assert int(L.status.item()) == 0
    assert torch.equal(L.out, ref)
    del arena2


def test_stale_slot_is_reported_and_left_out(arenas):
    """A slot whose key does not match sets MOE_ERANGE and that expert's term is left out of
    the sum; the other terms are as the oracle has them."""
    E, k, d, f = 64, 6, 1024, 512
    w = _workload(E, k, d, f)
    arena = _arena(arenas, w)
    xh = configs.gen_x(w)
    x = x_device(w, xh)
    lgh = configs.gen_logits(w, rotation=2)
    L = MoeLayer(1, E, k, d, f)
    ids, wt = oracle.route(lgh, k)
    stale = int(ids[0, 2])
    key = torch.arange(E, dtype=torch.int32, device="cuda")
    key[stale] = -7
    L.decode_token(x, dev(lgh), arena, w.entry_bytes, slot_key=key, key_base=0)
    torch.cuda.synchronize()
    assert int(L.status.item()) == moe.MOE_ERANGE
    keep = [j for j in range(k) if j != 2]
    y = oracle.expert_ffn(xh, ids, oracle_table(w, sorted(set(ids.ravel().tolist()))),
                          np.arange(k, dtype=np.int32))
    ref = (wt[0, keep, None] * y[keep]).sum(axis=0)[None]
    assert_close(L.out.cpu().numpy(), ref, bf16_tol(ref), "stale slot left out")


@pytest.mark.parametrize("E,k,d,f,dtype", [(256, 6, 4096, 2048, gen.BF16), (37, 5, 320, 192, gen.BF16),
                                           (256, 6, 4096, 2048, gen.MXFP4)])
def test_graph_replay_matches_eager(E, k, d, f, dtype, arenas):
    """The one-launch layer captured in a graph and replayed on new logits, with eager work and
    synchronisations between replays, gives the eager bits on every replay (each launch
    advances the workspace's epoch word by one; nothing is cleared by a memset node)."""
    w = _workload(E, k, d, f, dtype=dtype)
    arena = _arena(arenas, w)
    x = x_device(w, configs.gen_x(w))
    L = MoeLayer(1, E, k, d, f, w_dtype=w.dtype)
    assert L.fusable
    lg_in = torch.empty((1, E), dtype=torch.float32, device="cuda")
    outs = []
    for rot in range(4):
        lg_in.copy_(dev(configs.gen_logits(w, rotation=rot)))
        outs.append(L.forward(x, lg_in, arena, w.entry_bytes).clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.forward(x, lg_in, arena, w.entry_bytes, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            L.forward(x, lg_in, arena, w.entry_bytes, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for rot in range(4):
            lg_in.copy_(dev(configs.gen_logits(w, rotation=rot)))
            torch.cuda.synchronize()
            e0 = int(L.tok_ws[:4].view(torch.int32).item())
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(L.out, outs[rot]), (rep, rot)
            assert int(L.tok_ws[:4].view(torch.int32).item()) == e0 + 1
            # eager work between replays, on the same workspace
            if rot == 1:
                L.forward(x, lg_in, arena, w.entry_bytes)
                torch.cuda.synchronize()
                assert torch.equal(L.out, outs[rot])
    assert int(L.status.item()) == 0


def test_many_calls_in_a_row_on_one_stream(arenas):
    """Back-to-back calls with no host synchronisation between them (each call reads the epoch
    word the previous one advanced)."""
    E, k, d, f = 256, 6, 4096, 2048
    w = _workload(E, k, d, f)
    arena = _arena(arenas, w)
    x = x_device(w, configs.gen_x(w))
    L = MoeLayer(1, E, k, d, f)
    lgs = [dev(configs.gen_logits(w, rotation=r)) for r in range(4)]
    refs = []
    for lg in lgs:
        refs.append(L.forward(x, lg, arena, w.entry_bytes).clone())
    torch.cuda.synchronize()
    outs = []
    for i in range(40):
        L.forward(x, lgs[i % 4], arena, w.entry_bytes)
        if i % 10 == 9:
            outs.append((i % 4, L.out.clone()))
    torch.cuda.synchronize()
    for r, o in outs:
        assert torch.equal(o, refs[r])
    assert int(L.status.item()) == 0


def test_one_launch_beside_a_long_launch_on_another_stream(arenas):
    """The one-launch layer needs its workgroups resident together.  Started while a long
    grouped GEMM (the T=8192 prefill FFN, milliseconds) holds the compute units from another
    stream, its resident workgroups wait (bounded) until the GEMM's workgroups finish and the
    rest of the grid is placed; the result is the same bits and no status is raised."""
    E, k, d, f = 256, 6, 4096, 2048
    w = _workload(E, k, d, f)
    arena = _arena(arenas, w)
    x = x_device(w, configs.gen_x(w))
    lg = dev(configs.gen_logits(w, rotation=3))
    L = MoeLayer(1, E, k, d, f)
    ref = L.forward(x, lg, arena, w.entry_bytes).clone()
    torch.cuda.synchronize()
    # the prefill FFN on the same resident experts (weights of this workload), its own buffers
    wp = configs.with_(configs.PREFILL, seed=w.seed)
    P = MoeLayer(wp.T, E, k, d, f)
    xp = x_device(wp, configs.gen_x(wp))
    P.route_permute(dev(configs.gen_logits(wp)))
    torch.cuda.synchronize()
    side, main = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(side):
            P.ffn(xp, arena, w.entry_bytes, stream=side)
        with torch.cuda.stream(main):
            L.out.zero_()
            L.forward(x, lg, arena, w.entry_bytes, stream=main)
        torch.cuda.synchronize()
        assert torch.equal(L.out, ref)
    assert int(L.status.item()) == 0 and int(P.status.item()) == 0
