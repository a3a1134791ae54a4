"""Full-shape parity of the three multi-kernel workloads against the oracle, in the launch
configurations bench.py times:

* prefill, T=8192, E=256, k=6, d=4096, f=2048 (grouped GEMMs, bf16 y_perm): every y_perm row
  of the most, a median and the least loaded expert, Zipf 0.2 and 1, bf16 and MXFP4 experts;
* multi-layer decode through the LRU cache at its real shape (16 layers x 256 experts, 1024
  slots, d=2048, f=1024, batch 8, the 51.5 GB layer-major pinned pool): eight decode steps
  from a cold cache past the first evictions, host-issued and device-driven fills alternating,
  every layer's output against the oracle and the tables against the LRU simulator;
* streamed prefill at its real shape (E=128, k=8, d=2048, f=768, T=2048), four layers through
  the two streaming buffers: routing and grouping bit-exact, every y_perm row of each layer's
  most loaded expert and sampled token outputs within the bf16 rule.
"""
import ctypes

import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import HostPool, device_arena_all_experts, fill_entries_ptr, host_pool, torch_dtype
import oracle
from oracle import LruSim
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, bf16_tol, dev, np_of, oracle_table, x_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_grouping(L, lg, k, E):
    """ids, counts, offsets, perm and inv of a layer equal the oracle's, bit for bit."""
    ids, _ = oracle.route(lg, k)
    np.testing.assert_array_equal(L.ids.cpu().numpy(), ids)
    counts, offsets, perm, inv = oracle.permute(ids, E)
    np.testing.assert_array_equal(L.counts.cpu().numpy(), counts)
    np.testing.assert_array_equal(L.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(L.perm.cpu().numpy(), perm)
    np.testing.assert_array_equal(L.inv.cpu().numpy(), inv)
    return ids, counts, offsets, perm


def _check_expert_rows(L, w, x, ids, offsets, perm, e, layer=0, what=""):
    """Every y_perm row of expert e against the oracle's FFN of the same assignments."""
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    got = np_of(L.y_perm[lo:hi])
    ref = oracle.expert_ffn(x, ids, oracle_table(w, [e], layer), perm[lo:hi])
    assert_close(got, ref, bf16_tol(ref), f"{what} expert {e} ({hi - lo} rows)")


# ------------------------------------------------------------------ prefill, every GEMM row
@pytest.fixture(scope="module")
def prefill_arena():
    held = {}

    def get(dtype):
        if dtype not in held:
            held.clear()
            torch.cuda.empty_cache()
            held[dtype] = device_arena_all_experts(configs.with_(configs.PREFILL, dtype=dtype))
        return held[dtype]

    yield get
    held.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("alpha", [0.2, 1.0])
@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
def test_prefill_every_row_of_three_experts(alpha, dtype, prefill_arena):
    """T=8192 prefill with bf16 y_perm (the benchmark's configuration): routing and grouping
    bit-exact for all tokens, then every y_perm row of the most loaded, a median and the least
    loaded non-empty expert against the oracle.  The most loaded expert has 1189 rows at Zipf
    0.2 and about 7800 at Zipf 1, so every token tile, weight tile and k step of both grouped
    GEMMs at d=4096, f=2048 is compared, including the ragged last token tile."""
    w = configs.with_(configs.PREFILL, alpha=alpha, dtype=dtype)
    _say(f"[prefill rows] alpha={alpha} dtype={dtype}")
    arena = prefill_arena(dtype)
    x = configs.gen_x(w)
    lg = configs.gen_logits(w)
    L = MoeLayer(w.T, w.E, w.k, w.d, w.f, y_dtype=moe.MOE_BF16, w_dtype=w.dtype)
    L.forward(x_device(w, x), dev(lg), arena, w.entry_bytes)
    torch.cuda.synchronize()
    assert int(L.status.item()) == 0
    ids, counts, offsets, perm = _check_grouping(L, lg, w.k, w.E)
    nz = np.nonzero(counts)[0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    picks = [int(order[-1]), int(order[len(order) // 2]), int(order[0])]
    for e in picks:
        _check_expert_rows(L, w, x, ids, offsets, perm, e, what=f"prefill alpha={alpha}")
    assert counts[picks[0]] > 256 and counts[picks[2]] < 256


# ------------------------------------------------------------------ streamed prefill
@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
def test_streamed_prefill_real_shape(dtype):
    """Four layers of the streamed-prefill workload at its real shape (E=128, k=8, d=2048,
    f=768, T=2048, Zipf 0.2, bf16 y_perm) through the two streaming buffers: layer l+1's whole
    expert block is copied on a copy stream (after layer l-1's compute released the buffer)
    while layer l computes.  Per layer: routing and grouping bit-exact; every y_perm row of
    the most loaded expert; outputs of 16 tokens (first, last and spread)."""
    w = configs.with_(configs.STREAM_PREFILL, L=4, dtype=dtype)
    _say(f"[stream real shape] dtype={dtype}")
    pool = host_pool(w)
    layer_bytes = w.E * w.entry_bytes
    bufs = [torch.empty((w.E, w.entry_elems), dtype=torch_dtype(w), device="cuda")
            for _ in range(2)]
    xs = [configs.gen_x(w, l) for l in range(w.L)]
    lgs = [configs.gen_logits(w, layer=l) for l in range(w.L)]
    xs_d = [x_device(w, x) for x in xs]
    lgs_d = [dev(lg) for lg in lgs]
    layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, y_dtype=moe.MOE_BF16, w_dtype=w.dtype)
              for _ in range(w.L)]
    comp, copy = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(w.L)]
    free = [torch.cuda.Event() for _ in range(2)]
    for ev in ready:
        ev.record(copy)  # a recorded event has a HIP handle that can cross the C ABI
    for ev in free:
        ev.record(comp)
    torch.cuda.synchronize()
    moe.layer_stream_prefetch(pool.entry_ptr(0), bufs[0], layer_bytes, 1, copy, None, ready[0])
    for l in range(w.L):
        if l + 1 < w.L:
            nb = (l + 1) % 2
            moe.layer_stream_prefetch(pool.entry_ptr((l + 1) * w.E), bufs[nb], layer_bytes, 1,
                                      copy, free[nb] if l >= 1 else None, ready[l + 1])
        comp.wait_event(ready[l])
        layers[l].forward(xs_d[l], lgs_d[l], bufs[l % 2], w.entry_bytes, stream=comp)
        free[l % 2].record(comp)
    torch.cuda.synchronize()
    r = np.random.default_rng(5)
    for l in range(w.L):
        L = layers[l]
        assert int(L.status.item()) == 0
        ids, counts, offsets, perm = _check_grouping(L, lgs[l], w.k, w.E)
        big = int(np.argmax(counts))
        _check_expert_rows(L, w, xs[l], ids, offsets, perm, big, layer=l,
                           what=f"streamed layer {l}")
        toks = np.array(sorted({0, w.T - 1} | set(r.choice(w.T, 14, replace=False).tolist())),
                        dtype=np.int32)
        need = sorted(set(ids[toks].ravel().tolist()))
        _, _, ref = oracle.moe_layer(xs[l], lgs[l], w.k, oracle_table(w, need, layer=l),
                                     tokens=toks)
        assert_close(L.out.cpu().numpy()[toks], ref, bf16_tol(ref), f"streamed layer {l} out")
    pool.close()


# ------------------------------------------------------------------ multi-layer LRU decode
def _tables_equal(dc, sim):
    np.testing.assert_array_equal(dc["key_of"].cpu().numpy(), sim.key_of)
    np.testing.assert_array_equal(dc["slot_of"].cpu().numpy(), sim.slot_of)
    np.testing.assert_array_equal(dc["stamp"].cpu().numpy(), sim.stamp)
    assert int(dc["clock"].item()) == sim.clock
    st = dc["stats"].cpu().numpy()
    assert (st[0], st[1], st[2]) == (sim.accesses, sim.hits, sim.misses)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
def test_lru_decode_real_shape_through_fills(dtype):
    """The multi-layer decode workload at its real shape: 16 layers x 256 experts, top-6,
    d=2048, f=1024, bf16 or MXFP4 entries, 1024 slots, batch 8, Markov routing (p=0.7) from
    the benchmark's seed, and the real pinned pool (4096 entries, 51.5 GB bf16 or 13.7 GB
    MXFP4, layer-major; the entries the eight steps fill are generated, the others are never
    read).  Eight decode steps from a cold
    cache, the last two with evictions.  Even steps run as the benchmark's host-driven loop
    (lookup, fill list read on the host, cache_fill on a copy stream while the FFN of the hits
    runs, then the FFN of the misses); odd steps as its graph loop (hit/miss masks on the
    device, cache_fill_device on a side stream while the FFN of the hits runs).  Every call:
    expert_slot and fill records equal LruSim's; every layer's output equals the oracle's;
    all tables equal the simulator's after every step."""
    w = configs.with_(configs.LRU_DECODE, dtype=dtype)
    steps = 8
    ids_all, lg_all = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    sim = LruSim(w.L, w.E, w.S)
    needed = set()
    for s in range(steps):
        for l in range(w.L):
            needed |= {(f[1], f[2]) for f in sim.step(l, ids_all[s, l])[1]}
    assert needed
    _say(f"[lru real shape] generating {len(needed)} pool entries of {w.L * w.E}")
    pool = HostPool(w)
    for l, e in sorted(needed):
        fill_entries_ptr(w, [(l, e)], pool.entry_ptr(l * w.E + e), w.entry_elems)
    i32 = dict(dtype=torch.int32, device="cuda")
    i64 = dict(dtype=torch.int64, device="cuda")
    dc = dict(slot_of=torch.empty(w.L * w.E, **i32), key_of=torch.empty(w.S, **i32),
              stamp=torch.empty(w.S, **i64), clock=torch.empty(1, **i64),
              stats=torch.empty(4, **i64), status=torch.zeros(1, **i32),
              arena=torch.empty((w.S, w.entry_elems), dtype=torch_dtype(w), device="cuda"))
    desc = moe.moe_cache_t(w.L, w.E, w.S, w.L * w.E, w.entry_bytes,
                           *(dc[n].data_ptr() for n in ("slot_of", "key_of", "stamp", "clock",
                                                        "stats", "status", "arena")),
                           pool.data_ptr())
    moe.cache_init(desc)
    expert_slot = torch.empty(w.E, **i32)
    fills = torch.empty((w.E, 4), **i32)
    n_fills = torch.empty(1, **i32)
    hit = torch.empty(w.E, dtype=torch.uint8, device="cuda")
    miss = torch.empty_like(hit)
    records = (moe.moe_fill_t * w.E)()
    lay = MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype)
    xs = [configs.gen_x(w, l) for l in range(w.L)]
    xs_d = [x_device(w, x) for x in xs]
    lg_d = dev(lg_all)
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    weights = {}
    sim = LruSim(w.L, w.E, w.S)
    evictions = 0
    for s in range(steps):
        for l in range(w.L):
            lay.route(lg_d[s, l])
            moe.cache_lookup_update(desc, l, lay.ids, w.T, w.k, expert_slot, fills, n_fills)
            key = dict(slot_key=dc["key_of"], key_base=l * w.E)
            if s % 2 == 0:
                n = int(n_fills.item())  # synchronises: the one host read per layer
                for i, rec in enumerate(fills[:n].cpu().numpy()):
                    records[i] = moe.moe_fill_t(*(int(v) for v in rec))
                got_fills = [tuple(int(v) for v in rec) for rec in fills[:n].cpu().numpy()]
                missed = np.zeros(w.E, dtype=np.uint8)
                missed[[f[2] for f in got_fills]] = 1
                miss.copy_(torch.from_numpy(missed))
                hit.copy_(torch.from_numpy(1 - missed))
                side.wait_stream(comp)
                moe.cache_fill(desc, ctypes.addressof(records), n, side)
            else:
                moe.cache_fill_masks(expert_slot, fills, n_fills, w.E, hit, miss, dc["status"])
                side.wait_stream(comp)
                moe.cache_fill_device(desc, fills, n_fills, w.E, side)
            lay.permute()
            lay.ffn(xs_d[l], dc["arena"], w.entry_bytes, expert_slot, mask=hit, **key)
            comp.wait_stream(side)
            lay.ffn(xs_d[l], dc["arena"], w.entry_bytes, expert_slot, mask=miss, **key)
            lay.combine()
            torch.cuda.synchronize()
            ids = ids_all[s, l]
            slot_ref, fills_ref = sim.step(l, ids)
            np.testing.assert_array_equal(lay.ids.cpu().numpy(), ids)
            n = int(n_fills.item())
            assert [tuple(int(v) for v in r) for r in fills[:n].cpu().numpy()] == \
                [tuple(f) for f in fills_ref], (s, l)
            np.testing.assert_array_equal(expert_slot.cpu().numpy(), slot_ref)
            evictions += sum(1 for f in fills_ref if f[3] >= 0)
            used = sorted(set(ids.ravel().tolist()))
            for e in used:
                if (l, e) not in weights:
                    m = configs.gen_expert(w, l, e)
                    if w.dtype == gen.MXFP4:  # the exact dequantised weights
                        m = tuple(oracle.mxfp4_dequant(c, sc).astype(np.float32) for c, sc in m)
                    weights[(l, e)] = m
            table = oracle.ExpertTable(w.E, {e: weights[(l, e)] for e in used})
            _, _, ref = oracle.moe_layer(xs[l], lg_all[s, l], w.k, table)
            assert_close(lay.out.cpu().numpy(), ref, bf16_tol(ref), f"step {s} layer {l}")
        _tables_equal(dc, sim)
        _say(f"[lru real shape] step {s}: tables and outputs equal the oracle")
    assert evictions > 0
    assert int(dc["stats"][3].item()) == sim.misses * w.entry_bytes
    assert int(dc["status"].item()) == 0 and int(lay.status.item()) == 0
    pool.close()
