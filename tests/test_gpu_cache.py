"""GPU parity of the device LRU (tables, fills, counters) against the sequential simulator,
miss fills from a pinned host pool, stale-slot detection, and error paths."""
import ctypes

import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import host_pool, torch_dtype
import oracle
from oracle import LruSim
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, bf16_tol, dev, x_device, oracle_table

pytestmark = pytest.mark.gpu


class DevCache:
    """Device tables + descriptor for a cache of S slots over L x E entries."""

    def __init__(self, L, E, S, entry_bytes, arena=None, pool=None, pool_entries=None):
        i32 = dict(dtype=torch.int32, device="cuda")
        i64 = dict(dtype=torch.int64, device="cuda")
        self.slot_of = torch.empty(L * E, **i32)
        self.key_of = torch.empty(S, **i32)
        self.stamp = torch.empty(S, **i64)
        self.clock = torch.empty(1, **i64)
        self.stats = torch.empty(4, **i64)
        self.status = torch.empty(1, **i32)
        self.expert_slot = torch.empty(E, **i32)
        self.fills = torch.empty((max(E, 1), 4), **i32)
        self.n_fills = torch.empty(1, **i32)
        self.arena, self.pool = arena, pool
        if pool_entries is None:
            pool_entries = 0 if pool is None else L * E
        self.desc = moe.moe_cache_t(
            L, E, S, pool_entries, entry_bytes, self.slot_of.data_ptr(), self.key_of.data_ptr(),
            self.stamp.data_ptr(), self.clock.data_ptr(), self.stats.data_ptr(),
            self.status.data_ptr(), 0 if arena is None else arena.data_ptr(),
            0 if pool is None else pool.data_ptr())
        moe.cache_init(self.desc)

    def lookup(self, layer, ids_dev, T, k, stream=None):
        moe.cache_lookup_update(self.desc, layer, ids_dev, T, k, self.expert_slot, self.fills,
                                self.n_fills, stream)

    def fills_host(self):
        n = int(self.n_fills.item())
        return [tuple(int(v) for v in r) for r in self.fills[:n].cpu().numpy()]


def _compare_tables(dc, sim):
    np.testing.assert_array_equal(dc.key_of.cpu().numpy(), sim.key_of)
    np.testing.assert_array_equal(dc.slot_of.cpu().numpy(), sim.slot_of)
    np.testing.assert_array_equal(dc.stamp.cpu().numpy(), sim.stamp)
    assert int(dc.clock.item()) == sim.clock
    st = dc.stats.cpu().numpy()
    assert (st[0], st[1], st[2]) == (sim.accesses, sim.hits, sim.misses)


def test_lru_hand_traced_sequence_on_device():
    dc = DevCache(1, 8, 3, 64)
    sim = LruSim(1, 8, 3)
    for req in ([0, 1], [2], [0, 3], [1], [2, 3], [0, 1, 2]):
        ids = np.array([req], dtype=np.int32)
        dc.lookup(0, dev(ids), 1, len(req))
        _, fills = sim.step(0, req)
        assert dc.fills_host() == [tuple(f) for f in fills]
        _compare_tables(dc, sim)
    assert int(dc.status.item()) == 0


@pytest.mark.parametrize("L,E,S,steps", [(4, 64, 48, 150), (16, 256, 1024, 512)])
def test_lru_markov_trace_bit_exact(L, E, S, steps):
    """Every call: expert_slot, fill records and (every 16 calls and at the end) all tables
    equal the simulator's.  The second case is the full multi-layer decode workload
    (16 layers x 256 experts, 1024 slots, 512 steps of batch 8, top-6)."""
    w = configs.with_(configs.LRU_DECODE, L=L, E=E, S=S, steps=steps)
    ids, _ = gen.markov_routing(w.seed, steps, L, w.T, E, w.k, w.p_stay, w.zipf_s)
    ids_dev = dev(ids)
    dc = DevCache(L, E, S, w.entry_bytes)
    sim = LruSim(L, E, S)
    calls = 0
    for s in range(steps):
        for layer in range(L):
            dc.lookup(layer, ids_dev[s, layer], w.T, w.k)
            slot_ref, fills = sim.step(layer, ids[s, layer])
            assert dc.fills_host() == [tuple(f) for f in fills], (s, layer)
            np.testing.assert_array_equal(dc.expert_slot.cpu().numpy(), slot_ref)
            calls += 1
            if calls % 16 == 0:
                _compare_tables(dc, sim)
    _compare_tables(dc, sim)
    assert int(dc.stats[3].item()) == sim.misses * w.entry_bytes
    assert int(dc.status.item()) == 0


def test_lru_capacity_error_leaves_tables():
    dc = DevCache(1, 16, 4, 64)
    dc.lookup(0, dev(np.array([[1, 2]], dtype=np.int32)), 1, 2)
    before = [t.clone() for t in (dc.key_of, dc.slot_of, dc.stamp, dc.clock, dc.stats)]
    dc.lookup(0, dev(np.array([[0, 1, 2, 3, 4]], dtype=np.int32)), 1, 5)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == moe.MOE_ECAPACITY
    assert int(dc.n_fills.item()) == 0
    for a, b in zip(before, (dc.key_of, dc.slot_of, dc.stamp, dc.clock, dc.stats)):
        assert torch.equal(a, b)


def test_lru_bad_id_and_layer():
    dc = DevCache(2, 16, 4, 64)
    with pytest.raises(moe.MoeError) as ei:
        dc.lookup(2, dev(np.array([[1]], dtype=np.int32)), 1, 1)
    assert ei.value.status == moe.MOE_ERANGE
    dc.lookup(0, dev(np.array([[1, 16]], dtype=np.int32)), 1, 2)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == moe.MOE_ERANGE
    assert int(dc.clock.item()) == 0


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
def test_fill_then_ffn_through_slots_and_stale_slot_detection(dtype):
    """A small multi-layer cache: lookup -> D2H fill list -> cache_fill from the pinned pool ->
    FFN reading weights through expert_slot with the key check -> combine; every step's
    output equals the oracle.  Then a corrupted key makes the FFN report MOE_ERANGE."""
    w = configs.Workload("lru_small", seed=31, T=4, d=256, E=16, k=3, f=192, dtype=dtype,
                         L=3, S=14, alpha=0.5)  # S >= T*k; 3 layers x ~11 unique ids evict
    pool = host_pool(w)
    arena = torch.empty((w.S, w.entry_elems), dtype=torch_dtype(w), device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    lay = MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype)
    copy = torch.cuda.Stream()
    fills_host = (moe.moe_fill_t * w.E)()
    for step in range(6):
        for layer in range(w.L):
            x = configs.gen_x(w, layer, attempt=step)
            lg = gen.routing_logits(w.seed, gen.TAG_LOGIT + layer * 0x10000 + step * 0x100, w.T,
                                    w.E, w.k)
            lay.route(dev(lg))
            dc.lookup(layer, lay.ids, w.T, w.k)
            f = dc.fills_host()  # synchronises: the one host read per layer
            assert int(dc.status.item()) == 0, (step, layer)
            for i, (s, l, e, old) in enumerate(f):
                fills_host[i] = moe.moe_fill_t(s, l, e, old)
            copy.wait_stream(torch.cuda.current_stream())
            moe.cache_fill(dc.desc, ctypes.addressof(fills_host), len(f), copy)
            torch.cuda.current_stream().wait_stream(copy)
            lay.permute()
            lay.ffn(x_device(w, x), arena, w.entry_bytes, dc.expert_slot, slot_key=dc.key_of,
                    key_base=layer * w.E)
            lay.combine()
            torch.cuda.synchronize()
            ids, _, ref = oracle.moe_layer(x, lg, w.k, oracle_table(w, range(w.E), layer))
            np.testing.assert_array_equal(lay.ids.cpu().numpy(), ids)
            assert_close(lay.out.cpu().numpy(), ref, bf16_tol(ref), f"step {step} layer {layer}")
    assert int(dc.status.item()) == 0 and int(lay.status.item()) == 0
    # stale slot: overwrite the key of one slot used by the last layer's experts
    used = int(lay.ids[0, 0].item())
    s = int(dc.expert_slot[used].item())
    dc.key_of[s] = -7
    lay.ffn(x_device(w, x), arena, w.entry_bytes, dc.expert_slot, slot_key=dc.key_of,
            key_base=(w.L - 1) * w.E)
    torch.cuda.synchronize()
    assert int(lay.status.item()) == moe.MOE_ERANGE


def test_cache_fill_rejects_out_of_range_records():
    pool = torch.zeros((4, 64), dtype=torch.uint8, pin_memory=True)
    arena = torch.zeros((2, 64), dtype=torch.uint8, device="cuda")
    dc = DevCache(2, 2, 2, 64, arena, pool)
    bad = (moe.moe_fill_t * 1)(moe.moe_fill_t(2, 0, 0, -1))
    with pytest.raises(moe.MoeError) as ei:
        moe.cache_fill(dc.desc, ctypes.addressof(bad), 1)
    assert ei.value.status == moe.MOE_ERANGE


def _small_lru_workload(seed, dtype=gen.BF16):
    # S >= T*k; 3 layers x ~11 unique ids per layer evict every step
    return configs.Workload("lru_small", seed=seed, T=4, d=256, E=16, k=3, f=192, dtype=dtype,
                            L=3, S=14, alpha=0.5)


def _pool_entry(pool, w, layer, e):
    """Bytes of pool entry (layer, e) as uint16, read straight from the pinned buffer."""
    n = w.entry_elems
    buf = (ctypes.c_uint16 * n).from_address(pool.entry_ptr(layer * w.E + e))
    return np.frombuffer(buf, dtype=np.uint16).copy()


def test_device_fill_matches_host_fill_and_pool():
    """Device-driven fills (records and count read on the GPU, pool read over PCIe) leave the
    arena byte-identical to host-issued copies of the same records, and every filled slot
    holds its pool entry."""
    w = _small_lru_workload(33)
    pool = host_pool(w)
    arena_a = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    arena_b = torch.zeros_like(arena_a)
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena_a, pool)
    desc_b = moe.moe_cache_t.from_buffer_copy(dc.desc)
    desc_b.arena = arena_b.data_ptr()
    steps = 5
    ids, _ = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, 0.5, 1.1)
    ids_dev = dev(ids)
    rec = (moe.moe_fill_t * w.E)()
    filled = 0
    for s in range(steps):
        for layer in range(w.L):
            dc.lookup(layer, ids_dev[s, layer], w.T, w.k)
            moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
            f = dc.fills_host()
            for i, (slot, l, e, old) in enumerate(f):
                rec[i] = moe.moe_fill_t(slot, l, e, old)
            moe.cache_fill(desc_b, ctypes.addressof(rec), len(f))
            torch.cuda.synchronize()
            assert torch.equal(arena_a.view(torch.int16), arena_b.view(torch.int16)), (s, layer)
            for slot, l, e, _ in f:
                got = arena_a[slot].view(torch.int16).cpu().numpy().view(np.uint16)
                np.testing.assert_array_equal(got, _pool_entry(pool, w, l, e))
            filled += len(f)
    assert filled > steps * w.L  # evictions happened
    assert int(dc.status.item()) == 0


@pytest.mark.parametrize("overlap,dtype", [(False, gen.BF16), (True, gen.BF16), (True, gen.MXFP4)])
def test_decode_step_with_device_fills_replays_as_one_graph(overlap, dtype):
    """route -> lookup -> device fill -> permute -> FFN through slots (key-checked) -> combine
    for every layer, captured once and replayed over several steps with new routing written
    into the captured input between replays: every layer's output equals the oracle and the
    cache tables equal the sequential simulator's.  With overlap, the graph forks after the
    lookup: the fill runs on a side branch while the FFN of the hits runs, and the FFN of
    the misses follows the join.  MXFP4 entries take the same path (fills are byte copies)."""
    w = _small_lru_workload(35, dtype)
    pool = host_pool(w)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch_dtype(w), device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    sim = LruSim(w.L, w.E, w.S)
    layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype) for _ in range(w.L)]
    xs = [configs.gen_x(w, layer) for layer in range(w.L)]
    xs_dev = [x_device(w, x) for x in xs]
    tables = [oracle_table(w, range(w.E), layer) for layer in range(w.L)]
    lg_buf = torch.zeros((w.L, w.T, w.E), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    masks = torch.zeros((w.L, 2, w.E), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        for layer, lay in enumerate(layers):
            lay.route(lg_buf[layer])
            dc.lookup(layer, lay.ids, w.T, w.k)
            key = dict(slot_key=dc.key_of, key_base=layer * w.E)
            if overlap:
                hit, miss = masks[layer, 0], masks[layer, 1]
                moe.cache_fill_masks(dc.expert_slot, dc.fills, dc.n_fills, w.E, hit, miss,
                                     dc.status)
                side.wait_stream(s)
                moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E, side)
                lay.permute()
                lay.ffn(xs_dev[layer], arena, w.entry_bytes, dc.expert_slot, mask=hit, **key)
                s.wait_stream(side)
                lay.ffn(xs_dev[layer], arena, w.entry_bytes, dc.expert_slot, mask=miss, **key)
            else:
                moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
                lay.permute()
                lay.ffn(xs_dev[layer], arena, w.entry_bytes, dc.expert_slot, **key)
            lay.combine()
    for step in range(5):
        lgs = [gen.routing_logits(w.seed, gen.TAG_LOGIT + layer * 0x10000 + step * 0x100, w.T,
                                  w.E, w.k) for layer in range(w.L)]
        lg_buf.copy_(torch.from_numpy(np.stack(lgs)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer, lay in enumerate(layers):
            ids, _, ref = oracle.moe_layer(xs[layer], lgs[layer], w.k, tables[layer])
            np.testing.assert_array_equal(lay.ids.cpu().numpy(), ids)
            assert_close(lay.out.cpu().numpy(), ref, bf16_tol(ref), f"step {step} layer {layer}")
            sim.step(layer, ids.reshape(-1))
        _compare_tables(dc, sim)
        assert int(dc.status.item()) == 0
        assert all(int(lay.status.item()) == 0 for lay in layers)


def test_device_fill_error_records():
    """A record outside the tables sets MOE_ERANGE and is skipped while the others are copied;
    a count above max_fills sets MOE_ERANGE and copies nothing."""
    w = configs.Workload("fill_err", seed=37, T=1, d=64, E=2, k=1, f=64, dtype=gen.BF16, L=2, S=2)
    pool = host_pool(w)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    dc.fills[0] = torch.tensor([w.S, 0, 0, -1], dtype=torch.int32)  # slot out of range
    dc.fills[1] = torch.tensor([1, 1, 0, -1], dtype=torch.int32)    # good: (layer 1, expert 0)
    dc.n_fills.fill_(2)
    moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, 2)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == moe.MOE_ERANGE
    got = arena[1].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _pool_entry(pool, w, 1, 0))
    assert int(arena[0].view(torch.int16).abs().sum().item()) == 0
    dc2 = DevCache(w.L, w.E, w.S, w.entry_bytes, torch.zeros_like(arena), pool)
    dc2.fills[0] = torch.tensor([0, 0, 1, -1], dtype=torch.int32)
    dc2.n_fills.fill_(2)
    moe.cache_fill_device(dc2.desc, dc2.fills, dc2.n_fills, 1)
    torch.cuda.synchronize()
    assert int(dc2.status.item()) == moe.MOE_ERANGE
    assert int(dc2.arena.view(torch.int16).abs().sum().item()) == 0


def test_fills_past_a_short_pool_are_rejected():
    """The pool holds every (layer, expert) entry but declares only the first L*E - 1: a record
    for the last entry is out of range on both fill paths.  The host path returns MOE_ERANGE
    before enqueueing anything; the device path sets MOE_ERANGE, skips that record and copies
    the others.  (The undeclared entry is still inside the allocation, so a wrong read could
    not leave it.)"""
    w = configs.Workload("fill_short", seed=38, T=1, d=64, E=2, k=1, f=64, dtype=gen.BF16, L=2, S=2)
    pool = host_pool(w)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool, pool_entries=w.L * w.E - 1)
    last = (moe.moe_fill_t * 2)(moe.moe_fill_t(0, 0, 1, -1), moe.moe_fill_t(1, 1, 1, -1))
    with pytest.raises(moe.MoeError) as ei:
        moe.cache_fill(dc.desc, ctypes.addressof(last), 2)
    assert ei.value.status == moe.MOE_ERANGE
    torch.cuda.synchronize()
    assert int(arena.view(torch.int16).abs().sum().item()) == 0  # nothing was enqueued
    dc.fills[0] = torch.tensor([0, 0, 1, -1], dtype=torch.int32)  # entry 1: declared
    dc.fills[1] = torch.tensor([1, 1, 1, -1], dtype=torch.int32)  # entry 3: past the count
    dc.n_fills.fill_(2)
    moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, 2)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == moe.MOE_ERANGE
    got = arena[0].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _pool_entry(pool, w, 0, 1))
    assert int(arena[1].view(torch.int16).abs().sum().item()) == 0


def test_fill_masks_split_requested_experts():
    """hit_mask / miss_mask after each lookup equal the split of the requested experts by the
    fill records, and together cover exactly the requested set."""
    w = configs.with_(_small_lru_workload(39), L=2, S=20)  # room for reuse: hits and misses
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes)
    steps = 6
    ids, _ = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, 0.5, 1.1)
    ids_dev = dev(ids)
    hit = torch.empty(w.E, dtype=torch.uint8, device="cuda")
    miss = torch.empty_like(hit)
    saw_hit = saw_miss = False
    for s in range(steps):
        for layer in range(w.L):
            dc.lookup(layer, ids_dev[s, layer], w.T, w.k)
            moe.cache_fill_masks(dc.expert_slot, dc.fills, dc.n_fills, w.E, hit, miss, dc.status)
            filled = {e for _, _, e, _ in dc.fills_host()}
            req = set(int(e) for e in ids[s, layer].ravel())
            want_miss = np.array([e in filled for e in range(w.E)], dtype=np.uint8)
            want_hit = np.array([e in req and e not in filled for e in range(w.E)], dtype=np.uint8)
            np.testing.assert_array_equal(miss.cpu().numpy(), want_miss)
            np.testing.assert_array_equal(hit.cpu().numpy(), want_hit)
            saw_hit |= bool(want_hit.any())
            saw_miss |= bool(want_miss.any())
    assert saw_hit and saw_miss
    assert int(dc.status.item()) == 0
    dc.n_fills.fill_(w.E + 1)
    moe.cache_fill_masks(dc.expert_slot, dc.fills, dc.n_fills, w.E, hit, miss, dc.status)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == moe.MOE_ERANGE
    assert int(hit.sum().item()) == 0 and int(miss.sum().item()) == 0


@pytest.mark.parametrize("pcie,host", [(1000, 0), (0, 1000), (57000, 30000), (20000, 60000)])
def test_split_lookup_trace_bit_exact(pcie, host):
    """cache_lookup_update_split against LruSim.step_split on a Markov trace: expert_slot,
    fill records, host mask every call; all tables every 16 calls; counters at the end."""
    w = configs.with_(configs.LRU_DECODE, L=4, E=64, S=48, steps=60)
    ids, _ = gen.markov_routing(w.seed, w.steps, w.L, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    ids_dev = dev(ids)
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes)
    sim = LruSim(w.L, w.E, w.S)
    host_mask = torch.empty(w.E, dtype=torch.uint8, device="cuda")
    calls = fills_total = 0
    for s in range(w.steps):
        for layer in range(w.L):
            moe.cache_lookup_update_split(dc.desc, layer, ids_dev[s, layer], w.T, w.k, pcie, host,
                                          dc.expert_slot, dc.fills, dc.n_fills, host_mask)
            slot_ref, fills, to_host = sim.step_split(layer, ids[s, layer], pcie, host)
            assert dc.fills_host() == [tuple(f) for f in fills], (s, layer)
            np.testing.assert_array_equal(dc.expert_slot.cpu().numpy(), slot_ref)
            want = np.zeros(w.E, dtype=np.uint8)
            want[to_host] = 1
            np.testing.assert_array_equal(host_mask.cpu().numpy(), want)
            fills_total += len(fills)
            calls += 1
            if calls % 16 == 0:
                _compare_tables(dc, sim)
    _compare_tables(dc, sim)
    assert int(dc.stats[3].item()) == fills_total * w.entry_bytes
    assert int(dc.status.item()) == 0
    if host == 0:
        assert sim.host_runs == 0
    if pcie == 0:
        assert fills_total == 0 and sim.host_runs == sim.misses


def test_split_layer_with_host_rows_equals_oracle():
    """A decode layer under the q* split: lookup_split -> masks -> device fill -> FFN of hits
    and of filled misses on the GPU; the rows of the experts left to the host are written
    by the test from the oracle (standing in for host execution, which is not part of the
    library) -> combine.  Every layer's output equals the oracle's full layer."""
    w = _small_lru_workload(41)
    pool = host_pool(w)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    lay = MoeLayer(w.T, w.E, w.k, w.d, w.f)
    hit = torch.empty(w.E, dtype=torch.uint8, device="cuda")
    miss, host_mask = torch.empty_like(hit), torch.empty_like(hit)
    tables = [oracle_table(w, range(w.E), layer) for layer in range(w.L)]
    n_host = 0
    for step in range(4):
        for layer in range(w.L):
            x = configs.gen_x(w, layer, attempt=step)
            lg = gen.routing_logits(w.seed, gen.TAG_LOGIT + layer * 0x10000 + step * 0x100, w.T,
                                    w.E, w.k)
            lay.route(dev(lg))
            moe.cache_lookup_update_split(dc.desc, layer, lay.ids, w.T, w.k, 20000, 30000,
                                          dc.expert_slot, dc.fills, dc.n_fills, host_mask)
            moe.cache_fill_masks(dc.expert_slot, dc.fills, dc.n_fills, w.E, hit, miss, dc.status)
            moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
            lay.permute()
            key = dict(slot_key=dc.key_of, key_base=layer * w.E)
            lay.ffn(x_device(w, x), arena, w.entry_bytes, dc.expert_slot, mask=hit, **key)
            lay.ffn(x_device(w, x), arena, w.entry_bytes, dc.expert_slot, mask=miss, **key)
            torch.cuda.synchronize()
            ids = lay.ids.cpu().numpy()
            on_host = set(np.nonzero(host_mask.cpu().numpy())[0].tolist())
            assign = [a for a in range(w.T * w.k) if int(ids.flat[a]) in on_host]
            if assign:
                y = oracle.expert_ffn(x, ids, tables[layer], assign)
                pos = lay.inv.cpu().numpy()[assign]
                lay.y_perm[torch.from_numpy(pos).long().cuda()] = torch.from_numpy(y).float().cuda()
            n_host += len(on_host)
            lay.combine()
            torch.cuda.synchronize()
            _, _, ref = oracle.moe_layer(x, lg, w.k, tables[layer])
            assert_close(lay.out.cpu().numpy(), ref, bf16_tol(ref), f"step {step} layer {layer}")
    assert n_host > 0
    assert int(dc.status.item()) == 0 and int(lay.status.item()) == 0


def _arena_holds_pool(dc, arena, pool, w):
    """Every occupied slot of the device cache holds its pool entry."""
    keys = dc.key_of.cpu().numpy()
    for j in np.nonzero(keys >= 0)[0]:
        layer, e = divmod(int(keys[j]), w.E)
        got = arena[j].view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, _pool_entry(pool, w, layer, e), f"slot {j}")


def test_resize_shrink_grow_mid_trace_matches_oracle():
    """A trace with device fills, resized to fewer slots and then to more at safe points:
    after each resize and every later call the tables equal LruSim.resized's, the arena's
    occupied slots hold their pool entries, and lookups keep matching the simulator."""
    w = configs.Workload("lru_resize", seed=43, T=4, d=128, E=16, k=3, f=128, dtype=gen.BF16,
                         L=3, S=24, alpha=0.5)
    pool = host_pool(w)
    steps = 18
    ids, _ = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, 0.6, 1.1)
    ids_dev = dev(ids)
    sizes = {6: 13, 12: 30}  # step -> new slot count (shrink below residency, then grow)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    sim = LruSim(w.L, w.E, w.S)
    for s in range(steps):
        if s in sizes:
            S2 = sizes[s]
            arena2 = torch.zeros((S2, w.entry_elems), dtype=torch.bfloat16, device="cuda")
            dc2 = DevCache(w.L, w.E, S2, w.entry_bytes, arena2, pool)
            moe.cache_resize(dc.desc, dc2.desc)
            torch.cuda.synchronize()
            sim = sim.resized(S2)
            dc, arena = dc2, arena2
            _compare_tables(dc, sim)
            _arena_holds_pool(dc, arena, pool, w)
        for layer in range(w.L):
            dc.lookup(layer, ids_dev[s, layer], w.T, w.k)
            moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
            slot_ref, fills = sim.step(layer, ids[s, layer])
            assert dc.fills_host() == [tuple(f) for f in fills], (s, layer)
            np.testing.assert_array_equal(dc.expert_slot.cpu().numpy(), slot_ref)
        _compare_tables(dc, sim)
        _arena_holds_pool(dc, arena, pool, w)
    assert int(dc.status.item()) == 0


@pytest.mark.parametrize("sizes", [{0: 5}, {3: 1, 4: 7}, {5: 24}])
def test_resize_edge_cases_match_oracle(sizes):
    """Resize of a freshly initialised (empty) cache, a shrink to a single slot followed by a
    grow, and a resize to the same slot count: tables equal LruSim.resized's, the arena keeps
    the pool entries, and the later lookups match the simulator."""
    w = configs.Workload("lru_resize_edge", seed=53, T=1, d=64, E=12, k=1, f=64,
                         dtype=gen.BF16, L=2, S=24, alpha=0.5)
    pool = host_pool(w)
    steps = 8
    ids, _ = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, 0.6, 1.1)
    ids_dev = dev(ids)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch.bfloat16, device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    sim = LruSim(w.L, w.E, w.S)
    for s in range(steps):
        if s in sizes:
            S2 = sizes[s]
            arena2 = torch.zeros((S2, w.entry_elems), dtype=torch.bfloat16, device="cuda")
            dc2 = DevCache(w.L, w.E, S2, w.entry_bytes, arena2, pool)
            moe.cache_resize(dc.desc, dc2.desc)
            torch.cuda.synchronize()
            sim = sim.resized(S2)
            dc, arena = dc2, arena2
            _compare_tables(dc, sim)
            _arena_holds_pool(dc, arena, pool, w)
            assert int(dc.clock.item()) == sim.clock
        for layer in range(w.L):
            dc.lookup(layer, ids_dev[s, layer], w.T, w.k)
            moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
            slot_ref, fills = sim.step(layer, ids[s, layer])
            assert dc.fills_host() == [tuple(f) for f in fills], (s, layer)
            np.testing.assert_array_equal(dc.expert_slot.cpu().numpy(), slot_ref)
        _compare_tables(dc, sim)
        _arena_holds_pool(dc, arena, pool, w)
    assert int(dc.status.item()) == 0


def test_lru_split_and_resize_at_maximum_sizes():
    """The library's limits: E = 1024 experts (one lookup thread each), S = 4096 slots (every
    slot's key sorted in LDS, 4 slots per thread in the resize scan) and k = 16.  A trace with
    evictions from the second step, a resize below residency (4096 -> 1500 slots) and back to
    4096, then split lookups: every call's expert_slot and fill records, and all tables after
    every step and resize, equal the simulator's."""
    L, E, S, T, k, steps = 8, 1024, 4096, 64, 16, 8
    ids, _ = gen.markov_routing(97, steps, L, T, E, k, 0.5, 1.05)
    ids_dev = dev(ids)
    eb = 16  # tables only: a 16-byte arena entry per slot for the resize copy
    dc = DevCache(L, E, S, eb, torch.zeros(S * eb, dtype=torch.uint8, device="cuda"))
    sim = LruSim(L, E, S)
    host_mask = torch.empty(E, dtype=torch.uint8, device="cuda")
    sizes = {3: 1500, 5: 4096}
    evicted = 0
    for s in range(steps):
        if s in sizes:
            S2 = sizes[s]
            dc2 = DevCache(L, E, S2, eb, torch.zeros(S2 * eb, dtype=torch.uint8, device="cuda"))
            moe.cache_resize(dc.desc, dc2.desc)
            torch.cuda.synchronize()
            sim, dc = sim.resized(S2), dc2
            _compare_tables(dc, sim)
        for layer in range(L):
            if s < 6:
                dc.lookup(layer, ids_dev[s, layer], T, k)
                slot_ref, fills = sim.step(layer, ids[s, layer])
            else:
                moe.cache_lookup_update_split(dc.desc, layer, ids_dev[s, layer], T, k, 57000,
                                              30000, dc.expert_slot, dc.fills, dc.n_fills,
                                              host_mask)
                slot_ref, fills, to_host = sim.step_split(layer, ids[s, layer], 57000, 30000)
                want = np.zeros(E, dtype=np.uint8)
                want[to_host] = 1
                np.testing.assert_array_equal(host_mask.cpu().numpy(), want)
            assert dc.fills_host() == [tuple(f) for f in fills], (s, layer)
            np.testing.assert_array_equal(dc.expert_slot.cpu().numpy(), slot_ref)
            evicted += sum(1 for f in fills if f[3] >= 0)
        _compare_tables(dc, sim)
    assert evicted > 0
    assert int(dc.status.item()) == 0


@pytest.mark.parametrize("dtype,graph,slots", [(gen.BF16, False, "table"), (gen.BF16, True, "lookup"),
                                               (gen.MXFP4, True, "table")])
def test_one_token_decode_through_cache_with_one_launch_layer(dtype, graph, slots):
    """One token per step: route -> lookup -> device fill -> the one-launch layer on the
    routed ids (grouping, FFN through key-checked slots, combine) for every layer, eager or
    captured once and replayed with new logits.  Slots come from the layer's row of slot_of
    or from the lookup's expert_slot.  Every layer's output equals the oracle and the
    tables equal the sequential simulator's; 3 layers x 3 experts over 7 slots evict every
    step."""
    w = configs.Workload("lru_tok", seed=41, T=1, d=256, E=16, k=3, f=192, dtype=dtype, L=3,
                         S=7, alpha=0.5)
    pool = host_pool(w)
    arena = torch.zeros((w.S, w.entry_elems), dtype=torch_dtype(w), device="cuda")
    dc = DevCache(w.L, w.E, w.S, w.entry_bytes, arena, pool)
    sim = LruSim(w.L, w.E, w.S)
    layers = [MoeLayer(1, w.E, w.k, w.d, w.f, w_dtype=w.dtype) for _ in range(w.L)]
    assert all(lay.fusable for lay in layers)
    xs = [configs.gen_x(w, layer) for layer in range(w.L)]
    xs_dev = [x_device(w, x) for x in xs]
    tables = [oracle_table(w, range(w.E), layer) for layer in range(w.L)]
    lg_buf = torch.zeros((w.L, 1, w.E), dtype=torch.float32, device="cuda")

    def step_layers():
        for layer, lay in enumerate(layers):
            lay.route(lg_buf[layer])
            dc.lookup(layer, lay.ids, 1, w.k)
            moe.cache_fill_device(dc.desc, dc.fills, dc.n_fills, w.E)
            es = dc.slot_of[layer * w.E:(layer + 1) * w.E] if slots == "table" else dc.expert_slot
            lay.decode_token(xs_dev[layer], None, arena, w.entry_bytes, expert_slot=es,
                             slot_key=dc.key_of, key_base=layer * w.E)

    torch.cuda.synchronize()
    if graph:
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step_layers()
    for step in range(8):
        lgs = [gen.routing_logits(w.seed, gen.TAG_LOGIT + layer * 0x10000 + step * 0x100, 1,
                                  w.E, w.k) for layer in range(w.L)]
        lg_buf.copy_(torch.from_numpy(np.stack(lgs)))
        torch.cuda.synchronize()
        if graph:
            g.replay()
        else:
            step_layers()
        torch.cuda.synchronize()
        for layer, lay in enumerate(layers):
            ids, _, ref = oracle.moe_layer(xs[layer], lgs[layer], w.k, tables[layer])
            np.testing.assert_array_equal(lay.ids.cpu().numpy(), ids)
            assert_close(lay.out.cpu().numpy().reshape(ref.shape), ref, bf16_tol(ref),
                         f"step {step} layer {layer}")
            sim.step(layer, ids.reshape(-1))
            assert int(lay.status.item()) == 0, (step, layer)
        _compare_tables(dc, sim)
        assert int(dc.status.item()) == 0
    assert sim.misses > w.L * w.k  # evictions happened after the cold start
