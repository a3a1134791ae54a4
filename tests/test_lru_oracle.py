"""Pins of the LRU simulator: a hand-traced sequence, a textbook LRU, invariants."""
import os
from collections import OrderedDict

import numpy as np
import pytest

import gen
from gen import configs
import oracle
from oracle import LruSim, CapacityError, StaticPlacement

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_trace_s3.txt")


def _parse_golden():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        t, req, hits, fills, ev, keys, stamps = [c.strip() for c in line.split("|")]
        fl = [] if fills == "-" else [tuple(int(v) for v in f.split("<-")) for f in fills.split()]
        rows.append(dict(
            t=int(t), req=[int(v) for v in req.split()],
            hits=[] if hits == "-" else [int(v) for v in hits.split()],
            fills=fl, evicted=[] if ev == "-" else [int(v) for v in ev.split()],
            keys=[-1 if v == "-" else int(v) for v in keys.split()],
            stamps=[int(v) for v in stamps.split()]))
    return rows


def test_hand_traced_sequence():
    sim = LruSim(L=1, E=8, S=3)
    evictions = []
    for row in _parse_golden():
        slot, fills = sim.step(0, row["req"])
        assert sim.clock == row["t"]
        assert [(s, e) for s, _, e, _ in fills] == row["fills"]
        ev = [old for _, _, _, old in fills if old >= 0]
        assert ev == row["evicted"]
        evictions += ev
        assert list(sim.key_of) == row["keys"]
        assert list(sim.stamp) == row["stamps"]
        assert sorted(e for e in row["req"] if e not in [f[1] for f in row["fills"]]) == row["hits"]
        for e in row["req"]:
            assert sim.key_of[slot[e]] == e
    assert (sim.accesses, sim.misses, evictions) == (11, 7, [1, 2, 0, 3])


def test_single_request_calls_equal_textbook_lru():
    """One expert per call: no ties inside a call, so the hit/miss sequence and the
    resident set must equal a textbook move-to-end LRU (collections.OrderedDict)."""
    L, E, S = 3, 20, 7
    r = np.random.default_rng(0)
    sim = LruSim(L, E, S)
    book = OrderedDict()
    for _ in range(3000):
        layer = int(r.integers(L))
        e = int(min(r.zipf(1.3), E) - 1)
        key = layer * E + e
        hit_book = key in book
        if hit_book:
            book.move_to_end(key)
        else:
            if len(book) == S:
                book.popitem(last=False)
            book[key] = True
        _, fills = sim.step(layer, [e])
        assert (len(fills) == 0) == hit_book
        assert sim.resident_keys() == set(book.keys())


def test_capacity_error_leaves_state_unchanged():
    sim = LruSim(1, 16, 4)
    sim.step(0, [1, 2])
    before = (sim.key_of.copy(), sim.slot_of.copy(), sim.stamp.copy(), sim.clock)
    with pytest.raises(CapacityError):
        sim.step(0, [0, 1, 2, 3, 4])
    after = (sim.key_of, sim.slot_of, sim.stamp, sim.clock)
    for a, b in zip(before, after):
        np.testing.assert_array_equal(a, b)


def _check_invariants(sim, t, U_keys, fills, before_stamp, before_key):
    S = sim.S
    for s in range(S):  # slot_of and key_of are mutual inverses
        if sim.key_of[s] >= 0:
            assert sim.slot_of[sim.key_of[s]] == s
    assert np.count_nonzero(sim.slot_of >= 0) == np.count_nonzero(sim.key_of >= 0)
    misses = [k for k in U_keys if k not in set(before_key[before_key >= 0])]
    assert len(fills) == len(misses)
    evicted_slots = [s for s, _, _, old in fills if old >= 0]
    for s in evicted_slots:  # nothing stamped t is evicted at t
        assert before_stamp[s] < t
    if evicted_slots:  # nothing evicted was used more recently than anything kept
        newest_evicted = max(before_stamp[s] for s in evicted_slots)
        kept = [s for s in range(S) if before_key[s] >= 0 and s not in evicted_slots]
        for s in kept:
            assert sim.stamp[s] >= newest_evicted
    for k in U_keys:  # every requested entry is resident after the call
        assert sim.slot_of[k] >= 0 and sim.stamp[sim.slot_of[k]] == t


def test_invariants_on_markov_trace_and_lru_beats_static_placement():
    """Multi-layer Markov routing (p=0.7 re-pick, else Zipf(1.1)), 16 layers x 256 experts,
    1024 slots.  Invariants every call; LRU misses less than a routing-agnostic static
    placement of the same capacity (directional check of the pages' comparison of the
    global LRU with a static split: RTX-4090 page, "Benchmarks, comparisons, trade-offs")."""
    w = configs.LRU_DECODE
    steps = 64
    ids, logits = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    sim = LruSim(w.L, w.E, w.S)
    # static: the S/L most Zipf-popular experts of every layer, fixed
    per_layer = w.S // w.L
    static_keys = []
    for layer in range(w.L):
        rank = gen.rank_perm(w.seed, gen.TAG_MRANK + layer * 0x10000, w.E)
        static_keys += [layer * w.E + int(e) for e in np.argsort(rank)[:per_layer]]
    static = StaticPlacement(static_keys)
    for s in range(steps):
        for layer in range(w.L):
            before_stamp, before_key = sim.stamp.copy(), sim.key_of.copy()
            U = sorted(set(int(e) for e in ids[s, layer].ravel()))
            _, fills = sim.step(layer, ids[s, layer])
            _check_invariants(sim, sim.clock, [layer * w.E + e for e in U], fills, before_stamp,
                              before_key)
            static.step(layer, ids[s, layer], w.E)
    assert sim.accesses == static.accesses
    assert sim.misses < static.misses


def test_markov_logits_route_back_to_generated_ids():
    """The oracle's top-k of the synthesised logits reproduces the generated expert ids."""
    w = configs.LRU_DECODE
    ids, logits = gen.markov_routing(w.seed, 4, 3, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    got, _ = oracle.route(logits.reshape(-1, w.E), w.k)
    np.testing.assert_array_equal(got, ids.reshape(-1, w.k))


def test_qstar_closed_forms_and_hand_values():
    """q* (misses filled over PCIe, the rest run on the host) against what the balance fixes:
    no host bandwidth -> fill all; no PCIe -> fill none; equal bandwidths -> half, ties to
    the larger count; two hand-computed cases."""
    for m in range(0, 12):
        assert oracle.qstar(m, 1000, 0) == m
        assert oracle.qstar(m, 0, 1000) == 0
        assert oracle.qstar(m, 777, 777) == (m + 1) // 2
    # m=10, P=3, H=1: max(q*H, (m-q)*P) is 9 at q=7, 8 at q=8, 9 at q=9, so q*=8
    assert oracle.qstar(10, 3, 1) == 8
    # m=6 misses, PCIe 57 GB/s, host 100 GB/s: optimum 6*57/157 = 2.18; q=2 -> max(200000,
    # 228000), q=3 -> max(300000, 171000): q*=2
    assert oracle.qstar(6, 57000, 100000) == 2
    with pytest.raises(ValueError):
        oracle.qstar(3, 0, 0)


def test_qstar_is_a_neighbour_of_the_continuous_balance():
    """The integer optimum is floor or ceil of m*P/(P+H) (the balance point of the two
    linear times), chosen by the smaller max-time, ties to the larger: checked with exact
    fractions over a grid."""
    from fractions import Fraction
    for m in range(0, 17):
        for P in (0, 1, 2, 3, 5, 8, 57, 100):
            for H in (0, 1, 2, 3, 5, 8, 57, 100):
                if P + H == 0:
                    continue
                q0 = Fraction(m * P, P + H)
                lo, hi = int(q0), min(m, int(q0) + (q0.denominator != 1))
                t = lambda q: max(Fraction(q, P) if P else (0 if q == 0 else Fraction(10**9)),
                                  Fraction(m - q, H) if H else (0 if q == m else Fraction(10**9)))
                want = hi if t(hi) <= t(lo) else lo
                assert oracle.qstar(m, P, H) == want, (m, P, H)


def test_split_step_invariants_on_markov_trace():
    """step_split: with no host bandwidth it is step; otherwise the first q* misses (ascending
    id) are filled exactly as step fills them, the rest stay out of the cache, and the tables
    stay mutually consistent."""
    w = configs.with_(configs.LRU_DECODE, L=4, E=64, S=48)
    steps = 40
    ids, _ = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    plain, same = LruSim(w.L, w.E, w.S), LruSim(w.L, w.E, w.S)
    split = LruSim(w.L, w.E, w.S)
    P, H = 57000, 30000
    saw_host, n_host = False, 0
    for s in range(steps):
        for layer in range(w.L):
            a = plain.step(layer, ids[s, layer])
            b = same.step_split(layer, ids[s, layer], 1000, 0)
            np.testing.assert_array_equal(a[0], b[0])
            assert a[1] == b[1] and b[2] == []
            resident = split.resident_keys()
            U = sorted(set(int(e) for e in ids[s, layer].ravel()))
            misses = [e for e in U if layer * w.E + e not in resident]
            slot, fills, host = split.step_split(layer, ids[s, layer], P, H)
            q = oracle.qstar(len(misses), P, H)
            assert [e for _, _, e, _ in fills] == misses[:q]
            assert host == misses[q:]
            saw_host |= bool(host)
            n_host += len(host)
            for e in host:
                assert slot[e] == -1 and split.slot_of[layer * w.E + e] == -1
            for e in U:
                if e not in host:
                    assert split.key_of[slot[e]] == layer * w.E + e
            for sl in range(w.S):
                if split.key_of[sl] >= 0:
                    assert split.slot_of[split.key_of[sl]] == sl
    assert saw_host
    assert split.host_runs == n_host
    assert (plain.accesses, plain.hits, plain.misses) == (same.accesses, same.hits, same.misses)


def _markov_trace(L, E, S, steps, seed_shift=0):
    w = configs.with_(configs.LRU_DECODE, L=L, E=E, S=S, steps=steps)
    ids, _ = gen.markov_routing(w.seed + seed_shift, steps, L, w.T, E, w.k, w.p_stay, w.zipf_s)
    return w, ids


def test_resize_to_same_size_is_invisible_to_hits_and_residency():
    """Rebuilding at the same S only renumbers slots: the hit/miss sequence and the resident
    key sets of the rest of the trace equal those of the cache that was never rebuilt."""
    w, ids = _markov_trace(4, 64, 40, 60)
    a, b = LruSim(w.L, w.E, w.S), LruSim(w.L, w.E, w.S)
    for s in range(w.steps):
        if s == 25:
            b = b.resized(w.S)
            assert b.resident_keys() == a.resident_keys()
        for layer in range(w.L):
            _, fa = a.step(layer, ids[s, layer])
            _, fb = b.step(layer, ids[s, layer])
            assert [e for _, _, e, _ in fa] == [e for _, _, e, _ in fb]
            assert a.resident_keys() == b.resident_keys()
    assert (a.accesses, a.hits, a.misses, a.clock) == (b.accesses, b.hits, b.misses, b.clock)


def test_resize_keeps_the_most_recent_entries():
    """Shrinking keeps exactly S_new entries, none used less recently than any dropped one
    (recency tracked independently of the simulator); growing keeps everything and the next
    misses take the new empty slots first; later calls keep every LRU invariant."""
    w, ids = _markov_trace(4, 64, 48, 50, seed_shift=1)
    sim = LruSim(w.L, w.E, w.S)
    last = {}
    call = 0
    for s in range(30):
        for layer in range(w.L):
            sim.step(layer, ids[s, layer])
            call += 1
            for e in set(int(v) for v in ids[s, layer].ravel()):
                last[layer * w.E + e] = call
    before = sim.resident_keys()
    small = sim.resized(20)
    kept = small.resident_keys()
    assert len(kept) == 20 and kept <= before
    dropped = before - kept
    assert min(last[k] for k in kept) >= max(last[k] for k in dropped)
    assert small.clock == sim.clock and small.misses == sim.misses
    big = small.resized(64)
    assert big.resident_keys() == kept
    assert all(big.key_of[j] == -1 and big.stamp[j] == 0 for j in range(20, 64))
    for s in range(30, w.steps):
        for layer in range(w.L):
            before_stamp, before_key = big.stamp.copy(), big.key_of.copy()
            U = sorted(set(int(e) for e in ids[s, layer].ravel()))
            _, fills = big.step(layer, ids[s, layer])
            _check_invariants(big, big.clock, [layer * w.E + e for e in U], fills, before_stamp,
                              before_key)
            if s == 30 and layer == 0 and fills:
                assert fills[0][0] == 20 and fills[0][3] == -1  # first empty slot, no eviction
