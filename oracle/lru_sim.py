"""Sequential reference simulator of the global (layer, expert) LRU expert cache.

TEST INFRASTRUCTURE ONLY: used by the tests and by the benchmark's CPU
baseline leg, never by the product path.

Sources (FreeToken pages): the decode phase keeps one shared LRU cache of
recently routed experts, not fixed at start-up, across layers and tokens
(llama page, "Official project overview"; benchmark page, "How FreeToken serves
large MoE models"; RTX-4090 page, "How the MoE memory hierarchy works").  Cache
entries are whole (layer, expert) pairs under one logical mapping (RTX-4090
page, same section).  Misses are filled from the host-resident pool
(benchmark page, runtime-tier table; all misses are filled here since the
CPU-execution half of the miss split is out of scope).

The pages give no tie rules.  Reading taken (one call per (step, layer)):
  t = ++clock
  U = sorted unique requested expert ids (duplicates are one access)
  if |U| > S: capacity error, nothing changes (clock included)
  hits: every resident e in U gets stamp t
  misses: U minus hits, ascending id
  candidates: slots with stamp < t ordered by (stamp, slot) -- empty slots
              (stamp 0) first, in slot order; entries used in this call are
              never evicted by it
  the i-th miss takes the i-th candidate, evicting its old key; the fill
  record (slot, layer, expert, old key or -1) is emitted in miss order.
"""
import numpy as np


class LruSim:
    def __init__(self, L, E, S):
        self.L, self.E, self.S = L, E, S
        self.key_of = np.full(S, -1, dtype=np.int64)
        self.slot_of = np.full(L * E, -1, dtype=np.int64)
        self.stamp = np.zeros(S, dtype=np.int64)
        self.clock = 0
        self.accesses = self.hits = self.misses = 0

    def step(self, layer, ids):
        """One lookup/update for `layer` with requested expert ids (any shape).

        Returns (expert_slot[E] with -1 for unrequested experts, fills list of
        (slot, layer, expert, evicted_key)), or raises CapacityError.
        """
        U = sorted(set(int(e) for e in np.asarray(ids).ravel()))
        if len(U) > self.S:
            raise CapacityError(len(U), self.S)
        self.clock += 1
        t = self.clock
        expert_slot = np.full(self.E, -1, dtype=np.int64)
        misses = []
        for e in U:
            s = self.slot_of[layer * self.E + e]
            if s >= 0:
                self.stamp[s] = t
                expert_slot[e] = s
            else:
                misses.append(e)
        free = np.nonzero(self.stamp < t)[0]
        cand = free[np.lexsort((free, self.stamp[free]))]  # by (stamp, slot)
        fills = []
        for i, e in enumerate(misses):
            s = int(cand[i])
            old = int(self.key_of[s])
            if old >= 0:
                self.slot_of[old] = -1
            key = layer * self.E + e
            self.key_of[s] = key
            self.slot_of[key] = s
            self.stamp[s] = t
            expert_slot[e] = s
            fills.append((s, layer, e, old))
        self.accesses += len(U)
        self.hits += len(U) - len(misses)
        self.misses += len(misses)
        return expert_slot, fills

    def resident_keys(self):
        return set(int(k) for k in self.key_of if k >= 0)


class CapacityError(Exception):
    def __init__(self, need, have):
        super().__init__(f"{need} unique experts requested, cache has {have} slots")
        self.need, self.have = need, have


class StaticPlacement:
    """Routing-agnostic baseline: a fixed set of S entries, chosen once, never changed."""

    def __init__(self, resident_keys):
        self.resident = set(int(k) for k in resident_keys)
        self.accesses = self.hits = self.misses = 0

    def step(self, layer, ids, E):
        U = set(int(e) for e in np.asarray(ids).ravel())
        h = sum(1 for e in U if layer * E + e in self.resident)
        self.accesses += len(U)
        self.hits += h
        self.misses += len(U) - h
