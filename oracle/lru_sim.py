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
CPU-execution half of the miss split is out of scope; step_split decides only which
misses are filled and which are left to the host).

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


def qstar(m, pcie_mbps, host_mbps):
    """How many of m missed entries to fill over PCIe when the others run on the host.

    FreeToken pages: the runtime profiles host-side expert throughput and pinned PCIe
    bandwidth and uses the two measurements to decide how many misses move to the GPU and
    how many execute on the CPU, so both links work at once (benchmark page, "How FreeToken
    serves large MoE models", where the q-star policy is named, its runtime-tier table and
    the "adaptive cache miss" feature card; RTX-4090 page, "Setup and tuning workflow",
    step "Measure the system").  The pages give no formula.  Reading:
    the two paths run concurrently, so the step waits for the slower one; q* minimises
    max(q * B / P, (m - q) * B / H) over q = 0..m (B = entry bytes), ties to the larger q
    (more fills keep the cache warm).  Compared as max(q * H, (m - q) * P) in integers
    (bandwidths in MB/s), so no rounding decides the count.
    """
    if pcie_mbps < 0 or host_mbps < 0 or pcie_mbps + host_mbps == 0:
        raise ValueError("bandwidths must be >= 0 and not both 0")
    best_q, best_t = 0, None
    for q in range(m + 1):
        t = max(q * host_mbps, (m - q) * pcie_mbps)
        if best_t is None or t <= best_t:
            best_q, best_t = q, t
    return best_q


class LruSim:
    def __init__(self, L, E, S):
        self.L, self.E, self.S = L, E, S
        self.key_of = np.full(S, -1, dtype=np.int64)
        self.slot_of = np.full(L * E, -1, dtype=np.int64)
        self.stamp = np.zeros(S, dtype=np.int64)
        self.clock = 0
        self.accesses = self.hits = self.misses = 0
        self.host_runs = 0  # misses left to the host by step_split

    def step(self, layer, ids):
        """One lookup/update for `layer` with requested expert ids (any shape).

        Returns (expert_slot[E] with -1 for unrequested experts, fills list of
        (slot, layer, expert, evicted_key)), or raises CapacityError.
        """
        expert_slot, fills, _ = self._step(layer, ids, None)
        return expert_slot, fills

    def step_split(self, layer, ids, pcie_mbps, host_mbps):
        """As step, with the misses split by qstar: the first q* misses (ascending id) are
        filled as in step; the rest run on the host, so they take no slot, are not inserted
        and keep expert_slot -1.  Returns (expert_slot, fills, host_experts)."""
        return self._step(layer, ids, (pcie_mbps, host_mbps))

    def _step(self, layer, ids, split):
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
        n_fill = len(misses) if split is None else qstar(len(misses), *split)
        to_host = misses[n_fill:]
        free = np.nonzero(self.stamp < t)[0]
        cand = free[np.lexsort((free, self.stamp[free]))]  # by (stamp, slot)
        fills = []
        for i, e in enumerate(misses[:n_fill]):
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
        self.host_runs += len(to_host)
        return expert_slot, fills, to_host

    def resident_keys(self):
        return set(int(k) for k in self.key_of if k >= 0)

    def resized(self, S_new):
        """The cache rebuilt with S_new slots at a safe point, keeping the most recent entries.

        FreeToken pages: the GPU expert capacity can be reconfigured at a safe runtime point
        without restarting the engine or reloading the host-resident pool (benchmark page,
        "elastic cache" feature card; vram page, on the 2026 paper's elastic memory).  No
        rule is given for what survives.  Reading: keep the min(S_new, resident) entries
        used most recently (stamp descending, ties to the lower slot), place them in slots
        0..n-1 in ascending order of their old slot (so the relative order that breaks
        stamp ties is kept), keep their stamps; the clock and the counters carry over.
        """
        if S_new <= 0:
            raise ValueError("S_new must be positive")
        occ = [s for s in range(self.S) if self.key_of[s] >= 0]
        keep = sorted(occ, key=lambda s: (-int(self.stamp[s]), s))[:S_new]
        new = LruSim(self.L, self.E, S_new)
        for j, s in enumerate(sorted(keep)):
            key = int(self.key_of[s])
            new.key_of[j] = key
            new.slot_of[key] = j
            new.stamp[j] = self.stamp[s]
        new.clock = self.clock
        new.accesses, new.hits, new.misses = self.accesses, self.hits, self.misses
        new.host_runs = self.host_runs
        return new


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
