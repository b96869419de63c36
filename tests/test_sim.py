"""Pins of the placement / LRU-ring simulator: hand-worked traces (golden
file), an independent list-based LRU model on random traces, calibration
against a full sort, quota arithmetic, the uniform-placement cold-hit rate
under unbiased routing, and the online self-tuning step (against calibration,
and on hand-worked hysteresis, decay and ring cases)."""
import os
from collections import OrderedDict

import numpy as np
import pytest

import oracle


def _run_golden(path):
    sim = None
    checked = 0
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        tok = line.split()
        op, args = tok[0], [int(t) for t in tok[1:] if t.lstrip("-").isdigit()]
        if op == "trace":
            L, E, P, R = args
            sim = oracle.Sim(L, E, P, R, slot_bytes=100)
            sim.place_uniform()
            name = tok[1]
        elif op == "access":
            sim.decode_layer(args[0], np.array([args[1]]))
        elif op == "prefill":  # one token per listed expert: the layer's distinct experts
            sim.prefill_layer(args[0], np.array(args[1:], dtype=np.int32).reshape(-1, 1))
        elif op == "prefetch":
            hist = np.zeros(sim.E, np.int32)
            hist[args[1:]] = 1
            sim.prefetch(args[0], hist)
        elif op == "expect_prefetches":
            assert sim.stats()["prefetches"] == args[0], (name, sim.stats())
            checked += 1
        elif op == "expect_event_kind":
            assert int(sim.events()[args[0] - 1]["kind"]) == args[1], name
            checked += 1
        elif op == "calibrate":
            sim.calibrate(reset_counts=True)
        elif op == "expect_stats":
            st = sim.stats()
            got = [st[k] for k in ("accesses", "pinned_hits", "cold_hits", "ring_hits", "fills",
                                   "evictions")]
            assert got == args, (name, got, args)
            assert st["h2d_bytes"] == 100 * (st["fills"] + st["prefetches"])
            checked += 1
        elif op == "expect_event":
            ev = sim.events()
            seq, layer, expert, slot, victim = args
            e = ev[seq - 1]
            assert (int(e["seq"]), int(e["layer"]), int(e["expert"]), int(e["slot"]),
                    int(e["victim"])) == (seq, layer, expert, slot, victim), (name, e)
            checked += 1
        elif op == "expect_slot_of":
            slot_of = sim.placement()[0]
            assert list(slot_of[args[0]]) == args[1:], (name, slot_of)
            checked += 1
        elif op == "expect_ring":
            owner = sim.placement()[1]
            assert list(owner) == args, (name, owner)
            checked += 1
        elif op == "end":
            sim = None
    return checked


def test_golden_traces(golden_dir):
    assert _run_golden(os.path.join(golden_dir, "placement_traces.txt")) == 30


def test_quota_sums_to_budget():
    for L, P in [(40, 6144), (40, 3072), (40, 10240), (40, 0), (3, 7), (40, 39)]:
        q = [oracle.quota(L, P, l) for l in range(L)]
        assert sum(q) == P and max(q) - min(q) <= 1
        assert q == sorted(q, reverse=True)


class ListLRU:
    """Independent model: an ordered dict of ring residents, least recent
    first; free ring slots handed out lowest first."""

    def __init__(self, L, E, P, R):
        self.L, self.E, self.P, self.R = L, E, P, R
        self.pinned = {}
        nxt = 0
        for l in range(L):
            q = P // L + (1 if l < P % L else 0)
            for e in range(q):
                self.pinned[(l, e)] = nxt
                nxt += 1
        self.ring = OrderedDict()  # key -> ring slot index
        self.stats = dict(accesses=0, pinned_hits=0, cold_hits=0, ring_hits=0, fills=0,
                          evictions=0)
        self.events = []

    def access(self, l, e):
        s = self.stats
        s["accesses"] += 1
        if (l, e) in self.pinned:
            s["pinned_hits"] += 1
            return
        s["cold_hits"] += 1
        key = l * self.E + e
        if key in self.ring:
            s["ring_hits"] += 1
            self.ring.move_to_end(key)
            return
        s["fills"] += 1
        if len(self.ring) < self.R:
            used = set(self.ring.values())
            slot = min(set(range(self.R)) - used)
            victim = -1
        else:
            victim, slot = self.ring.popitem(last=False)
            s["evictions"] += 1
        self.ring[key] = slot
        self.events.append((len(self.events) + 1, l, e, self.P + slot, victim))

    def prefill_layer(self, l, experts):
        """A prefill batch's distinct experts of layer l, ascending; remembers
        how many cold experts the layer's last ring chunk (R at a time) holds."""
        distinct = sorted(set(int(e) for e in experts))
        cold = sum((l, e) not in self.pinned for e in distinct)
        for e in distinct:
            self.access(l, e)
        self.last_cold = 0 if cold == 0 or self.R == 0 else cold - self.R * ((cold - 1) // self.R)

    def prefetch(self, l, candidates):
        budget = self.R - getattr(self, "last_cold", 0)
        n = 0
        for e in sorted(set(int(c) for c in candidates)):
            if n >= budget:
                break
            key = l * self.E + e
            if (l, e) in self.pinned or key in self.ring:
                continue
            self.stats["prefetches"] = self.stats.get("prefetches", 0) + 1
            if len(self.ring) < self.R:
                slot = min(set(range(self.R)) - set(self.ring.values()))
                victim = -1
            else:
                victim, slot = self.ring.popitem(last=False)
                self.stats["evictions"] += 1
            self.ring[key] = slot
            self.events.append((len(self.events) + 1, l, e, self.P + slot, victim))
            n += 1
        return n


@pytest.mark.parametrize("L,E,P,R,K", [(4, 16, 24, 4, 2), (3, 32, 40, 8, 8), (2, 8, 0, 8, 4),
                                       (40, 256, 6144, 32, 8)])
def test_simulator_matches_list_lru_on_random_traces(L, E, P, R, K):
    rng = np.random.default_rng(L * 1000 + E + P + R)
    n_tokens = 200_000 // (L * K) + 1
    sim = oracle.Sim(L, E, P, R, slot_bytes=1)
    sim.place_uniform()
    ref = ListLRU(L, E, P, R)
    # Zipf-ish routing so that ring hits, fills and evictions all occur
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    for t in range(n_tokens):
        idx = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(L)]).astype(np.int32)
        sim.decode_token(idx)
        for l in range(L):
            for e in idx[l]:
                ref.access(l, int(e))
    st = sim.stats()
    for k, v in ref.stats.items():
        assert st[k] == v, (k, st[k], v)
    ev = sim.events()
    got = [(int(e["seq"]), int(e["layer"]), int(e["expert"]), int(e["slot"]), int(e["victim"]))
           for e in ev]
    assert got == ref.events
    assert st["fills"] > 0 and (P == 0 or st["pinned_hits"] > 0)
    if R < E * L - P:
        assert st["evictions"] > 0 and st["ring_hits"] > 0


@pytest.mark.parametrize("L,E,P,R", [(3, 32, 40, 8), (4, 64, 150, 12), (2, 16, 8, 4)])
def test_prefill_prefetch_matches_list_model_on_random_traces(L, E, P, R):
    """Random prefill layers (Zipf-skewed distinct sets, often more cold
    experts than ring slots) each followed by a prefetch of the next layer's
    random candidates: counters, the fill/prefetch log and the ring contents
    equal an independent list model."""
    rng = np.random.default_rng(L * 100 + E + P + R)
    sim = oracle.Sim(L, E, P, R, slot_bytes=1)
    sim.place_uniform()
    ref = ListLRU(L, E, P, R)
    ref.stats["prefetches"] = 0
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    for step in range(400):
        l = step % L
        idx = rng.choice(E, size=(int(rng.integers(1, 40)), 2), p=p).astype(np.int32)
        sim.prefill_layer(l, idx)
        ref.prefill_layer(l, idx.ravel())
        cand = rng.choice(E, size=int(rng.integers(0, 2 * R)), replace=False)
        hist = np.zeros(E, np.int32)
        hist[cand] = 1
        assert sim.prefetch((l + 1) % L, hist) == ref.prefetch((l + 1) % L, cand)
    st = sim.stats()
    for k, v in ref.stats.items():
        assert st[k] == v, (k, st[k], v)
    assert st["h2d_bytes"] == st["fills"] + st["prefetches"]
    got = [(int(e["seq"]), int(e["layer"]), int(e["expert"]), int(e["slot"]), int(e["victim"]))
           for e in sim.events()]
    assert got == ref.events
    kinds = [int(e["kind"]) for e in sim.events()]
    assert kinds.count(oracle.EV_PREFETCH) == st["prefetches"] > 0
    owner = sim.placement()[1]
    ring = {slot: key for key, slot in ref.ring.items()}
    assert [int(o) for o in owner] == [ring.get(r, -1) for r in range(R)]


def test_calibration_matches_full_sort_and_keeps_slots():
    rng = np.random.default_rng(12)
    L, E, P, R = 5, 32, 70, 6
    sim = oracle.Sim(L, E, P, R, slot_bytes=1)
    sim.place_uniform()
    for rnd in range(3):
        before = sim.placement()[0].copy()
        for _ in range(300):
            sim.decode_token(np.stack([rng.choice(E, 3, replace=False, p=None) for _ in range(L)])
                             .astype(np.int32))
        counts = sim.placement()[3].copy()
        sim.calibrate(reset_counts=True)
        slot_of, owner, stamp, counts_after = sim.placement()
        assert not counts_after.any()
        pinned_slots = slot_of[slot_of >= 0]
        assert sorted(pinned_slots.tolist()) == list(range(P))
        for l in range(L):
            q = oracle.quota(L, P, l)
            top = np.lexsort((np.arange(E), -counts[l]))[:q]
            assert set(np.flatnonzero(slot_of[l] >= 0)) == set(top.tolist())
            kept = (before[l] >= 0) & (slot_of[l] >= 0)
            assert np.array_equal(before[l][kept], slot_of[l][kept])
        new = (before < 0) & (slot_of >= 0)
        freed = np.sort(before[(before >= 0) & (slot_of < 0)])
        assert np.array_equal(slot_of[new], freed)  # (layer, expert) order gets ascending slots
        for r in range(R):  # no ring entry of a pinned expert survives
            if owner[r] >= 0:
                assert slot_of.ravel()[owner[r]] < 0


def test_prefill_accesses_distinct_experts_ascending():
    sim = oracle.Sim(1, 8, 2, 3, slot_bytes=1)
    sim.place_uniform()  # pins 0, 1
    idx = np.array([[5, 1], [3, 5], [7, 3], [0, 6]], dtype=np.int32)
    sim.prefill_layer(0, idx)
    st = sim.stats()
    assert st["accesses"] == 6  # distinct {0,1,3,5,6,7}
    assert st["pinned_hits"] == 2 and st["fills"] == 4 and st["evictions"] == 1
    ev = sim.events()
    assert [int(e["expert"]) for e in ev] == [3, 5, 6, 7]
    assert int(ev[3]["victim"]) == 3  # 7 evicts the least recent, 3
    counts = sim.placement()[3]
    assert counts[0].tolist() == [1, 1, 0, 2, 0, 2, 1, 1]


def test_uniform_placement_cold_rate_under_unbiased_routing():
    """Unbiased routing with a uniform 60% pinned set: cold-hit rate = 1 - 0.6
    up to sampling error."""
    rng = np.random.default_rng(13)
    L, E, K = 4, 256, 8
    P = int(0.6 * L * E)
    sim = oracle.Sim(L, E, P, 32, slot_bytes=1)
    sim.place_uniform()
    for _ in range(2000):
        sim.decode_token(np.stack([rng.choice(E, K, replace=False) for _ in range(L)])
                         .astype(np.int32))
    st = sim.stats()
    rate = st["cold_hits"] / st["accesses"]
    q = sum(oracle.quota(L, P, l) for l in range(L)) / (L * E)
    assert abs(rate - (1 - q)) < 0.01


def _sim_with_counts(counts, P, R):
    """A simulator whose layers have exactly these routing counts, reached by
    single-expert decode tokens (K = 1) in a shuffled order."""
    L, E = counts.shape
    sim = oracle.Sim(L, E, P, R, slot_bytes=1)
    sim.place_uniform()
    rng = np.random.default_rng(3)
    per_layer = [rng.permutation(np.repeat(np.arange(E), counts[l])) for l in range(L)]
    for t in range(max(len(p) for p in per_layer)):
        for l in range(L):
            if t < len(per_layer[l]):
                sim.decode_layer(l, np.array([per_layer[l][t]], np.int32))
    assert np.array_equal(sim.placement()[3], counts)
    return sim


def test_retune_without_hysteresis_reaches_the_calibrated_placement():
    """With distinct counts, no hysteresis and no decay, the swap walk ends at
    each layer's top q_l: the same slots, ring and counts as calibration."""
    rng = np.random.default_rng(21)
    L, E, P, R = 3, 16, 20, 4
    counts = np.stack([rng.permutation(E) + 1 for _ in range(L)]).astype(np.int64)
    a = _sim_with_counts(counts, P, R)
    b = _sim_with_counts(counts, P, R)
    swaps = a.retune(0, 0)
    b.calibrate(reset_counts=False)
    for got, ref in zip(a.placement(), b.placement()):
        assert np.array_equal(got, ref)
    before = _sim_with_counts(counts, P, R).placement()[0]
    assert swaps == int(((before < 0) & (a.placement()[0] >= 0)).sum())


def test_retune_hysteresis_decay_and_ring():
    """Hand-worked: one layer, 4 experts, 2 pinned (experts 0 and 1 after the
    uniform placement), counts 2, 10, 12, 1.  Ranked: 2, 1, 0, 3.  Pairs
    (strongest unpinned, weakest pinned): (2, 0), then (3, 1)."""
    counts = np.array([[2, 10, 12, 1]], np.int64)
    sim = _sim_with_counts(counts, P=2, R=2)
    slot_of, owner, _, _ = sim.placement()
    assert slot_of[0].tolist() == [0, 1, -1, -1]
    assert sorted(owner.tolist()) == [2, 3]   # both cold experts sit in the ring
    # 25%: 1200 > 125*2 swaps 2 for 0; 100 > 125*10 fails and ends the layer
    assert sim.retune(25, 1) == 1
    slot_of, owner, stamp, cnt = sim.placement()
    assert slot_of[0].tolist() == [-1, 1, 0, -1]   # expert 2 takes the slot expert 0 freed
    assert 2 not in owner.tolist() and 3 in owner.tolist()
    assert stamp[owner.tolist().index(-1)] == 0
    assert cnt[0].tolist() == [1, 5, 6, 0]           # counts >> 1
    # at 600% the first pair already fails (1200 > 700*2 is false): nothing moves
    sim2 = _sim_with_counts(counts, P=2, R=2)
    assert sim2.retune(600, 0) == 0
    assert sim2.placement()[0][0].tolist() == [0, 1, -1, -1]
    # equal counts never swap, even without hysteresis: counts 5, 5, 5, 1 rank
    # 0, 1, 2, 3 and the first pair (2, 1) has 500 > 500 false
    sim3 = _sim_with_counts(np.array([[5, 5, 5, 1]], np.int64), P=2, R=2)
    assert sim3.retune(0, 0) == 0
    assert sim3.placement()[0][0].tolist() == [0, 1, -1, -1]


@pytest.mark.parametrize("B", [1, 3, 8])
def test_batched_decode_matches_list_lru_in_layer_token_rank_order(B):
    """B tokens through the stack together access in (layer, token, rank)
    order; checked against the independent list model fed in that order, and
    B = 1 against decode_token."""
    L, E, P, R, K = 3, 32, 40, 8, 4
    rng = np.random.default_rng(100 + B)
    sim = oracle.Sim(L, E, P, R, slot_bytes=1)
    sim.place_uniform()
    one = oracle.Sim(L, E, P, R, slot_bytes=1)
    one.place_uniform()
    ref = ListLRU(L, E, P, R)
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    for step in range(300):
        idx = np.stack([np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(L)])
                        for _ in range(B)]).astype(np.int32)
        sim.decode_batch(idx)
        if B == 1:
            one.decode_token(idx[0])
        for l in range(L):
            for b in range(B):
                for e in idx[b, l]:
                    ref.access(l, int(e))
    st = sim.stats()
    for k, v in ref.stats.items():
        assert st[k] == v, (k, st[k], v)
    got = [(int(e["seq"]), int(e["layer"]), int(e["expert"]), int(e["slot"]), int(e["victim"]))
           for e in sim.events()]
    assert got == ref.events and st["ring_hits"] > 0 and st["evictions"] > 0
    if B == 1:
        assert st == one.stats()
