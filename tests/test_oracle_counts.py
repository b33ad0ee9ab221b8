"""Pins for counts, capacity, overflow, the redundancy plan and reroute.

Counts are checked against brute-force loops and conservation laws; the cap
and the overflow predicate against hand values and the page facts stored
under tests/golden; the greedy plan against hand-worked examples and its
invariants (load conservation, n_div <= c_e, no expert duplicated twice,
has_candidate stop).
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def prob(**kw):
    base = dict(tokens=16, seq_len=16, hidden=8, ffn=8, num_experts=8, top_k=2,
                num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=2)
    base.update(kw)
    return Problem(**base)


def random_idx(T, E, k, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    return oracle.route(lg, k, "softmax")[0]


@pytest.mark.parametrize("T,E,k,seed", [(16, 8, 2, 0), (40, 12, 3, 1), (33, 16, 8, 2)])
def test_expert_counts_brute_force(T, E, k, seed):
    idx = random_idx(T, E, k, seed)
    c = oracle.expert_counts(idx, E)
    want = [0] * E
    for t in range(T):
        for j in range(k):
            want[int(idx[t, j])] += 1
    assert c.tolist() == want
    assert c.sum() == T * k


@pytest.mark.parametrize("dedup", [False, True])
def test_shard_counts_brute_force(dedup):
    p = prob(tokens=40, seq_len=40, num_experts=12, top_k=3, num_shards=4, dedup=dedup)
    idx = random_idx(40, 12, 3, 5)
    slot = oracle.assign_slots(idx, p, np.zeros(12, np.int64), np.full(12, -1))
    sc = oracle.shard_counts(slot, p)
    El = p.e_loc
    want = [0] * 4
    for t in range(40):
        seen = set()
        for j in range(3):
            d = int(idx[t, j]) // El
            if dedup:
                if d in seen:
                    continue
                seen.add(d)
            want[d] += 1
    assert sc.tolist() == want
    if not dedup:
        assert sc.sum() == 40 * 3
    else:
        counts = oracle.expert_counts(idx, 12)
        for d in range(4):
            assert max(counts[d * El:(d + 1) * El]) <= sc[d] <= 40
        assert sc.sum() <= 40 * 3


def test_home_slots_without_redundancy():
    p = prob(num_experts=8, num_shards=4, slots_per_shard=2)
    idx = np.arange(8, dtype=np.int32).reshape(4, 2)
    slot = oracle.assign_slots(idx, p, np.zeros(8, np.int64), np.full(8, -1))
    # E_loc = 2, 4 slots per shard: expert e -> (e // 2) * 4 + e % 2
    assert slot.ravel().tolist() == [0, 1, 4, 5, 8, 9, 12, 13]


def test_capacity_hand_values():
    assert oracle.capacity(prob(tokens=4096, top_k=4, num_shards=8, factor=1.5)) == 3072
    assert oracle.capacity(prob(tokens=256, top_k=2, num_shards=4, factor=2.0)) == 256
    assert oracle.capacity(prob(tokens=32768, top_k=1, num_shards=16, factor=2.0)) == 4096
    # float32(0.1) = 0.100000001490116...: 0.1 * 512 / 4 = 12.8000002 -> 13
    assert oracle.capacity(prob(tokens=256, top_k=2, num_shards=4, factor=0.1)) == 13
    # 0.5 * 30 / 4 = 3.75 -> 4 (rounds up)
    assert oracle.capacity(prob(tokens=15, top_k=2, num_shards=4, factor=0.5)) == 4
    assert oracle.capacity(prob(factor=-1.0)) is None
    assert oracle.capacity(prob(factor=0.0)) is None


def test_overflow_is_strict():
    assert not oracle.overflow(np.array([8192, 100]), 8192)
    assert oracle.overflow(np.array([8193, 100]), 8192)
    assert oracle.overflow(np.array([0, 0, 0, 5]), 4)
    assert not oracle.overflow(np.array([10 ** 9]), None)


def test_capacity_page_facts():
    """Factor 0.1 overflows and -1 never does ([FALLBACK] Tests / Why)."""
    with open(os.path.join(GOLDEN, "capacity_facts.json")) as f:
        facts = json.load(f)["facts"]
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((64, 8)).astype(np.float32)
    for fact in facts:
        p = prob(tokens=64, seq_len=64, factor=fact["factor"])
        idx, _ = oracle.route(lg, 2, "softmax")
        slot = oracle.assign_slots(idx, p, np.zeros(8, np.int64), np.full(8, -1))
        assert oracle.overflow(oracle.shard_counts(slot, p), oracle.capacity(p)) == fact["overflow"]


def test_single_shard_overflow_flags():
    """Only one shard overflows, yet the flag is raised ([FALLBACK] Tests:
    the asymmetric-overflow case)."""
    p = prob(tokens=32, seq_len=32, num_experts=8, top_k=2, num_shards=4, factor=1.0)
    lg = np.zeros((32, 8), np.float32)
    lg[:, 0] = 5.0   # every token's first choice is expert 0 (shard 0)
    lg[:, 1] = 1.0 * (np.arange(32) % 2)  # second choice: expert 1 or 2
    lg[:, 2] = 1.0 * (1 - np.arange(32) % 2)
    idx, _ = oracle.route(lg, 2, "softmax")
    slot = oracle.assign_slots(idx, p, np.zeros(8, np.int64), np.full(8, -1))
    sc = oracle.shard_counts(slot, p)
    assert sc.tolist() == [48, 16, 0, 0]
    cap = oracle.capacity(p)
    assert cap == 16
    assert oracle.overflow(sc, cap)
    assert oracle.required_factor(sc, p) == 3.0


def test_plan_worked_example_partial_fraction():
    """S=2, E_loc=2, B=1, R=2, counts [6,2,1,1]: loads [8,2]; e0 goes to
    shard 1's redundant slot with n_div = min(6, (8-2)//2) = 3, loads [5,5];
    the second iteration stops because the only shard with a free slot is
    shard 0 and 5 <= 5."""
    p = prob(num_experts=4, num_shards=2, slots_per_shard=1, num_replicas=2)
    se, ndiv, rep = oracle.plan_redundancy(np.array([6, 2, 1, 1]), p)
    assert se.tolist() == [0, 1, -1, 2, 3, 0]
    assert ndiv.tolist() == [3, 0, 0, 0]
    assert rep.tolist() == [5, -1, -1, -1]


def test_plan_has_candidate_stop():
    """S=2, E_loc=1, B=2, R=3, counts [10, 0]: e0 -> shard 1 (n_div 5, loads
    [5,5]); next r_max is shard 0 again, whose only expert is duplicated, so
    planning stops ([DRED] has_candidate guard) instead of duplicating e0
    twice."""
    p = prob(num_experts=2, num_shards=2, slots_per_shard=2, num_replicas=3)
    se, ndiv, rep = oracle.plan_redundancy(np.array([10, 0]), p)
    assert se.tolist() == [0, -1, -1, 1, 0, -1]
    assert ndiv.tolist() == [5, 0]
    assert rep.tolist() == [4, -1]


def test_plan_fraction_one_and_second_iteration():
    """S=4, E_loc=2, B=1, R=2, counts [9,7,1,0,1,1,0,1]: loads [16,1,2,1].
    Iteration 1: r_max 0, hottest e0 (9), r_min shard 1 (load 1, lowest of the
    tied minima), n_div = min(9, 15//2=7) = 7 -> slot 1*3+2 = 5; loads
    [9,8,2,1].  Iteration 2: r_max 0, candidate e1 (7), r_min shard 3 (load 1;
    shard 1's slot is used), n_div = min(7, 8//2=4) = 4 -> slot 3*3+2 = 11;
    loads [5,8,2,5]."""
    p = prob(num_experts=8, num_shards=4, slots_per_shard=1, num_replicas=2)
    counts = np.array([9, 7, 1, 0, 1, 1, 0, 1])
    se, ndiv, rep = oracle.plan_redundancy(counts, p)
    assert se.tolist() == [0, 1, -1, 2, 3, 0, 4, 5, -1, 6, 7, 1]
    assert ndiv.tolist() == [7, 4, 0, 0, 0, 0, 0, 0]
    assert rep.tolist() == [5, 11, -1, -1, -1, -1, -1, -1]


@pytest.mark.parametrize("seed", range(8))
def test_plan_invariants(seed):
    rng = np.random.default_rng(seed)
    S, El, B, R = 6, 3, 2, 7
    p = prob(num_experts=S * El, num_shards=S, slots_per_shard=B, num_replicas=R)
    counts = (rng.zipf(1.5, S * El) % 50).astype(np.int64)
    se, ndiv, rep = oracle.plan_redundancy(counts, p)
    spd = El + B
    load = np.array([counts[d * El:(d + 1) * El].sum() for d in range(S)])
    moved = np.zeros(S, np.int64)
    dup = [e for e in range(S * El) if ndiv[e] > 0]
    assert len(dup) <= R
    assert len(set(dup)) == len(dup)
    for e in dup:
        s = rep[e]
        assert se[s] == e
        assert s % spd >= El                         # a redundant slot
        assert s // spd != e // El                   # on another shard
        assert 0 < ndiv[e] <= counts[e]
        moved[e // El] -= ndiv[e]
        moved[s // spd] += ndiv[e]
    assert (load + moved).sum() == load.sum()        # load is conserved
    for d in range(S):                               # slots fill from the first
        used = [se[d * spd + El + b] >= 0 for b in range(B)]
        assert used == sorted(used, reverse=True)


def test_reroute_first_ndiv_in_flat_order():
    p = prob(tokens=6, seq_len=6, num_experts=4, top_k=2, num_shards=2,
             slots_per_shard=1, num_replicas=1)
    idx = np.array([[0, 1], [2, 0], [0, 3], [1, 0], [0, 2], [3, 1]], np.int32)
    ndiv = np.array([2, 0, 0, 0])
    rep = np.array([5, -1, -1, -1])
    slot = oracle.assign_slots(idx, p, ndiv, rep)
    # expert 0 appears at flat positions 0, 3, 4, 7, 8: the first two reroute
    home = {0: 0, 1: 1, 2: 3, 3: 4}
    want = []
    seen0 = 0
    for t in range(6):
        for j in range(2):
            e = int(idx[t, j])
            if e == 0 and seen0 < 2:
                want.append(5)
                seen0 += 1
            else:
                want.append(home[e])
    assert slot.ravel().tolist() == want
    assert slot.ravel().tolist()[:5] == [5, 1, 3, 5, 0]
