"""Pins for the oracle's return-path dedup (partial combine at the receiving
shard, sum of the partial rows at the source).

* A hand-worked case: two tokens, two shards, slots chosen by hand, expert
  outputs and gates with values a reader can add up, so every expected row
  is written out below.
* Regrouping: without rounding, the partial rows of a token add up to the
  plain combine (every assignment with a row counted exactly once, with its
  own gate).  Checked on random problems, with capped drops and rerouting.
* Row count: one partial row per (token, resident shard) pair that kept the
  token, i.e. exactly the dedup rows of the pass.
"""

from dataclasses import replace

import numpy as np
import pytest

import oracle
from oracle import Problem


def test_hand_worked_two_tokens_two_shards():
    # 4 experts on 2 shards (shard 0: experts 0, 1; shard 1: experts 2, 3),
    # no redundant slots, so slot == expert.  Token 0 picks experts 0 and 1
    # (both on shard 0); token 1 picks experts 2 and 0 (shards 1 and 0).
    p = Problem(tokens=2, seq_len=2, hidden=2, ffn=2, num_experts=4, top_k=2, num_shards=2,
                res_lo=0, res_hi=2, factor=-1.0, num_chunks=1, bf16=False, dedup=True)
    slot = np.array([[0, 1], [2, 0]])
    gates = np.array([[0.75, 0.25], [0.5, 0.5]])
    lay = oracle.pass_layout(p, slot, np.arange(2), None)
    # rows in (slot, t, j) order: (0,0,0) (0,1,1) (1,0,1) (2,1,0)
    assert lay["sorted_assign"].tolist() == [0, 3, 1, 2]
    # dedup rows: shard 0 keeps tokens 0, 1; shard 1 keeps token 1
    assert lay["dedup_offsets"].tolist() == [0, 2, 3]
    assert lay["dedup_token"].tolist() == [0, 1, 1]
    out = np.array([[1.0, 2.0],     # row 0: token 0, expert 0
                    [10.0, 20.0],   # row 1: token 1, expert 0
                    [100.0, 0.0],   # row 2: token 0, expert 1
                    [0.0, 4.0]])    # row 3: token 1, expert 2
    part = oracle.combine_partial(p, out, lay["row_of_assign"], gates, slot,
                                  lay["dedup_offsets"], lay["dedup_token"])
    # (token 0, shard 0) = 0.75*[1,2] + 0.25*[100,0]
    # (token 1, shard 0) = 0.5*[10,20]
    # (token 1, shard 1) = 0.5*[0,4]
    assert part.tolist() == [[25.75, 1.5], [5.0, 10.0], [0.0, 2.0]]
    y = oracle.combine_from_partials(p, part, slot, lay["dedup_offsets"], lay["dedup_token"],
                                     np.arange(2))
    assert y.tolist() == [[25.75, 1.5], [5.0, 12.0]]


def random_case(seed, T=40, E=8, k=3, S=4, res=(0, 4), B=0, R=0, cap=None, zipf=0.0):
    p = Problem(tokens=T, seq_len=T, hidden=5, ffn=4, num_experts=E, top_k=k, num_shards=S,
                res_lo=res[0], res_hi=res[1], factor=1.0, num_chunks=1, bf16=False, dedup=True,
                slots_per_shard=B, num_replicas=R)
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        lg += (-zipf * np.log(np.arange(1, E + 1))).astype(np.float32)
    idx, gates = oracle.route(lg, k, "softmax")
    counts = oracle.expert_counts(idx, E)
    se, ndiv, rep = oracle.plan_redundancy(counts, p)
    slot = oracle.assign_slots(idx, p, ndiv, rep)
    lay = oracle.pass_layout(p, slot, np.arange(T), cap)
    out = rng.standard_normal((lay["num_rows"], p.hidden))
    return p, slot, gates, lay, out


@pytest.mark.parametrize("seed,kw", [
    (0, {}),
    (1, dict(res=(1, 3))),
    (2, dict(cap=6, zipf=1.5)),
    (3, dict(B=1, R=2, zipf=1.2)),
    (4, dict(k=4, E=16, S=8, res=(2, 7), zipf=0.8, cap=9)),
])
def test_partials_regroup_the_plain_combine(seed, kw):
    p, slot, gates, lay, out = random_case(seed, **kw)
    T = p.tokens
    part = oracle.combine_partial(p, out, lay["row_of_assign"], gates, slot,
                                  lay["dedup_offsets"], lay["dedup_token"])
    y_part = oracle.combine_from_partials(p, part, slot, lay["dedup_offsets"],
                                          lay["dedup_token"], np.arange(T))
    y = oracle.combine(p, out, lay["row_of_assign"], gates, np.arange(T))
    np.testing.assert_allclose(y_part, y, rtol=1e-12, atol=1e-12)
    # one partial row per (token, resident shard) pair that kept the token
    pairs = set()
    for t in range(T):
        for j in range(p.top_k):
            if lay["row_of_assign"][t * p.top_k + j] >= 0:
                pairs.add((t, int(slot[t, j]) // p.spd))
    assert len(pairs) == part.shape[0] == int(lay["dedup_offsets"][-1])


def test_partial_of_a_single_assignment_is_gate_times_row():
    # with one assignment per (token, shard) a partial row is g * out[row]
    p, slot, gates, lay, out = random_case(7, E=16, k=2, S=8, res=(0, 8))
    part = oracle.combine_partial(p, out, lay["row_of_assign"], gates, slot,
                                  lay["dedup_offsets"], lay["dedup_token"])
    k = p.top_k
    for u, t in enumerate(lay["dedup_token"]):
        js = [j for j in range(k) if lay["row_of_assign"][t * k + j] >= 0
              and lay["expand_idx"][lay["row_of_assign"][t * k + j]] == u]
        if len(js) == 1:
            j = js[0]
            np.testing.assert_array_equal(part[u], gates[t, j] * out[lay["row_of_assign"][t * k + j]])


def test_partials_are_not_rounded_and_y_is_rounded_once():
    # bf16 storage rounds y once at the source; the partial rows stay exact
    p, slot, gates, lay, out = random_case(5, zipf=1.0)
    p16 = replace(p, bf16=True)
    args = (out, lay["row_of_assign"], gates, slot, lay["dedup_offsets"], lay["dedup_token"])
    part64 = oracle.combine_partial(p, *args)
    part16 = oracle.combine_partial(p16, *args)
    np.testing.assert_array_equal(part16, part64)
    y64 = oracle.combine_from_partials(p, part64, slot, lay["dedup_offsets"],
                                       lay["dedup_token"], np.arange(p.tokens))
    y16 = oracle.combine_from_partials(p16, part16, slot, lay["dedup_offsets"],
                                       lay["dedup_token"], np.arange(p.tokens))
    np.testing.assert_array_equal(y16, oracle.round_bf16(y64))
