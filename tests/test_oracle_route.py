"""Pins for the oracle's router (top-k, gates) and its bf16 rounding.

Top-k is checked against a brute-force comparison sort written from the
definition (logit descending, ties to the lowest expert index), against
hand-built tie cases, and the gates against closed forms.  The bf16 rounding
is checked against torch's float32 -> bfloat16 conversion (round to nearest
even) and hand-computed ties.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_topk(row, k):
    keyed = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return keyed[:k]


@pytest.mark.parametrize("T,E,k", [(7, 5, 2), (16, 8, 3), (9, 33, 8), (5, 4, 4)])
def test_topk_matches_brute_force(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    # coarse values so that exact ties occur often
    lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
    idx, _ = oracle.route(lg, k, "softmax")
    for t in range(T):
        assert list(idx[t]) == brute_topk(lg[t], k)


def test_topk_hand_ties():
    lg = np.array([[1, 3, 3, 2],
                   [0, 0, 0, 0],
                   [0.0, -0.0, -1, 5],
                   [-0.0, 0.0, 0.0, -2]], dtype=np.float32)
    idx, _ = oracle.route(lg, 2, "softmax")
    assert idx.tolist() == [[1, 2], [0, 1], [3, 0], [0, 1]]


def test_softmax_gates_closed_form():
    lg = np.array([[2.0, -1.0, 0.5, 0.25]], dtype=np.float32)
    idx, g = oracle.route(lg, 2, "softmax")
    assert idx.tolist() == [[0, 2]]
    # two chosen logits: g0 = 1 / (1 + exp(l1 - l0))
    assert g[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(0.5 - 2.0)), rel=1e-15)
    assert g[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(2.0 - 0.5)), rel=1e-15)
    _, g1 = oracle.route(lg, 1, "softmax")
    assert g1[0, 0] == 1.0
    rng = np.random.default_rng(3)
    _, gs = oracle.route(rng.standard_normal((50, 16)).astype(np.float32), 5, "softmax")
    assert np.allclose(gs.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(gs, axis=1) <= 0)  # chosen in descending logit order


def test_sigmoid_gates_closed_form():
    lg = np.array([[0.0, -5.0], [math.log(3.0), -7.0]], dtype=np.float32)
    idx, g = oracle.route(lg, 1, "sigmoid")
    assert idx.tolist() == [[0], [0]]
    assert g[0, 0] == 0.5
    assert g[1, 0] == pytest.approx(0.75, rel=1e-7)  # float32(ln 3) rounding


def test_round_bf16_hand_cases():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 1.0,                     # tie, even neighbour 1.0
        one + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,     # tie, odd neighbour rounds up
        one + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7,  # just above the tie
        one + 2.0 ** -8 - 2.0 ** -30: 1.0,        # just below the tie
        -(one + 3 * 2.0 ** -8): -(1.0 + 2.0 ** -6),
        0.0: 0.0,
        3.0: 3.0,
        2.0 - 2.0 ** -9: 2.0,                     # carry into the exponent
    }
    for v, want in cases.items():
        assert oracle.round_bf16(np.array([v]))[0] == want, v


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000),
                        rng.standard_normal(1000)]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_default_chunk_count_golden():
    with open(os.path.join(GOLDEN, "fallback_chunk_count.json")) as f:
        gold = json.load(f)
    assert oracle.default_num_chunks(gold["num_shards"], gold["factor"]) == gold["num_chunks"]
