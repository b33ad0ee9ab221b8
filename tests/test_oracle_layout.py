"""Pins for the oracle's pass layout (stable expert-sorted order, capped
drops, dedup) and the permute.

The row order is checked against numpy's lexsort (a library sort that the
oracle does not use), bijection and stability invariants; capped drops
against per-bucket counting; dedup against brute-force sets and against the
direct permute (bitwise).
"""

import numpy as np
import pytest

import oracle
from oracle import Problem


def setup(T=24, L=None, E=8, k=3, S=4, res=(0, 4), B=0, R=0, dedup=False, seed=0, zipf=0.0):
    L = L or T
    p = Problem(tokens=T, seq_len=L, hidden=4, ffn=4, num_experts=E, top_k=k, num_shards=S,
                res_lo=res[0], res_hi=res[1], factor=1.0, num_chunks=2, dedup=dedup,
                slots_per_shard=B, num_replicas=R)
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        lg += (-zipf * np.log(np.arange(1, E + 1))).astype(np.float32)
    idx, g = oracle.route(lg, k, "softmax")
    counts = oracle.expert_counts(idx, E)
    se, ndiv, rep = oracle.plan_redundancy(counts, p)
    slot = oracle.assign_slots(idx, p, ndiv, rep)
    return p, idx, slot


def lexsort_rows(p, slot, tokens):
    spd = p.spd
    lo, hi = p.res_lo * spd, p.res_hi * spd
    s_list, t_list, j_list = [], [], []
    for t in tokens:
        for j in range(p.top_k):
            if lo <= slot[t, j] < hi:
                s_list.append(slot[t, j]); t_list.append(t); j_list.append(j)
    s_arr, t_arr, j_arr = map(np.asarray, (s_list, t_list, j_list))
    order = np.lexsort((j_arr, t_arr, s_arr))
    return s_arr[order], t_arr[order], j_arr[order]


@pytest.mark.parametrize("kw", [dict(), dict(res=(1, 3)), dict(B=2, R=3, zipf=1.5),
                                dict(T=40, k=1, E=16, S=8, res=(0, 1))])
def test_uncapped_layout_is_lexsort(kw):
    p, idx, slot = setup(**kw)
    toks = np.arange(p.tokens)
    lay = oracle.pass_layout(p, slot, toks, None)
    s, t, j = lexsort_rows(p, slot, toks)
    assert lay["sorted_assign"].tolist() == (t * p.top_k + j).tolist()
    lo = p.res_lo * p.spd
    sizes = np.bincount(s - lo, minlength=(p.res_hi - p.res_lo) * p.spd)
    assert lay["group_sizes"].tolist() == sizes.tolist()
    off = lay["group_offsets"]
    assert off[0] == 0 and np.array_equal(np.diff(off), sizes)
    n = lay["num_rows"]
    roa = lay["row_of_assign"]
    assert np.array_equal(roa[lay["sorted_assign"]], np.arange(n))     # inverse
    assert (roa >= 0).sum() == n                                        # bijection
    for a in range(p.tokens * p.top_k):                                 # the rest are
        if roa[a] < 0:                                                  # not resident
            sa = slot.ravel()[a]
            assert not (p.res_lo * p.spd <= sa < p.res_hi * p.spd)


def test_chunk_tokens_partition():
    p = Problem(tokens=24, seq_len=8, hidden=4, ffn=4, num_experts=4, top_k=1, num_shards=2,
                res_lo=0, res_hi=2, factor=1.0, num_chunks=4)
    chunks = [oracle.pass_tokens(p, 4, c) for c in range(4)]
    assert chunks[1].tolist() == [2, 3, 10, 11, 18, 19]
    allt = np.sort(np.concatenate(chunks))
    assert allt.tolist() == list(range(24))


def test_chunk_layout_is_restriction_of_full_order():
    p, idx, slot = setup(T=32, L=16, k=2)
    full = oracle.pass_layout(p, slot, np.arange(32), None)
    for c in range(4):
        toks = oracle.pass_tokens(p, 4, c)
        lay = oracle.pass_layout(p, slot, toks, None)
        mine = set(toks.tolist())
        restricted = [a for a in full["sorted_assign"] if a // p.top_k in mine]
        assert lay["sorted_assign"].tolist() == restricted


@pytest.mark.parametrize("cap", [0, 1, 5, 9, 1000])
def test_capped_drops_bucket_tail(cap):
    p, idx, slot = setup(T=30, k=2, S=4, E=8)
    toks = np.arange(30)
    full = oracle.pass_layout(p, slot, toks, None)
    lay = oracle.pass_layout(p, slot, toks, cap)
    spd = p.spd
    for d in range(4):
        bucket = [a for a in full["sorted_assign"] if slot.ravel()[a] // spd == d]
        kept = [a for a in lay["sorted_assign"] if slot.ravel()[a] // spd == d]
        assert kept == bucket[:cap]


@pytest.mark.parametrize("kw", [dict(), dict(res=(1, 4)), dict(B=2, R=2, zipf=2.0, k=4)])
def test_dedup_layout_brute_force(kw):
    p, idx, slot = setup(dedup=True, **kw)
    toks = np.arange(p.tokens)
    lay = oracle.pass_layout(p, slot, toks, None)
    spd = p.spd
    d_tok = lay["dedup_token"].tolist()
    d_off = lay["dedup_offsets"].tolist()
    for i, d in enumerate(range(p.res_lo, p.res_hi)):
        want = sorted({t for t in range(p.tokens) for j in range(p.top_k) if slot[t, j] // spd == d})
        assert d_tok[d_off[i]:d_off[i + 1]] == want
    x = np.random.default_rng(9).standard_normal((p.tokens, 5))
    _, xs_dedup = oracle.permute_dedup(x, lay["dedup_token"], lay["expand_idx"])
    xs = oracle.permute(x, lay["sorted_assign"], p.top_k)
    assert np.array_equal(xs, xs_dedup)
    # dedup does not change the row order
    p2 = Problem(**{**p.__dict__, "dedup": False})
    assert np.array_equal(oracle.pass_layout(p2, slot, toks, None)["sorted_assign"],
                          lay["sorted_assign"])


@pytest.mark.parametrize("cap", [0, 3, 7, 100])
def test_dedup_capped_truncates_unique_tokens(cap):
    p, idx, slot = setup(dedup=True, T=30, k=3)
    toks = np.arange(30)
    lay = oracle.pass_layout(p, slot, toks, cap)
    spd = p.spd
    d_off = lay["dedup_offsets"]
    for i, d in enumerate(range(4)):
        uniq = sorted({t for t in range(30) for j in range(3) if slot[t, j] // spd == d})
        kept = uniq[:cap]
        assert lay["dedup_token"][d_off[i]:d_off[i + 1]].tolist() == kept
        rows = [a for a in lay["sorted_assign"] if slot.ravel()[a] // spd == d]
        want = [t * 3 + j for t in range(30) for j in range(3)
                if slot[t, j] // spd == d and t in kept]
        assert sorted(rows) == sorted(want)


def test_permute_rows():
    x = np.arange(12.0).reshape(6, 2)
    xs = oracle.permute(x, np.array([5, 0, 3]), 2)
    assert xs.tolist() == [[4.0, 5.0], [0.0, 1.0], [2.0, 3.0]]
