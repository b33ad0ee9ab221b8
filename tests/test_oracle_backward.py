"""Pins for the oracle's backward (oracle/moe_backward.py).

Every gradient is checked against central differences of the forward
oracle in float64 (unrounded storage), which the forward's own pins tie to
the pages and to textbook routines; the permute's backward against its
adjoint identity; the gate derivatives against closed forms.  Logits are
perturbed by 2^-10, which float32 (the router's input type) represents
exactly at these magnitudes, so the differences see no input rounding.
"""

from dataclasses import replace

import numpy as np
import pytest

import oracle
from oracle import Problem

EPS = 1e-6
LEPS = 2.0 ** -10


def central(f, v, idx, eps):
    """(f(v + eps e_idx) - f(v - eps e_idx)) / (2 eps), v restored."""
    old = v[idx]
    v[idx] = old + eps
    fp = f()
    v[idx] = old - eps
    fm = f()
    v[idx] = old
    return (fp - fm) / (2 * eps)


def check_fd(f, v, grad, eps=EPS, rtol=1e-6, atol=1e-9, sample=None, rng=None):
    idxs = list(np.ndindex(v.shape))
    if sample is not None and len(idxs) > sample:
        idxs = [idxs[i] for i in rng.choice(len(idxs), size=sample, replace=False)]
    for idx in idxs:
        num = central(f, v, idx, eps)
        assert abs(num - grad[idx]) <= atol + rtol * abs(num), (idx, num, grad[idx])


def test_ffn_backward_central_differences():
    rng = np.random.default_rng(0)
    n, H, F = 5, 6, 4
    x = rng.standard_normal((n, H))
    wg, wu = rng.standard_normal((F, H)) * 0.5, rng.standard_normal((F, H)) * 0.5
    wd = rng.standard_normal((H, F)) * 0.5
    d_o = rng.standard_normal((n, H))
    dx, dwg, dwu, dwd = oracle.expert_ffn_bwd(x, wg, wu, wd, d_o, False)

    def loss():
        return float(np.sum(d_o * oracle.expert_ffn(x, wg, wu, wd, False)[1]))

    for v, g in ((x, dx), (wg, dwg), (wu, dwu), (wd, dwd)):
        check_fd(loss, v, g)


def test_silu_derivative_closed_form():
    # one row, one hidden unit, unit weights: d_hg = d_a * h_u * SiLU'(h_g)
    # with SiLU'(0) = 1/2 and SiLU'(z) -> 1 for large z
    for z, want in ((0.0, 0.5), (30.0, 1.0)):
        x = np.array([[z]])
        one = np.array([[1.0]])
        dx, dwg, dwu, dwd = oracle.expert_ffn_bwd(x, one, one, one, one, False)
        # d_a = 1, h_u = z: d_hg = z * SiLU'(z), d_hu = SiLU(z); dx = d_hg + d_hu
        silu = z / (1 + np.exp(-z))
        np.testing.assert_allclose(dx[0, 0], z * want + silu, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dwd[0, 0], silu * z, rtol=1e-12)


def small_problem(**kw):
    base = dict(tokens=12, seq_len=6, hidden=4, ffn=3, num_experts=8, top_k=2, num_shards=4,
                res_lo=0, res_hi=4, factor=1.0, num_chunks=2, bf16=False)
    base.update(kw)
    return Problem(**base)


def test_combine_backward_central_differences():
    rng = np.random.default_rng(1)
    p = small_problem()
    lg = rng.standard_normal((p.tokens, p.num_experts)).astype(np.float32)
    idx, gates = oracle.route(lg, p.top_k, p.gate)
    counts = oracle.expert_counts(idx, p.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, p)
    slot = oracle.assign_slots(idx, p, ndiv, rep)
    toks = oracle.pass_tokens(p, 2, 1)
    lay = oracle.pass_layout(p, slot, toks, None)
    out = rng.standard_normal((lay["num_rows"], p.hidden))
    dy = rng.standard_normal((p.tokens, p.hidden))
    gates = np.array(gates)
    d_out, d_gate = oracle.combine_bwd(p, dy, out, lay["row_of_assign"], gates, toks,
                                       lay["num_rows"])

    def loss():
        return float(np.sum(dy[toks] * oracle.combine(p, out, lay["row_of_assign"], gates, toks)))

    check_fd(loss, out, d_out)
    check_fd(loss, gates, d_gate)
    # tokens outside the pass get no gate gradient
    rest = np.setdiff1d(np.arange(p.tokens), toks)
    assert np.all(d_gate[rest] == 0)


@pytest.mark.parametrize("cap", [None, 2])
def test_permute_backward_is_the_adjoint(cap):
    # <dys, permute(x)> = <permute_bwd(dys), x> over the pass's tokens
    rng = np.random.default_rng(2)
    p = small_problem(num_experts=8, top_k=3)
    lg = rng.standard_normal((p.tokens, p.num_experts)).astype(np.float32)
    idx, _ = oracle.route(lg, p.top_k, p.gate)
    slot = oracle.assign_slots(idx, p, np.zeros(8, dtype=np.int64), np.full(8, -1))
    toks = np.arange(p.tokens)
    lay = oracle.pass_layout(p, slot, toks, cap)
    x = rng.standard_normal((p.tokens, p.hidden))
    dys = rng.standard_normal((lay["num_rows"], p.hidden))
    lhs = np.sum(dys * oracle.permute(x, lay["sorted_assign"], p.top_k))
    rhs = np.sum(oracle.permute_bwd(p, dys, lay["row_of_assign"], toks) * x)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)


def exact_logits(rng, T, E, k):
    """float32 logits on a 2^-6 grid whose k+1 largest of every token are
    at least 2^-4 apart, so a 2^-10 step changes neither the chosen set nor
    its order."""
    out = np.empty((T, E))
    for t in range(T):
        while True:
            row = np.round(rng.standard_normal(E) * 64) / 64
            s = -np.sort(-row)
            if np.all(s[:k] - s[1:k + 1] >= 2.0 ** -4):
                out[t] = row
                break
    return out.astype(np.float32)


@pytest.mark.parametrize("gate", ["softmax", "sigmoid"])
def test_route_backward_central_differences(gate):
    rng = np.random.default_rng(3)
    p = small_problem(gate=gate, top_k=3)
    lg = exact_logits(rng, p.tokens, p.num_experts, p.top_k).astype(np.float64)
    idx, g = oracle.route(lg, p.top_k, gate)
    dg = rng.standard_normal(g.shape)
    dl = oracle.route_bwd(p, idx, g, dg)

    def loss():
        i2, g2 = oracle.route(lg.astype(np.float32), p.top_k, gate)
        assert np.array_equal(i2, idx)
        return float(np.sum(dg * g2))

    check_fd(loss, lg, dl, eps=LEPS, rtol=1e-5, atol=1e-8)
    if gate == "softmax":
        # the gates sum to one, so their logit gradients sum to zero
        np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    else:
        # at logit 0 the sigmoid's slope is 1/4
        p1 = replace(p, tokens=1)
        d0 = oracle.route_bwd(p1, np.array([[0, 1, 2]]), np.full((1, 3), 0.5),
                              np.array([[1.0, 2.0, -4.0]]))
        np.testing.assert_allclose(d0[0, :3], [0.25, 0.5, -1.0], rtol=1e-15)


def test_grouped_gemm_backward_with_a_replica_group():
    # three groups, the third a replica of expert 0: its rows add into
    # expert 0's weight gradients
    rng = np.random.default_rng(4)
    p = small_problem(hidden=5, ffn=4)
    go = np.array([0, 3, 5, 9])
    ge = np.array([0, 1, 0])
    xs = rng.standard_normal((9, p.hidden))
    wg = rng.standard_normal((2, p.ffn, p.hidden)) * 0.5
    wu = rng.standard_normal((2, p.ffn, p.hidden)) * 0.5
    wd = rng.standard_normal((2, p.hidden, p.ffn)) * 0.5
    d_out = rng.standard_normal((9, p.hidden))
    dx, dwg, dwu, dwd = oracle.gmm_swiglu_bwd(p, xs, go, ge, wg, wu, wd, d_out)

    def loss():
        return float(np.sum(d_out * oracle.gmm_swiglu(p, xs, go, ge, wg, wu, wd)[1]))

    for v, g in ((xs, dx), (wg, dwg), (wu, dwu), (wd, dwd)):
        check_fd(loss, v, g)


LAYER_CASES = [
    # (mode, problem overrides): chunked fallback, capped drops, dropless,
    # redundant slots, a partial residency, sigmoid gates
    (oracle.MODE_LAYER, dict(factor=1.0)),
    (oracle.MODE_CAPPED_ONLY, dict(factor=0.5)),
    (oracle.MODE_FORCE_DROPLESS, dict(factor=-1.0)),
    (oracle.MODE_FORCE_CHUNKED, dict(slots_per_shard=1, num_replicas=2)),
    (oracle.MODE_LAYER, dict(res_lo=1, res_hi=3, gate="sigmoid")),
]


@pytest.mark.parametrize("mode,kw", LAYER_CASES)
def test_layer_backward_central_differences(mode, kw):
    rng = np.random.default_rng(5)
    p = small_problem(**kw)
    e_res = (p.res_hi - p.res_lo) * p.e_loc
    zipf = -1.5 * np.log(np.arange(1, p.num_experts + 1))
    lg = exact_logits(rng, p.tokens, p.num_experts, p.top_k).astype(np.float64)
    # Zipf-skewed routing (overflows the cap), kept on the grid and gapped
    lg = np.round((lg + zipf) * 64) / 64
    s = -np.sort(-lg, axis=1)
    bad = np.any(s[:, :p.top_k] - s[:, 1:p.top_k + 1] < 2.0 ** -4, axis=1)
    lg[bad] = exact_logits(rng, int(bad.sum()), p.num_experts, p.top_k)
    x = rng.standard_normal((p.tokens, p.hidden))
    wg = rng.standard_normal((e_res, p.ffn, p.hidden)) * 0.5
    wu = rng.standard_normal((e_res, p.ffn, p.hidden)) * 0.5
    wd = rng.standard_normal((e_res, p.hidden, p.ffn)) * 0.5
    dy = rng.standard_normal((p.tokens, p.hidden))
    g = oracle.layer_bwd(p, mode, lg, x, wg, wu, wd, dy)
    fwd = oracle.layer(p, mode, lg, x, wg, wu, wd)
    assert g["fallback_ran"] == fwd["fallback_ran"]

    def loss():
        r = oracle.layer(p, mode, lg.astype(np.float32), x, wg, wu, wd)
        assert np.array_equal(r["slot_of_assign"], fwd["slot_of_assign"])
        return float(np.sum(dy * r["y"]))

    check_fd(loss, x, g["dx"])
    for v, name in ((wg, "dw_gate"), (wu, "dw_up"), (wd, "dw_down")):
        check_fd(loss, v, g[name], sample=24, rng=rng)
    check_fd(loss, lg, g["d_logits"], eps=LEPS, rtol=1e-5, atol=1e-8)


def test_chunked_and_single_pass_gradients_agree():
    # both dropless modes compute the same function, so the chunked
    # backward (gradients carried across passes) equals the one-pass one
    rng = np.random.default_rng(6)
    p = small_problem(factor=-1.0, num_chunks=3, tokens=18, seq_len=9)
    lg = rng.standard_normal((p.tokens, p.num_experts)).astype(np.float32)
    x = rng.standard_normal((p.tokens, p.hidden))
    w = [rng.standard_normal((p.num_experts, p.ffn, p.hidden)),
         rng.standard_normal((p.num_experts, p.ffn, p.hidden)),
         rng.standard_normal((p.num_experts, p.hidden, p.ffn))]
    dy = rng.standard_normal((p.tokens, p.hidden))
    a = oracle.layer_bwd(p, oracle.MODE_FORCE_CHUNKED, lg, x, *w, dy)
    b = oracle.layer_bwd(p, oracle.MODE_FORCE_DROPLESS, lg, x, *w, dy)
    assert a["fallback_ran"] and not b["fallback_ran"]
    for name in ("dx", "d_logits", "d_gate", "dw_gate", "dw_up", "dw_down"):
        np.testing.assert_allclose(a[name], b[name], rtol=1e-12, atol=1e-12, err_msg=name)


def test_bf16_storage_stays_within_the_layer_tolerance():
    # rounding the stored intermediates to bf16 moves the gradients by
    # about the bf16 step, never by more than the layer's tolerance
    rng = np.random.default_rng(7)
    p = small_problem(hidden=16, ffn=8, factor=-1.0)
    lg = rng.standard_normal((p.tokens, p.num_experts)).astype(np.float32)
    r = oracle.round_bf16
    x = r(rng.standard_normal((p.tokens, p.hidden)))
    w = [r(rng.standard_normal((p.num_experts, p.ffn, p.hidden)) * 0.3),
         r(rng.standard_normal((p.num_experts, p.ffn, p.hidden)) * 0.3),
         r(rng.standard_normal((p.num_experts, p.hidden, p.ffn)) * 0.3)]
    dy = r(rng.standard_normal((p.tokens, p.hidden)))
    a = oracle.layer_bwd(p, oracle.MODE_FORCE_DROPLESS, lg, x, *w, dy)
    b = oracle.layer_bwd(replace(p, bf16=True), oracle.MODE_FORCE_DROPLESS, lg, x, *w, dy)
    for name in ("dx", "dw_gate", "dw_up", "dw_down", "d_logits"):
        ref = a[name]
        err = np.abs(b[name] - ref).max() / max(np.abs(ref).max(), 1e-30)
        assert 0 < err < 2e-2, (name, err)
    # dx is stored in bf16
    np.testing.assert_array_equal(b["dx"], r(b["dx"]))


def test_per_expert_tolerance_catches_a_zeroed_cold_expert():
    """The weight-gradient check of the GPU tests, expert by expert: a cold
    expert's slice 1e4 times below the hot one's, left at zero by a faulty
    kernel, passes the whole-tensor bound but fails the per-expert one."""
    import pytest
    from moe_cases import check_close_grad, check_close_grad_per_expert
    rng = np.random.default_rng(3)
    ref = np.stack([rng.standard_normal((8, 8)), 1e-4 * rng.standard_normal((8, 8))])
    got = ref.copy()
    got[1] = 0.0
    check_close_grad(got, ref)
    with pytest.raises(AssertionError):
        check_close_grad_per_expert(got, ref)
    check_close_grad_per_expert(ref * (1 + 1e-4), ref)
