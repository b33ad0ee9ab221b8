"""Pins for the oracle's expert FFN, combine and the layer modes.

The FFN is checked against torch's textbook SwiGLU MLP (torch.nn.functional
.silu, float64); the whole layer against a dense mixture that runs every
expert on every token with no sorting (pins permute + GEMM + combine
together); combine against identity experts; the modes against each other
([FALLBACK] Tests: the fallback matches dropless, the capped model
diverges) and dedup/redundancy against the plain layer.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import Problem


def make(T=32, L=None, H=16, F=24, E=8, k=2, S=4, res=(0, 4), factor=2.0, chunks=4,
         gate="softmax", bf16=False, dedup=False, B=0, R=0, seed=0, zipf=0.0):
    L = L or T
    p = Problem(tokens=T, seq_len=L, hidden=H, ffn=F, num_experts=E, top_k=k, num_shards=S,
                res_lo=res[0], res_hi=res[1], factor=factor, num_chunks=chunks, gate=gate,
                bf16=bf16, dedup=dedup, slots_per_shard=B, num_replicas=R)
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        lg += (-zipf * np.log(np.arange(1, E + 1))).astype(np.float32)
    x = rng.standard_normal((T, H))
    e_res = (res[1] - res[0]) * (E // S)
    wg = rng.standard_normal((e_res, F, H)) * 0.3
    wu = rng.standard_normal((e_res, F, H)) * 0.3
    wd = rng.standard_normal((e_res, H, F)) * 0.3
    if bf16:
        x, wg, wu, wd = (oracle.round_bf16(a) for a in (x, wg, wu, wd))
    return p, lg, x, wg, wu, wd


def torch_swiglu(x, wg, wu, wd):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    h = torch.nn.functional.silu(xt @ torch.from_numpy(wg).T) * (xt @ torch.from_numpy(wu).T)
    return (h @ torch.from_numpy(wd).T).numpy()


def test_expert_ffn_matches_torch_swiglu():
    p, lg, x, wg, wu, wd = make()
    _, o = oracle.expert_ffn(x, wg[1], wu[1], wd[1], bf16=False)
    assert np.allclose(o, torch_swiglu(x, wg[1], wu[1], wd[1]), rtol=1e-12, atol=1e-12)


def test_bf16_storage_points_are_bf16():
    p, lg, x, wg, wu, wd = make(bf16=True)
    a, o = oracle.expert_ffn(x, wg[0], wu[0], wd[0], bf16=True)
    assert np.array_equal(oracle.round_bf16(a), a)
    assert np.array_equal(oracle.round_bf16(o), o)
    _, o32 = oracle.expert_ffn(x, wg[0], wu[0], wd[0], bf16=False)
    assert np.max(np.abs(o - o32)) <= 0.05 * np.max(np.abs(o32))


def dense_mixture(p, lg, x, wg, wu, wd):
    """Every resident expert on every token, weighted by the gate mask."""
    idx, g = oracle.route(lg, p.top_k, p.gate)
    El = p.e_loc
    y = np.zeros((p.tokens, p.hidden))
    for e_loc in range(wg.shape[0]):
        e = p.res_lo * El + e_loc
        o = torch_swiglu(x, wg[e_loc], wu[e_loc], wd[e_loc])
        w = np.zeros(p.tokens)
        for t in range(p.tokens):
            for j in range(p.top_k):
                if idx[t, j] == e:
                    w[t] += g[t, j]
        y += w[:, None] * o
    return y


@pytest.mark.parametrize("kw", [dict(), dict(res=(1, 3)), dict(gate="sigmoid", k=1),
                                dict(k=4, E=16, S=4), dict(dedup=True, B=2, R=2, zipf=1.5)])
def test_layer_equals_dense_mixture(kw):
    p, lg, x, wg, wu, wd = make(**kw)
    out = oracle.layer(p, oracle.MODE_FORCE_DROPLESS, lg, x, wg, wu, wd)
    assert np.allclose(out["y"], dense_mixture(p, lg, x, wg, wu, wd), rtol=1e-11, atol=1e-11)


def test_layer_bf16_close_to_dense_mixture():
    p, lg, x, wg, wu, wd = make(bf16=True, T=64, H=32, F=48)
    y = oracle.layer(p, oracle.MODE_FORCE_DROPLESS, lg, x, wg, wu, wd)["y"]
    ref = dense_mixture(p, lg, x, wg, wu, wd)
    assert np.max(np.abs(y - ref)) <= 2e-2 * np.max(np.abs(ref))


def test_combine_identity_experts():
    """With o = x_sorted, combine returns (sum_j g_tj) x_t = x_t for softmax."""
    p, lg, x, *_ = make(T=20, k=3, E=8)
    idx, g = oracle.route(lg, 3, "softmax")
    slot = oracle.assign_slots(idx, p, np.zeros(8, np.int64), np.full(8, -1))
    toks = np.arange(20)
    lay = oracle.pass_layout(p, slot, toks, None)
    xs = oracle.permute(x, lay["sorted_assign"], 3)
    y = oracle.combine(p, xs, lay["row_of_assign"], g, toks)
    assert np.allclose(y, x, rtol=1e-14, atol=1e-14)
    y0 = oracle.combine(p, xs, lay["row_of_assign"], np.zeros_like(g), toks)
    assert not y0.any()


def test_nonresident_tokens_get_zero():
    p, lg, x, wg, wu, wd = make(res=(0, 1), E=8, S=4, k=1)
    out = oracle.layer(p, oracle.MODE_FORCE_DROPLESS, lg, x, wg, wu, wd)
    idx = out["topk_idx"]
    off = idx[:, 0] >= 2
    assert off.any() and not out["y"][off].any()
    assert np.all(np.abs(out["y"][~off]).sum(axis=1) > 0)


def overflow_case(**kw):
    return make(T=64, L=32, factor=1.0, zipf=2.5, chunks=4, **kw)


@pytest.mark.parametrize("kw", [dict(), dict(bf16=True), dict(dedup=True, B=1, R=2),
                                dict(res=(0, 2))])
def test_modes_agree(kw):
    p, lg, x, wg, wu, wd = overflow_case(**kw)
    plain = oracle.layer_plain(p, lg, x, wg, wu, wd)
    lay = oracle.layer(p, oracle.MODE_LAYER, lg, x, wg, wu, wd)
    assert lay["overflow"] and lay["fallback_ran"]
    for mode in (oracle.MODE_LAYER, oracle.MODE_FORCE_DROPLESS, oracle.MODE_FORCE_CHUNKED):
        y = oracle.layer(p, mode, lg, x, wg, wu, wd)["y"]
        assert np.allclose(y, plain, rtol=0, atol=1e-12), mode
    capped = oracle.layer(p, oracle.MODE_CAPPED_ONLY, lg, x, wg, wu, wd)["y"]
    assert not np.allclose(capped, plain, rtol=0, atol=1e-6)


def test_capped_factor_point_one_diverges():
    p, lg, x, wg, wu, wd = make(T=64, factor=0.1)
    out = oracle.layer(p, oracle.MODE_LAYER, lg, x, wg, wu, wd)
    assert out["overflow"] and out["cap"] == 4
    y_drop = oracle.layer(p, oracle.MODE_CAPPED_ONLY, lg, x, wg, wu, wd)["y"]
    assert not np.allclose(y_drop, out["y"])
    assert np.allclose(out["y"], oracle.layer_plain(p, lg, x, wg, wu, wd), atol=1e-12)


def test_no_overflow_takes_single_capped_pass():
    p, lg, x, wg, wu, wd = make(T=32, factor=4.0)
    out = oracle.layer(p, oracle.MODE_LAYER, lg, x, wg, wu, wd)
    assert not out["overflow"] and not out["fallback_ran"] and len(out["passes"]) == 1
    assert np.allclose(out["y"], oracle.layer_plain(p, lg, x, wg, wu, wd), atol=1e-12)


def test_dedup_and_redundancy_leave_output_unchanged():
    p, lg, x, wg, wu, wd = make(T=48, E=8, S=4, k=3, zipf=2.0, dedup=True, B=2, R=3)
    out = oracle.layer(p, oracle.MODE_FORCE_DROPLESS, lg, x, wg, wu, wd)
    assert out["ndiv"].sum() > 0
    p0 = Problem(**{**p.__dict__, "dedup": False, "slots_per_shard": 0, "num_replicas": 0})
    y0 = oracle.layer(p0, oracle.MODE_FORCE_DROPLESS, lg, x, wg, wu, wd)["y"]
    assert np.allclose(out["y"], y0, rtol=0, atol=1e-12)


def test_sampled_plain_equals_full():
    p, lg, x, wg, wu, wd = make(bf16=True, zipf=1.0, dedup=True, B=1, R=1)
    full = oracle.layer_plain(p, lg, x, wg, wu, wd)
    toks = np.array([3, 0, 17, 31])
    assert np.array_equal(oracle.layer_plain_tokens(p, lg, x, wg, wu, wd, toks), full[toks])
