"""GPU parity of the backward at the full workload sizes, in the passes the
layer takes there (LAYER mode: the GPU's own overflow flag picks the capped
pass or the chunked fallback; weight gradients accumulated across passes).

The float64 oracle's whole backward is out of reach at these sizes, so it
is evaluated on samples, each with the oracle's own functions:

* for a seeded sample of tokens: dx (the sum of expert_ffn_bwd over the
  token's rows), d_gate (<dy, expert_ffn output> per row) and d_logits
  (route_bwd of those gates);
* for the hottest resident expert and one other, a seeded sample of FFN
  columns f: rows f of dW_gate and dW_up and column f of dW_down over all of
  the expert's rows (replica groups included).  Column f of the backward
  depends only on column f of the FFN (h_g, h_u, d_a, d_hg, d_hu and the
  activation at f), so expert_ffn_bwd with the weights cut to the sampled
  columns gives exactly those gradient entries.

All to the layer's tolerance, taken relative to each gradient's scale
(check_close_grad: gradients are linear in dy, whose scale is arbitrary).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import LazyExperts, binding_problem, check_close_grad, host, oracle_problem, say
from workloads import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["dsv3_shard", "maverick_shard", "dedup_redundant", "dsv3_ep8_receive"]


def i32(n, fill=-7):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    t.fill_(fill)
    return t


def gpu_backward(g, w, p, inp, dy):
    """The backward of every pass LAYER mode takes, through the step API;
    returns device tensors."""
    T, k, H, F, E = w.tokens, w.top_k, w.hidden, w.ffn, w.num_experts
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ec, se, nd = i32(E), i32(p.num_slots), i32(E)
    soa, sc, st = i32(T * k), i32(w.num_shards), i32(4)
    g.moe_count_overflow(p, idx, ec, se, nd, soa, sc, st, ws)
    status = st.cpu().numpy()
    ovf = bool(status[1])
    passes = [(w.num_chunks, c, 0) for c in range(w.num_chunks)] if ovf else \
        [(1, 0, int(int(status[0]) >= 0))]
    wg, wu, wd = inp["weights"]
    dwg = torch.full((w.e_res, F, H), float("nan"), dtype=torch.float32, device="cuda")
    dwu = torch.full_like(dwg, float("nan"))
    dwd = torch.full((w.e_res, H, F), float("nan"), dtype=torch.float32, device="cuda")
    d_gate = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    dx = torch.full((T, H), float("nan"), dtype=p.dtype, device="cuda")
    roa = i32(T * k)
    for i, (n, c, capped) in enumerate(passes):
        say(f"  pass n={n} c={c} capped={capped}")
        rows, drows = g.pass_max_rows(p, n, capped)
        go, sa = i32(p.g_res + 1), i32(rows)
        xs = torch.empty((rows, H), dtype=p.dtype, device="cuda")
        if w.dedup:
            do, dt, ex = i32(p.s_res + 1), i32(drows), i32(rows)
            xd = torch.empty((drows, H), dtype=p.dtype, device="cuda")
        else:
            do = dt = ex = xd = None
        g.moe_permute(p, n, c, capped, inp["x"], soa, go, roa, sa, do, dt, ex, xd, xs, ws)
        act = torch.empty((rows, F), dtype=p.dtype, device="cuda")
        out = torch.empty((rows, H), dtype=p.dtype, device="cuda")
        g.moe_gmm_swiglu(p, xs, go, se, wg, wu, wd, act, out, ws)
        del act, xd
        d_out = torch.empty((rows, H), dtype=p.dtype, device="cuda")
        g.moe_combine_bwd(p, n, c, dy, out, roa, gate, d_out, d_gate)
        del out
        dxs = torch.empty((rows, H), dtype=p.dtype, device="cuda")
        bws = torch.empty(g.bwd_workspace_bytes(p, rows), dtype=torch.uint8, device="cuda")
        g.moe_gmm_swiglu_bwd(p, xs, go, se, wg, wu, wd, d_out, dxs, dwg, dwu, dwd, i > 0, bws)
        g.moe_permute_bwd(p, n, c, dxs, roa, dx)
        torch.cuda.synchronize()
        del xs, d_out, dxs, bws
    d_logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    g.moe_route_bwd(p, idx, gate, d_gate, d_logits)
    torch.cuda.synchronize()
    return dict(dx=dx, d_gate=d_gate, d_logits=d_logits, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                fallback_ran=ovf)


@pytest.mark.parametrize("name", FULL)
def test_full_size_backward_sampled(name):
    import grouped_gemm_shard_amd as g
    torch.cuda.empty_cache()
    w = CONFIGS[name]
    p, op = binding_problem(w), oracle_problem(w)
    say(f"[bwd-full] {name}: inputs")
    inp = workloads.make_inputs(w, device="cuda")
    dy = workloads.make_dy(w, device="cuda")
    say(f"[bwd-full] {name}: GPU backward")
    got = gpu_backward(g, w, p, inp, dy)

    say(f"[bwd-full] {name}: oracle routing")
    logits = inp["logits"].cpu().numpy()
    o_idx, o_gate = oracle.route(logits, w.top_k, w.gate)
    counts = oracle.expert_counts(o_idx, w.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, op)
    slot = oracle.assign_slots(o_idx, op, ndiv, rep)
    assert got["fallback_ran"] == oracle.overflow(oracle.shard_counts(slot, op),
                                                  oracle.capacity(op))
    spd, k = p.spd, w.top_k
    e0 = w.res_lo * w.e_loc

    def local_expert(t, j):
        s = int(slot[t, j])
        if not (w.res_lo <= s // spd < w.res_hi):
            return -1
        return int(se[s]) - e0

    wg, wu, wd = (LazyExperts(t) for t in inp["weights"])
    rd = oracle.round_bf16 if w.bf16 else (lambda v: v)

    say(f"[bwd-full] {name}: sampled tokens")
    rng = np.random.default_rng(11)
    resident = [t for t in range(w.tokens) if any(local_expert(t, j) >= 0 for j in range(k))]
    sample = np.sort(rng.choice(np.asarray(resident), size=min(12, len(resident)),
                                replace=False))
    want_dx, want_dg = [], []
    for t in sample:
        xt = host(inp["x"][int(t)])[None, :]
        dyt = host(dy[int(t)])
        acc = np.zeros(w.hidden)
        dg = np.zeros(k)
        for j in range(k):
            e = local_expert(t, j)
            if e < 0:
                continue
            wge, wue, wde = wg[e], wu[e], wd[e]
            out = oracle.expert_ffn(xt, wge, wue, wde, w.bf16)[1][0]
            dg[j] = float(np.dot(dyt, out))
            d_o = rd(o_gate[t, j] * dyt)[None, :]
            acc = acc + oracle.expert_ffn_bwd(xt, wge, wue, wde, d_o, w.bf16)[0][0]
        want_dx.append(rd(acc))
        want_dg.append(dg)
    ts = torch.from_numpy(sample).cuda()
    check_close_grad(host(got["dx"][ts]), np.stack(want_dx), f"dx {name} (sampled tokens)")
    want_dg = np.stack(want_dg)
    check_close_grad(host(got["d_gate"][ts]), want_dg, f"d_gate {name} (sampled tokens)")
    p_sub = replace(op, tokens=len(sample))
    want_dl = oracle.route_bwd(p_sub, o_idx[sample], o_gate[sample], want_dg)
    check_close_grad(host(got["d_logits"][ts]), want_dl, f"d_logits {name} (sampled tokens)")

    say(f"[bwd-full] {name}: sampled weight-gradient columns")
    rows_of = {}
    for t in range(w.tokens):
        for j in range(k):
            e = local_expert(t, j)
            if e >= 0:
                rows_of.setdefault(e, []).append((t, j))
    hot = max(rows_of, key=lambda e: len(rows_of[e]))
    others = [e for e in rows_of if e != hot]
    experts = [hot] + ([int(rng.choice(others))] if others else [])
    for e in experts:
        pairs = rows_of[e]
        tok = torch.from_numpy(np.asarray([t for t, _ in pairs])).cuda()
        X = host(inp["x"][tok])
        gates = np.asarray([o_gate[t, j] for t, j in pairs])
        d_o = rd(gates[:, None] * host(dy[tok]))
        cols = np.sort(rng.choice(w.ffn, size=4, replace=False))
        wge, wue, wde = wg[e], wu[e], wd[e]
        _, dwg_c, dwu_c, dwd_c = oracle.expert_ffn_bwd(X, wge[cols], wue[cols], wde[:, cols],
                                                       d_o, w.bf16)
        cs = torch.from_numpy(cols).cuda()
        say(f"  expert {e}: {len(pairs)} rows, columns {cols.tolist()}")
        check_close_grad(host(got["dw_gate"][e][cs]), dwg_c, f"dW_gate {name} expert {e}")
        check_close_grad(host(got["dw_up"][e][cs]), dwu_c, f"dW_up {name} expert {e}")
        check_close_grad(host(got["dw_down"][e][:, cs]), dwd_c, f"dW_down {name} expert {e}")
    # experts with no rows got exact zeros (first pass overwrites)
    empty = [e for e in range(w.e_res) if e not in rows_of]
    for e in empty[:4]:
        assert bool((got["dw_gate"][e] == 0).all()) and bool((got["dw_down"][e] == 0).all())
