"""GPU parity of the return-path dedup (moe_combine_partial and
moe_combine_from_partials) beyond the bf16 small cases that
test_pass_steps_parity covers.

* fp32: a small fp32 problem with dedup and redundant slots, every pass of
  the chunked mode, against the oracle's own pipeline.
* Full size (dedup_redundant): in test_gpu_fullsize_float.py, against
  the oracle's return path on the GPU's expert_out.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import binding_problem, check_close, host, ints, oracle_problem, say

pytestmark = pytest.mark.gpu

W = workloads.Workload
FP32 = W("fp32_dedup_small", tokens=128, seq_len=128, hidden=64, ffn=64, num_experts=8,
         top_k=3, num_shards=4, res_lo=0, res_hi=4, factor=1.0, num_chunks=2, bf16=False,
         dedup=True, slots_per_shard=1, num_replicas=2, zipf=1.5)


def i32(n, fill=-7):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    t.fill_(fill)
    return t


def step_api(g, p, w, inp, n, c, capped):
    """route, count, permute, grouped GEMM, combine and the return path of
    one pass through the step API."""
    idx = torch.empty((w.tokens, w.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ec, se, nd = i32(w.num_experts), i32(p.num_slots), i32(w.num_experts)
    soa, sc, st = i32(w.tokens * w.top_k), i32(w.num_shards), i32(4)
    g.moe_count_overflow(p, idx, ec, se, nd, soa, sc, st, ws)
    rows, drows = g.pass_max_rows(p, n, capped)
    go, roa, sa = i32(p.g_res + 1), i32(w.tokens * w.top_k), i32(rows)
    do, dt, ex = i32(p.s_res + 1), i32(drows), i32(rows)
    xd = torch.zeros((drows, w.hidden), dtype=p.dtype, device="cuda")
    xs = torch.zeros((rows, w.hidden), dtype=p.dtype, device="cuda")
    g.moe_permute(p, n, c, capped, inp["x"], soa, go, roa, sa, do, dt, ex, xd, xs, ws)
    act = torch.zeros((rows, w.ffn), dtype=p.dtype, device="cuda")
    out = torch.zeros((rows, w.hidden), dtype=p.dtype, device="cuda")
    g.moe_gmm_swiglu(p, xs, go, se, *inp["weights"], act, out, ws)
    y = torch.full((w.tokens, w.hidden), 7.0, dtype=p.dtype, device="cuda")
    g.moe_combine(p, n, c, out, roa, gate, y)
    part = torch.full((drows, w.hidden), 7.0, dtype=torch.float32, device="cuda")
    g.moe_combine_partial(p, n, c, capped, out, roa, gate, do, dt, ex, part)
    y2 = torch.full((w.tokens, w.hidden), 7.0, dtype=p.dtype, device="cuda")
    g.moe_combine_from_partials(p, n, c, capped, part, roa, ex, y2, rows)
    torch.cuda.synchronize()
    return dict(gate=gate, soa=soa, roa=roa, do=do, dt=dt, ex=ex, out=out, y=y, part=part, y2=y2,
                rows=rows)


@pytest.mark.parametrize("n,c", [(1, 0), (2, 0), (2, 1)])
def test_fp32_return_path_against_oracle(n, c):
    import grouped_gemm_shard_amd as g
    w = FP32
    p, op = binding_problem(w), oracle_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    say(f"[return-dedup] fp32 n={n} c={c}")
    r = step_api(g, p, w, inp, n, c, 0)
    logits, x = inp["logits"].cpu().numpy(), host(inp["x"])
    ws_h = [host(t) for t in inp["weights"]]
    o_idx, o_gate = oracle.route(logits, w.top_k, w.gate)
    counts = oracle.expert_counts(o_idx, w.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, op)
    slot = oracle.assign_slots(o_idx, op, ndiv, rep)
    toks = oracle.pass_tokens(op, n, c)
    lay = oracle.pass_layout(op, slot, toks, None)
    _, o_xs = oracle.permute_dedup(x, lay["dedup_token"], lay["expand_idx"])
    ge = np.asarray([int(se[w.res_lo * p.spd + q]) - w.res_lo * w.e_loc for q in range(p.g_res)])
    _, o_out = oracle.gmm_swiglu(op, o_xs, lay["group_offsets"], ge, *ws_h)
    o_part = oracle.combine_partial(op, o_out, lay["row_of_assign"], o_gate, slot,
                                    lay["dedup_offsets"], lay["dedup_token"])
    o_y2 = oracle.combine_from_partials(op, o_part, slot, lay["dedup_offsets"],
                                        lay["dedup_token"], toks)
    U = int(lay["dedup_offsets"][-1])
    assert np.array_equal(ints(r["do"]), lay["dedup_offsets"])
    part = host(r["part"])
    check_close(part[:U], o_part, f"fp32 partial n={n} c={c}")
    assert np.all(part[U:] == 7.0)
    y2 = host(r["y2"])
    check_close(y2[toks], o_y2, f"fp32 y from partials n={n} c={c}")
    rest = np.setdiff1d(np.arange(w.tokens), toks)
    assert np.all(y2[rest] == 7.0)
