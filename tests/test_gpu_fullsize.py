"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (LAYER mode).

* Routing, counts, plan, reroute, capacity/overflow and every pass layout
  the layer takes are compared with the oracle bit-exactly at full size.
* x_sorted (and the dedup buffers) are checked at full size by the property
  that defines them, on the GPU with torch indexing: x_sorted[n] ==
  x[sorted_assign[n] / k], x_dedup[u] == x[dedup_token[u]], x_sorted[n] ==
  x_dedup[expand_idx[n]].
* y of the whole LAYER call is compared on at least 512 tokens -- one in
  every group of every pass the layer took, then a seeded sample -- with
  the oracle's plain definition of the dropless layer (which the chunked
  fallback must equal), to the layer's tolerance; tokens with no resident
  assignment must be exactly 0.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import LazyExperts, binding_problem, check_close, host, ints, oracle_problem, say
from workloads import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["dsv3_shard", "maverick_shard", "dedup_redundant", "dsv3_ep8_receive"]
Y_SAMPLE = 512


class LazyRows:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, i):
        return host(self.t[i])


def i32(n, fill=-7):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    t.fill_(fill)
    return t


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    import grouped_gemm_shard_amd as g
    torch.cuda.empty_cache()
    w = CONFIGS[name]
    p, op = binding_problem(w), oracle_problem(w)
    say(f"[full] {name}: inputs")
    inp = workloads.make_inputs(w, device="cuda")
    logits = inp["logits"].cpu().numpy()

    say(f"[full] {name}: layer (LAYER mode)")
    run = g.LayerRunner(p, g.MODE_LAYER)
    y = run(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    info = ints(run.info).tolist()

    say(f"[full] {name}: oracle integer artefacts")
    o_idx, o_gate = oracle.route(logits, w.top_k, w.gate)
    counts = oracle.expert_counts(o_idx, w.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, op)
    slot = oracle.assign_slots(o_idx, op, ndiv, rep)
    sc = oracle.shard_counts(slot, op)
    cap = oracle.capacity(op)
    ovf = oracle.overflow(sc, cap)
    assert info == [int(ovf), int(ovf), -1 if cap is None else cap, int(sc.max()), 0]

    say(f"[full] {name}: step API route/count")
    idx = torch.empty((w.tokens, w.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ec, sev, ndv = i32(w.num_experts), i32(p.num_slots), i32(w.num_experts)
    soa, scv, st = i32(w.tokens * w.top_k), i32(w.num_shards), i32(4)
    g.moe_count_overflow(p, idx, ec, sev, ndv, soa, scv, st, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ints(idx), o_idx)
    check_close(gate.cpu().numpy(), o_gate, "gate")
    assert np.array_equal(ints(ec), counts)
    assert np.array_equal(ints(sev), se)
    assert np.array_equal(ints(ndv), ndiv)
    assert np.array_equal(ints(soa), slot.ravel())
    assert np.array_equal(ints(scv), sc)

    passes = [(w.num_chunks, c, 0) for c in range(w.num_chunks)] if ovf else [(1, 0, 1)]
    rng = np.random.default_rng(7)
    touch = set()  # one token per (pass, group) for the sampled y
    for (n, c, capped) in passes:
        say(f"[full] {name}: pass n={n} c={c} capped={capped}")
        rows, drows = g.pass_max_rows(p, n, capped)
        go, roa, sa = i32(p.g_res + 1), i32(w.tokens * w.top_k), i32(rows)
        xs = torch.empty((rows, w.hidden), dtype=p.dtype, device="cuda")
        if w.dedup:
            do, dt, ex = i32(p.s_res + 1), i32(drows), i32(rows)
            xd = torch.empty((drows, w.hidden), dtype=p.dtype, device="cuda")
        else:
            do = dt = ex = xd = None
        g.moe_permute(p, n, c, capped, inp["x"], soa, go, roa, sa, do, dt, ex, xd, xs, ws)
        toks = oracle.pass_tokens(op, n, c)
        lay = oracle.pass_layout(op, slot, toks, cap if capped else None)
        torch.cuda.synchronize()
        N = lay["num_rows"]
        o_go = lay["group_offsets"]
        for q in range(len(o_go) - 1):
            if o_go[q + 1] > o_go[q]:
                touch.add(int(lay["sorted_assign"][rng.integers(o_go[q], o_go[q + 1])]) // w.top_k)
        assert np.array_equal(ints(go), lay["group_offsets"])
        assert np.array_equal(ints(sa)[:N], lay["sorted_assign"])
        pass_a = (toks[:, None] * w.top_k + np.arange(w.top_k)[None, :]).ravel()
        assert np.array_equal(ints(roa)[pass_a], lay["row_of_assign"][pass_a])
        src = (sa[:N].long() // w.top_k)
        assert torch.equal(xs[:N], inp["x"][src])
        if w.dedup:
            U = int(lay["dedup_offsets"][-1])
            assert np.array_equal(ints(do), lay["dedup_offsets"])
            assert np.array_equal(ints(dt)[:U], lay["dedup_token"])
            assert np.array_equal(ints(ex)[:N], lay["expand_idx"])
            assert torch.equal(xd[:U], inp["x"][dt[:U].long()])
            assert torch.equal(xs[:N], xd[ex[:N].long()])
        del xs, xd

    say(f"[full] {name}: sampled y against the oracle")
    # a token in every group of every pass, then seeded tokens up to
    # Y_SAMPLE (non-resident ones included)
    resident = [t for t in range(w.tokens)
                if any(w.res_lo <= slot[t, j] // p.spd < w.res_hi for j in range(w.top_k))]
    sample = set(touch)
    for t in rng.permutation(w.tokens):
        if len(sample) >= Y_SAMPLE:
            break
        sample.add(int(t))
    sample = np.asarray(sorted(sample), dtype=np.int64)
    assert len(sample) >= min(Y_SAMPLE, w.tokens)
    wg, wu, wd = (LazyExperts(t) for t in inp["weights"])
    want = oracle.layer_plain_tokens(op, logits, LazyRows(inp["x"]), wg, wu, wd, sample)
    got = host(y[torch.from_numpy(sample).cuda()])
    check_close(got, want, f"y {name}")
    res_set = set(resident)
    nonres = [i for i, t in enumerate(sample) if t not in res_set]
    assert np.all(got[nonres] == 0)
