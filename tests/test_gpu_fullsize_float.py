"""Full-size floating-point parity of the grouped GEMM and the return path.

* act and expert_out of the step-API grouped GEMM at the full sizes of the
  DeepSeek-V3 shard, the Llama4-Maverick shard, the dedup + redundancy
  workload and the DeepSeek-V3 EP8 receive shape, compared element by
  element with oracle.gmm_swiglu on whole m-tiles (256 rows at these
  hidden sizes): in every pass the layer takes, the first and the last
  m-tile of the pass's hottest group and the last (remainder) m-tile of
  every group -- of a seeded sample of 48 groups where a pass has more --
  with consecutive passes issued on two different streams.  The oracle
  runs on its own layout (route, plan, reroute and pass layout), whose
  group offsets must equal the GPU's; its x_sorted rows come from
  oracle.permute.
* The full-size return path (dedup_redundant): every partial row, y from
  the partials for every token, and the plain combine for every token,
  against oracle.combine_partial, oracle.combine_from_partials and
  oracle.combine on the GPU's expert_out, with the oracle's own layout and
  gates.
"""

from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import binding_problem, check_close, host, ints, oracle_problem, say
from workloads import CONFIGS

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TILE = 256
MAX_GROUPS = 48


def i32(n, fill=-7):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    t.fill_(fill)
    return t


class CachedExperts:
    """w[e] -> float64 host copy of one resident expert's matrix, kept in a
    cache of bounded size (least recently used out first)."""

    def __init__(self, t: torch.Tensor, budget_bytes: int):
        self.t, self.budget, self.cache = t, budget_bytes, OrderedDict()

    def __getitem__(self, e):
        e = int(e)
        if e in self.cache:
            self.cache.move_to_end(e)
            return self.cache[e]
        m = host(self.t[e])
        self.cache[e] = m
        while len(self.cache) > 1 and sum(v.nbytes for v in self.cache.values()) > self.budget:
            self.cache.popitem(last=False)
        return m


def oracle_slots(w, op, logits):
    o_idx, o_gate = oracle.route(logits, w.top_k, w.gate)
    counts = oracle.expert_counts(o_idx, w.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, op)
    slot = oracle.assign_slots(o_idx, op, ndiv, rep)
    sc = oracle.shard_counts(slot, op)
    cap = oracle.capacity(op)
    return o_gate, se, slot, cap, oracle.overflow(sc, cap)


def layer_passes(w, ovf):
    """(num_chunks, chunk, capped) of every pass LAYER mode takes."""
    return [(w.num_chunks, c, 0) for c in range(w.num_chunks)] if ovf else [(1, 0, 1)]


def tile_rows(go, rng):
    """Row ranges to check in one pass: the first and the last m-tile of
    the hottest group and the last m-tile of every group (of a seeded
    sample of groups when there are many)."""
    sizes = np.diff(go)
    groups = [g for g in range(len(sizes)) if sizes[g] > 0]
    if not groups:
        return []
    hot = max(groups, key=lambda g: (sizes[g], -g))
    if len(groups) > MAX_GROUPS:
        keep = set(rng.choice(np.asarray(groups), size=MAX_GROUPS, replace=False).tolist())
        groups = [g for g in groups if g in keep or g == hot]
    ranges = {(int(go[hot]), int(min(go[hot] + TILE, go[hot + 1])))}
    for g in groups:
        a0, a1 = int(go[g]), int(go[g + 1])
        ranges.add((a0 + TILE * ((a1 - a0 - 1) // TILE), a1))
    return sorted(ranges)


def group_of(go, r):
    return int(np.searchsorted(go, r, side="right") - 1)


@pytest.mark.parametrize("name", ["dsv3_shard", "maverick_shard", "dedup_redundant",
                                  "dsv3_ep8_receive"])
def test_full_size_gemm_tiles(name):
    import grouped_gemm_shard_amd as g
    torch.cuda.empty_cache()
    w = CONFIGS[name]
    p, op = binding_problem(w), oracle_problem(w)
    say(f"[full-float] {name}: inputs")
    inp = workloads.make_inputs(w, device="cuda")
    logits = inp["logits"].cpu().numpy()
    x_host = host(inp["x"])
    _, o_se, o_slot, cap, ovf = oracle_slots(w, op, logits)
    ge = [int(o_se[w.res_lo * p.spd + q]) - w.res_lo * w.e_loc for q in range(p.g_res)]
    budget = 6 << 30
    wg, wu, wd = (CachedExperts(t, budget) for t in inp["weights"])

    say(f"[full-float] {name}: route and count (step API)")
    idx = torch.empty((w.tokens, w.top_k), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ec, sev, ndv = i32(w.num_experts), i32(p.num_slots), i32(w.num_experts)
    soa, scv, st = i32(w.tokens * w.top_k), i32(w.num_shards), i32(4)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    ws = [torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda") for _ in streams]
    g.moe_count_overflow(p, idx, ec, sev, ndv, soa, scv, st, ws[0])
    torch.cuda.synchronize()
    assert np.array_equal(ints(sev), o_se)
    assert np.array_equal(ints(soa), o_slot.ravel())

    rng = np.random.default_rng(11)
    checked = 0
    for i, (n, c, capped) in enumerate(layer_passes(w, ovf)):
        s = streams[i % 2]
        s.wait_stream(streams[0])
        rows, drows = g.pass_max_rows(p, n, capped)
        go, roa, sa = i32(p.g_res + 1), i32(w.tokens * w.top_k), i32(rows)
        xs = torch.empty((rows, w.hidden), dtype=p.dtype, device="cuda")
        act = torch.empty((rows, w.ffn), dtype=p.dtype, device="cuda")
        out = torch.empty((rows, w.hidden), dtype=p.dtype, device="cuda")
        stat = torch.zeros(1, dtype=torch.int32, device="cuda")
        if w.dedup:
            do, dt, ex = i32(p.s_res + 1), i32(drows), i32(rows)
            xd = torch.empty((drows, w.hidden), dtype=p.dtype, device="cuda")
        else:
            do = dt = ex = xd = None
        say(f"[full-float] {name}: pass n={n} c={c} capped={capped} on stream {i % 2}")
        with torch.cuda.stream(s):
            g.moe_permute(p, n, c, capped, inp["x"], soa, go, roa, sa, do, dt, ex, xd, xs, ws[i % 2])
            g.moe_gmm_swiglu(p, xs, go, sev, *inp["weights"], act, out, ws[i % 2], status=stat)
        torch.cuda.synchronize()
        assert int(stat.item()) == 0
        toks = oracle.pass_tokens(op, n, c)
        lay = oracle.pass_layout(op, o_slot, toks, cap if capped else None)
        o_go = lay["group_offsets"]
        assert np.array_equal(ints(go), o_go)
        if w.dedup:
            src = lay["dedup_token"][lay["expand_idx"]]
            src_k = 1
        else:
            src, src_k = lay["sorted_assign"], w.top_k
        for (r0, r1) in tile_rows(o_go, rng):
            grp = group_of(o_go, r0)
            xr = oracle.permute(x_host, src[r0:r1], src_k)
            o_act, o_out = oracle.gmm_swiglu(op, xr, np.asarray([0, r1 - r0]), [ge[grp]],
                                             wg, wu, wd)
            what = f"{name} pass {c}/{n} group {grp} rows {r0}:{r1}"
            check_close(host(act[r0:r1]), o_act, f"act {what}")
            check_close(host(out[r0:r1]), o_out, f"expert_out {what}")
            checked += r1 - r0
        del xs, act, out, xd
    say(f"[full-float] {name}: {checked} rows checked")
    assert checked > 0


def test_full_size_return_path_against_oracle():
    import grouped_gemm_shard_amd as g
    from test_gpu_return_dedup import step_api
    torch.cuda.empty_cache()
    w = CONFIGS["dedup_redundant"]
    p, op = binding_problem(w), oracle_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    say("[full-float] dedup_redundant: return path, one uncapped pass")
    r = step_api(g, p, w, inp, 1, 0, 0)
    o_gate, _, o_slot, _, _ = oracle_slots(w, op, inp["logits"].cpu().numpy())
    toks = oracle.pass_tokens(op, 1, 0)
    lay = oracle.pass_layout(op, o_slot, toks, None)
    U = int(lay["dedup_offsets"][-1])
    assert np.array_equal(ints(r["do"]), lay["dedup_offsets"])
    assert np.array_equal(ints(r["dt"])[:U], lay["dedup_token"])
    assert np.array_equal(ints(r["roa"]), lay["row_of_assign"])
    out = host(r["out"])
    say("[full-float] dedup_redundant: oracle partial rows")
    o_part = oracle.combine_partial(op, out, lay["row_of_assign"], o_gate, o_slot,
                                    lay["dedup_offsets"], lay["dedup_token"])
    check_close(host(r["part"][:U]), o_part, "partial rows (full size)")
    assert bool((r["part"][U:] == 7.0).all())
    say("[full-float] dedup_redundant: oracle y from partials and plain combine")
    o_y2 = oracle.combine_from_partials(op, o_part, o_slot, lay["dedup_offsets"],
                                        lay["dedup_token"], toks)
    check_close(host(r["y2"])[toks], o_y2, "y from partials (full size)")
    o_y = oracle.combine(op, out, lay["row_of_assign"], o_gate, toks)
    check_close(host(r["y"])[toks], o_y, "y (full size)")
