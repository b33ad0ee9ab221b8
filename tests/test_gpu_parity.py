"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every step (route, counts/plan/overflow, permute layout, grouped GEMM,
combine) and the whole layer in all four modes are compared on the same
seeded inputs: integer artefacts bit-exactly, floating point within the
layer's tolerance (tests/moe_cases.py).  The oracle always receives host
copies of the exact tensors the GPU path received.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import (SMALL_CASES, binding_problem, check_close, host, ints, oracle_problem,
                       say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import grouped_gemm_shard_amd as g
    return g


_INPUTS = {}


def inputs(name):
    if name not in _INPUTS:
        _INPUTS.clear()
        torch.cuda.empty_cache()
        w = SMALL_CASES[name]
        inp = workloads.make_inputs(w, device="cuda")
        hostc = dict(logits=inp["logits"].cpu().numpy(), x=host(inp["x"]),
                     w=[host(t) for t in inp["weights"]])
        _INPUTS[name] = (w, inp, hostc)
    return _INPUTS[name]


def i32(n, fill=None):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def gpu_route(g, p, logits):
    idx = i32((p.tokens, p.top_k))
    gate = torch.empty((p.tokens, p.top_k), dtype=torch.float32, device="cuda")
    g.moe_route(p, logits, idx, gate)
    return idx, gate


def gpu_count(g, p, idx):
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    out = dict(expert_counts=i32(p.num_experts, -7), slot_expert=i32(p.num_slots, -7),
               ndiv=i32(p.num_experts, -7), slot_of_assign=i32(p.tokens * p.top_k, -7),
               shard_counts=i32(p.num_shards, -7), status=i32(4, -7),
               required_factor=torch.full((1,), -7.0, dtype=torch.float32, device="cuda"))
    g.moe_count_overflow(p, idx, out["expert_counts"], out["slot_expert"], out["ndiv"],
                         out["slot_of_assign"], out["shard_counts"], out["status"], ws,
                         required_factor=out["required_factor"])
    return out


def oracle_count(op, idx_np):
    counts = oracle.expert_counts(idx_np, op.num_experts)
    se, ndiv, rep = oracle.plan_redundancy(counts, op)
    slot = oracle.assign_slots(idx_np, op, ndiv, rep)
    sc = oracle.shard_counts(slot, op)
    cap = oracle.capacity(op)
    return dict(expert_counts=counts, slot_expert=se, ndiv=ndiv, slot_of_assign=slot.ravel(),
                shard_counts=sc, cap=-1 if cap is None else cap,
                overflow=int(oracle.overflow(sc, cap)), max=int(sc.max()))


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_route_parity(g, name):
    w, inp, hc = inputs(name)
    p = binding_problem(w)
    say(f"[route] {name}")
    idx, gate = gpu_route(g, p, inp["logits"])
    torch.cuda.synchronize()
    o_idx, o_gate = oracle.route(hc["logits"], w.top_k, w.gate)
    assert np.array_equal(ints(idx), o_idx)
    check_close(gate.cpu().numpy(), o_gate, "gate")


def test_route_ties_and_signed_zero(g):
    p = g.Problem(tokens=8, seq_len=8, hidden=256, ffn=128, num_experts=70, top_k=5,
                  num_shards=2, res_lo=0, res_hi=2, factor=2.0, num_chunks=1)
    lg = np.zeros((8, 70), np.float32)
    lg[1, :] = 1.0                       # all equal: lowest indices
    lg[2, [3, 66, 9, 64]] = 2.0          # ties across lanes 3/2 and registers
    lg[3, 5], lg[3, 6] = -0.0, 0.0       # signed zeros compare equal
    lg[3, :5] = -1.0
    lg[4] = np.arange(70, dtype=np.float32) % 3
    lg[5] = -np.arange(70, dtype=np.float32)
    lg[6, 69] = 5.0
    lg[7] = np.random.default_rng(0).integers(-2, 3, 70).astype(np.float32)
    say("[route] ties")
    idx, gate = gpu_route(g, p, torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    o_idx, o_gate = oracle.route(lg, 5, "softmax")
    assert np.array_equal(ints(idx), o_idx)
    check_close(gate.cpu().numpy(), o_gate, "gate")


def _count_case(g, w, logits_np):
    p = binding_problem(w)
    op = oracle_problem(w)
    idx, _ = gpu_route(g, p, torch.from_numpy(logits_np).cuda())
    got = gpu_count(g, p, idx)
    torch.cuda.synchronize()
    o_idx, _ = oracle.route(logits_np, w.top_k, w.gate)
    assert np.array_equal(ints(idx), o_idx)
    want = oracle_count(op, o_idx)
    for key in ("expert_counts", "slot_expert", "ndiv", "slot_of_assign", "shard_counts"):
        assert np.array_equal(ints(got[key]).ravel(), np.asarray(want[key]).ravel()), key
    st = ints(got["status"])
    assert st.tolist() == [want["cap"], want["overflow"], want["max"], 0]
    # the figure [FALLBACK] Shortcomings logs, max shard count / (T*k/S), as
    # float32 (the integer quotient rounded once)
    rf = float(got["required_factor"].item())
    want_rf = oracle.required_factor(np.asarray(want["shard_counts"]), op)
    assert abs(rf - want_rf) <= 1e-6 * max(1.0, want_rf), (rf, want_rf)
    return want


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_count_parity(g, name):
    w, inp, hc = inputs(name)
    say(f"[count] {name}")
    _count_case(g, w, hc["logits"])


@pytest.mark.parametrize("factor,expect", [(0.1, 1), (-1.0, 0), (100.0, 0)])
def test_count_factor_cases(g, factor, expect):
    w = SMALL_CASES["dedup_small"].scaled(factor=factor)
    lg = workloads.make_logits(w, "cpu").numpy()
    say(f"[count] dedup_small factor={factor}")
    want = _count_case(g, w, lg)
    assert want["overflow"] == expect


def test_count_single_shard_overflow(g):
    """Only one shard overflows and the flag is raised (the fallback page's
    asymmetric-overflow test)."""
    w = SMALL_CASES["mid_bf16"].scaled(factor=1.0, zipf=0.0)
    lg = workloads.make_logits(w, "cpu").numpy()
    lg[: w.tokens // 2, 0] += 100.0       # half the tokens pick expert 0 (shard 0)
    say("[count] single-shard overflow")
    want = _count_case(g, w, lg)
    assert want["overflow"] == 1
    assert int(np.sum(want["shard_counts"] > want["cap"])) == 1


def _passes(w):
    out = [(1, 0, 0), (1, 0, 1)]
    out += [(w.num_chunks, c, 0) for c in range(w.num_chunks)]
    return out


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_pass_steps_parity(g, name):
    """permute -> grouped GEMM -> combine, pass by pass, against the oracle."""
    w, inp, hc = inputs(name)
    p, op = binding_problem(w), oracle_problem(w)
    idx, gate = gpu_route(g, p, inp["logits"])
    cnt = gpu_count(g, p, idx)
    o_idx, o_gate = oracle.route(hc["logits"], w.top_k, w.gate)
    want = oracle_count(op, o_idx)
    torch.cuda.synchronize()
    assert np.array_equal(ints(cnt["slot_of_assign"]), want["slot_of_assign"])
    slot_np = want["slot_of_assign"].reshape(w.tokens, w.top_k)
    cap = oracle.capacity(op)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    group_expert = np.asarray([int(want["slot_expert"][w.res_lo * p.spd + q]) - w.res_lo * w.e_loc
                               for q in range(p.g_res)])
    for (n, c, capped) in _passes(w):
        say(f"[pass] {name} n={n} c={c} capped={capped}")
        rows, drows = g.pass_max_rows(p, n, capped)
        go = i32(p.g_res + 1, -7)
        roa = i32(w.tokens * w.top_k, -7)
        sa = i32(rows, -7)
        xs = torch.zeros((rows, w.hidden), dtype=p.dtype, device="cuda")
        if w.dedup:
            do, dt, ex = i32(p.s_res + 1, -7), i32(drows, -7), i32(rows, -7)
            xd = torch.zeros((drows, w.hidden), dtype=p.dtype, device="cuda")
        else:
            do = dt = ex = xd = None
        g.moe_permute(p, n, c, capped, inp["x"], cnt["slot_of_assign"], go, roa, sa, do, dt, ex,
                      xd, xs, ws)
        toks = oracle.pass_tokens(op, n, c)
        lay = oracle.pass_layout(op, slot_np, toks, cap if capped else None)
        torch.cuda.synchronize()
        N = lay["num_rows"]
        assert np.array_equal(ints(go), lay["group_offsets"])
        assert np.array_equal(ints(sa)[:N], lay["sorted_assign"])
        roa_np = ints(roa)
        pass_a = (toks[:, None] * w.top_k + np.arange(w.top_k)[None, :]).ravel()
        assert np.array_equal(roa_np[pass_a], lay["row_of_assign"][pass_a])
        other = np.setdiff1d(np.arange(w.tokens * w.top_k), pass_a)
        assert np.all(roa_np[other] == -7)          # other tokens untouched
        if w.dedup:
            U = int(lay["dedup_offsets"][-1])
            assert np.array_equal(ints(do), lay["dedup_offsets"])
            assert np.array_equal(ints(dt)[:U], lay["dedup_token"])
            assert np.array_equal(ints(ex)[:N], lay["expand_idx"])
            _, o_xs = oracle.permute_dedup(hc["x"], lay["dedup_token"], lay["expand_idx"])
        else:
            o_xs = oracle.permute(hc["x"], lay["sorted_assign"], w.top_k)
        assert np.array_equal(host(xs[:N]), o_xs)   # bitwise
        # grouped GEMM on the GPU rows (bitwise equal to the oracle's rows)
        act = torch.zeros((rows, w.ffn), dtype=p.dtype, device="cuda")
        out = torch.zeros((rows, w.hidden), dtype=p.dtype, device="cuda")
        g.moe_gmm_swiglu(p, xs, go, cnt["slot_expert"], *inp["weights"], act, out, ws)
        o_act, o_out = oracle.gmm_swiglu(op, o_xs, lay["group_offsets"], group_expert, *hc["w"])
        torch.cuda.synchronize()
        check_close(host(act[:N]), o_act, f"act {name} pass {n}/{c}/{capped}")
        check_close(host(out[:N]), o_out, f"expert_out {name} pass {n}/{c}/{capped}")
        # combine
        y = torch.full((w.tokens, w.hidden), 7.0, dtype=p.dtype, device="cuda")
        g.moe_combine(p, n, c, out, roa, gate, y)
        o_y = oracle.combine(op, o_out, lay["row_of_assign"], o_gate, toks)
        torch.cuda.synchronize()
        y_np = host(y)
        check_close(y_np[toks], o_y, f"y {name} pass {n}/{c}/{capped}")
        rest = np.setdiff1d(np.arange(w.tokens), toks)
        assert np.all(y_np[rest] == 7.0)
        if w.dedup:
            # return-path dedup: one partial row per (token, shard), then the
            # sum at the source; the oracle regroups its own expert outputs
            part = torch.full((drows, w.hidden), 7.0, dtype=torch.float32, device="cuda")
            g.moe_combine_partial(p, n, c, capped, out, roa, gate, do, dt, ex, part)
            y2 = torch.full((w.tokens, w.hidden), 7.0, dtype=p.dtype, device="cuda")
            g.moe_combine_from_partials(p, n, c, capped, part, roa, ex, y2, rows)
            o_part = oracle.combine_partial(op, o_out, lay["row_of_assign"], o_gate, slot_np,
                                            lay["dedup_offsets"], lay["dedup_token"])
            o_y2 = oracle.combine_from_partials(op, o_part, slot_np, lay["dedup_offsets"],
                                                lay["dedup_token"], toks)
            torch.cuda.synchronize()
            part_np = host(part)
            check_close(part_np[:U], o_part, f"partial {name} pass {n}/{c}/{capped}")
            assert np.all(part_np[U:] == 7.0)
            y2_np = host(y2)
            check_close(y2_np[toks], o_y2, f"y from partials {name} pass {n}/{c}/{capped}")
            check_close(y2_np[toks], o_y, f"y from partials vs combine {name} pass {n}/{c}/{capped}")
            assert np.all(y2_np[rest] == 7.0)


MODES = {0: "LAYER", 1: "FORCE_DROPLESS", 2: "CAPPED_ONLY", 3: "FORCE_CHUNKED"}


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_layer_modes(g, name):
    w, inp, hc = inputs(name)
    p, op = binding_problem(w), oracle_problem(w)
    ys = {}
    for mode in MODES:
        say(f"[layer] {name} mode={MODES[mode]}")
        run = g.LayerRunner(p, mode)
        y = run(inp["x"], inp["logits"], *inp["weights"]).clone()
        info = ints(run.info)
        want = oracle.layer(op, mode, hc["logits"], hc["x"], *hc["w"])
        torch.cuda.synchronize()
        cap = -1 if want["cap"] is None else want["cap"]
        assert info.tolist() == [int(want["overflow"]), int(want["fallback_ran"]), cap,
                                 int(want["shard_counts"].max()), 0]
        check_close(host(y), want["y"], f"y {name} {MODES[mode]}")
        ys[mode] = y
        del run
    # dropless, chunked and (without overflow) capped layers are the same
    # computation per row: the GPU results agree bitwise
    assert torch.equal(ys[1], ys[3])
    assert torch.equal(ys[0], ys[1])


def test_dedup_and_redundancy_do_not_change_y(g):
    w = SMALL_CASES["dedup_small"]
    _, inp, _ = inputs("dedup_small")
    p = binding_problem(w)
    p0 = binding_problem(w.scaled(dedup=False, slots_per_shard=0, num_replicas=0))
    say("[layer] dedup/redundancy invariance")
    y1 = g.LayerRunner(p, g.MODE_FORCE_DROPLESS)(inp["x"], inp["logits"], *inp["weights"])
    y0 = g.LayerRunner(p0, g.MODE_FORCE_DROPLESS)(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_capped_dedup_drops_match_oracle(g):
    """Dedup with a cap small enough to cut every shard's buffer."""
    w = SMALL_CASES["dedup_small"].scaled(factor=0.2)
    _, inp, hc = inputs("dedup_small")
    p, op = binding_problem(w), oracle_problem(w)
    say("[layer] dedup capped drops")
    run = g.LayerRunner(p, g.MODE_CAPPED_ONLY)
    y = run(inp["x"], inp["logits"], *inp["weights"])
    want = oracle.layer(op, oracle.MODE_CAPPED_ONLY, hc["logits"], hc["x"], *hc["w"])
    torch.cuda.synchronize()
    check_close(host(y), want["y"], "y capped dedup")
    plain = oracle.layer_plain(op, hc["logits"], hc["x"], *hc["w"])
    assert not np.allclose(want["y"], plain)      # the capped model diverges


def test_repeat_is_bitwise_deterministic(g):
    w, inp, _ = inputs("mid_bf16")
    p = binding_problem(w)
    run = g.LayerRunner(p, g.MODE_LAYER)
    say("[layer] determinism")
    y1 = run(inp["x"], inp["logits"], *inp["weights"]).clone()
    y2 = run(inp["x"], inp["logits"], *inp["weights"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# Rows of exactly 16 KB and of 17 KB (bf16, H = 8192 and 8704) through the
# step API's permute: passes of at most 8192 elements take the one-launch
# permute, whose waves load a row of up to 16 KB before the layout and copy
# longer rows after it.
@pytest.mark.parametrize("hidden", [8192, 8704])
def test_permute_long_rows(g, hidden):
    w = workloads.Workload(f"long_rows_{hidden}", tokens=512, seq_len=256, hidden=hidden,
                           ffn=128, num_experts=8, top_k=2, num_shards=4, res_lo=1, res_hi=3,
                           factor=1.0, num_chunks=2, zipf=1.0)
    p, op = binding_problem(w), oracle_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    x_host = host(inp["x"])
    idx, _ = gpu_route(g, p, inp["logits"])
    cnt = gpu_count(g, p, idx)
    o_idx, _ = oracle.route(inp["logits"].cpu().numpy(), w.top_k, w.gate)
    want = oracle_count(op, o_idx)
    torch.cuda.synchronize()
    assert np.array_equal(ints(cnt["slot_of_assign"]), want["slot_of_assign"])
    slot_np = want["slot_of_assign"].reshape(w.tokens, w.top_k)
    cap = oracle.capacity(op)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    for (n, c, capped) in _passes(w):
        say(f"[permute] H={hidden} n={n} c={c} capped={capped}")
        rows, _ = g.pass_max_rows(p, n, capped)
        go, roa, sa = i32(p.g_res + 1, -7), i32(w.tokens * w.top_k, -7), i32(rows, -7)
        xs = torch.full((rows, w.hidden), 7.0, dtype=p.dtype, device="cuda")
        g.moe_permute(p, n, c, capped, inp["x"], cnt["slot_of_assign"], go, roa, sa, None, None,
                      None, None, xs, ws)
        toks = oracle.pass_tokens(op, n, c)
        lay = oracle.pass_layout(op, slot_np, toks, cap if capped else None)
        torch.cuda.synchronize()
        N = lay["num_rows"]
        assert np.array_equal(ints(go), lay["group_offsets"])
        assert np.array_equal(ints(sa)[:N], lay["sorted_assign"])
        assert np.array_equal(host(xs[:N]), oracle.permute(x_host, lay["sorted_assign"], w.top_k))
        assert bool((xs[N:] == 7.0).all())   # rows past the pass untouched


# The one-launch permute at its largest passes: 4097-8192 elements give each
# workgroup 32 elements, two rows per wave, with a ragged last workgroup.
# Rows of up to 10 KB (2 KB, and the Maverick-shaped 10 KB) are both loaded
# before the layout; rows of 14 KB load the first before it and copy the
# second after it; rows of 17 KB are all copied after it.
@pytest.mark.parametrize("tokens,hidden,res_lo,res_hi",
                         [(4096, 1024, 0, 4), (3000, 5120, 1, 3), (3000, 7168, 0, 4),
                          (2500, 8704, 0, 4)])
def test_permute_one_launch_large(g, tokens, hidden, res_lo, res_hi):
    w = workloads.Workload(f"perm_large_{tokens}_{hidden}", tokens=tokens, seq_len=tokens,
                           hidden=hidden, ffn=128, num_experts=16, top_k=2, num_shards=4,
                           res_lo=res_lo, res_hi=res_hi, factor=1.0, num_chunks=1, zipf=1.0)
    p, op = binding_problem(w), oracle_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    x_host = host(inp["x"])
    idx, _ = gpu_route(g, p, inp["logits"])
    cnt = gpu_count(g, p, idx)
    o_idx, _ = oracle.route(inp["logits"].cpu().numpy(), w.top_k, w.gate)
    want = oracle_count(op, o_idx)
    torch.cuda.synchronize()
    assert np.array_equal(ints(cnt["slot_of_assign"]), want["slot_of_assign"])
    slot_np = want["slot_of_assign"].reshape(w.tokens, w.top_k)
    cap = oracle.capacity(op)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    for (n, c, capped) in _passes(w):
        say(f"[permute large] T={tokens} H={hidden} n={n} c={c} capped={capped}")
        rows, _ = g.pass_max_rows(p, n, capped)
        go, roa, sa = i32(p.g_res + 1, -7), i32(w.tokens * w.top_k, -7), i32(rows, -7)
        xs = torch.full((rows, w.hidden), 7.0, dtype=p.dtype, device="cuda")
        g.moe_permute(p, n, c, capped, inp["x"], cnt["slot_of_assign"], go, roa, sa, None, None,
                      None, None, xs, ws)
        toks = oracle.pass_tokens(op, n, c)
        lay = oracle.pass_layout(op, slot_np, toks, cap if capped else None)
        torch.cuda.synchronize()
        N = lay["num_rows"]
        assert np.array_equal(ints(go), lay["group_offsets"])
        assert np.array_equal(ints(roa), lay["row_of_assign"].reshape(-1))
        assert np.array_equal(ints(sa)[:N], lay["sorted_assign"])
        assert np.array_equal(host(xs[:N]), oracle.permute(x_host, lay["sorted_assign"], w.top_k))
        assert bool((xs[N:] == 7.0).all())   # rows past the pass untouched
