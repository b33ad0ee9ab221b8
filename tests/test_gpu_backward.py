"""GPU parity of the backward (moe_combine_bwd, moe_gmm_swiglu_bwd,
moe_permute_bwd, moe_route_bwd) through the C ABI.

Each case runs the forward's steps and the backward's steps pass by pass,
as a caller of the step API would (the passes the GPU's own overflow flag
selects; weight gradients overwritten on the first pass and accumulated
after), and compares dx, d_logits, d_gate and the three weight gradients
with the float64 oracle's backward of the same layer (oracle.layer_bwd) on
the same seeded inputs and upstream gradient, to the layer's tolerance taken
relative to each gradient's scale (check_close_grad), and for the weight
gradients also expert by expert at each expert's own scale.
The pass choice is compared bit-exactly.

Cases: the fp32 path; the benchmark's mid-sized layer at full size (its
chunked fallback runs); reduced DeepSeek-V3 (one of 8 shards resident,
ragged groups), reduced Llama4-Maverick (sigmoid top-1, 256-row forward
tiles), dedup with redundant slots (replica groups add into their home
expert's gradients); and every mode on a small dedup problem.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import (MEDIUM, binding_problem, check_close_grad, check_close_grad_per_expert,
                        host, oracle_problem, say)

pytestmark = pytest.mark.gpu

W = workloads.Workload


def i32(n, fill=-7):
    t = torch.empty(n, dtype=torch.int32, device="cuda")
    t.fill_(fill)
    return t


def gpu_backward(g, w, mode, inp, dy):
    """Forward and backward through the step API; returns host arrays."""
    p = binding_problem(w)
    T, k, H, F, E = w.tokens, w.top_k, w.hidden, w.ffn, w.num_experts
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ec, se, nd = i32(E), i32(p.num_slots), i32(E)
    soa, sc, st = i32(T * k), i32(w.num_shards), i32(4)
    g.moe_count_overflow(p, idx, ec, se, nd, soa, sc, st, ws)
    status = st.cpu().numpy()
    capped_ok = int(status[0]) >= 0
    chunked = {g.MODE_LAYER: bool(status[1]), g.MODE_FORCE_DROPLESS: False,
               g.MODE_CAPPED_ONLY: False, g.MODE_FORCE_CHUNKED: True}[mode]
    capped = int(capped_ok and not chunked and mode != g.MODE_FORCE_DROPLESS)
    n = w.num_chunks if chunked else 1
    rows, drows = g.pass_max_rows(p, n, capped)
    e_res = w.e_res
    wg, wu, wd = inp["weights"]
    nan = float("nan")
    dwg = torch.full((e_res, F, H), nan, dtype=torch.float32, device="cuda")
    dwu = torch.full((e_res, F, H), nan, dtype=torch.float32, device="cuda")
    dwd = torch.full((e_res, H, F), nan, dtype=torch.float32, device="cuda")
    d_gate = torch.full((T, k), nan, dtype=torch.float32, device="cuda")
    dx = torch.full((T, H), nan, dtype=p.dtype, device="cuda")
    bws = torch.empty(g.bwd_workspace_bytes(p, rows), dtype=torch.uint8, device="cuda")
    roa = i32(T * k)
    for c in range(n):
        go, sa = i32(p.g_res + 1), i32(rows)
        do, dt, ex = i32(p.s_res + 1), i32(max(drows, 1)), i32(rows)
        xd = torch.zeros((max(drows, 1), H), dtype=p.dtype, device="cuda")
        xs = torch.zeros((rows, H), dtype=p.dtype, device="cuda")
        g.moe_permute(p, n, c, capped, inp["x"], soa, go, roa, sa, do if w.dedup else None,
                      dt if w.dedup else None, ex if w.dedup else None,
                      xd if w.dedup else None, xs, ws)
        act = torch.zeros((rows, F), dtype=p.dtype, device="cuda")
        out = torch.zeros((rows, H), dtype=p.dtype, device="cuda")
        g.moe_gmm_swiglu(p, xs, go, se, wg, wu, wd, act, out, ws)
        d_out = torch.zeros((rows, H), dtype=p.dtype, device="cuda")
        g.moe_combine_bwd(p, n, c, dy, out, roa, gate, d_out, d_gate)
        dxs = torch.zeros((rows, H), dtype=p.dtype, device="cuda")
        g.moe_gmm_swiglu_bwd(p, xs, go, se, wg, wu, wd, d_out, dxs, dwg, dwu, dwd, c > 0, bws)
        g.moe_permute_bwd(p, n, c, dxs, roa, dx)
    d_logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    g.moe_route_bwd(p, idx, gate, d_gate, d_logits)
    torch.cuda.synchronize()
    return dict(dx=host(dx), d_logits=host(d_logits), d_gate=host(d_gate), dw_gate=host(dwg),
                dw_up=host(dwu), dw_down=host(dwd), fallback_ran=chunked)


def oracle_backward(w, mode, inp, dy):
    return oracle.layer_bwd(oracle_problem(w), mode, inp["logits"].cpu().numpy(),
                            host(inp["x"]), *[host(t) for t in inp["weights"]], host(dy))


def compare(w, mode):
    import grouped_gemm_shard_amd as g
    say(f"[backward] {w.name} mode={mode}")
    # one draw of the seeded inputs feeds both sides
    inp = workloads.make_inputs(w, device="cuda")
    dy = workloads.make_dy(w, device="cuda")
    got = gpu_backward(g, w, mode, inp, dy)
    ref = oracle_backward(w, mode, inp, dy)
    assert got["fallback_ran"] == ref["fallback_ran"]
    for name in ("dx", "d_gate", "d_logits", "dw_gate", "dw_up", "dw_down"):
        assert np.all(np.isfinite(got[name])), name
        rel, mean = check_close_grad(got[name], ref[name], f"{w.name} {name}")
        say(f"  {name:9s} max-rel {rel:.2e} mean/max {mean:.2e}")
        if name.startswith("dw_"):
            check_close_grad_per_expert(got[name], ref[name], f"{w.name} {name}")


# factor 0.5: every shard's distinct tokens exceed the cap, so LAYER runs
# the chunked fallback and CAPPED_ONLY drops rows (and their gradients)
SMALL_DEDUP = W("bwd_dedup_small", tokens=256, seq_len=256, hidden=256, ffn=128, num_experts=16,
                top_k=4, num_shards=4, res_lo=0, res_hi=4, factor=0.5, num_chunks=2,
                dedup=True, slots_per_shard=1, num_replicas=2, zipf=1.2)


@pytest.mark.parametrize("name", ["tiny_fp32", "dsv3_small", "maverick_mid", "dedup_small"])
def test_backward_against_oracle(name):
    w = workloads.CONFIGS.get(name) or MEDIUM[name]
    compare(w, 0)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_backward_modes(mode):
    compare(SMALL_DEDUP, mode)


@pytest.mark.slow
def test_backward_mid_full_size():
    # the benchmark's layer at full size, through its chunked fallback
    compare(workloads.CONFIGS["mid_bf16"], 0)


# ---- the whole layer's backward in one call (moe_layer_bwd) ----------------

def compare_layer(w, mode):
    """moe_layer_bwd against the oracle's backward of the same layer call;
    every output starts as NaN so that anything left unwritten fails."""
    import grouped_gemm_shard_amd as g
    say(f"[layer-backward] {w.name} mode={mode}")
    p = binding_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    dy = workloads.make_dy(w, device="cuda")
    run = g.LayerBackwardRunner(p, mode)
    for t in (run.dx, run.d_logits, run.dw_gate, run.dw_up, run.dw_down):
        t.fill_(float("nan"))
    got = run(inp["x"], inp["logits"], *inp["weights"], dy)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in got.items()}
    ref = oracle_backward(w, mode, inp, dy)
    for name in ("dx", "d_logits", "dw_gate", "dw_up", "dw_down"):
        assert np.all(np.isfinite(got[name])), name
        rel, mean = check_close_grad(got[name], ref[name], f"{w.name} {name}")
        say(f"  {name:9s} max-rel {rel:.2e} mean/max {mean:.2e}")
        if name.startswith("dw_"):
            check_close_grad_per_expert(got[name], ref[name], f"{w.name} {name}")
    # no atomics anywhere: a second call gives the same bits
    again = run(inp["x"], inp["logits"], *inp["weights"], dy)
    torch.cuda.synchronize()
    for name in ("dx", "d_logits", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(host(again[name]), got[name]), name


NO_DEDUP_SMALL = W("bwd_small", tokens=512, seq_len=256, hidden=256, ffn=256, num_experts=16,
                   top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=1.0, num_chunks=4,
                   zipf=1.2)


@pytest.mark.parametrize("name", ["tiny_fp32", "dsv3_small", "maverick_mid", "dedup_small",
                                  "dsv3_ep8_small", "maverick_wide"])
def test_layer_backward_against_oracle(name):
    w = workloads.CONFIGS.get(name) or MEDIUM[name]
    compare_layer(w, 0)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("which", ["dedup", "plain"])
def test_layer_backward_modes(which, mode):
    compare_layer(SMALL_DEDUP if which == "dedup" else NO_DEDUP_SMALL, mode)


@pytest.mark.slow
def test_layer_backward_mid_full_size():
    compare_layer(workloads.CONFIGS["mid_bf16"], 0)


# 130 chunks in 65 passes of two (the 0.009x buffer holds 150 rows, a chunk
# 128, so passes of two chunks fit twice the buffer): in the layer call an
# expert's weight gradients span 65 groups, one per pass, more than the 64
# that the 256 x 256 weight-gradient kernel keeps in its register window, and
# the hottest experts are cut into chunks whose partials are added in chunk
# order.
MANY_PASSES = W("bwd_many_passes", tokens=8320, seq_len=8320, hidden=2048, ffn=256,
                num_experts=8, top_k=2, num_shards=1, res_lo=0, res_hi=1, factor=0.009,
                num_chunks=130, zipf=1.1)


@pytest.mark.slow
def test_layer_backward_many_passes():
    import grouped_gemm_shard_amd as g
    p = binding_problem(MANY_PASSES)
    assert MANY_PASSES.num_chunks // g.layer_chunks_per_pass(p, g.MODE_LAYER) == 65
    compare_layer(MANY_PASSES, 0)
