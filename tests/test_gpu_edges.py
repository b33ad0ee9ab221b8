"""GPU parity on degenerate and boundary problems, the whole layer in every
mode against the float64 oracle (info bit-exact, y within the layer's
tolerance, and the dropless, chunked and LAYER results bitwise equal).

The cases sit at the edges the method allows: every token choosing every
expert (k = E), one expert per shard with only some shards resident, a
fallback whose chunks hold one position of each sequence, a single token,
heavy capped drops, more resident slots than the fused layout holds, 256-row
GEMM tiles with F >= 4096, and the fp32 path with dedup and redundant
slots.  The grouped GEMM is also given malformed group offsets (both tile
heights): it must compute nothing, and the same workspace must then serve a
well-formed call.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import binding_problem, check_close, host, ints, oracle_problem, say

pytestmark = pytest.mark.gpu

W = workloads.Workload
EDGES = {
    # k = E: every token is routed to every expert
    "all_experts": W("all_experts", tokens=64, seq_len=64, hidden=256, ffn=128, num_experts=4,
                     top_k=4, num_shards=2, res_lo=0, res_hi=2, factor=2.0, num_chunks=2),
    # one expert per shard, shards 2..4 resident, skewed sigmoid routing
    "one_per_shard": W("one_per_shard", tokens=256, seq_len=64, hidden=256, ffn=256,
                       num_experts=8, top_k=2, num_shards=8, res_lo=2, res_hi=5, factor=1.0,
                       num_chunks=4, gate="sigmoid", zipf=1.0),
    # chunks of one position per sequence (32 chunks of 2 tokens)
    "chunk_per_position": W("chunk_per_position", tokens=64, seq_len=32, hidden=256, ffn=128,
                            num_experts=8, top_k=2, num_shards=4, res_lo=0, res_hi=4,
                            factor=0.5, num_chunks=32, zipf=1.2),
    # a single token
    "single_token": W("single_token", tokens=1, seq_len=1, hidden=256, ffn=128, num_experts=8,
                      top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=1),
    # a cap of a quarter of the balanced load: most rows drop when capped
    "capped_drops": W("capped_drops", tokens=256, seq_len=256, hidden=256, ffn=128,
                      num_experts=16, top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=0.25,
                      num_chunks=4, zipf=1.0),
    # 256 resident slots without dedup: the layout's three-launch path (the
    # fused scan/placement holds at most 128 slots' block counts in LDS)
    "many_slots": W("many_slots", tokens=512, seq_len=256, hidden=256, ffn=128,
                    num_experts=256, top_k=4, num_shards=2, res_lo=0, res_hi=2, factor=1.0,
                    num_chunks=2, zipf=0.8),
    # 256-row GEMM tiles (H >= 2048) with F >= 4096, single and chunked passes
    "big_tiles_split": W("big_tiles_split", tokens=256, seq_len=128, hidden=2048, ffn=4096,
                         num_experts=16, top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=2.0,
                         num_chunks=2, zipf=0.5),
    # fp32 with dedup and two redundant slots
    "fp32_dedup_redundant": W("fp32_dedup_redundant", tokens=128, seq_len=128, hidden=64,
                              ffn=64, num_experts=8, top_k=3, num_shards=4, res_lo=0, res_hi=4,
                              factor=1.0, num_chunks=2, bf16=False, dedup=True,
                              slots_per_shard=1, num_replicas=2, zipf=1.5),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_edge_layer_all_modes(name):
    import grouped_gemm_shard_amd as g
    w = EDGES[name]
    p, op = binding_problem(w), oracle_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    logits, x = inp["logits"].cpu().numpy(), host(inp["x"])
    ws = [host(t) for t in inp["weights"]]
    ys = {}
    for mode in (g.MODE_LAYER, g.MODE_FORCE_DROPLESS, g.MODE_CAPPED_ONLY, g.MODE_FORCE_CHUNKED):
        say(f"[edge] {name} mode={mode}")
        run = g.LayerRunner(p, mode)
        y = run(inp["x"], inp["logits"], *inp["weights"]).clone()
        info = ints(run.info)
        want = oracle.layer(op, mode, logits, x, *ws)
        torch.cuda.synchronize()
        cap = -1 if want["cap"] is None else want["cap"]
        assert info.tolist() == [int(want["overflow"]), int(want["fallback_ran"]), cap,
                                 int(want["shard_counts"].max()), 0], name
        check_close(host(y), want["y"], f"y {name} mode {mode}")
        ys[mode] = y
    assert torch.equal(ys[g.MODE_FORCE_DROPLESS], ys[g.MODE_FORCE_CHUNKED])
    assert torch.equal(ys[g.MODE_LAYER], ys[g.MODE_FORCE_DROPLESS])


MALFORMED = {
    # group offsets that are not non-decreasing within [0, rows]: the first
    # group ends before it starts
    "decreasing": lambda G, rows: [0, 64, 32] + [64] * (G - 2),
    # the last offset past the rows the buffers hold
    "past_rows": lambda G, rows: [0] + [rows + 1] * G,
    # a negative first offset
    "negative": lambda G, rows: [-8] + [16] * G,
}


@pytest.mark.parametrize("hidden,bf16", [(256, True), (2048, True), (256, False)])
@pytest.mark.parametrize("case", sorted(MALFORMED))
def test_gmm_malformed_offsets_touch_nothing(case, hidden, bf16):
    """The grouped GEMM given group offsets that are not a non-decreasing
    sequence within [0, rows] computes nothing (act and expert_out keep their
    contents: the tile schedule gives no tiles, so no workgroup waits or
    writes) and says so: MOE_ERR_BAD_OFFSETS in its status word.  Both bf16
    tile heights (128 rows, one launch; 256 rows) and fp32."""
    import grouped_gemm_shard_amd as g
    w = W(f"malformed_{hidden}", tokens=64, seq_len=64, hidden=hidden, ffn=256, num_experts=8,
          top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=2, bf16=bf16)
    dt = torch.bfloat16 if bf16 else torch.float32
    p = binding_problem(w)
    say(f"[gmm malformed] {case} H={hidden}")
    rows = 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    xs = torch.randn((rows, hidden), generator=gen, device="cuda").to(dt)
    wts = workloads.make_weights(w, device="cuda")
    se = torch.arange(p.num_slots, dtype=torch.int32, device="cuda")  # home slots, no replicas
    go = torch.tensor(MALFORMED[case](p.g_res, rows), dtype=torch.int32, device="cuda")
    assert go.numel() == p.g_res + 1
    act = torch.full((rows, w.ffn), 7.0, dtype=dt, device="cuda")
    out = torch.full((rows, hidden), 7.0, dtype=dt, device="cuda")
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    g.moe_gmm_swiglu(p, xs, go, se, *wts, act, out, ws, status=status)
    torch.cuda.synchronize()
    assert torch.all(act == 7.0) and torch.all(out == 7.0)
    assert int(status.item()) == g.ERR_BAD_OFFSETS
    # the same workspace then serves a well-formed call (counters re-zeroed)
    go_ok = torch.tensor([min(16 * i, rows) for i in range(p.g_res + 1)], dtype=torch.int32,
                         device="cuda")
    g.moe_gmm_swiglu(p, xs, go_ok, se, *wts, act, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    n = int(go_ok[-1].item())
    o_act, o_out = oracle.gmm_swiglu(oracle_problem(w), host(xs[:n]), ints(go_ok),
                                     np.arange(p.g_res), *[host(t) for t in wts])
    check_close(host(act[:n]), o_act, f"act after malformed {case} H={hidden}")
    check_close(host(out[:n]), o_out, f"expert_out after malformed {case} H={hidden}")
    assert torch.all(out[n:] == 7.0)
