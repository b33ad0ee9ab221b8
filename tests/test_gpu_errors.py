"""Device-side errors are reported, never silent.

The one-launch grouped GEMM (128-row tiles: GEMM1 and GEMM2 in one launch)
makes each GEMM2 tile wait, with a bound, for the GEMM1 tiles of its rows.
A tile that gives up leaves its rows of expert_out unwritten, so the call
must say so: MOE_ERR_GEMM_WAIT in info[4] of the layer call and in the
status word of moe_gmm_swiglu ("Moe dynamic redundancy", code review,
dedup truncation comment: the failure to avoid is losing rows silently).

The time-out is forced from the host through the test hook
moe_testing_set_gemm_wait_limit(-1) (every such wait gives up at once), so
every kernel still ends normally; the hook is restored afterwards and the
same buffers must then give the oracle's result with no error bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from moe_cases import SMALL_CASES, binding_problem, check_close, host, oracle_problem, say

pytestmark = pytest.mark.gpu


@pytest.fixture
def g():
    import grouped_gemm_shard_amd as gg
    yield gg
    gg.testing_set_gemm_wait_limit(0)   # the default bound, whatever the test did


def test_layer_reports_gemm_wait(g):
    w = SMALL_CASES["mid_bf16"]          # H = 1024: 128-row tiles, one-launch GEMM
    p = binding_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    run = g.LayerRunner(p, g.MODE_LAYER)
    say("[errors] layer with every GEMM wait giving up at once")
    g.testing_set_gemm_wait_limit(-1)
    run(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    info = run.info.cpu().tolist()
    assert info[4] & g.ERR_GEMM_WAIT, info
    say("[errors] layer with the default bound")
    g.testing_set_gemm_wait_limit(0)
    y = run(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    assert run.info[4].item() == 0
    op = oracle_problem(w)
    want = oracle.layer(op, oracle.MODE_LAYER, inp["logits"].cpu().numpy(), host(inp["x"]),
                        *[host(t) for t in inp["weights"]])
    check_close(host(y), want["y"], "y after the error path")


def test_step_gemm_reports_gemm_wait(g):
    w = SMALL_CASES["mid_bf16"]
    p = binding_problem(w)
    T, k, H, F = w.tokens, w.top_k, w.hidden, w.ffn
    rows = 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    xs = torch.randn((rows, H), generator=gen, device="cuda").to(torch.bfloat16)
    wts = workloads.make_weights(w, device="cuda")
    se = torch.arange(p.num_slots, dtype=torch.int32, device="cuda")
    go = torch.tensor([min(rows, (rows // p.g_res) * i + (37 if i else 0)) for i in
                       range(p.g_res)] + [rows], dtype=torch.int32, device="cuda")
    act = torch.zeros((rows, F), dtype=torch.bfloat16, device="cuda")
    out = torch.full((rows, H), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    say("[errors] step GEMM with every wait giving up at once")
    g.testing_set_gemm_wait_limit(-1)
    g.moe_gmm_swiglu(p, xs, go, se, *wts, act, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == g.ERR_GEMM_WAIT
    # the rows no GEMM2 tile wrote kept their contents
    assert torch.all(out == 3.0)
    say("[errors] step GEMM with the default bound")
    g.testing_set_gemm_wait_limit(0)
    g.moe_gmm_swiglu(p, xs, go, se, *wts, act, out, ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    o_act, o_out = oracle.gmm_swiglu(oracle_problem(w), host(xs), go.cpu().numpy(),
                                     np.arange(p.g_res), *[host(t) for t in wts])
    check_close(host(act), o_act, "act")
    check_close(host(out), o_out, "expert_out")
