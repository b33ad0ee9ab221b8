"""The layer captured in a HIP graph (torch.cuda.graph) and replayed.

The layer call only enqueues work (no host synchronisation, no allocation,
no memset), so it can be captured, its passes in order on the caller's
stream.  Every replay, with other eager work on the device between
replays, must give y and info bitwise equal to the eager call.
"""

import pytest
import torch

import workloads
from moe_cases import SMALL_CASES, binding_problem, say

pytestmark = pytest.mark.gpu

CASES = [
    ("mid_bf16", "LAYER"),            # one pass
    ("mid_bf16", "FORCE_CHUNKED"),    # passes of two chunks
    ("maverick_small", "LAYER"),      # pass slots chosen on the device
    ("dedup_small", "FORCE_CHUNKED"),  # dedup gather, several passes
    ("maverick_wide", "FORCE_DROPLESS"),  # one pass, F = 4096
]


@pytest.mark.parametrize("name,mode_name", CASES)
def test_layer_graph_replay(name, mode_name):
    import grouped_gemm_shard_amd as g
    mode = getattr(g, "MODE_" + mode_name)
    w = SMALL_CASES[name]
    p = binding_problem(w)
    inp = workloads.make_inputs(w, device="cuda")
    args = (inp["x"], inp["logits"], *inp["weights"])
    say(f"[graph] {name} {mode_name}")
    run = g.LayerRunner(p, mode)
    # eager reference (also caches launch shapes before the capture)
    y_ref = run(*args).clone()
    info_ref = run.info.clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*args)
    torch.cuda.synchronize()

    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        # eager work between replays: clear the outputs, touch other memory
        run.y.zero_()
        run.info.fill_(-7)
        scratch.normal_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(run.info, info_ref), (name, mode_name, rep)
        assert torch.equal(run.y, y_ref), (name, mode_name, rep)
        # an eager call between replays must not disturb the next replay
        y_eager = run(*args).clone()
        torch.cuda.synchronize()
        assert torch.equal(y_eager, y_ref), (name, mode_name, rep)
