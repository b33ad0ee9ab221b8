"""moe_gmm_swiglu_noalloc (the grouped GEMM without a workspace, for callers
that cannot allocate) against moe_gmm_swiglu, through the C ABI.

Both run the same kernels, so act and expert_out must agree bitwise, and
rows past the groups must stay untouched.  Two calls in a row, the second
with a smaller input, check that the shared scratch array is cleared for
each call (its counters start at zero whatever the last call left).  Cases:
128-row tiles (the one-launch GEMM, whose counters live in the scratch),
256-row tiles, and float32.
"""

import pytest
import torch

import workloads
from moe_cases import binding_problem, say

pytestmark = pytest.mark.gpu

W = workloads.Workload
CASES = {
    "bf16_h1024": (W("na_1024", tokens=2048, seq_len=2048, hidden=1024, ffn=512, num_experts=16,
                     top_k=4, num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=2),
                   [4096, 1000]),
    "bf16_h2048": (W("na_2048", tokens=1024, seq_len=1024, hidden=2048, ffn=768, num_experts=8,
                     top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=2),
                   [2048, 700]),
    "f32_h256": (W("na_f32", tokens=512, seq_len=512, hidden=256, ffn=128, num_experts=8,
                   top_k=2, num_shards=4, res_lo=0, res_hi=4, factor=2.0, num_chunks=2,
                   bf16=False), [1024, 100]),
}


def offsets(G, rows, seed):
    """Ragged, non-decreasing group offsets over `rows` rows (some groups
    empty, some longer than one tile)."""
    gen = torch.Generator().manual_seed(seed)
    cuts = torch.sort(torch.randint(0, rows + 1, (G - 1,), generator=gen)).values
    return torch.cat([torch.zeros(1, dtype=torch.long), cuts,
                      torch.tensor([rows])]).to(torch.int32)


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_matches_workspace_call(name):
    import grouped_gemm_shard_amd as g
    w, sizes = CASES[name]
    p = binding_problem(w)
    dt = p.dtype
    wts = workloads.make_weights(w, device="cuda")
    se = torch.arange(p.num_slots, dtype=torch.int32, device="cuda")
    cap = max(sizes) + 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    xs = torch.randn((cap, w.hidden), generator=gen, device="cuda").to(dt)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    for call, rows in enumerate(sizes):
        say(f"[noalloc] {name} call {call} rows={rows}")
        go = offsets(p.g_res, rows, seed=call).cuda()
        outs = []
        for fn in ("workspace", "noalloc"):
            act = torch.full((cap, w.ffn), 5.0, dtype=dt, device="cuda")
            out = torch.full((cap, w.hidden), 5.0, dtype=dt, device="cuda")
            status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
            if fn == "workspace":
                g.moe_gmm_swiglu(p, xs, go, se, *wts, act, out, ws, status=status)
            else:
                g.moe_gmm_swiglu_noalloc(p, xs, go, se, *wts, act, out, status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0, (fn, int(status.item()))
            outs.append((act, out))
        (a0, o0), (a1, o1) = outs
        assert torch.equal(a0, a1), f"act differs ({name}, call {call})"
        assert torch.equal(o0, o1), f"expert_out differs ({name}, call {call})"
        assert torch.all(a1[rows:] == 5.0) and torch.all(o1[rows:] == 5.0)
        assert not torch.all(o1[:rows] == 5.0)
