"""Shared pieces of the GPU parity tests: the cases, their problems for the
binding and the oracle, host copies of the inputs and the tolerance check.

Floating-point outputs (gates, act, expert_out, y) must meet the layer's
tolerance against the float64 oracle: max |diff| / max |ref| <= 2e-2 (a
normwise relative error, since elementwise relative error is undefined on
the exact zeros of non-resident tokens) and mean |diff| <= 1e-3.  Integer
artefacts are compared bit-exactly.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from workloads import CONFIGS

MAX_REL = 2e-2
MEAN_ABS = 1e-3

# Reduced versions of the three large workloads: same routing structure
# (experts, top-k, shards, skew, dedup, replicas, chunks), smaller T / H / F
# so that the float64 oracle finishes in seconds, still spanning several
# GEMM tiles per group and ragged tails.
MEDIUM = {
    "dsv3_small": CONFIGS["dsv3_shard"].scaled(name="dsv3_small", tokens=1024, seq_len=1024,
                                               hidden=1024, ffn=768),
    "maverick_small": CONFIGS["maverick_shard"].scaled(name="maverick_small", tokens=4096,
                                                       seq_len=1024, hidden=1024, ffn=2048),
    "dedup_small": CONFIGS["dedup_redundant"].scaled(name="dedup_small", tokens=512,
                                                     seq_len=512, hidden=256, ffn=128),
    # the DeepSeek-V3 receive shape: 8 source sequences, shard 0 resident
    "dsv3_ep8_small": CONFIGS["dsv3_ep8_receive"].scaled(name="dsv3_ep8_small", tokens=2048,
                                                         seq_len=256, hidden=1024, ffn=512),
    # hidden >= 2048 selects 256-row GEMM tiles (a group's last tile of at
    # most 128 rows runs as a 128-row tile)
    "maverick_mid": CONFIGS["maverick_shard"].scaled(name="maverick_mid", tokens=2048,
                                                     seq_len=512, hidden=2048, ffn=1024),
    # F >= 4096: long GEMM2 reductions
    "maverick_wide": CONFIGS["maverick_shard"].scaled(name="maverick_wide", tokens=1024,
                                                      seq_len=256, hidden=256, ffn=4096),
}
SMALL_CASES = {"tiny_fp32": CONFIGS["tiny_fp32"], "mid_bf16": CONFIGS["mid_bf16"], **MEDIUM}


def binding_problem(w: workloads.Workload):
    import grouped_gemm_shard_amd as g
    return g.Problem(**w.problem_kwargs())


def oracle_problem(w: workloads.Workload):
    return oracle.Problem(**w.problem_kwargs())


def host(t: torch.Tensor) -> np.ndarray:
    return workloads.to_f64(t)


def ints(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def check_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    scale = float(np.max(np.abs(ref)))
    rel = float(np.max(diff)) / scale if scale > 0 else float(np.max(diff))
    mean = float(np.mean(diff))
    assert rel <= MAX_REL, f"{what}: max rel {rel:.3e} > {MAX_REL}"
    assert mean <= MEAN_ABS, f"{what}: mean abs {mean:.3e} > {MEAN_ABS}"
    return rel, mean


def check_close_grad(got, ref, what=""):
    """The layer's tolerance for a gradient.  Gradients are linear in the
    upstream gradient dy, whose scale is arbitrary, so both bounds are taken
    relative to the reference's largest magnitude: max |diff| / max |ref| <=
    2e-2 (as for the outputs) and mean |diff| / max |ref| <= 1e-3 (the
    outputs' mean-abs bound, made scale-free)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    scale = float(np.max(np.abs(ref)))
    scale = scale if scale > 0 else 1.0
    rel = float(np.max(diff)) / scale
    mean = float(np.mean(diff)) / scale
    assert rel <= MAX_REL, f"{what}: max rel {rel:.3e} > {MAX_REL}"
    assert mean <= MEAN_ABS, f"{what}: mean abs / max |ref| {mean:.3e} > {MEAN_ABS}"
    return rel, mean


def check_close_grad_per_expert(got, ref, what=""):
    """check_close_grad on each expert's slice (axis 0) at that slice's own
    scale: under skewed routing a cold expert's weight gradient can be orders
    of magnitude below the hottest expert's, and the whole tensor's scale
    would let a wrong cold-expert slice (one left at zero, say) pass."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    for e in range(ref.shape[0]):
        check_close_grad(got[e], ref[e], f"{what} expert {e}")


class LazyExperts:
    """w[e] -> float64 host copy of one resident expert's matrix, fetched on
    demand so that full-size weights never sit on the host all at once."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return host(self.t[e])


def say(*a):
    print(*a, flush=True)
