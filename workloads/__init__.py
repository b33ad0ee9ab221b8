"""Seeded synthetic inputs for the one-shard MoE layer.

This module holds only input generation: shapes, seeds and value
distributions.  It holds none of the layer's arithmetic, so both the CPU
oracle and the GPU path may take their inputs from it.

Every workload is synthetic (the pages' runs use synthetic data as well).
Generators are torch generators seeded per (stream, index), so a tensor is
the same however many other tensors were drawn before it, and experts can be
generated one at a time.  The same seed gives different values on the CPU
and on the GPU (different torch generators); a test always hands the oracle
the exact tensors the GPU path received.

Streams: 0 router-logit noise [T,E]; 1 activations x [T,H]; 2/3/4 the gate,
up and down weights of expert e (index e).  Router logits are N(0,1) plus,
for skewed workloads, a Zipf bias -s*ln(rank) over expert rank (expert 0
hottest), added in float32.  Activations are N(0,1) and weights N(0, 0.02),
both rounded to bfloat16 (round to nearest even) for the bf16 workloads.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

MODE_LAYER, MODE_FORCE_DROPLESS, MODE_CAPPED_ONLY, MODE_FORCE_CHUNKED = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    seq_len: int
    hidden: int
    ffn: int
    num_experts: int
    top_k: int
    num_shards: int
    res_lo: int
    res_hi: int
    factor: float
    num_chunks: int
    gate: str = "softmax"
    bf16: bool = True
    dedup: bool = False
    slots_per_shard: int = 0
    num_replicas: int = 0
    zipf: float = 0.0
    weight_std: float = 0.02
    seed: int = 0

    @property
    def e_loc(self):
        return self.num_experts // self.num_shards

    @property
    def e_res(self):
        return (self.res_hi - self.res_lo) * self.e_loc

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)

    def problem_kwargs(self):
        """Fields shared by the oracle's Problem and the binding's problem."""
        return dict(tokens=self.tokens, seq_len=self.seq_len, hidden=self.hidden,
                    ffn=self.ffn, num_experts=self.num_experts, top_k=self.top_k,
                    num_shards=self.num_shards, res_lo=self.res_lo, res_hi=self.res_hi,
                    factor=self.factor, num_chunks=self.num_chunks, gate=self.gate,
                    bf16=self.bf16, dedup=self.dedup,
                    slots_per_shard=self.slots_per_shard,
                    num_replicas=self.num_replicas)


# The five workloads.  Derived choices: chunks default to ceil(S / factor)
# where the statement gives none; the Llama4-Maverick shard is 4 sequences
# of 8192; the dedup workload keeps the pages' recipe factor 2.0.
CONFIGS = {
    "tiny_fp32": Workload("tiny_fp32", tokens=256, seq_len=256, hidden=64, ffn=128,
                          num_experts=8, top_k=2, num_shards=4, res_lo=0, res_hi=4,
                          factor=2.0, num_chunks=2, gate="softmax", bf16=False),
    "mid_bf16": Workload("mid_bf16", tokens=4096, seq_len=4096, hidden=1024, ffn=512,
                         num_experts=32, top_k=4, num_shards=8, res_lo=0, res_hi=8,
                         factor=1.5, num_chunks=4, gate="softmax", zipf=1.1),
    "dsv3_shard": Workload("dsv3_shard", tokens=4096, seq_len=4096, hidden=7168, ffn=2048,
                           num_experts=256, top_k=8, num_shards=8, res_lo=0, res_hi=1,
                           factor=2.0, num_chunks=4, gate="softmax"),
    "maverick_shard": Workload("maverick_shard", tokens=32768, seq_len=8192, hidden=5120,
                               ffn=8192, num_experts=128, top_k=1, num_shards=16,
                               res_lo=0, res_hi=1, factor=2.0, num_chunks=8,
                               gate="sigmoid", zipf=1.3),
    # The DeepSeek-V3 shard as it receives under 8-way expert parallelism:
    # 8 sources (sequences) of 4096 tokens each route over all 256 experts,
    # and this GPU runs shard 0 (experts 0..31) on the union of the rows the
    # sources send it (~32.8k rows instead of ~4.1k from one source).
    "dsv3_ep8_receive": Workload("dsv3_ep8_receive", tokens=32768, seq_len=4096, hidden=7168,
                                 ffn=2048, num_experts=256, top_k=8, num_shards=8, res_lo=0,
                                 res_hi=1, factor=2.0, num_chunks=4, gate="softmax"),
    "dedup_redundant": Workload("dedup_redundant", tokens=8192, seq_len=8192, hidden=7168,
                                ffn=2048, num_experts=256, top_k=8, num_shards=16,
                                res_lo=0, res_hi=16, factor=2.0, num_chunks=8,
                                gate="softmax", dedup=True, slots_per_shard=2,
                                num_replicas=2, zipf=1.2),
}
ORDER = ["tiny_fp32", "mid_bf16", "dsv3_shard", "maverick_shard", "dedup_redundant",
         "dsv3_ep8_receive"]


def _seed(seed: int, stream: int, index: int) -> int:
    st = np.random.SeedSequence([seed, stream, index]).generate_state(2, dtype=np.uint32)
    return (int(st[0]) << 31) ^ int(st[1])


def _normal(shape, seed, stream, index, device, std=1.0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, stream, index))
    out = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        out.mul_(std)
    return out


def zipf_bias(num_experts: int, s: float) -> torch.Tensor:
    """-s * ln(rank), rank = e + 1, as float32 (computed in float64)."""
    r = np.arange(1, num_experts + 1, dtype=np.float64)
    return torch.from_numpy((-s * np.log(r)).astype(np.float32))


def make_logits(w: Workload, device="cpu") -> torch.Tensor:
    lg = _normal((w.tokens, w.num_experts), w.seed, 0, 0, device)
    if w.zipf:
        lg.add_(zipf_bias(w.num_experts, w.zipf).to(device))
    return lg


def make_x(w: Workload, device="cpu") -> torch.Tensor:
    x = _normal((w.tokens, w.hidden), w.seed, 1, 0, device)
    return x.to(torch.bfloat16) if w.bf16 else x


def make_weights(w: Workload, device="cpu"):
    """(w_gate [E_res,F,H], w_up [E_res,F,H], w_down [E_res,H,F]) for the
    resident experts; expert e draws from its own streams, so a subset is
    identical to the same experts of the full set."""
    dt = torch.bfloat16 if w.bf16 else torch.float32
    e0 = w.res_lo * w.e_loc
    n = w.e_res
    wg = torch.empty((n, w.ffn, w.hidden), dtype=dt, device=device)
    wu = torch.empty((n, w.ffn, w.hidden), dtype=dt, device=device)
    wd = torch.empty((n, w.hidden, w.ffn), dtype=dt, device=device)
    for i in range(n):
        e = e0 + i
        wg[i] = _normal((w.ffn, w.hidden), w.seed, 2, e, device, w.weight_std).to(dt)
        wu[i] = _normal((w.ffn, w.hidden), w.seed, 3, e, device, w.weight_std).to(dt)
        wd[i] = _normal((w.hidden, w.ffn), w.seed, 4, e, device, w.weight_std).to(dt)
    return wg, wu, wd


def make_dy(w: Workload, device="cpu") -> torch.Tensor:
    """Upstream gradient of the layer output, [T,H] standard normal, in the
    activation dtype (for the backward)."""
    dy = _normal((w.tokens, w.hidden), w.seed, 5, 0, device)
    return dy.to(torch.bfloat16) if w.bf16 else dy


def make_inputs(w: Workload, device="cpu"):
    return dict(logits=make_logits(w, device), x=make_x(w, device), weights=make_weights(w, device))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy on the host (bf16 and fp32 values are exact in f64)."""
    return t.detach().to("cpu", torch.float64).numpy()


def default_chunks(num_shards: int, factor: float) -> int:
    """ceil(S / factor): the fallback's chunk count read from the example
    the fallback page's Shortcomings example (16-way expert parallelism at
    factor 2 gives an eight-fold slowdown, i.e. eight chunks)."""
    return int(math.ceil(num_shards / factor))
