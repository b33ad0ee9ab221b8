"""Benchmark of the one-shard MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload maverick_shard]

A step is one call of the whole layer in LAYER mode (route, counts, plan,
capacity and overflow check, then the capped pass or the chunked dropless
fallback: layout, grouped SwiGLU GEMM gathering its rows, combine) on one
batch of seeded synthetic input already resident in HBM.  The default
workload is the Llama4-Maverick-shaped shard (T=32768 as 4 sequences of
8192, H=5120, F=8192, 8 resident experts of 128 in 16 virtual shards, top-1
sigmoid gate, Zipf(1.3) routing that overflows buffer factor 2.0, so the
layer runs the 8-chunk dropless fallback, one chunk per pass); the other
workloads are behind --workload.

After the timed steps, the grouped GEMM, the permute and the combine of the
same passes are timed one call at a time with HIP events on the stream they
run on, to give achieved TFLOP/s and GB/s against MI355X peaks; the grouped
GEMMs of all passes are also replayed on the layer's own schedule (passes
alternating between two streams) and timed as one span.  The backward of
the same passes (given the forward's saved x_sorted and expert outputs) is
timed as a whole and step by step ("backward" in the JSON), and so is the
whole-layer backward call (which also recomputes the routing, layouts,
x_sorted and expert outputs) and a training step's layer forward plus it.
The library's calibration kernels (a streaming copy and a matrix-core loop)
and the vendor library's dense bf16 GEMM are timed as what this machine reaches
outside the layer ("measured_peaks").  The CPU
oracle is then timed on the host cores on the same inputs (the whole layer
where it finishes within the budget, else the plain layer definition on a
stated sample of tokens).  One JSON line is printed at the end.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import grouped_gemm_shard_amd as g  # noqa: E402
import workloads  # noqa: E402

METRIC = "MoE layer routed tokens/s; grouped-GEMM % MFMA peak; permute HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM traffic of the grouped GEMM per layer (every GEMM launch of one LAYER
# call), from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) scaled by
# what the counters read for the calibration copy of 1 GiB (FETCH_SIZE
# x1.99997, WRITE_SIZE x1.0).  It holds only for the kernel source it was
# measured on (sha256 of gmm.hip), that workload and the layer's chunks per
# pass; otherwise the traffic is reported as null.
GEMM_TRAFFIC = {
    "maverick_shard": {
        "gmm_src_sha256": "2ee25cb014df7ce9608d68cb2f1860a7ebc712b43414fe8a5cbc49868e412a2f",
        "chunks_per_pass": 2,
        "bytes_per_layer": 20883169063},
    "mid_bf16": {
        "gmm_src_sha256": "2ee25cb014df7ce9608d68cb2f1860a7ebc712b43414fe8a5cbc49868e412a2f",
        "chunks_per_pass": 4,
        "bytes_per_layer": 268087767},
}


def recorded_gemm_traffic(workload, chunks_per_pass):
    import hashlib
    src = os.path.join(ROOT, "grouped_gemm_shard_amd", "csrc", "gmm.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = GEMM_TRAFFIC.get(workload)
    if rec is None or sha != rec["gmm_src_sha256"] or chunks_per_pass != rec["chunks_per_pass"]:
        return None
    return rec["bytes_per_layer"]


def cache_note(w, p):
    """Whether the step's working set (x, logits, weights, y and the layer
    workspace) fits MI355X's 256 MB last-level cache, so that repeated steps
    run partly from it (warm)."""
    es = 2 if w.bf16 else 4
    ws = (w.tokens * w.hidden * es * 2 + w.tokens * w.num_experts * 4 +
          3 * w.e_res * w.hidden * w.ffn * es + g.layer_workspace_bytes(p, g.MODE_LAYER))
    mb = ws / 1e6
    return (f"working set {mb:.0f} MB " +
            ("fits the 256 MB last-level cache: repeated steps run warm" if mb < 256
             else "exceeds the 256 MB last-level cache"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pass_list(p, info):
    """The passes LAYER mode took, as (chunks, chunk, capped) of the step API:
    when the flag fired, the dropless chunks q at a time (q consecutive
    chunks of n are chunk b of n/q), else the one capped pass."""
    if info[0]:
        n = p.num_chunks
        q = g.layer_chunks_per_pass(p, g.MODE_LAYER)
        if n % q:
            q = 1
        return [(n // q, b, 0) for b in range(n // q)]
    return [(1, 0, 1)]


def build_passes(p, w, inp, passes):
    """Runs route / counts / permute through the step API and keeps each
    pass's layout, so that single kernels can be timed on real data."""
    T, k = w.tokens, w.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    g.moe_route(p, inp["logits"], idx, gate)
    ws = torch.empty(g.workspace_bytes(p), dtype=torch.uint8, device="cuda")
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")  # noqa: E731
    cnt = dict(ec=i32(w.num_experts), se=i32(p.num_slots), nd=i32(w.num_experts),
               soa=i32(T * k), sc=i32(w.num_shards), st=i32(4))
    g.moe_count_overflow(p, idx, cnt["ec"], cnt["se"], cnt["nd"], cnt["soa"], cnt["sc"],
                         cnt["st"], ws)
    out = []
    for (n, c, capped) in passes:
        rows, drows = g.pass_max_rows(p, n, capped)
        b = dict(n=n, c=c, capped=capped, rows=rows, ws=torch.empty_like(ws),
                 go=i32(p.g_res + 1), roa=i32(T * k), sa=i32(rows),
                 xs=torch.empty((rows, w.hidden), dtype=p.dtype, device="cuda"),
                 act=torch.empty((rows, w.ffn), dtype=p.dtype, device="cuda"),
                 out=torch.empty((rows, w.hidden), dtype=p.dtype, device="cuda"),
                 y=torch.empty((T, w.hidden), dtype=p.dtype, device="cuda"))
        if w.dedup:
            b.update(do=i32(p.s_res + 1), dt=i32(drows), ex=i32(rows),
                     xd=torch.empty((drows, w.hidden), dtype=p.dtype, device="cuda"))
        else:
            b.update(do=None, dt=None, ex=None, xd=None)
        out.append(b)
    return idx, gate, cnt, out


def run_permute(p, inp, cnt, b):
    g.moe_permute(p, b["n"], b["c"], b["capped"], inp["x"], cnt["soa"], b["go"], b["roa"],
                  b["sa"], b["do"], b["dt"], b["ex"], b["xd"], b["xs"], b["ws"])


def run_gmm(p, inp, cnt, b):
    g.moe_gmm_swiglu(p, b["xs"], b["go"], cnt["se"], *inp["weights"], b["act"], b["out"],
                     b["ws"])


def run_combine(p, gate, b):
    g.moe_combine(p, b["n"], b["c"], b["out"], b["roa"], gate, b["y"])


def time_calls(fn, reps):
    """Mean duration (s) of fn() over reps calls, HIP events on the current
    stream (the stream every library call is enqueued on)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, z in ev:
        a.record(stream)
        fn()
        z.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(z) for a, z in ev) / reps / 1e3


def gemm_layer_schedule(p, inp, cnt, bufs, reps):
    """Duration (s) of the grouped GEMMs of every pass on the layer's own
    schedule, the passes in order on the caller's stream: the same GEMM
    calls are replayed that way (without the layer's layout and combine
    launches) and timed as one span, so the figure is a span of the layer
    step, never longer than it."""
    def serial():
        for b in bufs:
            run_gmm(p, inp, cnt, b)
    return time_calls(serial, reps)


def kernel_figures(p, w, inp, info, reps):
    passes = pass_list(p, info)
    idx, gate, cnt, bufs = build_passes(p, w, inp, passes)
    torch.cuda.synchronize()
    es = 2 if w.bf16 else 4
    rows = []
    t_perm = t_gmm = t_comb = 0.0
    for b in bufs:
        t_perm += time_calls(lambda: run_permute(p, inp, cnt, b), reps)
        t_gmm += time_calls(lambda: run_gmm(p, inp, cnt, b), reps)
        t_comb += time_calls(lambda: run_combine(p, gate, b), reps)
        rows.append(int(b["go"][-1].item()))
    n_rows = sum(rows)
    t_gmm_sched = gemm_layer_schedule(p, inp, cnt, bufs, reps)
    # algorithmic work per layer (all passes)
    gemm_flops = 6.0 * n_rows * w.hidden * w.ffn
    ec = cnt["ec"].cpu().numpy()
    # weights streamed once per pass for every expert with rows in that pass
    w_bytes = 0
    for b in bufs:
        go = b["go"].cpu().numpy()
        se = cnt["se"].cpu().numpy()
        used = set()
        for q in range(p.g_res):
            if go[q + 1] > go[q]:
                used.add(int(se[w.res_lo * p.spd + q]))
        w_bytes += len(used) * 3 * w.hidden * w.ffn * es
    gemm_bytes = w_bytes + n_rows * (2 * w.hidden + 2 * w.ffn) * es
    tokens_res = 0
    for b in bufs:
        roa = b["roa"].cpu().numpy().reshape(w.tokens, w.top_k)
        toks = workloads_pass_tokens(w, b["n"], b["c"])
        tokens_res += int(np.sum((roa[toks] >= 0).any(axis=1)))
    # each resident token's row read once and each pass row written once;
    # with dedup the rows go through x_dedup (one row per token and shard,
    # written and read once)
    u_all = sum(int(b["do"][-1].item()) for b in bufs) if w.dedup else 0
    perm_bytes = (tokens_res + 2 * u_all + n_rows) * w.hidden * es
    comb_bytes = n_rows * w.hidden * es + w.tokens * w.hidden * es
    del ec
    fig = dict(rows=n_rows, t_gmm=t_gmm, t_gmm_sched=t_gmm_sched, passes=len(bufs),
               t_perm=t_perm, t_comb=t_comb, gemm_flops=gemm_flops,
               gemm_bytes=gemm_bytes, perm_bytes=perm_bytes, comb_bytes=comb_bytes)
    if w.dedup:
        # return-path dedup: partial rows at the receiving shard (reads every
        # expert_out row once, writes one row per token and shard), then the
        # sum at the source (reads the partial rows, writes y)
        t_part = t_src = 0.0
        u_rows = 0
        for b in bufs:
            part = torch.empty((b["dt"].shape[0], w.hidden), dtype=torch.float32, device="cuda")
            y2 = torch.empty_like(b["y"])
            t_part += time_calls(lambda: g.moe_combine_partial(
                p, b["n"], b["c"], b["capped"], b["out"], b["roa"], gate, b["do"], b["dt"],
                b["ex"], part), reps)
            t_src += time_calls(lambda: g.moe_combine_from_partials(
                p, b["n"], b["c"], b["capped"], part, b["roa"], b["ex"], y2, b["rows"]), reps)
            u_rows += int(b["do"][-1].item())
        fig.update(u_rows=u_rows, t_part=t_part, t_src=t_src,
                   part_bytes=n_rows * w.hidden * es + u_rows * w.hidden * 4,
                   src_bytes=u_rows * w.hidden * 4 + w.tokens * w.hidden * es)
    return fig


def backward_figures(p, w, inp, info, reps):
    """The backward of the same passes (the forward's saved x_sorted and
    expert_out kept): per pass the combine's backward, the grouped GEMM's backward (weight gradients carried across
    the passes) and the permute's backward, then the gates' backward into
    the logits.  Timed as a whole and call by call with HIP events."""
    passes = pass_list(p, info)
    idx, gate, cnt, bufs = build_passes(p, w, inp, passes)
    dy = workloads.make_dy(w, device="cuda")
    T, k, H, F, E = w.tokens, w.top_k, w.hidden, w.ffn, w.num_experts
    wg, wu, wd = inp["weights"]
    dev = "cuda"
    for b in bufs:
        run_permute(p, inp, cnt, b)
        run_gmm(p, inp, cnt, b)
        b["d_out"] = torch.empty((b["rows"], H), dtype=p.dtype, device=dev)
        b["dxs"] = torch.empty((b["rows"], H), dtype=p.dtype, device=dev)
        b["bws"] = torch.empty(g.bwd_workspace_bytes(p, b["rows"]), dtype=torch.uint8, device=dev)
    dwg = torch.empty((w.e_res, F, H), dtype=torch.float32, device=dev)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((w.e_res, H, F), dtype=torch.float32, device=dev)
    d_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    dx = torch.empty((T, H), dtype=p.dtype, device=dev)
    d_logits = torch.empty((T, E), dtype=torch.float32, device=dev)

    def comb(b):
        g.moe_combine_bwd(p, b["n"], b["c"], dy, b["out"], b["roa"], gate, b["d_out"], d_gate)

    def gmm(b, acc):
        g.moe_gmm_swiglu_bwd(p, b["xs"], b["go"], cnt["se"], wg, wu, wd, b["d_out"], b["dxs"],
                             dwg, dwu, dwd, acc, b["bws"])

    def perm(b):
        g.moe_permute_bwd(p, b["n"], b["c"], b["dxs"], b["roa"], dx)

    def route():
        g.moe_route_bwd(p, idx, gate, d_gate, d_logits)

    def step():
        for i, b in enumerate(bufs):
            comb(b)
            gmm(b, i > 0)
            perm(b)
        route()

    torch.cuda.synchronize()
    t_step = time_calls(step, reps)
    t_cb = sum(time_calls(lambda: comb(b), reps) for b in bufs)
    t_gb = sum(time_calls(lambda: gmm(b, 1), reps) for b in bufs)
    t_pb = sum(time_calls(lambda: perm(b), reps) for b in bufs)
    t_rb = time_calls(route, reps)
    n_rows = sum(int(b["go"][-1].item()) for b in bufs)
    # d_a (2NHF), gate/up recompute (4NHF), dx_sorted (4NHF), dWg+dWu (4NHF),
    # dWd (2NHF)
    flops = 16.0 * n_rows * H * F
    # algorithmic bytes of the grouped-GEMM backward calls (the timed ones
    # accumulate): per launch, its operands once and its outputs once.
    # x_sorted and d_out are read twice (recompute / d_a, then the weight
    # gradients), Wg and Wu twice (recompute, dx) and Wd once for every
    # expert with rows in the pass; d_a written and read, d_h written and
    # read twice, act written and read, dx_sorted written; the float32
    # weight gradients of the resident experts read and written.
    es = 2 if w.bf16 else 4
    se = cnt["se"].cpu().numpy()
    w_bytes = 0
    for b in bufs:
        go = b["go"].cpu().numpy()
        used = {int(se[w.res_lo * p.spd + q]) for q in range(p.g_res) if go[q + 1] > go[q]}
        w_bytes += len(used) * 5 * H * F * es
    row_bytes = n_rows * (4 * H + 2 * F + 6 * F + 2 * F + H) * es
    dw_bytes = len(bufs) * 2 * w.e_res * 3 * H * F * 4
    return dict(t_step=t_step, t_cb=t_cb, t_gb=t_gb, t_pb=t_pb, t_rb=t_rb,
                flops=flops, rows=n_rows, gemm_bytes=w_bytes + row_bytes + dw_bytes)


def run_calib_copy():
    """The calibration copy of 1 GiB, 3 times: the reference that HBM
    counters of the same run are scaled by."""
    log("[bench] calibration copy: moe_calib_copy of 1 GiB, 3 times")
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        g.calib_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst


def measured_peaks(reps=10):
    """What this machine reaches outside the layer, as context for the fractions
    of the spec peaks: the library's own calibration kernels
    (include/moe_calib.h) -- a streaming copy of 1 GiB (bytes read +
    written per second) and a matrix-core loop of bf16 MFMAs on registers --
    and, for comparison, the vendor library's dense bf16 GEMM (torch.mm,
    hipBLASLt) at 8192^3.  Timed with HIP events on the current stream."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    t_copy = time_calls(lambda: g.calib_copy(src, dst), reps)
    t_torch = time_calls(lambda: dst.copy_(src), reps)
    del src, dst
    sink = torch.empty(512, dtype=torch.float32, device="cuda")
    blocks = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    flops = g.calib_mfma(blocks, 4000, sink)
    t_mfma = time_calls(lambda: g.calib_mfma(blocks, 4000, sink), reps)
    m = 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    a = torch.randn((m, m), generator=gen, device="cuda").to(torch.bfloat16)
    b = torch.randn((m, m), generator=gen, device="cuda").to(torch.bfloat16)
    c = torch.empty((m, m), dtype=torch.bfloat16, device="cuda")
    t_mm = time_calls(lambda: torch.mm(a, b, out=c), reps)
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(2 * n / t_copy / 1e9, 1),
            "torch_copy_gbs": round(2 * n / t_torch / 1e9, 1),
            "mfma_loop_tflops": round(flops / t_mfma / 1e12, 1),
            "vendor_dense_bf16_gemm_tflops": round(2.0 * m ** 3 / t_mm / 1e12, 1),
            "method": "moe_calib_copy and torch copy_ of 1 GiB (read + written bytes); moe_calib_mfma "
                      f"({blocks} workgroups x 8 waves x 4000 rounds of 8 16x16x32 bf16 MFMAs); "
                      f"torch.mm bf16 8192^3; HIP events, mean of {reps}"}


def workloads_pass_tokens(w, n, c):
    lc = w.seq_len // n
    b = np.arange(w.tokens // w.seq_len)[:, None] * w.seq_len
    return (b + c * lc + np.arange(lc)[None, :]).ravel()


def host_info():
    """Host cores this process may run on, the CPU model, and the BLAS
    library and thread count numpy uses."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = None, None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas, threads = i.get("internal_api"), int(i.get("num_threads", 1))
                break
    except Exception:
        pass
    return dict(affinity_cores=cores, cpu_model=model, blas=blas, blas_threads=threads)


def cpu_baseline(w, inp, budget_s, n_rows):
    """The float64 oracle on the host cores, on the same inputs.  When one
    whole layer fits the budget, whole layers are timed (LAYER mode, median
    over the budget).  Otherwise the oracle's plain definition of the layer
    output (oracle.layer_plain_tokens: routing, counts and plan over all T
    tokens, then each sampled token's expert FFNs and gate-weighted sum) is
    timed on a sample of evenly spaced tokens sized from a first small run
    to fill the budget; tokens/s is the sample's tokens over its time, which
    charges the whole routing to the sample (a lower bound on the oracle's
    whole-layer rate)."""
    import oracle
    hi = host_info()
    op = oracle.Problem(**w.problem_kwargs())
    logits = inp["logits"].cpu().numpy()
    x64 = workloads.to_f64(inp["x"])
    ws = [workloads.to_f64(t) for t in inp["weights"]]
    # float64 flops of one whole oracle layer (the FFN of every resident row;
    # the host's numpy reaches ~100 GFLOP/s or more in float64)
    full_flops = 6.0 * n_rows * w.hidden * w.ffn
    cores = hi["blas_threads"] or hi["affinity_cores"]
    if full_flops < 1e11 * budget_s:
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.layer(op, oracle.MODE_LAYER, logits, x64, *ws)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s:
                break
        t = float(np.median(times))
        return dict(value=w.tokens / t, unit="tokens/s", cores=int(cores), kind="oracle",
                    sample=f"whole {w.name} layer in LAYER mode, median of {len(times)} run(s) "
                           f"({sum(times):.1f} s of CPU work), {t:.2f} s each, float64 numpy",
                    host=hi)

    def run(n):
        toks = np.linspace(0, w.tokens - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.layer_plain_tokens(op, logits, x64, *ws, toks)
        return time.perf_counter() - t0

    # fixed cost (routing over all T) and cost per sampled token from two
    # small runs, then the largest sample that fills the budget
    n0, n1 = 8, 64
    t0, t1 = run(n0), run(n1)
    per_tok = max((t1 - t0) / (n1 - n0), 1e-6)
    fixed = max(t0 - n0 * per_tok, 0.0)
    n = int(min(w.tokens, max(n1, (budget_s - t0 - t1 - fixed) / per_tok)))
    t = run(n)
    if n == w.tokens:
        return dict(value=n / t, unit="tokens/s", cores=int(cores), kind="oracle",
                    sample=f"oracle.layer_plain_tokens on all {n} tokens of the {w.name} "
                           f"workload (the plain definition of the dropless layer output, "
                           f"which the chunked fallback equals), {t:.1f} s, float64 numpy",
                    host=hi)
    return dict(value=n / t, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"oracle.layer_plain_tokens on {n} evenly spaced tokens of the "
                       f"{w.name} workload (routing, counts and plan over all {w.tokens} "
                       f"tokens included), {t:.1f} s, float64 numpy; the sample's tokens "
                       f"over its time", host=hi)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="maverick_shard", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the layer's passes")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run the calibration copy of 1 GiB (reference for HBM counters)")
    ap.add_argument("--layer-backward-only", action="store_true",
                    help="time only the whole-layer backward call (one untimed call, then "
                         "--steps timed ones) and print its mean duration; for profiling")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build runs one expert-parallel shard per "
              "GPU and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    w = workloads.CONFIGS[args.workload]
    p = g.Problem(**w.problem_kwargs())
    torch.cuda.set_device(0)
    log(f"[bench] workload {w.name}: generating inputs")
    inp = workloads.make_inputs(w, device="cuda")
    if args.layer_backward_only:
        brun = g.LayerBackwardRunner(p, g.MODE_LAYER)
        dy = workloads.make_dy(w, device="cuda")
        t = time_calls(lambda: brun(inp["x"], inp["logits"], *inp["weights"], dy), args.steps)
        if args.calib_copy:
            run_calib_copy()
        print(json.dumps({"workload": w.name, "layer_backward_calls": args.steps,
                          "layer_call_us": round(t * 1e6, 2)}), flush=True)
        return
    run = g.LayerRunner(p, g.MODE_LAYER)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run(inp["x"], inp["logits"], *inp["weights"])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) / args.steps * 1e3
    tokens_s = w.tokens / (ms / 1e3)
    # the flag and pass choice of the calls just timed (every call of the
    # same inputs takes the same)
    info = run.info.cpu().tolist()
    log(f"[bench] overflow={info[0]} fallback={info[1]}")

    # the same layer in the other modes: the capped pass alone (rows beyond
    # the buffer dropped), the chunked dropless fallback always, and the
    # single uncapped pass (worst-case buffer)
    # (a mode whose buffers this build cannot address, e.g. the single
    # uncapped pass of the EP8 receive shape, is reported as null)
    mode_ms = {}
    for name, mode in (("capped_only", g.MODE_CAPPED_ONLY), ("force_chunked", g.MODE_FORCE_CHUNKED),
                       ("force_dropless", g.MODE_FORCE_DROPLESS)):
        try:
            mrun = g.LayerRunner(p, mode)
            mode_ms[name] = time_calls(lambda: mrun(inp["x"], inp["logits"], *inp["weights"]),
                                       args.kernel_reps) * 1e3
            del mrun
        except g.MoeError as err:
            log(f"[bench] mode {name}: {err}")
            mode_ms[name] = None
    torch.cuda.empty_cache()

    log("[bench] per-kernel timing")
    kf = kernel_figures(p, w, inp, info, args.kernel_reps)
    peak_mm = PEAK_BF16_TFLOPS if w.bf16 else PEAK_FP32_TFLOPS
    # the grouped GEMM on the layer's own schedule (every pass, as the layer
    # overlaps them) is the headline figure; the serial step-API calls are
    # the per-call figure
    gemm_tflops = kf["gemm_flops"] / kf["t_gmm_sched"] / 1e12
    gemm_gbs = kf["gemm_bytes"] / kf["t_gmm_sched"] / 1e9
    gemm_tflops_serial = kf["gemm_flops"] / kf["t_gmm"] / 1e12
    ai = kf["gemm_flops"] / kf["gemm_bytes"]
    gemm_bound = "mfma" if ai * PEAK_HBM_GBS / 1e3 >= peak_mm else "hbm"
    perm_gbs = kf["perm_bytes"] / kf["t_perm"] / 1e9
    comb_gbs = kf["comb_bytes"] / kf["t_comb"] / 1e9
    if gemm_bound == "mfma":
        roof = dict(bound="mfma", achieved=round(gemm_tflops, 2), peak=peak_mm, unit="TFLOP/s",
                    frac=round(gemm_tflops / peak_mm, 4), traffic=None)
    else:
        roof = dict(bound="hbm", achieved=round(gemm_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(gemm_gbs / PEAK_HBM_GBS, 4), traffic=None)
    roof["traffic"] = recorded_gemm_traffic(w.name, g.layer_chunks_per_pass(p, g.MODE_LAYER))
    # 128-row tiles (hidden < 2048) run GEMM1 and GEMM2 as one launch
    sched = "the layer's schedule (passes in order on the caller's stream)"
    roof["kernel"] = ("grouped SwiGLU GEMM of every pass of the layer (" +
                      ("GEMM1 and GEMM2 in one launch" if w.hidden < 2048
                       else "GEMM1 and GEMM2 launches") +
                      " per pass, with the step call's tile schedule), timed as one span on " +
                      sched)

    bwd = None
    if not args.no_backward:
        log("[bench] backward timing")
        bf = backward_figures(p, w, inp, info, args.kernel_reps)
        # the whole layer's backward in one call: routing, layouts, x_sorted
        # and the expert outputs recomputed, then every pass's backward
        brun = g.LayerBackwardRunner(p, g.MODE_LAYER)
        dy = workloads.make_dy(w, device="cuda")
        t_layer_bwd = time_calls(lambda: brun(inp["x"], inp["logits"], *inp["weights"], dy),
                                 args.kernel_reps)
        del brun
        bt = bf["flops"] / bf["t_gb"] / 1e12
        bgbs = bf["gemm_bytes"] / bf["t_gb"] / 1e9
        bai = bf["flops"] / bf["gemm_bytes"]
        if bai * PEAK_HBM_GBS / 1e3 >= peak_mm:
            broof = dict(bound="mfma", achieved=round(bt, 2), peak=peak_mm, unit="TFLOP/s",
                         frac=round(bt / peak_mm, 4))
        else:
            broof = dict(bound="hbm", achieved=round(bgbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                         frac=round(bgbs / PEAK_HBM_GBS, 4))
        broof.update(traffic=None, arith_intensity=round(bai, 1),
                     kernel="grouped-GEMM backward call (d_a, gate/up recompute, dx_sorted, "
                            "weight gradients; accumulating)")
        # the layer call's grouped-GEMM work (16 N H F: d_a, the gate/up
        # recompute, dx_sorted and the weight gradients; bf16 takes the gate
        # gradients from the recompute's epilogue) over the whole call's
        # time: its weight gradients are taken once over every pass's rows,
        # not accumulated pass by pass
        lt = bf["flops"] / t_layer_bwd / 1e12
        bwd = {"layer_call_us": round(t_layer_bwd * 1e6, 2),
               "layer_call_gemm_tflops": round(lt, 2),
               "layer_call_frac_mfma_peak": round(lt / peak_mm, 4),
               "train_step_us": round((ms / 1e3 + t_layer_bwd) * 1e6, 2),
               "us_per_layer": round(bf["t_step"] * 1e6, 2),
               "tokens_s": round(w.tokens / bf["t_step"], 1),
               "gemm_us": round(bf["t_gb"] * 1e6, 2), "gemm_tflops": round(bt, 2),
               "gemm_frac_mfma_peak": round(bt / peak_mm, 4),
               "combine_bwd_us": round(bf["t_cb"] * 1e6, 2),
               "permute_bwd_us": round(bf["t_pb"] * 1e6, 2),
               "route_bwd_us": round(bf["t_rb"] * 1e6, 2), "rows": bf["rows"],
               "roofline": broof}

    if args.calib_copy:
        run_calib_copy()

    log("[bench] measured peaks (calibration copy and MFMA loop, vendor dense GEMM)")
    peaks = measured_peaks()
    roof["frac_of_measured"] = round(
        roof["achieved"] / (peaks["hbm_copy_gbs"] if roof["bound"] == "hbm"
                            else peaks["mfma_loop_tflops"] if w.bf16 else peak_mm), 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(w, inp, args.cpu_budget, kf["rows"])

    res = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden, "ffn": w.ffn,
                   "experts": w.num_experts, "top_k": w.top_k, "shards": w.num_shards,
                   "buffer_factor": w.factor, "chunks": w.num_chunks, "mode": "LAYER",
                   "fallback_ran": int(info[1]),
                   "chunks_per_pass": g.layer_chunks_per_pass(p, g.MODE_LAYER),
                   "cache": cache_note(w, p)},
        "gemm": {"tflops": round(gemm_tflops, 2), "frac_mfma_peak": round(gemm_tflops / peak_mm, 4),
                 "frac_of_mfma_loop": (round(gemm_tflops / peaks["mfma_loop_tflops"], 4)
                                       if w.bf16 else None),
                 "frac_of_vendor_gemm": (round(gemm_tflops / peaks["vendor_dense_bf16_gemm_tflops"], 4)
                                         if w.bf16 else None),
                 "gbs": round(gemm_gbs, 1), "arith_intensity": round(ai, 1),
                 "us_per_layer": round(kf["t_gmm_sched"] * 1e6, 2),
                 "schedule": "every pass's GEMM calls replayed on " + sched + ", one span",
                 "passes": kf["passes"], "rows": kf["rows"],
                 "serial_calls": {"us_per_layer": round(kf["t_gmm"] * 1e6, 2),
                                  "tflops": round(gemm_tflops_serial, 2),
                                  "frac_mfma_peak": round(gemm_tflops_serial / peak_mm, 4)}},
        "permute": {"gbs": round(perm_gbs, 1), "frac_hbm_peak": round(perm_gbs / PEAK_HBM_GBS, 4),
                    "frac_measured_copy": round(perm_gbs / peaks["hbm_copy_gbs"], 4),
                    "us_per_layer": round(kf["t_perm"] * 1e6, 2)},
        "combine": {"gbs": round(comb_gbs, 1), "frac_hbm_peak": round(comb_gbs / PEAK_HBM_GBS, 4),
                    "frac_measured_copy": round(comb_gbs / peaks["hbm_copy_gbs"], 4),
                    "us_per_layer": round(kf["t_comb"] * 1e6, 2)},
        "measured_peaks": peaks,
        "roofline": roof,
        "layer_modes": {
            "assignments_per_s": round(kf["rows"] / (ms / 1e3), 1),
            "ms_layer": round(ms, 4),
            **{f"ms_{k}": (round(v, 4) if v is not None else None) for k, v in mode_ms.items()},
            "layer_over_capped_only": (round(ms / mode_ms["capped_only"], 3)
                                       if mode_ms["capped_only"] else None),
            "note": "assignments/s: rows of the passes LAYER mode took per second of the "
                    "layer step; the other modes are timed one call at a time with HIP events"},
        "cpu_baseline": cpu,
        "backward": bwd,
    }
    if "u_rows" in kf:
        res["return_dedup"] = {
            "rows_per_assignment": kf["rows"], "rows_per_token_shard": kf["u_rows"],
            "partial_gbs": round(kf["part_bytes"] / kf["t_part"] / 1e9, 1),
            "partial_us_per_layer": round(kf["t_part"] * 1e6, 2),
            "source_sum_gbs": round(kf["src_bytes"] / kf["t_src"] / 1e9, 1),
            "source_sum_us_per_layer": round(kf["t_src"] * 1e6, 2)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
