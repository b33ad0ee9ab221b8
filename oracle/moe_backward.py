"""Plain float64 reference of the backward of the one-shard MoE layer.

TEST INFRASTRUCTURE ONLY: nothing on the product path may import this
module (the package docstring states the rule).

The pages describe the backward only in outline: [FALLBACK] How runs the
chunked passes in a scan, and the scan's backward redoes each chunk's
forward and keeps the weight gradients as a running sum across chunks; [RING] (title and What)
saves the expert-sorted input x_sorted for the backward and computes the
combine's backward.  The derivatives themselves are those of the forward
functions of moe_oracle, written out here by the chain rule:

  combine      y_t = sum_j g_tj o_r(t,j)
                 -> d_o[r(t,j)] = g_tj dy_t,   d_g[t,j] = <dy_t, o_r(t,j)>
  FFN          h_g = x Wg^T, h_u = x Wu^T, a = SiLU(h_g) h_u, o = a Wd^T
                 -> d_a = d_o Wd,  d_hu = d_a SiLU(h_g),
                    d_hg = d_a h_u SiLU'(h_g),  SiLU'(z) = s(z) (1 + z (1 - s(z))),
                    d_x = d_hg Wg + d_hu Wu,
                    dWg = d_hg^T x, dWu = d_hu^T x, dWd = d_o^T a
  permute      x_sorted[n] = x[t_n]          -> dx_t = sum over the rows of t
  gates        softmax over the k chosen:   d_l_j = g_j (d_g_j - sum_i g_i d_g_i)
               sigmoid:                     d_l_j = d_g_j g_j (1 - g_j)
  (logits that are not chosen get 0: the top-k selection is piecewise
  constant.)

bf16 storage: where the GPU path stores a bfloat16 intermediate (d_o, d_a,
d_hg, d_hu, the recomputed activation a, dx_sorted, dx) the float64 value
is rounded to the nearest bfloat16 at that point, as the forward oracle
does; weight gradients and gate/logit gradients are not rounded (the GPU
keeps them in float32).  The recomputed activation is the forward's own
(same rounding).

Pinned by tests/test_oracle_backward.py: central differences of the
forward oracle in float64, the adjoint identity of the permute, and
closed forms of the gate derivatives.
"""

from __future__ import annotations

import numpy as np

from .moe_oracle import (MODE_CAPPED_ONLY, MODE_FORCE_CHUNKED, MODE_FORCE_DROPLESS, MODE_LAYER,
                         Problem, _resident_expert, assign_slots, capacity, expert_counts,
                         gmm_swiglu, overflow, pass_layout, pass_tokens, permute,
                         plan_redundancy, round_bf16, route, shard_counts)

__all__ = ["combine_bwd", "expert_ffn_bwd", "gmm_swiglu_bwd", "permute_bwd", "route_bwd",
           "layer_bwd"]


def _r(p_bf16: bool, v):
    return round_bf16(v) if p_bf16 else v


def combine_bwd(p: Problem, dy, expert_out, row_of_assign, gates, tokens, num_rows):
    """Backward of the gate-weighted combine for the tokens of one pass.

    d_out[r] = g_tj * dy[t] for the row r = row(t, j) of every assignment
    with a row; d_gate[t, j] = <dy[t], expert_out[r]> (0 for an assignment
    with no row in the pass, and for tokens outside the pass).  d_out is
    rounded to bfloat16 with bf16 storage.  Returns (d_out [num_rows, H],
    d_gate [T, k])."""
    k = p.top_k
    dy = np.asarray(dy, dtype=np.float64)
    d_out = np.zeros((num_rows, p.hidden), dtype=np.float64)
    d_gate = np.zeros((p.tokens, k), dtype=np.float64)
    for t in tokens:
        t = int(t)
        for j in range(k):
            r = int(row_of_assign[t * k + j])
            if r < 0:
                continue
            d_out[r] = gates[t, j] * dy[t]
            d_gate[t, j] = float(np.dot(dy[t], np.asarray(expert_out[r], dtype=np.float64)))
    return _r(p.bf16, d_out), d_gate


def expert_ffn_bwd(rows, wg, wu, wd, d_o, bf16: bool):
    """Backward of the SwiGLU expert FFN on a block of rows (float64).

    Recomputes h_g = x Wg^T, h_u = x Wu^T and a = SiLU(h_g) h_u (rounded
    like the forward's stored activation), then the chain rule of the
    module docstring.  Returns (d_x [n, H], dWg [F, H], dWu [F, H],
    dWd [H, F]); d_x is rounded with bf16 storage, the weight gradients
    are not."""
    x = np.asarray(rows, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    wu = np.asarray(wu, dtype=np.float64)
    wd = np.asarray(wd, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    hg = x @ wg.T
    hu = x @ wu.T
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-hg))
    silu = hg * s
    a = _r(bf16, silu * hu)
    d_a = _r(bf16, d_o @ wd)
    d_hu = _r(bf16, d_a * silu)
    d_hg = _r(bf16, d_a * hu * s * (1.0 + hg * (1.0 - s)))
    d_x = _r(bf16, d_hg @ wg + d_hu @ wu)
    return d_x, d_hg.T @ x, d_hu.T @ x, d_o.T @ a


def gmm_swiglu_bwd(p: Problem, x_sorted, group_offsets, group_expert, w_gate, w_up, w_down,
                   d_out):
    """Backward of the grouped SwiGLU GEMM of one pass.

    Group g's rows ran resident expert group_expert[g]; their input
    gradients are that expert's FFN backward, and every group of an expert
    (a replica slot's group included) adds into the expert's weight
    gradients.  Returns (dx_sorted [N, H], dw_gate [E_res, F, H], dw_up
    [E_res, F, H], dw_down [E_res, H, F])."""
    n = int(group_offsets[-1])
    e_res = np.asarray(w_gate).shape[0]
    dx = np.zeros((n, p.hidden), dtype=np.float64)
    dwg = np.zeros((e_res, p.ffn, p.hidden), dtype=np.float64)
    dwu = np.zeros_like(dwg)
    dwd = np.zeros((e_res, p.hidden, p.ffn), dtype=np.float64)
    for g in range(len(group_offsets) - 1):
        a0, a1 = int(group_offsets[g]), int(group_offsets[g + 1])
        if a1 == a0:
            continue
        e = int(group_expert[g])
        gx, gg, gu, gd = expert_ffn_bwd(x_sorted[a0:a1], w_gate[e], w_up[e], w_down[e],
                                        d_out[a0:a1], p.bf16)
        dx[a0:a1] = gx
        dwg[e] += gg
        dwu[e] += gu
        dwd[e] += gd
    return dx, dwg, dwu, dwd


def permute_bwd(p: Problem, dx_sorted, row_of_assign, tokens):
    """Backward of the permute: dx[t] = sum over j ascending of
    dx_sorted[row(t, j)] over the token's rows in the pass (0 with none),
    rounded with bf16 storage.  Returns dx rows for `tokens` in order."""
    k = p.top_k
    dx = np.zeros((len(tokens), p.hidden), dtype=np.float64)
    for i, t in enumerate(tokens):
        acc = np.zeros(p.hidden, dtype=np.float64)
        for j in range(k):
            r = int(row_of_assign[int(t) * k + j])
            if r >= 0:
                acc = acc + np.asarray(dx_sorted[r], dtype=np.float64)
        dx[i] = acc
    return _r(p.bf16, dx)


def route_bwd(p: Problem, idx, gates, d_gate):
    """Logit gradients of the gates.  The chosen set is piecewise constant
    in the logits, so only the k chosen logits of a token get a gradient:
    softmax over the chosen, d_l_j = g_j (d_g_j - sum_i g_i d_g_i); sigmoid,
    d_l_j = d_g_j g_j (1 - g_j).  Returns d_logits [T, E] float64."""
    idx = np.asarray(idx, dtype=np.int64)
    g = np.asarray(gates, dtype=np.float64)
    dg = np.asarray(d_gate, dtype=np.float64)
    if p.gate == "softmax":
        dl = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    elif p.gate == "sigmoid":
        dl = dg * g * (1.0 - g)
    else:
        raise ValueError(p.gate)
    out = np.zeros((p.tokens, p.num_experts), dtype=np.float64)
    for t in range(p.tokens):
        for j in range(p.top_k):
            out[t, idx[t, j]] += dl[t, j]
    return out


def layer_bwd(p: Problem, mode: int, logits, x, w_gate, w_up, w_down, dy):
    """Backward of the layer ([FALLBACK] How: the same passes as the
    forward, each recomputed from x; the weight gradients are carried
    across the passes and summed).

    Routing, plan, cap and the pass choice are those of the forward (they
    do not depend on dy).  Per pass: combine backward, x_sorted from x, the
    grouped GEMM backward, the permute backward into dx for the pass's
    tokens.  Then the gate gradients of all passes go to the logits.
    Returns dict(dx [T,H], d_logits [T,E], d_gate [T,k], dw_gate, dw_up,
    dw_down)."""
    idx, gates = route(logits, p.top_k, p.gate)
    counts = expert_counts(idx, p.num_experts)
    slot_expert, ndiv, replica_slot = plan_redundancy(counts, p)
    slot = assign_slots(idx, p, ndiv, replica_slot)
    cap = capacity(p)
    ovf = overflow(shard_counts(slot, p), cap)
    if mode == MODE_LAYER:
        chunked, pass_cap = ovf, cap
    elif mode == MODE_FORCE_DROPLESS:
        chunked, pass_cap = False, None
    elif mode == MODE_CAPPED_ONLY:
        chunked, pass_cap = False, cap
    elif mode == MODE_FORCE_CHUNKED:
        chunked, pass_cap = True, None
    else:
        raise ValueError(mode)
    n = p.num_chunks if chunked else 1
    xs = np.asarray(x, dtype=np.float64)
    g_res = (p.res_hi - p.res_lo) * p.spd
    group_expert = np.asarray([_resident_expert(p, slot_expert, g) for g in range(g_res)])
    e_res = np.asarray(w_gate).shape[0]
    dx = np.zeros((p.tokens, p.hidden), dtype=np.float64)
    d_gate = np.zeros((p.tokens, p.top_k), dtype=np.float64)
    dwg = np.zeros((e_res, p.ffn, p.hidden), dtype=np.float64)
    dwu = np.zeros_like(dwg)
    dwd = np.zeros((e_res, p.hidden, p.ffn), dtype=np.float64)
    for c in range(n):
        toks = pass_tokens(p, n, c)
        lay = pass_layout(p, slot, toks, None if chunked else pass_cap)
        x_sorted = permute(xs, lay["sorted_assign"], p.top_k)
        # the forward's expert outputs, for the gate gradients
        _, out = gmm_swiglu(p, x_sorted, lay["group_offsets"], group_expert, w_gate, w_up,
                            w_down)
        d_out, dg = combine_bwd(p, dy, out, lay["row_of_assign"], gates, toks, lay["num_rows"])
        d_gate[toks] = dg[toks]
        dxs, gg, gu, gd = gmm_swiglu_bwd(p, x_sorted, lay["group_offsets"], group_expert,
                                         w_gate, w_up, w_down, d_out)
        dwg += gg
        dwu += gu
        dwd += gd
        dx[toks] = permute_bwd(p, dxs, lay["row_of_assign"], toks)
    d_logits = route_bwd(p, idx, gates, d_gate)
    return dict(dx=dx, d_logits=d_logits, d_gate=d_gate, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                fallback_ran=chunked)
