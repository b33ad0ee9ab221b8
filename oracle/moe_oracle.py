"""Plain, slow, float64 reference of the one-shard expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

Page tags used in the citations below:
  [DRED]     "Moe dynamic redundancy"
  [FALLBACK] "Support moe_dropless_fallback=layer on the ragged all-to-all MoE path"
  [RING]     "MoE ring-of-experts: TC Pallas ring all-gather for the combine
              backward + x_sorted remat save"

Layout conventions (shared with the GPU path only by specification):
  logits  float32 [T, E]            router logits, given
  x       [T, H]                    token activations (bf16 values or fp32)
  w_gate  [E_res, F, H]             gate projection, output-major (K = H contiguous)
  w_up    [E_res, F, H]             up projection
  w_down  [E_res, H, F]             down projection (K = F contiguous)
  slots   shard d owns slots [d*(E_loc+B), (d+1)*(E_loc+B)): its E_loc home
          experts in order, then B redundant slots.

Pinned by tests/test_oracle_*.py (brute force, closed forms, invariants and
hand-worked fixtures under tests/golden/).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "MODE_LAYER", "MODE_FORCE_DROPLESS", "MODE_CAPPED_ONLY", "MODE_FORCE_CHUNKED",
    "Problem", "round_bf16", "route", "expert_counts", "plan_redundancy",
    "assign_slots", "shard_counts", "capacity", "overflow", "required_factor",
    "default_num_chunks", "pass_tokens", "pass_layout", "permute", "permute_dedup", "expert_ffn",
    "gmm_swiglu", "combine", "combine_partial", "combine_from_partials", "layer", "layer_plain",
    "layer_plain_tokens",
]

MODE_LAYER = 0           # overflow check, capped pass or chunked dropless fallback
MODE_FORCE_DROPLESS = 1  # one pass with the worst-case (uncapped) buffer
MODE_CAPPED_ONLY = 2     # one capped pass, rows beyond the cap are dropped
MODE_FORCE_CHUNKED = 3   # always the chunked dropless path


@dataclass(frozen=True)
class Problem:
    """Statement of one layer call.

    The pages state the problem as tokens, top-k, experts, expert-parallel
    shards, a ragged buffer factor (-1 = no cap) and sequence chunks
    ([FALLBACK] Why / How); redundant slots per shard come from [DRED]
    (rerouting comment: the slots are appended to the group sizes).
    """

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
    gate: str = "softmax"        # "softmax" (over the k chosen) | "sigmoid"
    bf16: bool = True
    dedup: bool = False
    slots_per_shard: int = 0     # B redundant slots per shard
    num_replicas: int = 0        # R replicas planned per call

    @property
    def e_loc(self) -> int:
        return self.num_experts // self.num_shards

    @property
    def spd(self) -> int:
        """Slots per shard: home experts plus redundant slots."""
        return self.e_loc + self.slots_per_shard

    @property
    def num_slots(self) -> int:
        return self.num_shards * self.spd

    @property
    def batch(self) -> int:
        return self.tokens // self.seq_len


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even.

    bfloat16 keeps the top 7 of float64's 52 fraction bits (same exponent
    range as float32), so the low 45 bits are rounded away: add half an ulp
    minus one, plus the lowest kept bit (ties to even), then clear them.
    Valid for zero and for magnitudes inside bfloat16's normal range, which
    is all this layer produces.
    """
    a = np.ascontiguousarray(v, dtype=np.float64)
    bits = a.view(np.uint64)
    keep_lsb = (bits >> np.uint64(45)) & np.uint64(1)
    half_m1 = np.uint64((1 << 44) - 1)
    mask = ~np.uint64((1 << 45) - 1)
    out = ((bits + half_m1 + keep_lsb) & mask).view(np.float64)
    return out.reshape(np.shape(v))


# --------------------------------------------------------------------------
# a1: router top-k and gates
# --------------------------------------------------------------------------

def route(logits: np.ndarray, k: int, gate: str):
    """Top-k experts per token and their gate weights.

    [FALLBACK] How: the overflow check is computed "from the router's
    top-k".  Selection order: logit descending, equal logits broken to the
    lowest expert index (a stable sort of the negated logits keeps index
    order among equals; -0.0 and +0.0 compare equal).

    Gates: "softmax" renormalises over the k chosen logits,
    g_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0); "sigmoid" is 1/(1+exp(-l_j)).
    """
    lg = np.asarray(logits, dtype=np.float32)
    order = np.argsort(-lg, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(lg, idx.astype(np.int64), axis=1).astype(np.float64)
    if gate == "softmax":
        z = np.exp(chosen - chosen[:, :1])
        g = z / z.sum(axis=1, keepdims=True)
    elif gate == "sigmoid":
        g = 1.0 / (1.0 + np.exp(-chosen))
    else:
        raise ValueError(gate)
    return idx, g


# --------------------------------------------------------------------------
# a2/a3: counts, redundancy plan, reroute, capacity and overflow
# --------------------------------------------------------------------------

def expert_counts(idx: np.ndarray, num_experts: int) -> np.ndarray:
    """Assignments per expert (the planner's tokens-per-expert, [DRED])."""
    return np.bincount(np.asarray(idx).ravel(), minlength=num_experts).astype(np.int64)


def plan_redundancy(counts: np.ndarray, p: Problem):
    """Greedy duplication plan ([DRED], planner comments).

    Repeats up to R times:
      1. r_max = most loaded shard (ties: lowest index);
      2. its hottest expert not yet duplicated (ties: lowest index); stop if
         none is left (the reviewer's has_candidate guard);
      3. r_min = least loaded shard that still has a free redundant slot
         (ties: lowest index); stop if no shard has one;
      4. stop unless load[r_max] > load[r_min] (can_balance);
      5. divert n_div = min(c_e, (load[r_max] - load[r_min]) // 2) of the
         expert's assignments (stop if that is 0) into r_min's first free
         slot and move the load.
    Loads are assignment counts per shard.

    Returns (slot_expert [G] int: expert hosted by each slot, -1 for an
    unused redundant slot; ndiv [E] int; replica_slot [E] int, -1 if none).
    """
    S, El, B, spd = p.num_shards, p.e_loc, p.slots_per_shard, p.spd
    E = p.num_experts
    slot_expert = np.full(S * spd, -1, dtype=np.int64)
    for d in range(S):
        for i in range(El):
            slot_expert[d * spd + i] = d * El + i
    ndiv = np.zeros(E, dtype=np.int64)
    replica_slot = np.full(E, -1, dtype=np.int64)
    if p.num_replicas <= 0 or B <= 0:
        return slot_expert, ndiv, replica_slot
    load = [int(sum(int(counts[d * El + i]) for i in range(El))) for d in range(S)]
    used = [0] * S
    duplicated = [False] * E
    for _ in range(p.num_replicas):
        r_max = 0
        for d in range(1, S):
            if load[d] > load[r_max]:
                r_max = d
        cand = -1
        for e in range(r_max * El, (r_max + 1) * El):
            if duplicated[e]:
                continue
            if cand < 0 or counts[e] > counts[cand]:
                cand = e
        if cand < 0:
            break
        r_min = -1
        for d in range(S):
            if used[d] >= B:
                continue
            if r_min < 0 or load[d] < load[r_min]:
                r_min = d
        if r_min < 0:
            break
        if load[r_max] <= load[r_min]:
            break
        n = min(int(counts[cand]), (load[r_max] - load[r_min]) // 2)
        if n <= 0:
            break
        s = r_min * spd + El + used[r_min]
        used[r_min] += 1
        slot_expert[s] = cand
        replica_slot[cand] = s
        ndiv[cand] = n
        duplicated[cand] = True
        load[r_max] -= n
        load[r_min] += n
    return slot_expert, ndiv, replica_slot


def assign_slots(idx: np.ndarray, p: Problem, ndiv: np.ndarray, replica_slot: np.ndarray):
    """Slot of every assignment ([DRED], rerouting comment).

    Home slot of expert e: (e // E_loc) * (E_loc + B) + e % E_loc.  For a
    duplicated expert the first ndiv[e] of its assignments in flat (t, j)
    order go to its replica slot; the rest stay home.
    """
    flat = np.asarray(idx, dtype=np.int64).ravel()
    El, spd = p.e_loc, p.spd
    slot = (flat // El) * spd + flat % El
    for e in np.nonzero(ndiv > 0)[0]:
        where = np.nonzero(flat == e)[0]
        slot[where[: int(ndiv[e])]] = replica_slot[e]
    return slot.reshape(np.shape(idx))


def shard_counts(slot: np.ndarray, p: Problem) -> np.ndarray:
    """Rows each destination shard would receive.

    Without dedup one row per assignment; with dedup one row per distinct
    (token, shard) pair, since a token is sent once per destination shard
    and expanded by the receiver ([DRED], summary and dedup comment).
    """
    shard = np.asarray(slot, dtype=np.int64) // p.spd
    S = p.num_shards
    if not p.dedup:
        return np.bincount(shard.ravel(), minlength=S).astype(np.int64)
    out = np.zeros(S, dtype=np.int64)
    for t in range(shard.shape[0]):
        for d in set(int(v) for v in shard[t]):
            out[d] += 1
    return out


def capacity(p: Problem):
    """Receive-buffer cap per shard: ceil(factor * balanced), balanced = T*k/S.

    [FALLBACK] Why: with a positive factor each shard's receive buffer holds
    factor x balanced rows; -1 (any factor <= 0 here) means no cap, which is
    returned as None.  The factor is the float32 value the caller passed.
    """
    f = float(np.float32(p.factor))
    if f <= 0.0:
        return None
    return int(math.ceil(f * float(p.tokens * p.top_k) / float(p.num_shards)))


def overflow(counts_per_shard: np.ndarray, cap) -> bool:
    """True when some shard would receive more rows than its buffer holds
    ([FALLBACK] How, the ragged overflow check; strictly more)."""
    if cap is None:
        return False
    return bool(np.any(np.asarray(counts_per_shard) > cap))


def required_factor(counts_per_shard: np.ndarray, p: Problem) -> float:
    """Smallest factor that would have fit: max shard rows / balanced
    ([FALLBACK] Shortcomings names this figure)."""
    balanced = p.tokens * p.top_k / p.num_shards
    return float(np.max(counts_per_shard)) / balanced


# --------------------------------------------------------------------------
# a4/a5: pass layout (stable expert-sorted order, dedup) and permute
# --------------------------------------------------------------------------

def default_num_chunks(num_shards: int, factor: float) -> int:
    """Chunk count when none is given: ceil(S / factor), the reading of
    [FALLBACK] Shortcomings (its example: 16 shards at factor 2, an
    eight-fold slowdown, i.e. eight chunks)."""
    return int(math.ceil(num_shards / float(np.float32(factor))))


def pass_tokens(p: Problem, num_chunks: int, chunk: int) -> np.ndarray:
    """Tokens of sequence chunk `chunk` of `num_chunks` ([FALLBACK] How: the
    fallback runs the layer over sequence chunks).  Token t = b*L + s; the
    chunk holds s in [c*L/n, (c+1)*L/n) for every sequence b, in ascending t."""
    L, n = p.seq_len, num_chunks
    lc = L // n
    out = []
    for b in range(p.batch):
        for s in range(chunk * lc, (chunk + 1) * lc):
            out.append(b * L + s)
    return np.asarray(out, dtype=np.int64)


def pass_layout(p: Problem, slot: np.ndarray, tokens: np.ndarray, cap):
    """Row layout of one pass over `tokens` (a chunk, or all tokens).

    Rows are the assignments (t, j) of the pass whose slot belongs to a
    resident shard, sorted by (slot, t, j): the expert-sorted order of the
    routed input ([RING] What calls it x_sorted; [DRED] rerouting comment:
    group sizes per local expert followed by the redundant slots).

    cap is None for the worst-case (dropless) buffer.  Otherwise each
    resident shard's receive buffer keeps only its first `cap` rows and the
    rest are dropped ([FALLBACK] Why: rows beyond the cap are silently
    dropped): without dedup the buffer rows are the shard's assignments in
    slot-sorted order; with dedup they are the shard's distinct tokens in
    ascending t, and an assignment drops with its token.

    Returns a dict with
      group_sizes [G_res], group_offsets [G_res+1], sorted_assign [N]
      (flat id t*k+j per row), row_of_assign [T*k] (-1 when the assignment
      is not a row of this pass), and with dedup dedup_offsets [S_res+1],
      dedup_token [U], expand_idx [N].
    """
    k, spd = p.top_k, p.spd
    lo, hi = p.res_lo * spd, p.res_hi * spd
    g_res = hi - lo
    slot = np.asarray(slot, dtype=np.int64)
    cand = []
    for t in tokens:
        for j in range(k):
            s = int(slot[t, j])
            if lo <= s < hi:
                cand.append((s, int(t), j))
    cand.sort()

    kept_tokens = {}
    if p.dedup:
        for d in range(p.res_lo, p.res_hi):
            toks = sorted({t for (s, t, j) in cand if s // spd == d})
            if cap is not None:
                toks = toks[:cap]
            kept_tokens[d] = toks
        kept_sets = {d: set(v) for d, v in kept_tokens.items()}
        rows = [(s, t, j) for (s, t, j) in cand if t in kept_sets[s // spd]]
    else:
        rows = []
        pos_in_bucket = {}
        for (s, t, j) in cand:
            d = s // spd
            q = pos_in_bucket.get(d, 0)
            pos_in_bucket[d] = q + 1
            if cap is not None and q >= cap:
                continue
            rows.append((s, t, j))

    n = len(rows)
    sizes = np.zeros(g_res, dtype=np.int64)
    for (s, t, j) in rows:
        sizes[s - lo] += 1
    offsets = np.zeros(g_res + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    sorted_assign = np.asarray([t * k + j for (s, t, j) in rows], dtype=np.int64)
    row_of_assign = np.full(p.tokens * k, -1, dtype=np.int64)
    row_of_assign[sorted_assign] = np.arange(n)
    out = dict(group_sizes=sizes, group_offsets=offsets, sorted_assign=sorted_assign,
               row_of_assign=row_of_assign, num_rows=n)
    if p.dedup:
        s_res = p.res_hi - p.res_lo
        d_off = np.zeros(s_res + 1, dtype=np.int64)
        d_tok = []
        rank = {}
        for i, d in enumerate(range(p.res_lo, p.res_hi)):
            for r, t in enumerate(kept_tokens[d]):
                rank[(d, t)] = int(d_off[i]) + r
                d_tok.append(t)
            d_off[i + 1] = d_off[i] + len(kept_tokens[d])
        expand = np.asarray([rank[(s // spd, t)] for (s, t, j) in rows], dtype=np.int64)
        out.update(dedup_offsets=d_off, dedup_token=np.asarray(d_tok, dtype=np.int64),
                   expand_idx=expand)
    return out


def permute(x: np.ndarray, sorted_assign: np.ndarray, k: int) -> np.ndarray:
    """x_sorted[n] = x[t_n] with t_n = sorted_assign[n] // k ([RING] What:
    the routed, expert-sorted MoE input)."""
    return np.asarray(x)[np.asarray(sorted_assign, dtype=np.int64) // k]


def permute_dedup(x: np.ndarray, dedup_token: np.ndarray, expand_idx: np.ndarray):
    """Dedup path: x_dedup[u] = x[dedup_token[u]] (one row per token and
    destination shard), then x_sorted[n] = x_dedup[expand_idx[n]] ([DRED]:
    the receiver re-expands with expand_indices)."""
    x_dedup = np.asarray(x)[np.asarray(dedup_token, dtype=np.int64)]
    return x_dedup, x_dedup[np.asarray(expand_idx, dtype=np.int64)]


# --------------------------------------------------------------------------
# a6: grouped SwiGLU FFN
# --------------------------------------------------------------------------

def expert_ffn(rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, bf16: bool):
    """SwiGLU expert FFN on a block of rows (float64).

    a = SiLU(x Wg^T) * (x Wu^T), SiLU(z) = z / (1 + exp(-z)); o = a Wd^T.
    With bf16 storage, a and o are rounded to bfloat16 where the GPU path
    stores them.
    """
    xr = np.asarray(rows, dtype=np.float64)
    hg = xr @ np.asarray(wg, dtype=np.float64).T
    hu = xr @ np.asarray(wu, dtype=np.float64).T
    with np.errstate(over="ignore"):
        a = hg / (1.0 + np.exp(-hg)) * hu
    if bf16:
        a = round_bf16(a)
    o = a @ np.asarray(wd, dtype=np.float64).T
    if bf16:
        o = round_bf16(o)
    return a, o


def gmm_swiglu(p: Problem, x_sorted, group_offsets, group_expert, w_gate, w_up, w_down):
    """Grouped GEMM over ragged groups ([DRED], rerouting comment: a grouped
    matmul over the local experts' group sizes): group g's rows use the
    weights of resident expert group_expert[g] (a replica slot uses its home
    expert's weights).  Returns (act [N,F], out [N,H])."""
    n = int(group_offsets[-1])
    act = np.zeros((n, p.ffn), dtype=np.float64)
    out = np.zeros((n, p.hidden), dtype=np.float64)
    for g in range(len(group_offsets) - 1):
        a0, a1 = int(group_offsets[g]), int(group_offsets[g + 1])
        if a1 == a0:
            continue
        e = int(group_expert[g])
        act[a0:a1], out[a0:a1] = expert_ffn(x_sorted[a0:a1], w_gate[e], w_up[e], w_down[e], p.bf16)
    return act, out


# --------------------------------------------------------------------------
# a7: combine
# --------------------------------------------------------------------------

def combine(p: Problem, expert_out, row_of_assign, gates, tokens):
    """y_t = sum over j ascending of g_tj * out[row(t, j)] for the rows of
    this pass, float64; a token with no row gets 0.  With bf16 storage y is
    rounded to bfloat16.  Returns y rows for `tokens` in the given order."""
    k = p.top_k
    y = np.zeros((len(tokens), p.hidden), dtype=np.float64)
    for i, t in enumerate(tokens):
        acc = np.zeros(p.hidden, dtype=np.float64)
        for j in range(k):
            r = int(row_of_assign[t * k + j])
            if r >= 0:
                acc = acc + gates[t, j] * expert_out[r]
        y[i] = acc
    if p.bf16:
        y = round_bf16(y)
    return y


# --------------------------------------------------------------------------
# Return-path dedup: partial combine at the receiving shard, sum at the source
# --------------------------------------------------------------------------
#
# The pages deduplicate the dispatch: a token goes once to each destination
# shard and is re-expanded there ([DRED] code review: dedup and
# expand_indices).  The return path applied the same way: the receiving
# shard sums its own assignments of a token, gate-weighted, into one row per
# (token, shard), and the token's source adds those rows.  The partial rows
# are not rounded to the activation dtype (float32 on the GPU): the sum is
# the combine regrouped by shard, rounded once at the source.


def combine_partial(p: Problem, expert_out, row_of_assign, gates, slot, dedup_offsets,
                    dedup_token):
    """partial[u] for every dedup row u of a pass (token t on resident shard
    d): the sum over j ascending, over the token's assignments whose slot
    lies on shard d and that have a row in this pass, of g_tj * out[row(t, j)],
    float64 and not rounded (whatever the storage of the activations)."""
    k, spd = p.top_k, p.spd
    slot = np.asarray(slot, dtype=np.int64)
    u_total = int(dedup_offsets[-1])
    partial = np.zeros((u_total, p.hidden), dtype=np.float64)
    for i, d in enumerate(range(p.res_lo, p.res_hi)):
        for u in range(int(dedup_offsets[i]), int(dedup_offsets[i + 1])):
            t = int(dedup_token[u])
            acc = np.zeros(p.hidden, dtype=np.float64)
            for j in range(k):
                r = int(row_of_assign[t * k + j])
                if r >= 0 and int(slot[t, j]) // spd == d:
                    acc = acc + gates[t, j] * expert_out[r]
            partial[u] = acc
    return partial


def combine_from_partials(p: Problem, partial, slot, dedup_offsets, dedup_token, tokens):
    """Source side of the return-path dedup: y_t = the sum of the token's
    partial rows, one per resident shard that kept the token, taken in the
    order of the token's first assignment on each shard; 0 for a token with
    none.  Rounded to bfloat16 with bf16 storage.  Returns y rows for
    `tokens` in the given order."""
    k, spd = p.top_k, p.spd
    slot = np.asarray(slot, dtype=np.int64)
    row_of = {}
    for i, d in enumerate(range(p.res_lo, p.res_hi)):
        for u in range(int(dedup_offsets[i]), int(dedup_offsets[i + 1])):
            row_of[(d, int(dedup_token[u]))] = u
    y = np.zeros((len(tokens), p.hidden), dtype=np.float64)
    for n, t in enumerate(tokens):
        t = int(t)
        seen = set()
        acc = np.zeros(p.hidden, dtype=np.float64)
        for j in range(k):
            d = int(slot[t, j]) // spd
            if d in seen or (d, t) not in row_of:
                continue
            seen.add(d)
            acc = acc + partial[row_of[(d, t)]]
        y[n] = acc
    if p.bf16:
        y = round_bf16(y)
    return y


# --------------------------------------------------------------------------
# a8: the layer with the capped pass or the chunked dropless fallback
# --------------------------------------------------------------------------

def _resident_expert(p: Problem, slot_expert, g_local):
    e = int(slot_expert[p.res_lo * p.spd + g_local])
    return -1 if e < 0 else e - p.res_lo * p.e_loc


def layer(p: Problem, mode: int, logits, x, w_gate, w_up, w_down):
    """The layer, step by step ([FALLBACK] How).

    Route, count, plan and reroute once per call; compute the cap and the
    overflow flag.  LAYER: without overflow one capped pass (nothing drops,
    every shard fits), with overflow one dropless pass per sequence chunk.
    FORCE_DROPLESS: one uncapped pass.  FORCE_CHUNKED: always the chunks.
    CAPPED_ONLY: one capped pass that drops rows beyond the cap.
    Returns every integer artefact plus y [T,H] (float64).
    """
    idx, gates = route(logits, p.top_k, p.gate)
    counts = expert_counts(idx, p.num_experts)
    slot_expert, ndiv, replica_slot = plan_redundancy(counts, p)
    slot = assign_slots(idx, p, ndiv, replica_slot)
    sc = shard_counts(slot, p)
    cap = capacity(p)
    ovf = overflow(sc, cap)
    if mode == MODE_LAYER:
        chunked = ovf
        pass_cap = cap
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
    y = np.zeros((p.tokens, p.hidden), dtype=np.float64)
    g_res = (p.res_hi - p.res_lo) * p.spd
    group_expert = np.asarray([_resident_expert(p, slot_expert, g) for g in range(g_res)])
    passes = []
    for c in range(n):
        toks = pass_tokens(p, n, c)
        lay = pass_layout(p, slot, toks, None if chunked else pass_cap)
        if p.dedup:
            _, x_sorted = permute_dedup(xs, lay["dedup_token"], lay["expand_idx"])
        else:
            x_sorted = permute(xs, lay["sorted_assign"], p.top_k)
        _, out = gmm_swiglu(p, x_sorted, lay["group_offsets"], group_expert, w_gate, w_up, w_down)
        y[toks] = combine(p, out, lay["row_of_assign"], gates, toks)
        passes.append(lay)
    return dict(topk_idx=idx, topk_gate=gates, expert_counts=counts, slot_expert=slot_expert,
                ndiv=ndiv, replica_slot=replica_slot, slot_of_assign=slot, shard_counts=sc,
                cap=cap, overflow=ovf, fallback_ran=chunked,
                required_factor=required_factor(sc, p), group_expert=group_expert,
                passes=passes, y=y)


def layer_plain_tokens(p: Problem, logits, x, w_gate, w_up, w_down, tokens):
    """The plain definition of the (dropless) layer output for a list of
    tokens: y_t = sum over j ascending of g_tj * FFN_slot(t,j)(x_t) over the
    assignments on resident shards.  Dedup, rerouting and chunking do not
    change it ([FALLBACK] Tests: the fallback matches the dropless model;
    [DRED]: a replica computes its home expert's function).  Used at full
    sizes on a sample of tokens; each expert's weights are read once
    (w_gate[e] etc. may be lazy accessors)."""
    idx, gates = route(logits, p.top_k, p.gate)
    counts = expert_counts(idx, p.num_experts)
    slot_expert, ndiv, replica_slot = plan_redundancy(counts, p)
    slot = assign_slots(idx, p, ndiv, replica_slot)
    k, spd = p.top_k, p.spd
    tokens = [int(t) for t in tokens]
    by_expert = {}
    for t in tokens:
        for j in range(k):
            s = int(slot[t, j])
            if p.res_lo <= s // spd < p.res_hi:
                e = int(slot_expert[s]) - p.res_lo * p.e_loc
                by_expert.setdefault(e, []).append((t, j))
    o = {}
    for e in sorted(by_expert):
        pairs = by_expert[e]
        rows = np.stack([np.asarray(x[t], dtype=np.float64) for (t, _) in pairs])
        _, out = expert_ffn(rows, w_gate[e], w_up[e], w_down[e], p.bf16)
        for r, tj in enumerate(pairs):
            o[tj] = out[r]
    y = np.zeros((len(tokens), p.hidden), dtype=np.float64)
    for i, t in enumerate(tokens):
        acc = np.zeros(p.hidden, dtype=np.float64)
        for j in range(k):
            if (t, j) in o:
                acc = acc + gates[t, j] * o[(t, j)]
        y[i] = acc
    if p.bf16:
        y = round_bf16(y)
    return y


def layer_plain(p: Problem, logits, x, w_gate, w_up, w_down):
    """layer_plain_tokens over every token."""
    return layer_plain_tokens(p, logits, x, w_gate, w_up, w_down, np.arange(p.tokens))
