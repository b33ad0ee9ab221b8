/*
 * moe_shard.h -- C ABI of the one-shard expert-parallel MoE layer on MI355X.
 *
 * The layer follows three maxtext pull-request pages, cited by title and
 * section:
 *   [DRED]     "Moe dynamic redundancy" (automated code review comments on
 *              rerouting, dedup truncation and the duplication planner);
 *   [FALLBACK] "Support moe_dropless_fallback=layer on the ragged all-to-all
 *              MoE path" (sections Why, How, Shortcomings, Tests);
 *   [RING]     "MoE ring-of-experts: TC Pallas ring all-gather for the
 *              combine backward + x_sorted remat save" (section What).
 *
 * One GPU stands for one expert-parallel shard.  The all-to-all of the
 * pages becomes local bucketing by virtual destination shard: counts and the
 * overflow check cover every shard, while permute, grouped GEMM and combine
 * run only for the resident shards [res_shard_lo, res_shard_hi).
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers unless stated otherwise; the
 *    problem struct and size outputs are host pointers.
 *  - The caller owns every buffer.  The library allocates no device memory
 *    and is reentrant across streams; the only state it keeps is one side
 *    stream and two events per device, created on first use.  Scratch
 *    comes from the caller's workspace `ws` of `ws_bytes` bytes (256-byte
 *    aligned), sized by moe_workspace_bytes / moe_layer_workspace_bytes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work: nothing synchronises the host, so integer outputs are
 *    valid once the stream reaches them.  moe_gmm_swiglu_bwd and moe_layer_bwd
 *    put part of their work (dx_sorted) on the side stream, forked from
 *    `stream` and joined back to it by events inside the call, so everything
 *    is complete when `stream` reaches the point after the call.  Concurrent
 *    calls on one device serialise only that enqueue (a mutex), not their
 *    GPU work.
 *  - Errors: a negative moe_status, returned after validating every argument
 *    on the host and before any launch.  A failed launch returns MOE_EHIP.
 *    The library never truncates silently: too small a buffer is
 *    MOE_ECAPACITY ([DRED], dedup truncation comment).
 *  - Index arrays produced by moe_route are trusted by later calls; indices
 *    outside [0, E) are skipped by the kernels (no out-of-bounds access) and
 *    raise MOE_ERR_BAD_INDEX.
 *  - Errors only the device can see (the data decides them) are reported as
 *    the MOE_ERR_* bits below in a device word the call writes: status[3] of
 *    moe_count_overflow, info[4] of moe_layer_dropless_chunked, *status of
 *    moe_gmm_swiglu.  Nothing is ever dropped without a bit saying so
 *    ([DRED], dedup truncation comment: silent loss is the failure to avoid).
 *  - Layouts are row-major.  dtype MOE_BF16: x, weights, act, expert_out and
 *    y are bfloat16 (fp32 accumulation; act, expert_out and y rounded to
 *    nearest even); MOE_F32: all float32.  Logits and gates are float32.
 *  - Weights are output-major with the reduction dimension contiguous:
 *      w_gate, w_up [E_res, F, H],  w_down [E_res, H, F]
 *    for the E_res = (res_shard_hi - res_shard_lo) * E/S resident experts,
 *    resident expert i being global expert res_shard_lo*E/S + i.
 *  - Slots: shard d owns slots [d*(E/S+B), (d+1)*(E/S+B)): its E/S home
 *    experts in order, then B redundant slots ([DRED], rerouting comment:
 *    the redundant slots are appended to the group sizes).  G = S*(E/S+B)
 *    slots in all, G_res = (res_shard_hi-res_shard_lo)*(E/S+B) resident.
 */
#ifndef MOE_SHARD_H
#define MOE_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,      /* a size, enum or pointer argument is invalid        */
  MOE_EUNSUPPORTED = -2,/* valid problem this build does not run (see text)  */
  MOE_ECAPACITY = -3,   /* a caller buffer or the workspace is too small      */
  MOE_EHIP = -4         /* a HIP launch or copy failed                         */
} moe_status;

/* Device-side error bits (OR-ed together). */
enum {
  MOE_ERR_BAD_INDEX = 1,   /* a top-k expert index outside [0, E) was skipped       */
  MOE_ERR_BAD_OFFSETS = 2, /* group offsets not non-decreasing within [0, max_rows]:
                              the grouped GEMM computed nothing                      */
  MOE_ERR_GEMM_WAIT = 4    /* a grouped-GEMM tile gave up its bounded wait for its
                              input rows (another tile of the same launch never
                              finished them): its rows of expert_out were not
                              written                                                */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gate of the chosen experts.  SOFTMAX: softmax over the k chosen logits
 * (renormalised top-k); SIGMOID: 1/(1+exp(-logit)), not normalised. */
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate;

/* How moe_layer_dropless_chunked handles the ragged buffer ([FALLBACK] How):
 *  LAYER          overflow check; no overflow -> one capped pass, overflow ->
 *                 one dropless pass per sequence chunk (decided on the device,
 *                 the host never waits);
 *  FORCE_DROPLESS one pass with the worst-case buffer (force_dropless);
 *  CAPPED_ONLY    one capped pass that drops rows beyond the cap (the capped
 *                 model the page's tests show diverging);
 *  FORCE_CHUNKED  always the chunked dropless passes. */
typedef enum {
  MOE_MODE_LAYER = 0,
  MOE_MODE_FORCE_DROPLESS = 1,
  MOE_MODE_CAPPED_ONLY = 2,
  MOE_MODE_FORCE_CHUNKED = 3
} moe_mode;

/* Statement of one layer call ([FALLBACK] Why/How: tokens, top-k, experts,
 * EP shards, ragged buffer factor with -1 for no cap, sequence chunks;
 * [DRED]: redundant slots per shard). */
typedef struct {
  int32_t tokens;          /* T = batch * seq_len                              */
  int32_t seq_len;         /* L; chunks split every sequence, L % chunks == 0  */
  int32_t hidden;          /* H                                                */
  int32_t ffn;             /* F (SwiGLU inner size)                            */
  int32_t num_experts;     /* E, global experts                                */
  int32_t top_k;           /* k, 1 <= k <= min(E, 32)                          */
  int32_t num_shards;      /* S virtual destination shards, E % S == 0         */
  int32_t res_shard_lo;    /* resident shards [lo, hi), 0 <= lo < hi <= S      */
  int32_t res_shard_hi;
  float buffer_factor;     /* ragged_buffer_factor; <= 0 means no cap          */
  int32_t num_chunks;      /* fallback chunks; 0 = ceil(S / factor)            */
  int32_t gate;            /* moe_gate                                         */
  int32_t dtype;           /* moe_dtype                                        */
  int32_t dedup;           /* 1: one buffer row per (token, shard) ([DRED])    */
  int32_t slots_per_shard; /* B redundant slots per shard                      */
  int32_t num_replicas;    /* R replicas planned per call, R <= S*B; R > 0
                              needs every shard resident (replica weights
                              alias their home expert's weights)               */
} moe_problem;

/* Limits of this build (MOE_EUNSUPPORTED beyond them): E <= 1024,
 * G <= 1024, T*k < 2^24.  MOE_BF16 also needs H % 256 == 0 and F % 128 == 0. */

/* ---- sizes --------------------------------------------------------------- */

/* Scratch bytes any single step call below may need. */
int moe_workspace_bytes(const moe_problem* p, size_t* bytes);

/* Row bounds of one pass: `num_chunks` chunks (1 = all tokens), capped or
 * not.  *max_rows bounds the expert-sorted rows, *max_dedup_rows the dedup
 * rows (0 without dedup).  Capped: every resident shard keeps at most cap =
 * ceil(factor*T*k/S) buffer rows ([FALLBACK] Why); uncapped: the worst case
 * T/n * min(k, E/S+B) rows per resident shard ([FALLBACK] How:
 * force_dropless sizes for the worst case). */
int moe_pass_max_rows(const moe_problem* p, int32_t num_chunks, int32_t capped,
                      int64_t* max_rows, int64_t* max_dedup_rows);

/* Workspace bytes of moe_layer_dropless_chunked in `mode` (all of its
 * intermediate buffers, sized for the larger of the passes it may take). */
int moe_layer_workspace_bytes(const moe_problem* p, int32_t mode, size_t* bytes);

/* Chunks of the dropless fallback that moe_layer_dropless_chunked runs as
 * one pass in `mode`: the most consecutive chunks whose worst-case rows fit
 * the buffers the call is sized for.  Those hold the rows of the capped
 * buffer ([FALLBACK] How: the fallback keeps each chunk's worst case within
 * the capped buffer, so the layer's peak HBM stays that of the capped
 * layer), or twice those where that leaves two or more passes: a pass
 * streams every resident expert's weights once, so twice the chunks per
 * pass halve that traffic, for a constant factor of two on the pass
 * buffers.  The passes run in order on the caller's stream.  The tokens of
 * the chunks are disjoint and every grouped-GEMM row is computed on its
 * own, so y is the same as chunk by chunk.  1 = one chunk per pass. */
int moe_layer_chunks_per_pass(const moe_problem* p, int32_t mode, int32_t* chunks);

/* ---- the hot path -------------------------------------------------------- */

/* a1. Router top-k ([FALLBACK] How: the check works "from the router's
 * top-k").  logits [T,E] fp32 -> topk_idx [T,k] int32 in descending logit
 * order, equal logits broken to the lowest index; topk_gate [T,k] fp32. */
int moe_route(const moe_problem* p, const float* logits, int32_t* topk_idx,
              float* topk_gate, void* stream);

/* a2+a3. Counts, redundancy plan, reroute, capacity and overflow
 * ([FALLBACK] How: _check_ragged_overflow; [DRED]: plan_expert_duplication
 * with the has_candidate guard, tokens rerouted to the replicas).
 * Outputs (device):
 *   expert_counts [E]    assignments per expert;
 *   slot_expert   [G]    global expert hosted by each slot, -1 = unused;
 *   ndiv          [E]    assignments diverted to the expert's replica;
 *   slot_of_assign[T*k]  slot of every assignment (the first ndiv[e]
 *                        assignments of e in (t,j) order go to the replica);
 *   shard_counts  [S]    rows each shard would receive (assignments, or
 *                        distinct tokens with dedup);
 *   status        [4]    cap (-1 = uncapped), overflow (0/1: some shard
 *                        count > cap), max shard count, MOE_ERR_* bits;
 *   required_factor [1]  float32, may be NULL: the smallest buffer factor
 *                        that would have fit, max shard count / (T*k/S)
 *                        ([FALLBACK] Shortcomings: the figure the overflow
 *                        log reports). */
int moe_count_overflow(const moe_problem* p, const int32_t* topk_idx,
                       int32_t* expert_counts, int32_t* slot_expert, int32_t* ndiv,
                       int32_t* slot_of_assign, int32_t* shard_counts, int32_t* status,
                       float* required_factor, void* ws, size_t ws_bytes, void* stream);

/* a4+a5. Layout and permute of one pass: chunk `chunk` of `num_chunks`
 * (token t = b*L + s is in chunk c when s*n/L == c; num_chunks 1 = all
 * tokens), capped (rows past the cap of a resident shard's buffer are
 * dropped) or not.  Rows are the pass's assignments on resident slots in
 * stable (slot, t, j) order ([RING] What: the expert-sorted MoE input).
 * Outputs (device):
 *   group_offsets [G_res+1]  exclusive scan of the rows per resident slot;
 *   row_of_assign [T*k]      row of each assignment of the pass, -1 if it is
 *                            no row; entries of other tokens untouched;
 *   sorted_assign [max_rows] flat assignment id t*k+j of each row;
 *   x_sorted [max_rows, H]   x_sorted[n] = x[sorted_assign[n] / k];
 *   with dedup ([DRED]: a token goes once to each destination shard and the
 *   receiver re-expands it): dedup_offsets [S_res+1], dedup_token
 *   [max_dedup_rows] (the distinct tokens of each resident shard in
 *   ascending order, cut at the cap when capped), x_dedup [max_dedup_rows,H],
 *   expand_idx [max_rows] (x_sorted[n] = x_dedup[expand_idx[n]]).  Without
 *   dedup these four may be NULL.
 * max_rows / max_dedup_rows must be at least moe_pass_max_rows' bounds. */
int moe_permute(const moe_problem* p, int32_t num_chunks, int32_t chunk, int32_t capped,
                const void* x, const int32_t* slot_of_assign,
                int32_t* group_offsets, int32_t* row_of_assign, int32_t* sorted_assign,
                int32_t* dedup_offsets, int32_t* dedup_token, int32_t* expand_idx,
                void* x_dedup, void* x_sorted, int64_t max_rows, int64_t max_dedup_rows,
                void* ws, size_t ws_bytes, void* stream);

/* a6. Grouped SwiGLU FFN over ragged groups ([DRED], rerouting comment: a
 * grouped matmul over the local experts' group sizes).  Group g holds rows
 * [group_offsets[g], group_offsets[g+1]) of x_sorted and runs the expert in
 * resident slot g (slot_expert[res_shard_lo*(E/S+B) + g]; a replica slot
 * uses its home expert's weights):
 *   act[n]        = SiLU(x_sorted[n] Wg^T) * (x_sorted[n] Wu^T)   [max_rows,F]
 *   expert_out[n] = act[n] Wd^T                                   [max_rows,H]
 * SiLU(z) = z/(1+exp(-z)).  Rows past group_offsets[G_res] are untouched.
 * status (device, one int32, may be NULL) receives the MOE_ERR_* bits of
 * the call: offsets that are not a non-decreasing sequence within [0,
 * min(max_rows, T*k)] compute nothing (act and expert_out untouched) and
 * set MOE_ERR_BAD_OFFSETS; a tile that gave up its bounded wait sets
 * MOE_ERR_GEMM_WAIT.  The return value is still MOE_OK in both cases, since
 * the offsets are read on the device only. */
int moe_gmm_swiglu(const moe_problem* p, const void* x_sorted, const int32_t* group_offsets,
                   const int32_t* slot_expert, const void* w_gate, const void* w_up,
                   const void* w_down, void* act, void* expert_out, int64_t max_rows,
                   int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* moe_gmm_swiglu for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results, with no workspace argument.
 * Its scratch (the tile schedule and the one-launch kernel's counters, a
 * few KB for the workloads here) lives in a fixed 2 MiB device array inside
 * the library, one per GPU, held until the process ends; a problem whose
 * scratch (G_res+1 + 3*(T*k/128 + G_res + 1) + 128 ints, rounded) exceeds
 * it returns MOE_ECAPACITY.  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.  Every call on one GPU shares
 * that GPU's array and clears the parts it needs at its start, so calls
 * that overlap on one GPU (concurrent streams) race and must be serialised
 * by the caller. */
int moe_gmm_swiglu_noalloc(const moe_problem* p, const void* x_sorted,
                           const int32_t* group_offsets, const int32_t* slot_expert,
                           const void* w_gate, const void* w_up, const void* w_down, void* act,
                           void* expert_out, int64_t max_rows, int32_t* status, void* stream);

/* a7. Gate-weighted combine of one pass: for every token t of the pass,
 *   y[t] = sum over j ascending of topk_gate[t,j] * expert_out[row_of_assign[t*k+j]]
 * over the assignments with a row (fp32 accumulation); 0 for a token with
 * none (all its experts elsewhere or dropped).  Rows of other tokens of y
 * are untouched. */
int moe_combine(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                const void* expert_out, const int32_t* row_of_assign,
                const float* topk_gate, void* y, void* stream);

/* Return-path dedup (receiving side).  The pages deduplicate the dispatch:
 * with dedup a token goes once to each destination shard and is re-expanded
 * there ([DRED], code review: dedup and expand_indices).  This applies the
 * same to the return: for every dedup row u < dedup_offsets[S_res] of a
 * pass (chunk `chunk` of num_chunks, capped or not: token t = dedup_token[u]
 * on one resident shard, the arrays that moe_permute wrote for that pass),
 *   partial[u] = sum over j ascending, over the assignments (t, j) whose row
 *                r = row_of_assign[t*k+j] lies in [0, max_rows) and has
 *                expand_idx[r] == u (its slot is on u's shard),
 *                of topk_gate[t,j] * expert_out[r]
 * with fp32 accumulation, stored as float32: one row per (token, shard)
 * instead of one per assignment.  The rows stay fp32 (not the activation
 * dtype) so that y is rounded once, at the source: a second bf16 rounding
 * exceeds the layer's error bound at DeepSeek-V3-sized rows.  partial is
 * float32 [max_dedup_rows, H]; rows past dedup_offsets[S_res] are
 * untouched.  max_rows (rows of expert_out and expand_idx) and
 * max_dedup_rows must hold the pass's worst case (moe_pass_max_rows), else
 * MOE_ECAPACITY.  MOE_EINVAL when the problem has no dedup. */
int moe_combine_partial(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                        int32_t capped, const void* expert_out, const int32_t* row_of_assign,
                        const float* topk_gate, const int32_t* dedup_offsets,
                        const int32_t* dedup_token, const int32_t* expand_idx, void* partial,
                        int64_t max_rows, int64_t max_dedup_rows, void* stream);

/* Return-path dedup (source side): for every token t of chunk `chunk` of
 * num_chunks (the pass moe_combine_partial served),
 *   y[t] = sum of partial[u] over the distinct dedup rows u = expand_idx[r]
 *          of the token's assignments with a row r in [0, max_rows), each
 *          taken once, at the token's first assignment on its shard (j
 *          ascending)
 * with fp32 accumulation (partial is float32), stored in the activation
 * dtype; 0 for a token with none: moe_combine regrouped by shard.  Rows of
 * other tokens of y are untouched.  Bounds as for moe_combine_partial.
 * MOE_EINVAL when the problem has no dedup. */
int moe_combine_from_partials(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                              int32_t capped, const void* partial,
                              const int32_t* row_of_assign, const int32_t* expand_idx, void* y,
                              int64_t max_rows, int64_t max_dedup_rows, void* stream);

/* a8. The whole layer ([FALLBACK] How): route, counts, plan, capacity and
 * overflow once, then the passes `mode` selects, writing y [T,H].  In LAYER
 * mode the device picks between the capped pass and the num_chunks dropless
 * chunks (moe_layer_chunks_per_pass of them per pass) from the overflow
 * flag, with no host synchronisation.
 * info (device, may be NULL) receives [overflow, fallback_ran, cap, max
 * shard count, MOE_ERR_* bits] (5 int32).  ws must hold
 * moe_layer_workspace_bytes(p, mode). */
int moe_layer_dropless_chunked(const moe_problem* p, int32_t mode, const void* x,
                               const float* logits, const void* w_gate, const void* w_up,
                               const void* w_down, void* y, int32_t* info,
                               void* ws, size_t ws_bytes, void* stream);

/* ---- backward of the hot path ------------------------------------------- */
/*
 * The backward of one pass, step by step, as the chain rule of the steps
 * above.  [FALLBACK] How runs the chunked passes in a scan; the scan's
 * backward redoes each chunk's forward and keeps the weight gradients as a
 * running sum across chunks; [RING] (title, What) keeps the expert-sorted input x_sorted
 * for the backward.  A caller runs, per pass of the forward (the same
 * num_chunks / chunk / capped, and the arrays moe_permute wrote for it):
 * moe_combine_bwd, moe_gmm_swiglu_bwd (accumulate = 0 on the first pass,
 * 1 after), moe_permute_bwd; then once moe_route_bwd.  Gradients of
 * weights, gates and logits are float32; row gradients (d_out, dx_sorted,
 * dx) use the activation dtype.
 */

/* Scratch bytes of moe_gmm_swiglu_bwd for `max_rows` pass rows. */
int moe_bwd_workspace_bytes(const moe_problem* p, int64_t max_rows, size_t* bytes);

/* Backward of moe_combine for the tokens of chunk `chunk` of num_chunks:
 * for each assignment (t, j) with a row r = row_of_assign[t*k+j] in
 * [0, max_rows),
 *   d_out[r]       = topk_gate[t,j] * dy[t]         (activation dtype)
 *   d_gate[t*k+j]  = <dy[t], expert_out[r]>         (float32, fp32 sum)
 * and d_gate = 0 for an assignment without a row.  Rows of d_out no
 * assignment of the pass points at, and d_gate of other tokens, are
 * untouched.  dy [T,H]; expert_out and d_out [max_rows, H]. */
int moe_combine_bwd(const moe_problem* p, int32_t num_chunks, int32_t chunk, const void* dy,
                    const void* expert_out, const int32_t* row_of_assign,
                    const float* topk_gate, void* d_out, float* d_gate, int64_t max_rows,
                    void* stream);

/* Backward of moe_gmm_swiglu over the same groups (group g runs resident
 * slot g's expert, a replica slot its home expert).  With h_g = x Wg^T,
 * h_u = x Wu^T, s = sigmoid(h_g):
 *   d_a = d_out Wd;  d_hg = d_a h_u s (1 + h_g (1 - s));  d_hu = d_a h_g s;
 *   dx_sorted = d_hg Wg + d_hu Wu                      [max_rows, H]
 *   dw_gate[e] (+)= d_hg^T x_sorted,  dw_up[e] (+)= d_hu^T x_sorted  [E_res,F,H]
 *   dw_down[e] (+)= d_out^T a,  a = SiLU(h_g) h_u (recomputed)        [E_res,H,F]
 * summed over every row of every group of expert e (float32).  accumulate
 * 0 overwrites the weight gradients (experts without rows get 0), 1 adds
 * to them (the carry across passes).  d_a, d_hg, d_hu and a are rounded to
 * the activation dtype where they are stored (in ws).  The weights are
 * read as they are (no transposed copies).  Rows of dx_sorted past
 * group_offsets[G_res] are untouched.  ws holds moe_bwd_workspace_bytes(p,
 * max_rows); the weight gradients are 16-byte aligned. */
int moe_gmm_swiglu_bwd(const moe_problem* p, const void* x_sorted, const int32_t* group_offsets,
                       const int32_t* slot_expert, const void* w_gate, const void* w_up,
                       const void* w_down, const void* d_out, void* dx_sorted, float* dw_gate,
                       float* dw_up, float* dw_down, int32_t accumulate, int64_t max_rows,
                       void* ws, size_t ws_bytes, void* stream);

/* Backward of moe_permute for the tokens of chunk `chunk` of num_chunks:
 *   dx[t] = sum over j ascending of dx_sorted[row_of_assign[t*k+j]]
 * over the rows in [0, max_rows) (fp32 sum, one rounding); 0 for a token
 * with none.  Rows of other tokens of dx are untouched. */
int moe_permute_bwd(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                    const void* dx_sorted, const int32_t* row_of_assign, void* dx,
                    int64_t max_rows, void* stream);

/* Backward of the gates into the logits, every token: only the k chosen
 * logits get a gradient (the choice is piecewise constant);
 *   SOFTMAX: d_l[idx_j] = g_j (d_g_j - sum_i g_i d_g_i)
 *   SIGMOID: d_l[idx_j] = d_g_j g_j (1 - g_j)
 * d_logits [T,E] float32 is written in full. */
int moe_route_bwd(const moe_problem* p, const int32_t* topk_idx, const float* topk_gate,
                  const float* d_gate, float* d_logits, void* stream);

/* Workspace bytes of moe_layer_bwd in `mode`. */
int moe_layer_bwd_workspace_bytes(const moe_problem* p, int32_t mode, size_t* bytes);

/* Backward of moe_layer_dropless_chunked(p, mode, x, logits, weights) for
 * the upstream gradient dy [T,H] ([FALLBACK] How: the chunked scan's
 * backward recomputes each chunk and carries the weight gradients across
 * the chunks).  Routing, counts, plan, the overflow flag and the pass
 * layouts are recomputed from x and logits, and the device takes the same
 * passes as the forward (LAYER: the capped pass or the dropless chunk
 * batches, from the flag, with no host synchronisation).  Per pass:
 * x_sorted recomputed (and in fp32 the expert outputs), then the combine,
 * grouped GEMM and permute backward of that pass; in bf16 the gate
 * gradients <dy, expert output> are taken as <dy Wd, act> in the grouped
 * GEMM's recompute, so no expert output is recomputed (the bf16 rounding
 * points differ from the step calls': dy Wd and gate * act are rounded
 * instead of gate * dy and the expert output).  In bf16 with two or more pass
 * slots (and every operand offset within 31 bits) the weight gradients are
 * not carried from pass to pass: each pass keeps its rows in the workspace
 * and the gradients of all passes are one reduction after the last pass,
 * written once (the same sum in another order).  Outputs:
 *   dx [T,H] (activation dtype; 0 for a token with no resident row),
 *   d_logits [T,E] float32 (only chosen logits are nonzero),
 *   dw_gate, dw_up [E_res,F,H], dw_down [E_res,H,F] float32, overwritten
 *   (the sum over every pass).
 * Pointers 16-byte aligned; ws holds moe_layer_bwd_workspace_bytes(p, mode)
 * (which includes those per-pass rows). */
int moe_layer_bwd(const moe_problem* p, int32_t mode, const void* x, const float* logits,
                  const void* w_gate, const void* w_up, const void* w_down, const void* dy,
                  void* dx, float* d_logits, float* dw_gate, float* dw_up, float* dw_down,
                  void* ws, size_t ws_bytes, void* stream);

/* Text of a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SHARD_H */
