// C ABI of the one-shard MoE layer: argument validation, buffer bounds,
// workspace layout and the order of launches.  Every entry point validates
// on the host and returns a moe_status before launching anything.
#include <math.h>
#include <string.h>

#include "common.h"
#include "moe_testing.h"
#include "sort.h"

using namespace moe;

namespace {

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// Validates the problem and derives its dimensions.
int make_dims(const moe_problem* p, Dims* d) {
  if (p == nullptr || d == nullptr) return MOE_EINVAL;
  memset(d, 0, sizeof(*d));
  if (p->tokens < 1 || p->seq_len < 1 || p->tokens % p->seq_len != 0) return MOE_EINVAL;
  if (p->hidden < 1 || p->ffn < 1 || p->num_experts < 1 || p->num_shards < 1) return MOE_EINVAL;
  if (p->num_experts % p->num_shards != 0) return MOE_EINVAL;
  if (p->top_k < 1 || p->top_k > p->num_experts) return MOE_EINVAL;
  if (p->res_shard_lo < 0 || p->res_shard_lo >= p->res_shard_hi ||
      p->res_shard_hi > p->num_shards)
    return MOE_EINVAL;
  if (p->gate != MOE_GATE_SOFTMAX && p->gate != MOE_GATE_SIGMOID) return MOE_EINVAL;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_EINVAL;
  if (p->dedup != 0 && p->dedup != 1) return MOE_EINVAL;
  if (p->slots_per_shard < 0 || p->num_replicas < 0) return MOE_EINVAL;
  if ((long long)p->num_replicas > (long long)p->num_shards * p->slots_per_shard)
    return MOE_EINVAL;
  if (!(p->buffer_factor == p->buffer_factor)) return MOE_EINVAL;  // NaN
  if (p->num_chunks < 0) return MOE_EINVAL;
  // replica slots compute with their home expert's weights, so planning
  // needs every expert's weights on this device
  if (p->num_replicas > 0 && (p->res_shard_lo != 0 || p->res_shard_hi != p->num_shards))
    return MOE_EUNSUPPORTED;
  if (p->top_k > kMaxTopK || p->num_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  const long long spd = p->num_experts / p->num_shards + p->slots_per_shard;
  if (spd * p->num_shards > kMaxSlots) return MOE_EUNSUPPORTED;
  if ((long long)p->tokens * p->top_k >= (1ll << 24)) return MOE_EUNSUPPORTED;
  if (p->dtype == MOE_BF16 && (p->hidden % 256 != 0 || p->ffn % 128 != 0))
    return MOE_EUNSUPPORTED;
  if (p->dtype == MOE_F32 && p->hidden % 4 != 0) return MOE_EUNSUPPORTED;

  d->T = p->tokens;
  d->L = p->seq_len;
  d->H = p->hidden;
  d->F = p->ffn;
  d->E = p->num_experts;
  d->k = p->top_k;
  d->S = p->num_shards;
  d->El = d->E / d->S;
  d->B = p->slots_per_shard;
  d->R = p->num_replicas;
  d->spd = d->El + d->B;
  d->G = d->S * d->spd;
  d->res_lo = p->res_shard_lo;
  d->res_hi = p->res_shard_hi;
  d->S_res = d->res_hi - d->res_lo;
  d->lo_slot = d->res_lo * d->spd;
  d->G_res = d->S_res * d->spd;
  d->e_base = d->res_lo * d->El;
  d->gate = p->gate;
  d->bf16 = p->dtype == MOE_BF16;
  d->dedup = p->dedup;
  // cap = ceil(factor * balanced), balanced = T*k/S ("Support
  // moe_dropless_fallback=layer on the ragged all-to-all MoE path", Why)
  double f = (double)p->buffer_factor;
  if (f > 0.0) {
    double c = ceil(f * (double)((long long)d->T * d->k) / (double)d->S);
    if (c > 2147483647.0) return MOE_EINVAL;
    d->cap = (int)c;
  } else {
    d->cap = -1;
  }
  // chunks: given, or ceil(S / factor) (the same page's Shortcomings:
  // example: 16 shards at factor 2 make eight chunks)
  int n = p->num_chunks;
  if (n == 0) n = f > 0.0 ? (int)ceil((double)d->S / f) : 1;
  if (n < 1 || n > d->L || d->L % n != 0) return MOE_EINVAL;
  d->n_default = n;
  // tall tiles halve the operand traffic per flop where the reduction is
  // long; short ones waste less on small groups
  d->gemm_bm = d->H >= MOE_GEMM_BIG_MIN_H ? 256 : 128;
  return MOE_OK;
}

// Row bounds of a pass over a window of lw positions of every sequence,
// capped or not.
void window_bounds(const Dims& d, int lw, int capped, int64_t* rows, int64_t* drows) {
  const int64_t tc = (int64_t)(d.T / d.L) * lw;
  const int64_t per_tok = d.k < d.spd ? d.k : d.spd;  // a token's rows on one shard
  int64_t r = tc * d.k;
  int64_t u = d.dedup ? tc * d.S_res : 0;
  if (d.dedup && u > r) u = r;
  int64_t worst = (int64_t)d.S_res * tc * per_tok;
  if (worst < r) r = worst;
  if (capped && d.cap >= 0) {
    int64_t c = d.dedup ? (int64_t)d.S_res * d.cap * per_tok : (int64_t)d.S_res * d.cap;
    if (c < r) r = c;
    if (d.dedup && (int64_t)d.S_res * d.cap < u) u = (int64_t)d.S_res * d.cap;
  }
  *rows = r;
  *drows = u;
}

// Row bounds of chunk passes of n chunks.
void pass_bounds(const Dims& d, int n, int capped, int64_t* rows, int64_t* drows) {
  window_bounds(d, d.L / n, capped, rows, drows);
}

// The passes a layer call in `mode` may take, as bounds.
void layer_bounds(const Dims& d, int mode, int64_t* rows, int64_t* drows) {
  int64_t r1 = 0, u1 = 0, r2 = 0, u2 = 0;
  switch (mode) {
    case MOE_MODE_LAYER:
      pass_bounds(d, 1, 1, &r1, &u1);
      if (d.cap >= 0) pass_bounds(d, d.n_default, 0, &r2, &u2);
      break;
    case MOE_MODE_FORCE_DROPLESS: pass_bounds(d, 1, 0, &r1, &u1); break;
    case MOE_MODE_CAPPED_ONLY: pass_bounds(d, 1, 1, &r1, &u1); break;
    default: pass_bounds(d, d.n_default, 0, &r1, &u1); break;
  }
  *rows = r1 > r2 ? r1 : r2;
  *drows = u1 > u2 ? u1 : u2;
}

// The layout set of a single static pass (chunk c of n, capped or not).
LayoutSet single_layout(const Dims& d, int n, int c, int capped) {
  LayoutSet ls;
  memset(&ls, 0, sizeof(ls));
  if (n == 1) {
    ls.has_single = 1;
    ls.single_capped = capped;
  } else {
    ls.win = d.L / n;
    ls.w_lo = c;
    ls.w_cnt = 1;
    ls.w_capped = capped;
  }
  return ls;
}

// Chunks of the dropless fallback that run as one pass: the most
// consecutive chunks whose worst-case rows still fit the buffers sized for
// the call (rows, drows), so that running them together never needs more
// memory than the capped buffer.  Their tokens are disjoint and every row
// of the grouped GEMM is computed independently of the others, so y is the
// same as chunk by chunk.
int chunk_batch(const Dims& d, int64_t rows, int64_t drows) {
  const int n = d.n_default, lc = d.L / n;
  int q = 1;
  for (int cand = 2; cand <= n; ++cand) {
    int64_t r, u;
    window_bounds(d, cand * lc, 0, &r, &u);
    if (r > rows || u > drows) break;
    q = cand;
  }
  return q;
}

// The passes of a layer call in `mode`.  LAYER with a cap: the single pass
// (layout 0) or the dropless chunks in batches of q (layouts 1..), chosen on
// the device by the overflow flag.  Without overflow no shard exceeds the
// cap, so the single pass keeps every row and is laid out uncapped.
LayoutSet layer_layout(const Dims& d, int mode, int q, const int* ovf) {
  LayoutSet ls;
  memset(&ls, 0, sizeof(ls));
  const int n = d.n_default;
  ls.win = (d.L / n) * q;
  switch (mode) {
    case MOE_MODE_LAYER:
      ls.has_single = 1;
      if (d.cap >= 0) {
        ls.w_cnt = (n + q - 1) / q;
        ls.ovf = ovf;
      }
      break;
    case MOE_MODE_FORCE_DROPLESS: ls.has_single = 1; break;
    case MOE_MODE_CAPPED_ONLY: ls.has_single = 1; ls.single_capped = 1; break;
    default: ls.w_cnt = (n + q - 1) / q; break;
  }
  return ls;
}

// Static pass arguments of layout j.
PassArgs static_pass(const Dims& d, const LayoutSet& ls, int j) {
  int s0, lw, capped;
  size_t e0;
  layout_pass(d, ls, j, &s0, &lw, &capped, &e0);
  return static_pass_args(s0, lw, capped, j, d.L);
}

size_t step_scratch(const Dims& d) {
  size_t a = count_scratch_bytes(d), b = layout_scratch_bytes(d, single_layout(d, 1, 0, 1)),
         c = gmm_scratch_bytes(d);
  size_t m = a > b ? a : b;
  return m > c ? m : c;
}

// Workspace layout of the layer.
struct LayerWs {
  int* topk_idx;
  float* topk_gate;
  int* expert_counts;
  int* slot_expert;
  int* ndiv;
  int* slot_of_assign;
  int* shard_counts;
  int* status;
  void* count_scratch;
  void* layout_scratch;
  // pass buffers (the passes run in order on the caller's stream)
  void* x_dedup;
  void* act;
  void* out;
  // one-launch grouped GEMM counters, one block of sync_stride ints per pass
  // slot (bf16), zeroed by the route launch of the call
  int* gsync;
  int sync_stride, sync_slots;
  // where the grouped GEMM reports MOE_ERR_* bits (not carved: the caller's
  // info word, else status[3])
  int* err;
  size_t bytes;
};

// Pass slots a layer call enqueues: with the device-side choice (LAYER with
// a cap) one per chunk batch, the first also standing for the single pass;
// otherwise one per layout.
int layer_pass_slots(const LayoutSet& ls) {
  return (ls.has_single && ls.w_cnt > 0) ? ls.w_cnt : layout_num_passes(ls);
}

bool fits_rsrc(const Dims& d, int64_t rows, int64_t drows);

// Row bounds and chunks per pass of a layer call in `mode`.  The passes run
// in order on the caller's stream with one set of pass buffers.  With two or
// more chunk passes the buffers hold twice the rows the bounds give (the
// memory that two sets would take to overlap consecutive passes on two
// streams) and each pass as many chunks as they hold: every pass streams
// each resident expert's weights once, so twice the chunks per pass halve
// that traffic.  (Measured on MI355X, Llama4-Maverick-shaped shard: 6.8-6.9
// ms per layer against 7.85 ms for one-chunk passes overlapped on two
// streams.)
struct LayerPlan {
  int64_t rows, drows;
  int q;
};

LayerPlan layer_plan(const Dims& d, int mode) {
  LayerPlan pl;
  layer_bounds(d, mode, &pl.rows, &pl.drows);
  pl.q = chunk_batch(d, pl.rows, pl.drows);
  if (layer_layout(d, mode, pl.q, nullptr).w_cnt >= 2) {
    const int q2 = chunk_batch(d, 2 * pl.rows, 2 * pl.drows);
    int64_t r, u;
    window_bounds(d, q2 * (d.L / d.n_default), 0, &r, &u);
    r = r > pl.rows ? r : pl.rows;
    u = u > pl.drows ? u : pl.drows;
    if (q2 > pl.q && fits_rsrc(d, r, u)) {
      pl.q = q2;
      pl.rows = r;
      pl.drows = u;
    }
  }
  return pl;
}

LayerWs carve_layer(const Dims& d, const LayoutSet& ls, int64_t rows, int64_t drows, char* base) {
  LayerWs w;
  size_t off = 0;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += al256(b > 0 ? b : 1);
    return (void*)p;
  };
  const size_t tk = (size_t)d.T * d.k;
  const size_t es = d.bf16 ? 2 : 4;
  w.topk_idx = (int*)take(tk * 4);
  w.topk_gate = (float*)take(tk * 4);
  w.expert_counts = (int*)take((size_t)d.E * 4);
  w.slot_expert = (int*)take((size_t)d.G * 4);
  w.ndiv = (int*)take((size_t)d.E * 4);
  w.slot_of_assign = (int*)take(tk * 4);
  w.shard_counts = (int*)take((size_t)d.S * 4);
  w.status = (int*)take(4 * 4);
  w.count_scratch = take(count_scratch_bytes(d));
  w.layout_scratch = take(layout_scratch_bytes(d, ls));
  w.x_dedup = take(d.dedup ? (size_t)drows * d.H * es : 0);
  w.act = take((size_t)rows * d.F * es);
  w.out = take((size_t)rows * d.H * es);
  w.sync_stride = (int)(gmm_sync_bytes(d) / 4);
  w.sync_slots = d.bf16 ? layer_pass_slots(ls) : 0;
  w.gsync = w.sync_slots > 0 ? (int*)take((size_t)w.sync_slots * gmm_sync_bytes(d)) : nullptr;
  w.err = w.status != nullptr ? w.status + 3 : nullptr;
  w.bytes = off;
  return w;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

// The GEMMs address their bf16 operands through 32-bit buffer offsets.
bool fits_rsrc(const Dims& d, int64_t rows, int64_t drows) {
  if (!d.bf16) return true;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t wide = d.H > d.F ? d.H : d.F;
  return (int64_t)d.T * d.H * 2 < lim && rows * wide * 2 < lim && drows * d.H * 2 < lim;
}

// One pass of the layer: with dedup the pass's distinct tokens are copied
// once per shard (the dedup buffer) and GEMM1 re-expands them through
// expand_idx; without, GEMM1 gathers its rows from x through sorted_assign.
// Then the combine of the pass's tokens.
int run_pass(const Dims& d, const PassArgs& pa, const LayoutSet& ls, const LayoutBuffers& lb,
             const void* x, const void* wg, const void* wu, const void* wd, void* y,
             const LayerWs& w, int slot, int64_t rows, int64_t drows,
             hipStream_t s) {
  const long long tk = (long long)d.T * d.k;
  const int es = d.bf16 ? 2 : 4;
  GemmPass gp;
  if (d.dedup) {
    hipError_t e = launch_gather_rows(lb.meta + 1, kLayoutMeta, lb.dedup_token, tk, 1, x,
                                      w.x_dedup, d.H * es, d.T, drows, pa, s);
    if (e != hipSuccess) return MOE_EHIP;
    gp.a_src = w.x_dedup;
    gp.a_src_rows = (int)drows;
    gp.a_index = lb.expand_idx;
    gp.a_div = 1;
  } else {
    gp.a_src = x;
    gp.a_src_rows = d.T;
    gp.a_index = lb.sorted_assign;
    gp.a_div = d.k;
  }
  gp.a_index_stride = tk;
  gp.group_offsets = lb.group_offsets;
  gp.tile_off = lb.tile_off;
  gp.tile_group = lb.tile_group;
  gp.go_stride = d.G_res + 1;
  gp.tg_stride = tile_map_len(d);
  gp.sync = w.gsync != nullptr ? w.gsync + (size_t)slot * w.sync_stride : nullptr;
  gp.err = w.err;
  hipError_t e = launch_gmm(d, pa, gp, w.slot_expert, wg, wu, wd, w.act, w.out, rows,
                            nullptr, s);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_combine(d, pa, ls, w.out, lb.row_of_assign, tk, rows, w.topk_gate, y, s);
  return hip_status(e);
}

}  // namespace

extern "C" {

int moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_EINVAL;
  *bytes = step_scratch(d);
  return MOE_OK;
}

int moe_pass_max_rows(const moe_problem* p, int32_t num_chunks, int32_t capped,
                      int64_t* max_rows, int64_t* max_dedup_rows) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (max_rows == nullptr || max_dedup_rows == nullptr) return MOE_EINVAL;
  if (num_chunks < 1 || d.L % num_chunks != 0 || (capped != 0 && capped != 1)) return MOE_EINVAL;
  pass_bounds(d, num_chunks, capped, max_rows, max_dedup_rows);
  return MOE_OK;
}

int moe_layer_workspace_bytes(const moe_problem* p, int32_t mode, size_t* bytes) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (bytes == nullptr || mode < MOE_MODE_LAYER || mode > MOE_MODE_FORCE_CHUNKED)
    return MOE_EINVAL;
  const LayerPlan pl = layer_plan(d, mode);
  *bytes = carve_layer(d, layer_layout(d, mode, pl.q, nullptr), pl.rows, pl.drows, nullptr).bytes;
  return MOE_OK;
}

int moe_layer_chunks_per_pass(const moe_problem* p, int32_t mode, int32_t* chunks) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (chunks == nullptr || mode < MOE_MODE_LAYER || mode > MOE_MODE_FORCE_CHUNKED)
    return MOE_EINVAL;
  *chunks = layer_plan(d, mode).q;
  return MOE_OK;
}

int moe_route(const moe_problem* p, const float* logits, int32_t* topk_idx, float* topk_gate,
              void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_gate) return MOE_EINVAL;
  return hip_status(launch_route(d, logits, topk_idx, topk_gate, nullptr, (hipStream_t)stream));
}

int moe_count_overflow(const moe_problem* p, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* slot_expert, int32_t* ndiv, int32_t* slot_of_assign,
                       int32_t* shard_counts, int32_t* status, float* required_factor, void* ws,
                       size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!topk_idx || !expert_counts || !slot_expert || !ndiv || !slot_of_assign || !shard_counts ||
      !status || !ws)
    return MOE_EINVAL;
  if (misaligned(ws, 256)) return MOE_EINVAL;
  if (ws_bytes < count_scratch_bytes(d)) return MOE_ECAPACITY;
  return hip_status(launch_count(d, topk_idx, expert_counts, slot_expert, ndiv, slot_of_assign,
                                 shard_counts, status, ws, 0, nullptr, 0, required_factor,
                                 (hipStream_t)stream));
}

int moe_permute(const moe_problem* p, int32_t num_chunks, int32_t chunk, int32_t capped,
                const void* x, const int32_t* slot_of_assign, int32_t* group_offsets,
                int32_t* row_of_assign, int32_t* sorted_assign, int32_t* dedup_offsets,
                int32_t* dedup_token, int32_t* expand_idx, void* x_dedup, void* x_sorted,
                int64_t max_rows, int64_t max_dedup_rows, void* ws, size_t ws_bytes,
                void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (num_chunks < 1 || d.L % num_chunks != 0 || chunk < 0 || chunk >= num_chunks ||
      (capped != 0 && capped != 1))
    return MOE_EINVAL;
  if (!x || !slot_of_assign || !group_offsets || !row_of_assign || !sorted_assign || !x_sorted ||
      !ws)
    return MOE_EINVAL;
  if (d.dedup && (!dedup_offsets || !dedup_token || !expand_idx || !x_dedup)) return MOE_EINVAL;
  if (misaligned(ws, 256) || misaligned(x, 16) || misaligned(x_sorted, 16) ||
      (d.dedup && misaligned(x_dedup, 16)))
    return MOE_EINVAL;
  int64_t rb, ub;
  pass_bounds(d, num_chunks, capped, &rb, &ub);
  if (max_rows < rb || (d.dedup && max_dedup_rows < ub)) return MOE_ECAPACITY;
  const LayoutSet ls = single_layout(d, num_chunks, chunk, capped);
  if (ws_bytes < layout_scratch_bytes(d, ls)) return MOE_ECAPACITY;
  if (max_rows >= (1ll << 31) || max_dedup_rows >= (1ll << 31)) return MOE_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // the layout writes the caller's arrays directly; the rest stays in ws
  LayoutBuffers lb = carve_layout(d, ls, ws);
  lb.group_offsets = group_offsets;
  lb.row_of_assign = row_of_assign;
  lb.sorted_assign = sorted_assign;
  if (d.dedup) {
    lb.dedup_offsets = dedup_offsets;
    lb.dedup_token = dedup_token;
    lb.expand_idx = expand_idx;
  }
  const int row_bytes = d.H * (d.bf16 ? 2 : 4);
  hipError_t e = launch_permute_one(d, ls, slot_of_assign, lb, x, x_sorted, row_bytes, max_rows, s);
  if (e != hipErrorNotSupported) return hip_status(e);
  e = launch_layout(d, ls, slot_of_assign, 0, lb, nullptr, s);
  if (e != hipSuccess) return MOE_EHIP;
  const int lc = d.L / num_chunks;
  const PassArgs pa = static_pass_args(chunk * lc, lc, capped, 0, d.L);
  if (d.dedup) {
    e = launch_gather_rows(lb.meta + 1, kLayoutMeta, dedup_token, 0, 1, x, x_dedup, row_bytes,
                           d.T, max_dedup_rows, pa, s);
    if (e != hipSuccess) return MOE_EHIP;
    e = launch_gather_rows(lb.meta, kLayoutMeta, expand_idx, 0, 1, x_dedup, x_sorted, row_bytes,
                           (int)max_dedup_rows, max_rows, pa, s);
  } else {
    e = launch_gather_rows(lb.meta, kLayoutMeta, sorted_assign, 0, d.k, x, x_sorted, row_bytes,
                           d.T, max_rows, pa, s);
  }
  return hip_status(e);
}

int moe_gmm_swiglu(const moe_problem* p, const void* x_sorted, const int32_t* group_offsets,
                   const int32_t* slot_expert, const void* w_gate, const void* w_up,
                   const void* w_down, void* act, void* expert_out, int64_t max_rows,
                   int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!x_sorted || !group_offsets || !slot_expert || !w_gate || !w_up || !w_down || !act ||
      !expert_out || !ws || max_rows < 0)
    return MOE_EINVAL;
  if (misaligned(ws, 256) || misaligned(x_sorted, 16) || misaligned(act, 16) ||
      misaligned(w_gate, 16) || misaligned(w_up, 16) || misaligned(w_down, 16))
    return MOE_EINVAL;
  if (max_rows >= (1ll << 31) / 2) return MOE_EUNSUPPORTED;
  if (ws_bytes < gmm_scratch_bytes(d)) return MOE_ECAPACITY;
  if (!fits_rsrc(d, max_rows, 0)) return MOE_EUNSUPPORTED;
  const PassArgs pa = static_pass_args(0, d.L, 0, 0, d.L);
  GemmPass gp;
  memset(&gp, 0, sizeof(gp));
  gp.a_src = x_sorted;
  gp.a_src_rows = (int)max_rows;
  gp.a_div = 1;
  gp.group_offsets = group_offsets;
  // the step call runs on the caller's stream only (a layer call may split
  // a long-F single pass over its side stream)
  gp.err = status;
  return hip_status(launch_gmm(d, pa, gp, slot_expert, w_gate, w_up, w_down, act, expert_out,
                               max_rows, ws, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Scratch of moe_gmm_swiglu_noalloc: the tile schedule and the one-launch
// kernel's counters, in a file-scope device array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)2 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of this device's scratch array, or null if the lookup
// failed (first call on each device, with that device current).
void* noalloc_scratch() {
  static void* ptr[kMaxDevices] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = a;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

int moe_gmm_swiglu_noalloc(const moe_problem* p, const void* x_sorted,
                           const int32_t* group_offsets, const int32_t* slot_expert,
                           const void* w_gate, const void* w_up, const void* w_down, void* act,
                           void* expert_out, int64_t max_rows, int32_t* status, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!x_sorted || !group_offsets || !slot_expert || !w_gate || !w_up || !w_down || !act ||
      !expert_out || max_rows < 0)
    return MOE_EINVAL;
  if (misaligned(x_sorted, 16) || misaligned(act, 16) || misaligned(w_gate, 16) ||
      misaligned(w_up, 16) || misaligned(w_down, 16))
    return MOE_EINVAL;
  if (max_rows >= (1ll << 31) / 2) return MOE_EUNSUPPORTED;
  if (!fits_rsrc(d, max_rows, 0)) return MOE_EUNSUPPORTED;
  // the problem's scratch must fit the fixed array
  if (gmm_scratch_bytes(d) > kNoAllocScratchBytes) return MOE_ECAPACITY;
  void* ws = noalloc_scratch();
  if (ws == nullptr) return MOE_EHIP;
  const PassArgs pa = static_pass_args(0, d.L, 0, 0, d.L);
  GemmPass gp;
  memset(&gp, 0, sizeof(gp));
  gp.a_src = x_sorted;
  gp.a_src_rows = (int)max_rows;
  gp.a_div = 1;
  gp.group_offsets = group_offsets;
  gp.err = status;
  // the same launches as moe_gmm_swiglu; its first launch (the tile
  // schedule) clears the counters the later ones expect at zero
  return hip_status(launch_gmm(d, pa, gp, slot_expert, w_gate, w_up, w_down, act, expert_out,
                               max_rows, ws, (hipStream_t)stream));
}

int moe_combine(const moe_problem* p, int32_t num_chunks, int32_t chunk, const void* expert_out,
                const int32_t* row_of_assign, const float* topk_gate, void* y, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (num_chunks < 1 || d.L % num_chunks != 0 || chunk < 0 || chunk >= num_chunks)
    return MOE_EINVAL;
  if (!expert_out || !row_of_assign || !topk_gate || !y) return MOE_EINVAL;
  if (misaligned(expert_out, 16) || misaligned(y, 16)) return MOE_EINVAL;
  const int lc = d.L / num_chunks;
  const PassArgs pa = static_pass_args(chunk * lc, lc, 0, 0, d.L);
  const LayoutSet ls = single_layout(d, num_chunks, chunk, 0);
  return hip_status(launch_combine(d, pa, ls, expert_out, row_of_assign, 0, INT64_MAX, topk_gate,
                                   y, (hipStream_t)stream));
}

// Row bounds of the pass the return-path entry points serve: the buffers
// must hold its worst case (no silent truncation).
int return_path_bounds(const Dims& d, int num_chunks, int chunk, int capped, int64_t max_rows,
                       int64_t max_dedup_rows) {
  if (!d.dedup) return MOE_EINVAL;
  if (num_chunks < 1 || d.L % num_chunks != 0 || chunk < 0 || chunk >= num_chunks ||
      (capped != 0 && capped != 1))
    return MOE_EINVAL;
  if (max_rows < 0 || max_dedup_rows < 0) return MOE_EINVAL;
  int64_t rb, ub;
  pass_bounds(d, num_chunks, capped, &rb, &ub);
  if (max_rows < rb || max_dedup_rows < ub) return MOE_ECAPACITY;
  if (max_rows >= (1ll << 31) || max_dedup_rows >= (1ll << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int moe_combine_partial(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                        int32_t capped, const void* expert_out, const int32_t* row_of_assign,
                        const float* topk_gate, const int32_t* dedup_offsets,
                        const int32_t* dedup_token, const int32_t* expand_idx, void* partial,
                        int64_t max_rows, int64_t max_dedup_rows, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!d.dedup) return MOE_EINVAL;
  if (!expert_out || !row_of_assign || !topk_gate || !dedup_offsets || !dedup_token ||
      !expand_idx || !partial)
    return MOE_EINVAL;
  if (misaligned(expert_out, 16) || misaligned(partial, 16)) return MOE_EINVAL;
  st = return_path_bounds(d, num_chunks, chunk, capped, max_rows, max_dedup_rows);
  if (st != MOE_OK) return st;
  return hip_status(launch_combine_partial(d, dedup_offsets + d.S_res, dedup_token, row_of_assign,
                                           expand_idx, topk_gate, expert_out, max_rows,
                                           max_dedup_rows, partial, (hipStream_t)stream));
}

int moe_combine_from_partials(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                              int32_t capped, const void* partial,
                              const int32_t* row_of_assign, const int32_t* expand_idx, void* y,
                              int64_t max_rows, int64_t max_dedup_rows, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!d.dedup) return MOE_EINVAL;
  if (!partial || !row_of_assign || !expand_idx || !y) return MOE_EINVAL;
  if (misaligned(partial, 16) || misaligned(y, 16)) return MOE_EINVAL;
  st = return_path_bounds(d, num_chunks, chunk, capped, max_rows, max_dedup_rows);
  if (st != MOE_OK) return st;
  const int lc = d.L / num_chunks;
  const PassArgs pa = static_pass_args(chunk * lc, lc, 0, 0, d.L);
  return hip_status(launch_combine_from_partials(d, pa, row_of_assign, expand_idx, partial,
                                                 max_rows, max_dedup_rows, y,
                                                 (hipStream_t)stream));
}

int moe_layer_dropless_chunked(const moe_problem* p, int32_t mode, const void* x,
                               const float* logits, const void* w_gate, const void* w_up,
                               const void* w_down, void* y, int32_t* info, void* ws,
                               size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (mode < MOE_MODE_LAYER || mode > MOE_MODE_FORCE_CHUNKED) return MOE_EINVAL;
  if (!x || !logits || !w_gate || !w_up || !w_down || !y || !ws) return MOE_EINVAL;
  if (misaligned(ws, 256) || misaligned(x, 16) || misaligned(y, 16) || misaligned(w_gate, 16) ||
      misaligned(w_up, 16) || misaligned(w_down, 16))
    return MOE_EINVAL;
  const LayerPlan pl = layer_plan(d, mode);
  const int64_t rows = pl.rows, drows = pl.drows;
  if (!fits_rsrc(d, rows, drows)) return MOE_EUNSUPPORTED;
  const int q = pl.q;
  LayerWs w0 = carve_layer(d, layer_layout(d, mode, q, nullptr), rows, drows, nullptr);
  if (ws_bytes < w0.bytes) return MOE_ECAPACITY;
  // status[1] (the overflow flag) lives in the workspace
  LayerWs w = carve_layer(d, layer_layout(d, mode, q, nullptr), rows, drows, (char*)ws);
  // the count step writes the error bits found so far to info[4] (and
  // status[3]); the grouped GEMM adds its own to the same word
  if (info != nullptr) w.err = info + 4;
  const LayoutSet ls = layer_layout(d, mode, q, w.status + 1);
  hipStream_t s = (hipStream_t)stream;

  hipError_t e = launch_route(d, logits, w.topk_idx, w.topk_gate,
                              count_hist_area(d, w.count_scratch), s, w.gsync,
                              w.sync_slots * w.sync_stride);
  if (e != hipSuccess) return MOE_EHIP;
  // without rerouting every assignment goes to its expert's home slot, so
  // the layout reads the top-k directly; when the layout fuses its scan and
  // placement, the count step runs inside that launch too
  const bool reroute = d.R > 0 && d.B > 0;
  const LayoutBuffers lb = carve_layout(d, ls, w.layout_scratch);
  if (!reroute && layout_fused(d)) {
    const CountArgs c = layer_count_args(d, w.topk_idx, w.expert_counts, w.slot_expert, w.ndiv,
                                         w.shard_counts, w.status, w.count_scratch, info, mode);
    e = launch_layout(d, ls, w.topk_idx, 1, lb, &c, s);
    if (e != hipSuccess) return MOE_EHIP;
  } else {
    e = launch_count(d, w.topk_idx, w.expert_counts, w.slot_expert, w.ndiv,
                     reroute ? w.slot_of_assign : nullptr, w.shard_counts, w.status,
                     w.count_scratch, 1, info, mode, nullptr, s);
    if (e != hipSuccess) return MOE_EHIP;
    e = launch_layout(d, ls, reroute ? w.slot_of_assign : w.topk_idx, reroute ? 0 : 1, lb,
                      nullptr, s);
    if (e != hipSuccess) return MOE_EHIP;
  }

  // The passes run in order on the caller's stream (layer_plan); each
  // reuses the pass buffers after the previous one, which stream order puts
  // first.
  const int slots = layer_pass_slots(ls);
  for (int b = 0; b < slots && st == MOE_OK; ++b) {
    PassArgs pa;
    if (ls.ovf != nullptr) {
      // the device decides: the single pass alone, or the batches of
      // dropless chunks
      const int s0 = b * ls.win;
      pa = static_pass_args(s0, ls.win < d.L - s0 ? ls.win : d.L - s0, 0, b, d.L);
      pa.ovf = ls.ovf;
    } else {
      pa = static_pass(d, ls, b);
    }
    st = run_pass(d, pa, ls, lb, x, w_gate, w_up, w_down, y, w, b, rows, drows, s);
  }
  return st;
}

// ---- backward -----------------------------------------------------------

int moe_bwd_workspace_bytes(const moe_problem* p, int64_t max_rows, size_t* bytes) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (bytes == nullptr || max_rows < 0) return MOE_EINVAL;
  *bytes = gmm_bwd_scratch_bytes(d, max_rows);
  return MOE_OK;
}

int moe_combine_bwd(const moe_problem* p, int32_t num_chunks, int32_t chunk, const void* dy,
                    const void* expert_out, const int32_t* row_of_assign,
                    const float* topk_gate, void* d_out, float* d_gate, int64_t max_rows,
                    void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (num_chunks < 1 || d.L % num_chunks != 0 || chunk < 0 || chunk >= num_chunks)
    return MOE_EINVAL;
  if (!dy || !expert_out || !row_of_assign || !topk_gate || !d_out || !d_gate || max_rows < 0)
    return MOE_EINVAL;
  if (misaligned(dy, 16) || misaligned(expert_out, 16) || misaligned(d_out, 16))
    return MOE_EINVAL;
  const int lc = d.L / num_chunks;
  const PassArgs pa = static_pass_args(chunk * lc, lc, 0, 0, d.L);
  return hip_status(launch_combine_bwd(d, pa, single_layout(d, num_chunks, chunk, 0), dy,
                                       expert_out, row_of_assign, 0, topk_gate, d_out, d_gate,
                                       max_rows, 3, (hipStream_t)stream));
}

int moe_gmm_swiglu_bwd(const moe_problem* p, const void* x_sorted, const int32_t* group_offsets,
                       const int32_t* slot_expert, const void* w_gate, const void* w_up,
                       const void* w_down, const void* d_out, void* dx_sorted, float* dw_gate,
                       float* dw_up, float* dw_down, int32_t accumulate, int64_t max_rows,
                       void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!x_sorted || !group_offsets || !slot_expert || !w_gate || !w_up || !w_down || !d_out ||
      !dx_sorted || !dw_gate || !dw_up || !dw_down || !ws || max_rows < 0 ||
      (accumulate != 0 && accumulate != 1))
    return MOE_EINVAL;
  if (misaligned(ws, 256) || misaligned(x_sorted, 16) || misaligned(d_out, 16) ||
      misaligned(w_gate, 16) || misaligned(w_up, 16) || misaligned(w_down, 16) ||
      misaligned(dx_sorted, 4) || misaligned(dw_gate, 16) || misaligned(dw_up, 16) ||
      misaligned(dw_down, 16))
    return MOE_EINVAL;
  // buffer resources address A operands with 32-bit byte offsets
  const int64_t wide = d.H > 2 * d.F ? d.H : 2 * d.F;
  if (max_rows * wide * 2 >= ((int64_t)1 << 31)) return MOE_EUNSUPPORTED;
  if (ws_bytes < gmm_bwd_scratch_bytes(d, max_rows)) return MOE_ECAPACITY;
  GemmBwdArgs a;
  a.x_sorted = x_sorted;
  a.group_offsets = group_offsets;
  a.go_stride = 0;
  a.pa = static_pass_args(0, d.L, 0, 0, d.L);
  a.slot_expert = slot_expert;
  a.wg = w_gate;
  a.wu = w_up;
  a.wd = w_down;
  a.d_out = d_out;
  a.dx_sorted = dx_sorted;
  a.dwg = dw_gate;
  a.dwu = dw_up;
  a.dwd = dw_down;
  a.accumulate = accumulate;
  a.max_rows = max_rows;
  a.scratch = ws;
  a.out_recompute = nullptr;
  return hip_status(launch_gmm_bwd(d, a, (hipStream_t)stream));
}

int moe_permute_bwd(const moe_problem* p, int32_t num_chunks, int32_t chunk,
                    const void* dx_sorted, const int32_t* row_of_assign, void* dx,
                    int64_t max_rows, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (num_chunks < 1 || d.L % num_chunks != 0 || chunk < 0 || chunk >= num_chunks)
    return MOE_EINVAL;
  if (!dx_sorted || !row_of_assign || !dx || max_rows < 0) return MOE_EINVAL;
  if (misaligned(dx_sorted, 16) || misaligned(dx, 16)) return MOE_EINVAL;
  const int lc = d.L / num_chunks;
  const PassArgs pa = static_pass_args(chunk * lc, lc, 0, 0, d.L);
  return hip_status(launch_permute_bwd(d, pa, single_layout(d, num_chunks, chunk, 0),
                                       dx_sorted, row_of_assign, 0, dx, max_rows,
                                       (hipStream_t)stream));
}

int moe_route_bwd(const moe_problem* p, const int32_t* topk_idx, const float* topk_gate,
                  const float* d_gate, float* d_logits, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!topk_idx || !topk_gate || !d_gate || !d_logits) return MOE_EINVAL;
  return hip_status(launch_route_bwd(d, topk_idx, topk_gate, d_gate, d_logits,
                                     (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Whether a layer backward takes the weight gradients of all its passes in
// one launch at the end (bf16, two or more pass slots, every pass's groups
// together within kMaxSlots, every operand offset within 31 bits).  The
// passes then keep their x_sorted, d_out, d_h and act rows, and the float32
// gradients are written once instead of read and written once per pass
// (the pages' scan carries them from chunk to chunk; holding every chunk's
// rows at once is what a GPU with this much memory can afford).
bool defer_wgrad(const Dims& d, int slots, int64_t rows) {
  if (!d.bf16 || slots < 2 || (int64_t)slots * d.G_res > kMaxSlots) return false;
  const int64_t wide = d.H > 2 * d.F ? d.H : 2 * d.F;
  return (int64_t)slots * rows * wide * 2 < ((int64_t)1 << 31);
}

// Workspace of moe_layer_bwd: the forward layer's (routing, counts, layouts,
// one set of pass buffers), then x_sorted and d_out rows (per pass slot
// when the weight gradients are deferred, else one set), dx_sorted rows, the
// gate gradients, the grouped-GEMM backward's scratch and, deferred, every
// pass's d_h and act rows and group offsets and the weight gradients'
// scratch.
struct LayerBwdWs {
  LayerWs fwd;
  bool defer;
  void* x_sorted;
  void* d_out;
  void* dxs;
  float* d_gate;
  void* gmm;
  void* d_h_all;
  void* act_all;
  int* go_all;
  void* wgrad;
  float* row_gate;  // bf16: each row's gate (the gated mode of launch_gmm_bwd)
  float* dg_part;   // bf16: the rows' gate-gradient parts [rows, F/32]
  size_t bytes;
};

LayerBwdWs carve_layer_bwd(const Dims& d, const LayoutSet& ls, int64_t rows, int64_t drows,
                           char* base) {
  LayerBwdWs w;
  // the backward's passes run on the caller's stream and use the first
  // buffer set of the forward's layout (one set is enough)
  w.fwd = carve_layer(d, ls, rows, drows, base);
  size_t off = w.fwd.bytes;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += al256(b > 0 ? b : 1);
    return (void*)p;
  };
  const size_t es = d.bf16 ? 2 : 4;
  const int slots = layer_pass_slots(ls);
  w.defer = defer_wgrad(d, slots, rows);
  const size_t sets = w.defer ? (size_t)slots : 1;
  w.x_sorted = take(sets * rows * d.H * es);
  w.d_out = take(sets * rows * d.H * es);
  w.dxs = take((size_t)rows * d.H * es);
  w.d_gate = (float*)take((size_t)d.T * d.k * 4);
  w.gmm = take(gmm_bwd_scratch_bytes(d, rows));
  w.row_gate = w.dg_part = nullptr;
  if (d.bf16) {
    w.row_gate = (float*)take((size_t)rows * 4);
    w.dg_part = (float*)take((size_t)rows * (d.F / 32) * 4);
  }
  w.d_h_all = w.act_all = w.wgrad = nullptr;
  w.go_all = nullptr;
  if (w.defer) {
    w.d_h_all = take(sets * rows * 2 * d.F * es);
    w.act_all = take(sets * rows * d.F * es);
    w.go_all = (int*)take(sets * (d.G_res + 1) * 4);
    w.wgrad = take(wgrad_sets_scratch_bytes(d, slots, rows));
  }
  w.bytes = off;
  return w;
}

}  // namespace

extern "C" {

int moe_layer_bwd_workspace_bytes(const moe_problem* p, int32_t mode, size_t* bytes) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (bytes == nullptr || mode < MOE_MODE_LAYER || mode > MOE_MODE_FORCE_CHUNKED)
    return MOE_EINVAL;
  const LayerPlan pl = layer_plan(d, mode);
  *bytes = carve_layer_bwd(d, layer_layout(d, mode, pl.q, nullptr), pl.rows, pl.drows,
                           nullptr).bytes;
  return MOE_OK;
}

int moe_layer_bwd(const moe_problem* p, int32_t mode, const void* x, const float* logits,
                  const void* w_gate, const void* w_up, const void* w_down, const void* dy,
                  void* dx, float* d_logits, float* dw_gate, float* dw_up, float* dw_down,
                  void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (mode < MOE_MODE_LAYER || mode > MOE_MODE_FORCE_CHUNKED) return MOE_EINVAL;
  if (!x || !logits || !w_gate || !w_up || !w_down || !dy || !dx || !d_logits || !dw_gate ||
      !dw_up || !dw_down || !ws)
    return MOE_EINVAL;
  if (misaligned(ws, 256) || misaligned(x, 16) || misaligned(dy, 16) || misaligned(dx, 16) ||
      misaligned(w_gate, 16) || misaligned(w_up, 16) || misaligned(w_down, 16) ||
      misaligned(dw_gate, 16) || misaligned(dw_up, 16) || misaligned(dw_down, 16))
    return MOE_EINVAL;
  const LayerPlan pl = layer_plan(d, mode);
  const int64_t rows = pl.rows, drows = pl.drows;
  if (!fits_rsrc(d, rows, drows)) return MOE_EUNSUPPORTED;
  const int64_t wide = d.H > 2 * d.F ? d.H : 2 * d.F;
  if (d.bf16 && rows * wide * 2 >= ((int64_t)1 << 31)) return MOE_EUNSUPPORTED;
  const int q = pl.q;
  const LayerBwdWs w0 = carve_layer_bwd(d, layer_layout(d, mode, q, nullptr), rows, drows,
                                        nullptr);
  if (ws_bytes < w0.bytes) return MOE_ECAPACITY;
  const LayerBwdWs w = carve_layer_bwd(d, layer_layout(d, mode, q, nullptr), rows, drows,
                                       (char*)ws);
  const LayerWs& f = w.fwd;
  const LayoutSet ls = layer_layout(d, mode, q, f.status + 1);
  hipStream_t s = (hipStream_t)stream;

  // the forward's routing, counts, plan, overflow flag and pass layouts,
  // recomputed from x (the pass choice stays on the device)
  hipError_t e = launch_route(d, logits, f.topk_idx, f.topk_gate,
                              count_hist_area(d, f.count_scratch), s);
  if (e != hipSuccess) return MOE_EHIP;
  const bool reroute = d.R > 0 && d.B > 0;
  const LayoutBuffers lb = carve_layout(d, ls, f.layout_scratch);
  if (!reroute && layout_fused(d)) {
    const CountArgs c = layer_count_args(d, f.topk_idx, f.expert_counts, f.slot_expert, f.ndiv,
                                         f.shard_counts, f.status, f.count_scratch, nullptr,
                                         mode);
    e = launch_layout(d, ls, f.topk_idx, 1, lb, &c, s);
    if (e != hipSuccess) return MOE_EHIP;
  } else {
    e = launch_count(d, f.topk_idx, f.expert_counts, f.slot_expert, f.ndiv,
                     reroute ? f.slot_of_assign : nullptr, f.shard_counts, f.status,
                     f.count_scratch, 1, nullptr, mode, nullptr, s);
    if (e != hipSuccess) return MOE_EHIP;
    e = launch_layout(d, ls, reroute ? f.slot_of_assign : f.topk_idx, reroute ? 0 : 1, lb,
                      nullptr, s);
    if (e != hipSuccess) return MOE_EHIP;
  }

  // per pass: x_sorted and the expert outputs recomputed ([FALLBACK] How:
  // the scan's backward recomputes each chunk), then the combine, grouped
  // GEMM and permute backward; the weight gradients are overwritten by the
  // first pass slot and accumulated by the others (a slot the device does
  // not take leaves them alone), or, deferred (defer_wgrad), taken over all
  // pass slots' rows after the loop
  const long long tk = (long long)d.T * d.k;
  const int es = d.bf16 ? 2 : 4;
  const int slots = layer_pass_slots(ls);
  for (int b = 0; b < slots; ++b) {
    PassArgs pa;
    if (ls.ovf != nullptr) {
      const int s0 = b * ls.win;
      pa = static_pass_args(s0, ls.win < d.L - s0 ? ls.win : d.L - s0, 0, b, d.L);
      pa.ovf = ls.ovf;
    } else {
      pa = static_pass(d, ls, b);
    }
    // this pass's x_sorted and d_out rows (their own per pass slot when
    // the weight gradients come at the end)
    const size_t set = w.defer ? (size_t)b : 0;
    void* xs_b = (char*)w.x_sorted + set * rows * d.H * es;
    void* dout_b = (char*)w.d_out + set * rows * d.H * es;
    e = launch_gather_rows(lb.meta, kLayoutMeta, lb.sorted_assign, tk, d.k, x, xs_b, d.H * es,
                           d.T, rows, pa, s);
    if (e != hipSuccess) return MOE_EHIP;
    // bf16: the rows go ungated (dy) with each row's gate, d_a = dy Wd is
    // ungated, and the grouped-GEMM backward's recompute applies the gate
    // and returns the gate gradients in parts, <dy Wd, act> = <dy, act Wd^T>
    // = <dy, expert output>, so no expert output is recomputed; fp32
    // recomputes the forward first
    if (!d.bf16) {
      GemmPass gp;
      memset(&gp, 0, sizeof(gp));
      gp.a_src = xs_b;
      gp.a_src_rows = (int)rows;
      gp.a_div = 1;
      gp.group_offsets = lb.group_offsets;
      gp.tile_off = lb.tile_off;
      gp.tile_group = lb.tile_group;
      gp.go_stride = d.G_res + 1;
      gp.tg_stride = tile_map_len(d);
          e = launch_gmm(d, pa, gp, f.slot_expert, w_gate, w_up, w_down, f.act, f.out, rows,
                     nullptr, s);
      if (e != hipSuccess) return MOE_EHIP;
    }
    e = launch_combine_bwd(d, pa, ls, dy, f.out, lb.row_of_assign, tk, f.topk_gate, dout_b,
                           w.d_gate, rows, d.bf16 ? 1 | 4 : 3, s, w.row_gate, nullptr);
    if (e != hipSuccess) return MOE_EHIP;
    GemmBwdArgs a;
    a.x_sorted = xs_b;
    a.group_offsets = lb.group_offsets;
    a.go_stride = d.G_res + 1;
    a.pa = pa;
    a.slot_expert = f.slot_expert;
    a.wg = w_gate;
    a.wu = w_up;
    a.wd = w_down;
    a.d_out = dout_b;
    a.dx_sorted = w.dxs;
    a.dwg = dw_gate;
    a.dwu = dw_up;
    a.dwd = dw_down;
    a.accumulate = b > 0;
    a.max_rows = rows;
    a.scratch = w.gmm;
    a.out_recompute = nullptr;
    a.row_gate = w.row_gate;
    a.dg_part = w.dg_part;
    if (w.defer) {
      a.go_out = w.go_all + set * (d.G_res + 1);
      a.d_h_ext = (char*)w.d_h_all + set * rows * 2 * d.F * es;
      a.act_ext = (char*)w.act_all + set * rows * d.F * es;
      a.wgrad = 0;
    }
    e = launch_gmm_bwd(d, a, s);
    if (e != hipSuccess) return MOE_EHIP;
    if (d.bf16) {
      e = launch_combine_bwd(d, pa, ls, dy, nullptr, lb.row_of_assign, tk, f.topk_gate, nullptr,
                             w.d_gate, rows, 2 | 8, s, nullptr, w.dg_part);
      if (e != hipSuccess) return MOE_EHIP;
    }
    e = launch_permute_bwd(d, pa, ls, w.dxs, lb.row_of_assign, tk, dx, rows, s);
    if (e != hipSuccess) return MOE_EHIP;
  }
  if (w.defer) {
    // every pass slot's weight gradients in one plan (a slot the device did
    // not take has no rows), written once
    e = launch_wgrad(d, slots, w.go_all, rows, f.slot_expert, w.d_h_all, w.x_sorted, w.d_out,
                     w.act_all, dw_gate, dw_up, dw_down, 0, w.wgrad, s);
    if (e != hipSuccess) return MOE_EHIP;
  }
  return hip_status(launch_route_bwd(d, f.topk_idx, f.topk_gate, w.d_gate, d_logits, s));
}

int moe_testing_set_gemm_wait_limit(int32_t spins) {
  set_gemm_wait_limit(spins);
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "problem outside the limits of this build";
    case MOE_ECAPACITY: return "buffer or workspace too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
