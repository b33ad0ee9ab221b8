// C ABI of the one-shard MoE layer: argument validation, buffer bounds,
// workspace layout and the order of launches.  Every entry point validates
// on the host and returns a moe_status before launching anything.
#include <math.h>
#include <string.h>

#include "common.h"
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
  // "8x for EP16 / factor 2")
  int n = p->num_chunks;
  if (n == 0) n = f > 0.0 ? (int)ceil((double)d->S / f) : 1;
  if (n < 1 || n > d->L || d->L % n != 0) return MOE_EINVAL;
  d->n_default = n;
  // tall tiles halve the operand traffic per flop where the reduction is
  // long; short ones waste less on small groups
  d->gemm_bm = d->H >= 2048 ? 256 : 128;
  return MOE_OK;
}

// Row bounds of a pass of n chunks, capped or not.
void pass_bounds(const Dims& d, int n, int capped, int64_t* rows, int64_t* drows) {
  const int64_t tc = d.T / n;
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

size_t step_scratch(const Dims& d) {
  size_t a = count_scratch_bytes(d), b = pass_scratch_bytes(d), c = gmm_scratch_bytes(d);
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
  void* pass_scratch;
  int* group_offsets;
  int* row_of_assign;
  int* sorted_assign;
  int* dedup_offsets;
  int* dedup_token;
  int* expand_idx;
  void* x_dedup;
  void* x_sorted;
  void* act;
  void* out;
  size_t bytes;
};

LayerWs carve_layer(const Dims& d, int64_t rows, int64_t drows, char* base) {
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
  w.pass_scratch = take(pass_scratch_bytes(d));
  w.group_offsets = (int*)take((size_t)(d.G_res + 1) * 4);
  w.row_of_assign = (int*)take(tk * 4);
  w.sorted_assign = (int*)take((size_t)rows * 4);
  w.dedup_offsets = (int*)take((size_t)(d.S_res + 1) * 4);
  w.dedup_token = (int*)take((size_t)drows * 4);
  w.expand_idx = (int*)take((size_t)rows * 4);
  w.x_dedup = take((size_t)drows * d.H * es);
  w.x_sorted = take((size_t)rows * d.H * es);
  w.act = take((size_t)rows * d.F * es);
  w.out = take((size_t)rows * d.H * es);
  w.bytes = off;
  return w;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

int run_pass(const Dims& d, const PassArgs& pa, const void* x, const void* wg, const void* wu,
             const void* wd, void* y, const LayerWs& w, int64_t rows, hipStream_t s) {
  PassBuffers pb = carve_pass(d, w.pass_scratch);
  hipError_t e = launch_permute(d, pa, x, w.slot_of_assign, pb, w.group_offsets, w.row_of_assign,
                                w.sorted_assign, w.dedup_offsets, w.dedup_token, w.expand_idx,
                                w.x_dedup, w.x_sorted, s);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_gmm(d, pa, w.x_sorted, w.group_offsets, pb.tile_off, pb.tile_group, w.slot_expert,
                 wg, wu, wd, w.act, w.out, rows, nullptr, s);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_combine(d, pa, w.out, w.row_of_assign, w.topk_gate, y, s);
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
  int64_t rows, drows;
  layer_bounds(d, mode, &rows, &drows);
  *bytes = carve_layer(d, rows, drows, nullptr).bytes;
  return MOE_OK;
}

int moe_route(const moe_problem* p, const float* logits, int32_t* topk_idx, float* topk_gate,
              void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_gate) return MOE_EINVAL;
  return hip_status(launch_route(d, logits, topk_idx, topk_gate, (hipStream_t)stream));
}

int moe_count_overflow(const moe_problem* p, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* slot_expert, int32_t* ndiv, int32_t* slot_of_assign,
                       int32_t* shard_counts, int32_t* status, void* ws, size_t ws_bytes,
                       void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!topk_idx || !expert_counts || !slot_expert || !ndiv || !slot_of_assign || !shard_counts ||
      !status || !ws)
    return MOE_EINVAL;
  if (misaligned(ws, 256)) return MOE_EINVAL;
  if (ws_bytes < count_scratch_bytes(d)) return MOE_ECAPACITY;
  return hip_status(launch_count(d, topk_idx, expert_counts, slot_expert, ndiv, slot_of_assign,
                                 shard_counts, status, ws, nullptr, 0, (hipStream_t)stream));
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
  if (ws_bytes < pass_scratch_bytes(d)) return MOE_ECAPACITY;
  PassArgs pa{num_chunks, chunk, capped, nullptr};
  PassBuffers pb = carve_pass(d, ws);
  return hip_status(launch_permute(d, pa, x, slot_of_assign, pb, group_offsets, row_of_assign,
                                   sorted_assign, dedup_offsets, dedup_token, expand_idx, x_dedup,
                                   x_sorted, (hipStream_t)stream));
}

int moe_gmm_swiglu(const moe_problem* p, const void* x_sorted, const int32_t* group_offsets,
                   const int32_t* slot_expert, const void* w_gate, const void* w_up,
                   const void* w_down, void* act, void* expert_out, int64_t max_rows, void* ws,
                   size_t ws_bytes, void* stream) {
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
  PassArgs pa{1, 0, 0, nullptr};
  return hip_status(launch_gmm(d, pa, x_sorted, group_offsets, nullptr, nullptr, slot_expert,
                               w_gate, w_up, w_down, act, expert_out, max_rows, ws,
                               (hipStream_t)stream));
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
  PassArgs pa{num_chunks, chunk, 0, nullptr};
  return hip_status(
      launch_combine(d, pa, expert_out, row_of_assign, topk_gate, y, (hipStream_t)stream));
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
  int64_t rows, drows;
  layer_bounds(d, mode, &rows, &drows);
  LayerWs w = carve_layer(d, rows, drows, (char*)ws);
  if (ws_bytes < w.bytes) return MOE_ECAPACITY;
  hipStream_t s = (hipStream_t)stream;

  hipError_t e = launch_route(d, logits, w.topk_idx, w.topk_gate, s);
  if (e != hipSuccess) return MOE_EHIP;
  e = launch_count(d, w.topk_idx, w.expert_counts, w.slot_expert, w.ndiv, w.slot_of_assign,
                   w.shard_counts, w.status, w.count_scratch, info, mode, s);
  if (e != hipSuccess) return MOE_EHIP;

  const int n = d.n_default;
  if (mode == MOE_MODE_LAYER && d.cap >= 0) {
    // the device decides: capped pass 0 alone, or n dropless chunks
    for (int c = 0; c < n; ++c) {
      PassArgs pa{n, c, 1, w.status + 1};
      st = run_pass(d, pa, x, w_gate, w_up, w_down, y, w, rows, s);
      if (st != MOE_OK) return st;
    }
  } else if (mode == MOE_MODE_FORCE_CHUNKED) {
    for (int c = 0; c < n; ++c) {
      PassArgs pa{n, c, 0, nullptr};
      st = run_pass(d, pa, x, w_gate, w_up, w_down, y, w, rows, s);
      if (st != MOE_OK) return st;
    }
  } else {
    int capped = (mode == MOE_MODE_CAPPED_ONLY) ? 1 : 0;
    PassArgs pa{1, 0, capped, nullptr};
    st = run_pass(d, pa, x, w_gate, w_up, w_down, y, w, rows, s);
    if (st != MOE_OK) return st;
  }
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
