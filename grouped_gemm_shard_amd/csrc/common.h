// Internal definitions shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "moe_shard.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxSlots = 1024;     // G limit (keys of the slot sort)
constexpr int kMaxExperts = 1024;   // E limit (route keeps E/64 logits per lane)
constexpr int kMaxTopK = 32;        // one lane per chosen expert in route/combine
constexpr int kSortBlocks = 64;     // blocks of the stable counting sort
constexpr int kGemmBMMin = 128;     // smallest grouped-GEMM tile height
// Hidden sizes from which the grouped GEMM runs 256-row tiles (long
// reductions, where the taller tile halves the operand traffic per flop).
#ifndef MOE_GEMM_BIG_MIN_H
#define MOE_GEMM_BIG_MIN_H 2048
#endif
constexpr int kMaxChunks = 64;      // sequence chunks of the fallback

// Problem dimensions, derived once on the host and passed by value.
struct Dims {
  int T, L, H, F, E, k, S;
  int El;        // experts per shard
  int spd;       // slots per shard = El + B
  int G;         // all slots
  int res_lo, res_hi, S_res;
  int lo_slot;   // first resident slot
  int G_res;     // resident slots
  int e_base;    // first resident expert (global index)
  int B, R;
  int gate, bf16, dedup;
  int cap;       // ceil(factor*T*k/S), -1 when uncapped
  int n_default; // chunks of the fallback
  int gemm_bm;   // grouped-GEMM tile height (128 or 256)
};

// A pass covers the window [s0, s0 + lw) of every sequence: token t = b*L + s
// belongs to it when s0 <= s < s0 + lw.  The single pass over all tokens is
// (0, L), chunk c of n is (c*L/n, L/n), and a batch of q consecutive chunks
// is the window (c*L/n, q*L/n).  Static passes (ovf == nullptr) carry their
// window and the index j of their layout.  A dynamic pass is slot j of a
// LAYER-mode call: when *ovf is set it is batch j of the dropless chunks
// (layout 1 + j, window as given), else slot 0 runs the single pass
// (layout 0, window (0, L)) and the other slots are inactive.  Every kernel
// of a pass resolves this itself, so the host never waits for the flag.
struct PassArgs {
  int s0, lw, capped;
  const int* ovf;
  int j;
  int L;  // sequence length (window of the single pass)
};

struct PassInfo {
  int active, s0, lw, capped, j;
};

__host__ __device__ __forceinline__ PassArgs static_pass_args(int s0, int lw, int capped, int j,
                                                              int L) {
  PassArgs a;
  a.s0 = s0; a.lw = lw; a.capped = capped; a.ovf = nullptr; a.j = j; a.L = L;
  return a;
}

__device__ __forceinline__ PassInfo resolve_pass(const PassArgs& a) {
  PassInfo p;
  if (a.ovf == nullptr) {
    p.active = 1; p.s0 = a.s0; p.lw = a.lw; p.capped = a.capped; p.j = a.j;
  } else if (*a.ovf != 0) {
    p.active = 1; p.s0 = a.s0; p.lw = a.lw; p.capped = 0; p.j = 1 + a.j;
  } else {
    p.active = (a.j == 0); p.s0 = 0; p.lw = a.L; p.capped = 0; p.j = 0;
  }
  return p;
}

// The passes whose layouts are computed together: an optional single pass
// over all tokens (layout 0), then windows w_lo .. w_lo + w_cnt - 1 of
// width `win` (the last one clipped at L), in order.  The single pass's
// rows use one row_of_assign array ("set" 0) and the windows share the next
// one (their tokens are disjoint).  With `ovf` set (a LAYER-mode call) the
// device computes only the layouts the flag selects: the single pass when
// *ovf == 0, the windows otherwise.
struct LayoutSet {
  int has_single, single_capped;
  int win, w_lo, w_cnt, w_capped;
  const int* ovf;
};

__device__ __forceinline__ bool layout_live(const LayoutSet& ls, int j) {
  if (ls.ovf == nullptr) return true;
  return (ls.has_single && j == 0) ? (*ls.ovf == 0) : (*ls.ovf != 0);
}

__host__ __device__ __forceinline__ int layout_num_passes(const LayoutSet& ls) {
  return ls.has_single + ls.w_cnt;
}
__host__ __device__ __forceinline__ int layout_num_sets(const LayoutSet& ls) {
  return ls.has_single + (ls.w_cnt > 0 ? 1 : 0);
}
__host__ __device__ __forceinline__ int layout_set_of(const LayoutSet& ls, int j) {
  return (ls.has_single && j == 0) ? 0 : ls.has_single;
}
// Window of layout j; its rows and elements start at j * T*k in the
// per-element arrays (each layout gets room for all T*k assignments).
__host__ __device__ __forceinline__ void layout_pass(const Dims& d, const LayoutSet& ls, int j,
                                                     int* s0, int* lw, int* capped, size_t* e0) {
  if (ls.has_single && j == 0) {
    *s0 = 0; *lw = d.L; *capped = ls.single_capped;
  } else {
    const int w0 = (ls.w_lo + (j - ls.has_single)) * ls.win;
    *s0 = w0;
    *lw = ls.win < d.L - w0 ? ls.win : d.L - w0;
    *capped = ls.w_capped;
  }
  *e0 = (size_t)j * d.T * d.k;
}
__host__ __device__ __forceinline__ size_t layout_row_base(const Dims& d, const LayoutSet& ls, int j) {
  return (size_t)j * d.T * d.k;
}
__host__ __device__ __forceinline__ size_t layout_dedup_base(const Dims& d, const LayoutSet& ls,
                                                             int j) {
  return (size_t)j * d.T * d.k;
}
__host__ __device__ __forceinline__ size_t layout_total_elems(const Dims& d, const LayoutSet& ls) {
  return (size_t)layout_num_passes(ls) * d.T * d.k;
}
__host__ __device__ __forceinline__ size_t layout_total_dedup(const Dims& d, const LayoutSet& ls) {
  return d.dedup ? layout_total_elems(d, ls) : 1;
}
// Widest window of the set.
__host__ __device__ __forceinline__ int layout_max_lw(const Dims& d, const LayoutSet& ls) {
  if (ls.has_single) return d.L;
  return ls.win < d.L ? ls.win : d.L;
}

constexpr int kLayoutMeta = 8;  // per layout: [0] rows, [1] dedup rows

// Token of the i-th position of a pass, in ascending t = b*L + s.
__host__ __device__ __forceinline__ int window_token(int L, int s0, int lw, int i) {
  int b = i / lw;
  return b * L + s0 + (i - b * lw);
}

__device__ __forceinline__ int pass_token(const Dims& d, const PassInfo& p, int i) {
  return window_token(d.L, p.s0, p.lw, i);
}

__device__ __forceinline__ int pass_tokens(const Dims& d, const PassInfo& p) {
  return (d.T / d.L) * p.lw;
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// accesses, not for its global loads, so prefetches stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Capacity of the m-tile -> group map: rows never exceed T*k.
__host__ __device__ __forceinline__ int tile_map_len(const Dims& d) {
  return (int)(((long long)d.T * d.k) / kGemmBMMin) + d.G_res + 1;
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------
// Host-side launchers (defined in the .hip files).  Each returns hipError_t.
// ---------------------------------------------------------------------------

// Rows of the per-block expert histograms the route step can leave for the
// count step (one per route block).
__host__ __device__ __forceinline__ int route_hist_blocks(const Dims& d) {
  const int nb = (d.T + 15) / 16;  // 16 waves per block, a token per wave
  return nb < 256 ? nb : 256;
}

// Router top-k.  With ph non-null (route_hist_blocks(d) x E ints) it also
// leaves per-block expert histograms for launch_count.
// zero / zero_n: ints the route launch also clears (counters that later
// launches of the same call expect at zero), or none.
hipError_t launch_route(const Dims& d, const float* logits, int* idx, float* gate, int* ph,
                        hipStream_t s, int* zero = nullptr, int zero_n = 0);

// Scratch of the count step: per-block expert histograms and error flags,
// and for rerouting kSortBlocks*R ints of block histograms and T*k packed
// keys.
size_t count_scratch_bytes(const Dims& d);
// The per-block histogram area of the count scratch (route may fill it).
int* count_hist_area(const Dims& d, void* scratch);
// Counts, plan, slots, shard counts and the overflow check from the top-k.
// hist_ready: the route step already left its histograms in the scratch.
// Without rerouting (R == 0 or B == 0) slot_of_assign may be null: every
// assignment then goes to its expert's home slot.
hipError_t launch_count(const Dims& d, const int* idx, int* expert_counts, int* slot_expert,
                        int* ndiv, int* slot_of_assign, int* shard_counts, int* status,
                        void* scratch, int hist_ready, int* info_out, int info_mode,
                        float* rfactor, hipStream_t s);

// Arguments of the count step without rerouting (one workgroup): the top-k,
// per-block expert histograms ph [nb][E] (pbad: per-block bad-id flags, or
// null), and its outputs.
struct CountArgs {
  const int* idx;
  const int* ph;
  const int* pbad;
  int nb;
  int* expert_counts;
  int* slot_expert;
  int* ndiv;
  int* slot_of_assign;  // may be null
  int* shard_counts;
  int* status;
  int* info;            // may be null
  int info_mode;
  float* rfactor;       // may be null
};
// The CountArgs of a layer call whose route step left its histograms in the
// count scratch.
CountArgs layer_count_args(const Dims& d, const int* idx, int* expert_counts, int* slot_expert,
                           int* ndiv, int* shard_counts, int* status, void* scratch, int* info,
                           int info_mode);

// Layout state of every pass of a LayoutSet (arrays are per layout j with
// the strides used by the kernels below).
struct LayoutBuffers {
  unsigned* skey;       // [elems] packed slot key / local rank
  unsigned* dkey;       // [elems] packed dedup key / local rank
  int* bh_slot;         // [np][kSortBlocks][G_res] block counts -> bases
  int* bh_dedup;        // [np][kSortBlocks][S_res]
  int* kept;            // [np][G_res] kept rows per slot
  int* dedup_kept;      // [np][S_res]
  int* group_offsets;   // [np][G_res + 1]
  int* tile_off;        // [np][G_res + 1] m-tile prefix (tile height gemm_bm)
  int* tile_group;      // [np][tile_map_len] group of every m-tile
  int* dedup_offsets;   // [np][S_res + 1]
  int* meta;            // [np][kLayoutMeta]
  int* row_of_assign;   // [sets][T*k]
  int* sorted_assign;   // [elems] rows of layout j start at its first element
  int* expand_idx;      // [elems]
  int* dedup_token;     // [elems] (dedup only)
};
size_t layout_scratch_bytes(const Dims& d, const LayoutSet& ls);
LayoutBuffers carve_layout(const Dims& d, const LayoutSet& ls, void* scratch);
// slots: slot_of_assign [T*k], or with home != 0 the top-k expert ids, each
// assignment then going to its expert's home slot (no rerouting).
// Layouts without dedup and with at most kFusedBases / kSortBlocks resident
// slots take two launches: local ranks, then scan and placement together.
constexpr int kFusedBases = 8192;
bool layout_fused(const Dims& d);
// cnt (no rerouting, and layout_fused; may be null otherwise): the count
// step runs inside the layout, in one extra workgroup of the scan/place
// launch, and every candidate pass is laid out, so the layout does not wait
// for the overflow flag.
hipError_t launch_layout(const Dims& d, const LayoutSet& ls, const int* slots, int home,
                         const LayoutBuffers& lb, const CountArgs* cnt, hipStream_t s);

// dst[r] = src[index[r] / div] for r < *count, per pass: count, index are
// base pointers advanced by count_stride / index_stride per layout j.
// The standalone permute of a single small pass without dedup in one
// launch (layout and x_sorted); hipErrorNotSupported where it does not
// apply.
hipError_t launch_permute_one(const Dims& d, const LayoutSet& ls, const int* soa,
                              const LayoutBuffers& lb, const void* x, void* x_sorted,
                              int row_bytes, int64_t max_rows, hipStream_t s);
hipError_t launch_gather_rows(const int* count, int count_stride, const int* index,
                              long long index_stride, int div, const void* src, void* dst,
                              int row_bytes, int src_rows, int64_t max_rows, const PassArgs& pa,
                              hipStream_t s);

// Grouped GEMM of one pass.  GEMM1 reads its rows through a_index when it
// is non-null (row n of the pass = src[a_index[n] / a_div]), else rows are
// contiguous in x_sorted.  Per-pass arrays advance by the given strides per
// layout j; tile_off / tile_group may be null, and are then computed into
// scratch from group_offsets.
struct GemmPass {
  const void* a_src;      // GEMM1 row source: x, x_dedup or x_sorted
  int a_src_rows;         // rows of a_src (bounds of the gather)
  const int* a_index;     // per-row source index or null
  long long a_index_stride;
  int a_div;
  const int* group_offsets;
  const int* tile_off;
  const int* tile_group;
  int go_stride, tg_stride;
  int* err;               // MOE_ERR_* bits of the GEMM are OR-ed into *err (may be null)
  int* sync;              // bf16: counters of the one-launch GEMM1+GEMM2 kernel
                          // (gmm_sync_bytes), zeroed by an earlier launch of the
                          // call; null: in scratch (zeroed with the tile map) when
                          // tile_off is null, else two launches
};
size_t gmm_scratch_bytes(const Dims& d);
// bf16 C = A B^T over one pass's groups with the forward's second-GEMM
// kernel: A [rows, K] in row order, B [e_res][N][K], C [rows, N]; scratch of
// gmm_scratch_bytes(d) for the tile map.  hipErrorNotSupported for fp32 or
// when K is not a multiple of the kernel's reduction step or N of 256.
hipError_t launch_gmm_plain(const Dims& d, const int* group_offsets, const int* slot_expert,
                            const void* A, int64_t a_rows, const void* B, size_t b_stride, int K,
                            int N, void* C, int64_t max_rows, void* scratch, hipStream_t s);
// bf16 with 256-row tiles: C = A B over one pass's groups on the forward's
// 256-row kernel with B stored reduction-major: rows [0, k_split) of the
// reduction from B0 [e_res][k_split][N] (experts b_stride apart), the rest
// from B1 [e_res][K - k_split][N]; hipErrorNotSupported otherwise.
hipError_t launch_gmm_plain_kmajor(const Dims& d, const int* group_offsets,
                                   const int* slot_expert, const void* A, int64_t a_rows,
                                   const void* B0, const void* B1, int k_split, size_t b_stride,
                                   int K, int N, void* C, int64_t max_rows, void* scratch,
                                   hipStream_t s);
// bf16: the backward's gate/up recompute on the forward's first-GEMM kernel
// with the SwiGLU backward in its epilogue: act and d_h = (d_hg | d_hu)
// [rows, 2F] of x_sorted [rows, H] and d_a [rows, F]; scratch as above.
hipError_t launch_gmm_swiglu_recompute(const Dims& d, const int* group_offsets,
                                       const int* slot_expert, const void* x_sorted,
                                       int64_t a_rows, const void* wg, const void* wu,
                                       const void* d_a, void* d_h, void* act, int64_t max_rows,
                                       void* scratch, hipStream_t s,
                                       const float* row_gate = nullptr, float* dg_part = nullptr);
size_t gmm_sync_bytes(const Dims& d);
int gmm_sync_ints(const Dims& d);  // ints of gmm_sync_bytes the kernel expects at zero

// A second stream per device (default priority), with the events that fork
// work onto it from a caller's stream and join it back.  Whoever enqueues
// work on it holds side_mutex() from the fork to the join, so concurrent
// callers cannot interleave their fork/join records.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false;
};
SideStream* side_stream();
std::mutex& side_mutex();
// Bound of the grouped GEMM's wait for rows another tile of the same launch
// produces, in sleeps; < 0 makes every such wait give up at once (tests of
// the MOE_ERR_GEMM_WAIT path).
int gemm_wait_limit();
void set_gemm_wait_limit(int spins);  // 0 restores the default
hipError_t launch_gmm(const Dims& d, const PassArgs& pa, const GemmPass& gp,
                      const int* slot_expert, const void* wg, const void* wu, const void* wd,
                      void* act, void* out, int64_t max_rows, void* scratch, hipStream_t s);

// Combine of one pass; row_of_assign advances by roa_stride per row_of_assign
// set of the pass's layout.  Rows at or past max_rows are treated as absent.
// Return-path dedup: partial[u] for u < *u_count (one row per token and
// resident shard; rows of expert_out at or past max_rows count as absent),
// and y of the pass's tokens from those rows.
hipError_t launch_combine_partial(const Dims& d, const int* u_count, const int* dedup_token,
                                  const int* row_of_assign, const int* expand_idx,
                                  const float* gate, const void* out, int64_t max_rows,
                                  int64_t max_urows, void* partial, hipStream_t s);
hipError_t launch_combine_from_partials(const Dims& d, const PassArgs& pa,
                                        const int* row_of_assign, const int* expand_idx,
                                        const void* partial, int64_t max_rows, int64_t max_urows,
                                        void* y, hipStream_t s);
hipError_t launch_combine(const Dims& d, const PassArgs& pa, const LayoutSet& ls, const void* out,
                          const int* row_of_assign, long long roa_stride, int64_t max_rows,
                          const float* gate, void* y, hipStream_t s);

// ---- backward ---------------------------------------------------------------

// Grouped-GEMM backward of one pass.  Weight gradients are float32,
// overwritten or (accumulate) added to.  scratch holds
// gmm_bwd_scratch_bytes(d, max_rows).
struct GemmBwdArgs {
  const void* x_sorted;
  const int* group_offsets;  // of layout pa's j, go_stride ints per layout
  int go_stride;
  PassArgs pa;
  const int* slot_expert;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* d_out;
  void* dx_sorted;
  float* dwg;
  float* dwu;
  float* dwd;
  int accumulate;
  int64_t max_rows;
  void* scratch;
  void* out_recompute;  // bf16: if set, expert outputs from the recomputed activation
  // bf16, a layer call taking every pass's weight gradients at the end: the
  // pass's group offsets, d_h [rows, 2F] and act [rows, F] go to these
  // buffers instead of the scratch, and wgrad = 0 skips the pass's weight
  // gradients (launch_wgrad over all passes follows)
  int* go_out = nullptr;
  void* d_h_ext = nullptr;
  void* act_ext = nullptr;
  int wgrad = 1;
  // bf16, the layer call's gated mode: d_out holds the ungated rows dy (so
  // d_a = dy Wd is ungated), row_gate [rows] each row's gate; the recompute
  // applies the gate, stores gate * act as the activation (dWd = dy^T
  // (gate act)) and writes the gate-gradient parts dg_part [rows, F/32]
  const float* row_gate = nullptr;
  float* dg_part = nullptr;
};
size_t gmm_bwd_scratch_bytes(const Dims& d, int64_t max_rows);
hipError_t launch_gmm_bwd(const Dims& d, const GemmBwdArgs& a, hipStream_t s);
// bf16 weight gradients over `sets` row sets of `rows` rows each (set s's
// group offsets at group_offsets + s (G_res + 1), its rows at s * rows of
// d_h [., 2F], x_sorted [., H], d_out [., H] and act [., F]); at most
// kMaxSlots groups in all.  Scratch: wgrad_sets_scratch_bytes.
size_t wgrad_sets_scratch_bytes(const Dims& d, int sets, int64_t rows_per_set);
hipError_t launch_wgrad(const Dims& d, int sets, const int* group_offsets, int64_t rows,
                        const int* slot_expert, const void* d_h, const void* x_sorted,
                        const void* d_out, const void* act, float* dwg, float* dwu, float* dwd,
                        int accumulate, void* scratch, hipStream_t s);
// Combine / permute backward of a pass; row_of_assign advances by
// roa_stride per row_of_assign set of the pass's layout (as launch_combine).
// what: bit 0 the rows g * dy into d_out, bit 1 the gate gradients <dy, out>
// (reads out); bit 2 (with bit 0) the rows dy ungated and each row's gate
// into row_gate; bit 3 (with bit 1) the gate gradients as the sum of the
// row's parts dg_part [rows, F/32] instead of reading out.
hipError_t launch_combine_bwd(const Dims& d, const PassArgs& pa, const LayoutSet& ls,
                              const void* dy, const void* out, const int* roa,
                              long long roa_stride, const float* gate, void* d_out,
                              float* d_gate, int64_t max_rows, int what, hipStream_t s,
                              float* row_gate = nullptr, const float* dg_part = nullptr);
hipError_t launch_permute_bwd(const Dims& d, const PassArgs& pa, const LayoutSet& ls,
                              const void* dxs, const int* roa, long long roa_stride, void* dx,
                              int64_t max_rows, hipStream_t s);
hipError_t launch_route_bwd(const Dims& d, const int* idx, const float* gate,
                            const float* d_gate, float* d_logits, hipStream_t s);

}  // namespace moe
