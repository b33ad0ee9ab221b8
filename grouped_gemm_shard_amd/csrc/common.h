// Internal definitions shared by the HIP kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
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

// One pass of the permute / GEMM / combine sequence.  Static passes carry
// (n, c, capped) directly.  A dynamic pass (ovf != nullptr) is one of the
// LAYER-mode passes: when *ovf is set it is chunk c of n, dropless; else
// pass 0 covers every token with the capped buffer and passes c > 0 are
// inactive.  Every kernel of a pass resolves this itself, so the host never
// waits for the overflow flag.
struct PassArgs {
  int n, c, capped;
  const int* ovf;
};

struct PassInfo {
  int active, n, c, capped;
};

__device__ __forceinline__ PassInfo resolve_pass(const PassArgs& a) {
  PassInfo p;
  if (a.ovf == nullptr) {
    p.active = 1; p.n = a.n; p.c = a.c; p.capped = a.capped;
  } else if (*a.ovf != 0) {
    p.active = 1; p.n = a.n; p.c = a.c; p.capped = 0;
  } else {
    p.active = (a.c == 0); p.n = 1; p.c = 0; p.capped = 1;
  }
  return p;
}

// Token of the i-th position of a pass: chunk c of n holds s in
// [c*L/n, (c+1)*L/n) of every sequence b, in ascending t = b*L + s.
__device__ __forceinline__ int pass_token(const Dims& d, const PassInfo& p, int i) {
  int lc = d.L / p.n;
  int b = i / lc;
  return b * d.L + p.c * lc + (i - b * lc);
}

__device__ __forceinline__ int pass_tokens(const Dims& d, const PassInfo& p) {
  return d.T / p.n;
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

hipError_t launch_route(const Dims& d, const float* logits, int* idx, float* gate,
                        hipStream_t s);

// Scratch of the count step: kSortBlocks*R ints of block histograms and T*k
// packed keys.
size_t count_scratch_bytes(const Dims& d);
hipError_t launch_count(const Dims& d, const int* idx, int* expert_counts, int* slot_expert,
                        int* ndiv, int* slot_of_assign, int* shard_counts, int* status,
                        void* scratch, int* info_out, int info_mode, hipStream_t s);

// Per-pass layout state carved from the workspace.
struct PassBuffers {
  unsigned* skey;      // [T*k] packed slot key / local rank
  unsigned* dkey;      // [T*k] packed dedup key / local rank
  int* bh_slot;        // [kSortBlocks * G_res] block counts -> bases
  int* bh_dedup;       // [kSortBlocks * S_res]
  int* kept;           // [G_res] kept rows per slot
  int* dedup_kept;     // [S_res]
  int* tile_off;       // [G_res + 1] m-tile prefix (tile height gemm_bm)
  int* tile_group;     // [tile_map_len] group of every m-tile
  int* meta;           // [8]: rows, dedup rows, ...
};
size_t pass_scratch_bytes(const Dims& d);
PassBuffers carve_pass(const Dims& d, void* scratch);

hipError_t launch_permute(const Dims& d, const PassArgs& pa, const void* x,
                          const int* slot_of_assign, const PassBuffers& pb,
                          int* group_offsets, int* row_of_assign, int* sorted_assign,
                          int* dedup_offsets, int* dedup_token, int* expand_idx,
                          void* x_dedup, void* x_sorted, hipStream_t s);

// Grouped GEMM.  tile_off / tile_group may be null: they are then computed
// into scratch from group_offsets.
size_t gmm_scratch_bytes(const Dims& d);
hipError_t launch_gmm(const Dims& d, const PassArgs& pa, const void* x_sorted,
                      const int* group_offsets, const int* tile_off, const int* tile_group,
                      const int* slot_expert,
                      const void* wg, const void* wu, const void* wd, void* act, void* out,
                      int64_t max_rows, void* scratch, hipStream_t s);

hipError_t launch_combine(const Dims& d, const PassArgs& pa, const void* out,
                          const int* row_of_assign, const float* gate, void* y,
                          hipStream_t s);

}  // namespace moe
