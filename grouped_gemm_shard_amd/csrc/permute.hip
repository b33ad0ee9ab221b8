// a4 + a5: layout and permute of one pass.
//
// Rows of a pass are its assignments on resident slots in stable (slot, t,
// j) order: the expert-sorted MoE input ("MoE ring-of-experts: TC Pallas
// ring all-gather for the combine backward + x_sorted remat save", section
// What).  With a capped buffer each resident shard keeps its first `cap`
// rows ("Support moe_dropless_fallback=layer on the ragged all-to-all MoE
// path", section Why: rows beyond the cap are dropped).  With dedup a token
// is stored once per destination shard and re-expanded ("Moe dynamic
// redundancy", code review: dedup and expand_indices), and the buffer is
// never truncated below the exact count (the same review's truncation
// comment).
//
// Kernels of a pass: local ranks (one wave per sort block), one scan block
// (bases, group offsets, kept rows, GEMM tile schedule), then scatter-copies
// of whole rows with 16-byte vector loads and stores, one wave per row.
#include "sort.h"

namespace moe {

namespace {

__device__ __forceinline__ int slot_key(const Dims& d, int s) {
  return (s >= d.lo_slot && s < d.lo_slot + d.G_res) ? s - d.lo_slot : -1;
}

// First assignment j' <= j of the token on the same shard as slot s.
__device__ __forceinline__ int first_on_shard(const Dims& d, const int* row, int j, int s) {
  int sh = s / d.spd;
  for (int jj = 0; jj < j; ++jj) {
    int s2 = row[jj];
    if (s2 >= 0 && s2 / d.spd == sh) return jj;
  }
  return j;
}

// Dedup key: local resident shard of the token's first assignment on it.
__device__ __forceinline__ int dedup_key(const Dims& d, const int* row, int j) {
  int s = row[j];
  if (slot_key(d, s) < 0) return -1;
  if (first_on_shard(d, row, j, s) != j) return -1;
  return s / d.spd - d.res_lo;
}

// Rank of element e in its dedup shard (relative to the shard start).
__device__ __forceinline__ int dedup_rank(const Dims& d, const unsigned* dkey, const int* bh_dedup,
                                          int blk, int e, int* key_out) {
  unsigned v = dkey[e];
  int kd = packed_key(v);
  *key_out = kd;
  return bh_dedup[(e / blk) * d.S_res + kd] + packed_rank(v);
}

template <int WHICH>  // bit 0: slot keys, bit 1: dedup keys
__global__ __launch_bounds__(64) void pass_local_kernel(Dims d, PassArgs pa,
                                                        const int* __restrict__ soa,
                                                        unsigned* skey, unsigned* dkey,
                                                        int* bh_slot, int* bh_dedup,
                                                        int drop_check) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  __shared__ int run_s[kMaxSlots];
  __shared__ int run_d[kMaxSlots];
  const int n = pass_tokens(d, pi) * d.k;
  const int blk = sort_block_len(n);
  const int e0 = blockIdx.x * blk, e1 = min(n, e0 + blk);
  const int nb_s = key_bits(d.G_res), nb_d = key_bits(d.S_res);
  for (int q = threadIdx.x; q < d.G_res; q += 64) run_s[q] = 0;
  for (int q = threadIdx.x; q < d.S_res; q += 64) run_d[q] = 0;
  __syncthreads();
  for (int base = e0; base < e1; base += 64) {
    const int e = base + lane_id();
    const bool in = e < e1;
    int i = 0, j = 0;
    const int* row = soa;
    if (in) {
      i = e / d.k;
      j = e - i * d.k;
      row = soa + (size_t)pass_token(d, pi, i) * d.k;
    }
    if (WHICH & 1) {
      int ks = in ? slot_key(d, row[j]) : -1;
      if (drop_check && ks >= 0) {
        // the token was cut from this shard's dedup buffer: drop the row
        int jr = first_on_shard(d, row, j, row[j]);
        int kd;
        int r = dedup_rank(d, dkey, bh_dedup, blk, i * d.k + jr, &kd);
        if (r >= d.cap) ks = -1;
      }
      int r = wave_rank_step(ks, nb_s, run_s);
      if (in) skey[e] = pack_key(ks, r);
    }
    if (WHICH & 2) {
      int kd = in ? dedup_key(d, row, j) : -1;
      int r = wave_rank_step(kd, nb_d, run_d);
      if (in) dkey[e] = pack_key(kd, r);
    }
  }
  __syncthreads();
  if (WHICH & 1)
    for (int q = threadIdx.x; q < d.G_res; q += 64) bh_slot[blockIdx.x * d.G_res + q] = run_s[q];
  if (WHICH & 2)
    for (int q = threadIdx.x; q < d.S_res; q += 64) bh_dedup[blockIdx.x * d.S_res + q] = run_d[q];
}

// Scan block.  Slot part: block bases, rows per slot, kept rows (without
// dedup, a capped shard keeps the first `cap` rows of its bucket, i.e. a
// prefix of each slot), group offsets, GEMM m-tile offsets.  Dedup part:
// distinct tokens per shard, cut at the cap when capped, and their offsets.
__global__ __launch_bounds__(1024) void pass_scan_kernel(Dims d, PassArgs pa, int which,
                                                         int* bh_slot, int* bh_dedup, int* kept,
                                                         int* group_offsets, int* tile_off,
                                                         int* tile_group, int* dedup_kept,
                                                         int* dedup_offsets, int* meta) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  __shared__ int tmp[16];
  __shared__ int excl[kMaxSlots];
  __shared__ int totals[kMaxSlots];
  __shared__ int dtotals[kMaxSlots];
  const bool capped = pi.capped && d.cap >= 0;
  const int g = threadIdx.x;
  if (which & 1) scan_keys_over_blocks(bh_slot, d.G_res, totals);
  if (which & 2) scan_keys_over_blocks(bh_dedup, d.S_res, dtotals);
  __syncthreads();
  if (which & 1) {
    const bool own = g < d.G_res;
    int tot = own ? totals[g] : 0;
    int all;
    int ex = block_exscan_1024(tot, tmp, &all);
    if (own) excl[g] = ex;
    __syncthreads();
    int kp = tot;
    if (own && capped && !d.dedup) {
      int first = ((g + d.lo_slot) / d.spd) * d.spd - d.lo_slot;
      int bstart = ex - excl[first];
      kp = min(max(d.cap - bstart, 0), tot);
    }
    if (own) kept[g] = kp;
    int nrows;
    int off = block_exscan_1024(own ? kp : 0, tmp, &nrows);
    if (own) group_offsets[g] = off;
    int ntiles;
    const int tiles = own ? (kp + d.gemm_bm - 1) / d.gemm_bm : 0;
    int toff = block_exscan_1024(tiles, tmp, &ntiles);
    if (own) {
      tile_off[g] = toff;
      for (int m = 0; m < tiles; ++m) tile_group[toff + m] = g;
    }
    if (g == 0) {
      group_offsets[d.G_res] = nrows;
      tile_off[d.G_res] = ntiles;
      meta[0] = nrows;
    }
  }
  if (which & 2) {
    const bool own = g < d.S_res;
    int u = own ? dtotals[g] : 0;
    int ku = capped ? min(u, d.cap) : u;
    if (own) dedup_kept[g] = ku;
    int nu;
    int off = block_exscan_1024(own ? ku : 0, tmp, &nu);
    if (own) dedup_offsets[g] = off;
    if (g == 0) {
      dedup_offsets[d.S_res] = nu;
      meta[1] = nu;
    }
  }
}

// Copies one row of `nbytes` (a multiple of 16) with the whole wavefront.
__device__ __forceinline__ void wave_copy_row(char* __restrict__ dst, const char* __restrict__ src,
                                              int nbytes) {
  int off = lane_id() * 16;
  for (; off + 3 * 1024 < nbytes; off += 4 * 1024) {
    uint4 v0 = *(const uint4*)(src + off);
    uint4 v1 = *(const uint4*)(src + off + 1024);
    uint4 v2 = *(const uint4*)(src + off + 2048);
    uint4 v3 = *(const uint4*)(src + off + 3072);
    *(uint4*)(dst + off) = v0;
    *(uint4*)(dst + off + 1024) = v1;
    *(uint4*)(dst + off + 2048) = v2;
    *(uint4*)(dst + off + 3072) = v3;
  }
  for (; off < nbytes; off += 1024) *(uint4*)(dst + off) = *(const uint4*)(src + off);
}

__global__ __launch_bounds__(256) void dedup_scatter_kernel(Dims d, PassArgs pa,
                                                            const unsigned* __restrict__ dkey,
                                                            const int* __restrict__ bh_dedup,
                                                            const int* __restrict__ dedup_kept,
                                                            const int* __restrict__ dedup_offsets,
                                                            const char* __restrict__ x,
                                                            int* dedup_token, char* x_dedup) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int n = pass_tokens(d, pi) * d.k;
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (e >= n) return;
  const int blk = sort_block_len(n);
  if (packed_key(dkey[e]) < 0) return;
  int kd;
  int r = dedup_rank(d, dkey, bh_dedup, blk, e, &kd);
  if (r >= dedup_kept[kd]) return;
  const int dpos = dedup_offsets[kd] + r;
  const int t = pass_token(d, pi, e / d.k);
  if (lane_id() == 0) dedup_token[dpos] = t;
  const int rb = d.H * (d.bf16 ? 2 : 4);
  wave_copy_row(x_dedup + (size_t)dpos * rb, x + (size_t)t * rb, rb);
}

__global__ __launch_bounds__(256) void row_scatter_kernel(Dims d, PassArgs pa,
                                                          const int* __restrict__ soa,
                                                          const unsigned* __restrict__ skey,
                                                          const unsigned* __restrict__ dkey,
                                                          const int* __restrict__ bh_slot,
                                                          const int* __restrict__ bh_dedup,
                                                          const int* __restrict__ kept,
                                                          const int* __restrict__ group_offsets,
                                                          const int* __restrict__ dedup_offsets,
                                                          const char* __restrict__ src_x,
                                                          const char* __restrict__ x_dedup,
                                                          int* row_of_assign, int* sorted_assign,
                                                          int* expand_idx, char* x_sorted) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int n = pass_tokens(d, pi) * d.k;
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (e >= n) return;
  const int blk = sort_block_len(n);
  const int i = e / d.k, j = e - i * d.k;
  const int t = pass_token(d, pi, i);
  const int a = t * d.k + j;
  unsigned v = skey[e];
  int ks = packed_key(v);
  int pos = -1;
  if (ks >= 0) {
    int r = bh_slot[(e / blk) * d.G_res + ks] + packed_rank(v);
    if (r < kept[ks]) pos = group_offsets[ks] + r;
  }
  if (lane_id() == 0) row_of_assign[a] = pos;
  if (pos < 0) return;
  if (lane_id() == 0) sorted_assign[pos] = a;
  const int rb = d.H * (d.bf16 ? 2 : 4);
  const char* src;
  if (d.dedup) {
    const int* row = soa + (size_t)t * d.k;
    int jr = first_on_shard(d, row, j, row[j]);
    int kd;
    int r = dedup_rank(d, dkey, bh_dedup, blk, i * d.k + jr, &kd);
    int dpos = dedup_offsets[kd] + r;
    if (lane_id() == 0) expand_idx[pos] = dpos;
    src = x_dedup + (size_t)dpos * rb;
  } else {
    src = src_x + (size_t)t * rb;
  }
  wave_copy_row(x_sorted + (size_t)pos * rb, src, rb);
}

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t pass_scratch_bytes(const Dims& d) {
  size_t n = (size_t)d.T * d.k;
  return al256(n * 4) * 2 + al256((size_t)kSortBlocks * d.G_res * 4) +
         al256((size_t)kSortBlocks * d.S_res * 4) + al256((size_t)d.G_res * 4) +
         al256((size_t)d.S_res * 4) + al256((size_t)(d.G_res + 1) * 4) +
         al256((size_t)tile_map_len(d) * 4) + al256(8 * 4);
}

PassBuffers carve_pass(const Dims& d, void* scratch) {
  size_t n = (size_t)d.T * d.k;
  char* p = (char*)scratch;
  PassBuffers b;
  b.skey = (unsigned*)p;       p += al256(n * 4);
  b.dkey = (unsigned*)p;       p += al256(n * 4);
  b.bh_slot = (int*)p;         p += al256((size_t)kSortBlocks * d.G_res * 4);
  b.bh_dedup = (int*)p;        p += al256((size_t)kSortBlocks * d.S_res * 4);
  b.kept = (int*)p;            p += al256((size_t)d.G_res * 4);
  b.dedup_kept = (int*)p;      p += al256((size_t)d.S_res * 4);
  b.tile_off = (int*)p;        p += al256((size_t)(d.G_res + 1) * 4);
  b.tile_group = (int*)p;      p += al256((size_t)tile_map_len(d) * 4);
  b.meta = (int*)p;
  return b;
}

hipError_t launch_permute(const Dims& d, const PassArgs& pa, const void* x,
                          const int* soa, const PassBuffers& pb, int* group_offsets,
                          int* row_of_assign, int* sorted_assign, int* dedup_offsets,
                          int* dedup_token, int* expand_idx, void* x_dedup, void* x_sorted,
                          hipStream_t s) {
  // Elements of the largest pass this call can take (the grid is sized for
  // it; kernels of a smaller pass stop at their own count).
  const int nmax = (d.T / (pa.ovf != nullptr ? 1 : pa.n)) * d.k;
  const dim3 lb(64), lg(kSortBlocks), sb(1024), one(1);
  // Static capped + dedup: the cut of each shard's dedup buffer decides which
  // rows drop, so the dedup ranks are scanned before the slot keys.
  const bool two_round = d.dedup && pa.ovf == nullptr && pa.capped && d.cap >= 0;
  if (!d.dedup) {
    hipLaunchKernelGGL(pass_local_kernel<1>, lg, lb, 0, s, d, pa, soa, pb.skey, pb.dkey,
                       pb.bh_slot, pb.bh_dedup, 0);
    hipLaunchKernelGGL(pass_scan_kernel, one, sb, 0, s, d, pa, 1, pb.bh_slot, pb.bh_dedup,
                       pb.kept, group_offsets, pb.tile_off, pb.tile_group, pb.dedup_kept, dedup_offsets,
                       pb.meta);
  } else if (!two_round) {
    hipLaunchKernelGGL(pass_local_kernel<3>, lg, lb, 0, s, d, pa, soa, pb.skey, pb.dkey,
                       pb.bh_slot, pb.bh_dedup, 0);
    hipLaunchKernelGGL(pass_scan_kernel, one, sb, 0, s, d, pa, 3, pb.bh_slot, pb.bh_dedup,
                       pb.kept, group_offsets, pb.tile_off, pb.tile_group, pb.dedup_kept, dedup_offsets,
                       pb.meta);
  } else {
    hipLaunchKernelGGL(pass_local_kernel<2>, lg, lb, 0, s, d, pa, soa, pb.skey, pb.dkey,
                       pb.bh_slot, pb.bh_dedup, 0);
    hipLaunchKernelGGL(pass_scan_kernel, one, sb, 0, s, d, pa, 2, pb.bh_slot, pb.bh_dedup,
                       pb.kept, group_offsets, pb.tile_off, pb.tile_group, pb.dedup_kept, dedup_offsets,
                       pb.meta);
    hipLaunchKernelGGL(pass_local_kernel<1>, lg, lb, 0, s, d, pa, soa, pb.skey, pb.dkey,
                       pb.bh_slot, pb.bh_dedup, 1);
    hipLaunchKernelGGL(pass_scan_kernel, one, sb, 0, s, d, pa, 1, pb.bh_slot, pb.bh_dedup,
                       pb.kept, group_offsets, pb.tile_off, pb.tile_group, pb.dedup_kept, dedup_offsets,
                       pb.meta);
  }
  const dim3 cg((nmax + 3) / 4), cb(256);
  if (d.dedup)
    hipLaunchKernelGGL(dedup_scatter_kernel, cg, cb, 0, s, d, pa, pb.dkey, pb.bh_dedup,
                       pb.dedup_kept, dedup_offsets, (const char*)x, dedup_token,
                       (char*)x_dedup);
  hipLaunchKernelGGL(row_scatter_kernel, cg, cb, 0, s, d, pa, soa, pb.skey, pb.dkey, pb.bh_slot,
                     pb.bh_dedup, pb.kept, group_offsets, dedup_offsets, (const char*)x,
                     (const char*)x_dedup, row_of_assign, sorted_assign, expand_idx,
                     (char*)x_sorted);
  return hipGetLastError();
}

}  // namespace moe
