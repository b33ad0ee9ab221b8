// a4 + a5: layouts of the passes and the permute.
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
// The layouts of every pass a call may take (the single pass and each
// sequence chunk) are computed together, before any pass runs: local ranks
// (up to 16 waves per sort block and pass), the scan (bases, group offsets, kept
// rows, GEMM tile schedule) and the placement of every element
// (sorted_assign, row_of_assign, dedup lists, expand indices).  Without
// dedup, scan and placement share one launch: each placement workgroup
// recomputes its pass's scan in LDS; with dedup they are separate launches
// (one scan block per pass).  Row copies are separate: the dedup buffer of a
// pass and, for the standalone permute, x_sorted, one wavefront per row with
// 16-byte loads and stores.  The standalone permute of a small pass without
// dedup instead runs as one launch that recounts the pass's keys in every
// workgroup (permute_one_launch_kernel).
#include <string.h>

#include "count_body.h"
#include "sort.h"

namespace moe {

namespace {

__device__ __forceinline__ int slot_key(const Dims& d, int s) {
  return (s >= d.lo_slot && s < d.lo_slot + d.G_res) ? s - d.lo_slot : -1;
}

// Slot of assignment j of a token whose row starts at `row`: the row holds
// slots, or (home != 0: nothing was rerouted) expert ids, whose slot is the
// expert's home slot.
__device__ __forceinline__ int slot_at(const Dims& d, const int* row, int home, int j) {
  const int v = row[j];
  if (!home) return v;
  if (v < 0 || v >= d.E) return -1;
  const int sh = v / d.El;
  return sh * d.spd + (v - sh * d.El);
}

// First assignment j' <= j of the token on the same shard as slot s.
__device__ __forceinline__ int first_on_shard(const Dims& d, const int* row, int home, int j,
                                              int s) {
  int sh = s / d.spd;
  for (int jj = 0; jj < j; ++jj) {
    int s2 = slot_at(d, row, home, jj);
    if (s2 >= 0 && s2 / d.spd == sh) return jj;
  }
  return j;
}

// Dedup key: local resident shard of the token's first assignment on it.
__device__ __forceinline__ int dedup_key(const Dims& d, const int* row, int home, int j) {
  int s = slot_at(d, row, home, j);
  if (slot_key(d, s) < 0) return -1;
  if (first_on_shard(d, row, home, j, s) != j) return -1;
  return s / d.spd - d.res_lo;
}

struct PassGeom {
  int s0, lw, capped, nelem, blk;
  size_t e0;  // first element of the pass in the per-element arrays
};

__device__ __forceinline__ PassGeom pass_geom(const Dims& d, const LayoutSet& ls, int j) {
  PassGeom g;
  layout_pass(d, ls, j, &g.s0, &g.lw, &g.capped, &g.e0);
  g.nelem = (d.T / d.L) * g.lw * d.k;
  g.blk = sort_block_len(g.nelem);
  return g;
}

__device__ __forceinline__ int elem_token(const Dims& d, const PassGeom& g, int e) {
  return window_token(d.L, g.s0, g.lw, e / d.k);
}

// Rank of pass element e (relative to its dedup shard), from the packed
// local rank and the block base.
__device__ __forceinline__ int dedup_rank(const Dims& d, const LayoutBuffers& lb, const PassGeom& g,
                                          int j, int e, int* key_out) {
  unsigned v = lb.dkey[g.e0 + e];
  int kd = packed_key(v);
  *key_out = kd;
  return lb.bh_dedup[((size_t)j * kSortBlocks + e / g.blk) * d.S_res + kd] + packed_rank(v);
}

// Local ranks of one sort block of pass j: blockDim / 64 waves split the
// block's elements into contiguous parts; each wave ranks its part against
// running counts of its own (LDS), then the waves' counts per key become
// exclusive bases (wave order = element order), which a second sweep adds
// to the ranks.  Leaves per element the packed (key, rank within the sort
// block) and per block the count of every key.
constexpr int kLocalLds = 16384;  // ints of LDS for the waves' running counts

template <int WHICH>  // bit 0: slot keys, bit 1: dedup keys
__global__ __launch_bounds__(1024) void layout_local_kernel(Dims d, LayoutSet ls,
                                                            const int* __restrict__ soa,
                                                            int home, LayoutBuffers lb,
                                                            int drop_check) {
  __shared__ int runs[kLocalLds];
  const int j = blockIdx.y;
  if (!layout_live(ls, j)) return;
  const PassGeom g = pass_geom(d, ls, j);
  const int nw = blockDim.x >> 6, w = threadIdx.x >> 6;
  const int GS = (WHICH & 1) ? d.G_res : 0, GD = (WHICH & 2) ? d.S_res : 0;
  int* run_s = runs + w * (GS + GD);
  int* run_d = run_s + GS;
  const int b0 = blockIdx.x * g.blk, b1 = min(g.nelem, b0 + g.blk);
  // this wave's part of the block, in whole rounds of 64 elements
  const int part = (((b1 > b0 ? b1 - b0 : 0) + nw * 64 - 1) / (nw * 64)) * 64;
  const int e0 = min(b1, b0 + w * part), e1 = min(b1, e0 + part);
  const int nb_s = key_bits(d.G_res), nb_d = key_bits(d.S_res);
  for (int q = threadIdx.x; q < nw * (GS + GD); q += blockDim.x) runs[q] = 0;
  __syncthreads();
  for (int base = e0; base < e1; base += 64) {
    const int e = base + lane_id();
    const bool in = e < e1;
    int jj = 0;
    const int* row = soa;
    if (in) {
      jj = e % d.k;
      row = soa + (size_t)elem_token(d, g, e) * d.k;
    }
    if (WHICH & 1) {
      const int sl = in ? slot_at(d, row, home, jj) : -1;
      int ks = in ? slot_key(d, sl) : -1;
      if (drop_check && g.capped && ks >= 0) {
        // the token was cut from this shard's dedup buffer: drop the row
        int jr = first_on_shard(d, row, home, jj, sl);
        int kd;
        int r = dedup_rank(d, lb, g, j, e - jj + jr, &kd);
        if (r >= d.cap) ks = -1;
      }
      int r = wave_rank_step(ks, nb_s, run_s);
      if (in) lb.skey[g.e0 + e] = pack_key(ks, r);
    }
    if (WHICH & 2) {
      int kd = in ? dedup_key(d, row, home, jj) : -1;
      int r = wave_rank_step(kd, nb_d, run_d);
      if (in) lb.dkey[g.e0 + e] = pack_key(kd, r);
    }
  }
  __syncthreads();
  // per key: the waves' exclusive bases (in place) and the block's count
  const int K = GS + GD;
  for (int q = threadIdx.x; q < K; q += blockDim.x) {
    int acc = 0;
    for (int v = 0; v < nw; ++v) {
      const int c = runs[v * K + q];
      runs[v * K + q] = acc;
      acc += c;
    }
    if (q < GS) lb.bh_slot[((size_t)j * kSortBlocks + blockIdx.x) * d.G_res + q] = acc;
    else lb.bh_dedup[((size_t)j * kSortBlocks + blockIdx.x) * d.S_res + (q - GS)] = acc;
  }
  __syncthreads();
  if (w == 0) return;  // the first wave's bases are all zero
  for (int e = e0 + lane_id(); e < e1; e += 64) {
    if (WHICH & 1) {
      const unsigned v = lb.skey[g.e0 + e];
      const int ks = packed_key(v);
      if (ks >= 0) lb.skey[g.e0 + e] = pack_key(ks, packed_rank(v) + run_s[ks]);
    }
    if (WHICH & 2) {
      const unsigned v = lb.dkey[g.e0 + e];
      const int kd = packed_key(v);
      if (kd >= 0) lb.dkey[g.e0 + e] = pack_key(kd, packed_rank(v) + run_d[kd]);
    }
  }
}

// Slot part of pass j's scan, from the rows per slot in totals (LDS): rows
// kept per slot (without dedup, a capped shard keeps the first `cap` rows of
// its bucket, i.e. a prefix of each slot), group offsets and the GEMM m-tile
// schedule.  With `write` they go to the pass's layout buffers; kept rows
// and offsets also go to kept_l / go_l (LDS) when those are set.  Every
// thread of the 1024-thread block calls it (it holds barriers).
__device__ __forceinline__ void slot_scan(const Dims& d, int j, bool capped, const int* totals,
                                          int* excl, int* tmp, bool write,
                                          const LayoutBuffers& lb, int* kept_l, int* go_l) {
  const int g = threadIdx.x;
  int* kept = lb.kept + (size_t)j * d.G_res;
  int* go = lb.group_offsets + (size_t)j * (d.G_res + 1);
  int* toff = lb.tile_off + (size_t)j * (d.G_res + 1);
  int* tgrp = lb.tile_group + (size_t)j * tile_map_len(d);
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
  int nrows;
  int off = block_exscan_1024(own ? kp : 0, tmp, &nrows);
  if (own && kept_l != nullptr) {
    kept_l[g] = kp;
    go_l[g] = off;
  }
  if (!write) return;
  if (own) {
    kept[g] = kp;
    go[g] = off;
  }
  int ntiles;
  const int tiles = own ? (kp + d.gemm_bm - 1) / d.gemm_bm : 0;
  int to = block_exscan_1024(tiles, tmp, &ntiles);
  if (own) {
    toff[g] = to;
    for (int m = 0; m < tiles; ++m) tgrp[to + m] = g;
  }
  if (g == 0) {
    go[d.G_res] = nrows;
    toff[d.G_res] = ntiles;
    lb.meta[(size_t)j * kLayoutMeta] = nrows;
  }
}

// One block per pass.  Slot part: block bases, rows per slot, kept rows
// (without dedup, a capped shard keeps the first `cap` rows of its bucket,
// i.e. a prefix of each slot), group offsets, GEMM m-tile offsets and the
// m-tile -> group map.  Dedup part: distinct tokens per shard, cut at the
// cap when capped, and their offsets.
__global__ __launch_bounds__(1024) void layout_scan_kernel(Dims d, LayoutSet ls, int which,
                                                           LayoutBuffers lb) {
  __shared__ int tmp[16];
  __shared__ int excl[kMaxSlots];
  __shared__ int totals[kMaxSlots];
  __shared__ int dtotals[kMaxSlots];
  const int j = blockIdx.x;
  if (!layout_live(ls, j)) return;
  const PassGeom pg = pass_geom(d, ls, j);
  const bool capped = pg.capped && d.cap >= 0;
  const int g = threadIdx.x;
  int* bh_s = lb.bh_slot + (size_t)j * kSortBlocks * d.G_res;
  int* bh_d = lb.bh_dedup + (size_t)j * kSortBlocks * d.S_res;
  if (which & 1) scan_keys_over_blocks(bh_s, d.G_res, totals);
  if (which & 2) scan_keys_over_blocks(bh_d, d.S_res, dtotals);
  __syncthreads();
  int* meta = lb.meta + (size_t)j * kLayoutMeta;
  if (which & 1) slot_scan(d, j, capped, totals, excl, tmp, true, lb, nullptr, nullptr);
  if (which & 2) {
    int* dkept = lb.dedup_kept + (size_t)j * d.S_res;
    int* doff = lb.dedup_offsets + (size_t)j * (d.S_res + 1);
    const bool own = g < d.S_res;
    int u = own ? dtotals[g] : 0;
    int ku = capped ? min(u, d.cap) : u;
    if (own) dkept[g] = ku;
    int nu;
    int off = block_exscan_1024(own ? ku : 0, tmp, &nu);
    if (own) doff[g] = off;
    if (g == 0) {
      doff[d.S_res] = nu;
      meta[1] = nu;
    }
  }
}

// Scan and placement in one launch (no dedup, kSortBlocks * G_res <=
// kFusedBases): every 1024-thread workgroup of pass j recomputes the pass's
// scan in LDS (per-key block bases, kept rows, group offsets) from the local
// counts and places its 1024 elements; workgroup 0 of the pass also writes
// the scan's results for the GEMM and the combine.  With has_count, row
// np of the grid runs the count step in its first workgroup.
__global__ __launch_bounds__(1024) void layout_scan_place_kernel(Dims d, LayoutSet ls,
                                                                 LayoutBuffers lb, CountArgs cnt,
                                                                 int has_count) {
  __shared__ int bases[kFusedBases];
  __shared__ int tmp[16];
  __shared__ int excl[kMaxSlots];
  __shared__ int totals[kMaxSlots];
  __shared__ int kept_l[kMaxSlots];
  __shared__ int go_l[kMaxSlots];
  const int j = blockIdx.y;
  if (has_count && j == layout_num_passes(ls)) {
    if (blockIdx.x == 0) count_fused_body(d, cnt);
    return;
  }
  if (!layout_live(ls, j)) return;
  const PassGeom g = pass_geom(d, ls, j);
  if (blockIdx.x > 0 && blockIdx.x * 1024 >= g.nelem) return;  // block-uniform
  const int G = d.G_res;
  // per-key exclusive bases over the sort blocks: one wave per key, one lane
  // per block
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int* bh = lb.bh_slot + (size_t)j * kSortBlocks * G;
  for (int key = w; key < G; key += 16) {
    const int v = bh[lane * G + key];
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    bases[lane * G + key] = x - v;
    if (lane == 63) totals[key] = x;
  }
  __syncthreads();
  slot_scan(d, j, g.capped && d.cap >= 0, totals, excl, tmp, blockIdx.x == 0, lb, kept_l, go_l);
  __syncthreads();
  const int e = blockIdx.x * 1024 + threadIdx.x;
  if (e >= g.nelem) return;
  const int jj = e % d.k;
  const int t = elem_token(d, g, e);
  const int a = t * d.k + jj;
  const unsigned v = lb.skey[g.e0 + e];
  const int ks = packed_key(v);
  int pos = -1;
  if (ks >= 0) {
    const int r = bases[(e / g.blk) * G + ks] + packed_rank(v);
    if (r < kept_l[ks]) pos = go_l[ks] + r;
  }
  lb.row_of_assign[(size_t)layout_set_of(ls, j) * ((size_t)d.T * d.k) + a] = pos;
  if (pos >= 0) lb.sorted_assign[layout_row_base(d, ls, j) + pos] = a;
}

// Places every element of every pass: row_of_assign, sorted_assign and, with
// dedup, the dedup token lists and the expand indices.
__global__ __launch_bounds__(256) void layout_place_kernel(Dims d, LayoutSet ls,
                                                           const int* __restrict__ soa,
                                                           int home, LayoutBuffers lb) {
  const int j = blockIdx.y;
  if (!layout_live(ls, j)) return;
  const PassGeom g = pass_geom(d, ls, j);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= g.nelem) return;
  const int jj = e % d.k;
  const int t = elem_token(d, g, e);
  const int a = t * d.k + jj;
  const size_t srow = layout_row_base(d, ls, j);
  int* roa = lb.row_of_assign + (size_t)layout_set_of(ls, j) * ((size_t)d.T * d.k);
  if (d.dedup) {
    unsigned vd = lb.dkey[g.e0 + e];
    int kd = packed_key(vd);
    if (kd >= 0) {
      int r = lb.bh_dedup[((size_t)j * kSortBlocks + e / g.blk) * d.S_res + kd] + packed_rank(vd);
      if (r < lb.dedup_kept[(size_t)j * d.S_res + kd])
        lb.dedup_token[layout_dedup_base(d, ls, j) + lb.dedup_offsets[(size_t)j * (d.S_res + 1) + kd] + r] = t;
    }
  }
  unsigned v = lb.skey[g.e0 + e];
  int ks = packed_key(v);
  int pos = -1;
  if (ks >= 0) {
    int r = lb.bh_slot[((size_t)j * kSortBlocks + e / g.blk) * d.G_res + ks] + packed_rank(v);
    if (r < lb.kept[(size_t)j * d.G_res + ks]) pos = lb.group_offsets[(size_t)j * (d.G_res + 1) + ks] + r;
  }
  roa[a] = pos;
  if (pos < 0) return;
  lb.sorted_assign[srow + pos] = a;
  if (d.dedup) {
    const int* row = soa + (size_t)t * d.k;
    int jr = first_on_shard(d, row, home, jj, slot_at(d, row, home, jj));
    int kd;
    int r = dedup_rank(d, lb, g, j, e - jj + jr, &kd);
    lb.expand_idx[srow + pos] = lb.dedup_offsets[(size_t)j * (d.S_res + 1) + kd] + r;
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
  // the rest (at most 3 chunks per lane): every load before the stores
  const bool p0 = off < nbytes, p1 = off + 1024 < nbytes, p2 = off + 2048 < nbytes;
  uint4 v0, v1, v2;
  if (p0) v0 = *(const uint4*)(src + off);
  if (p1) v1 = *(const uint4*)(src + off + 1024);
  if (p2) v2 = *(const uint4*)(src + off + 2048);
  if (p0) *(uint4*)(dst + off) = v0;
  if (p1) *(uint4*)(dst + off + 1024) = v1;
  if (p2) *(uint4*)(dst + off + 2048) = v2;
}

// dst[r] = src[index[r] / div] for r < count (count read on the device),
// one wavefront per row; count and index belong to the pass's layout j.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int* __restrict__ count,
                                                          int count_stride,
                                                          const int* __restrict__ index,
                                                          long long index_stride, int div,
                                                          const char* __restrict__ src,
                                                          char* __restrict__ dst, int row_bytes,
                                                          int src_rows, long long max_rows,
                                                          PassArgs pa) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int r = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int cnt = count[(size_t)pi.j * count_stride];
  if (r >= cnt || r >= max_rows) return;
  const int s = index[(size_t)pi.j * index_stride + r] / div;
  if (s < 0 || s >= src_rows) return;
  wave_copy_row(dst + (size_t)r * row_bytes, src + (size_t)s * row_bytes, row_bytes);
}

// Copies one row of `nbytes` (a multiple of 16) with the whole wavefront,
// up to 16 KB in flight: every load of a 16 KB piece before its stores.
__device__ __forceinline__ void wave_copy_row_deep(char* __restrict__ dst,
                                                   const char* __restrict__ src, int nbytes) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  constexpr int U = 16;
  for (int base = 0; base < nbytes; base += U * 1024) {
    v4i v[U];  // registers (a select, not a guarded assignment, keeps them out of scratch)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o = base + u * 1024 + lane_id() * 16;
      v[u] = o < nbytes ? *(const v4i*)(src + o) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int o = base + u * 1024 + lane_id() * 16;
      if (o < nbytes) *(v4i*)(dst + o) = v[u];
    }
  }
}

// The standalone permute of one pass without dedup in a single launch.
// Every 1024-thread workgroup counts the pass's keys itself (over all
// elements: the rows per slot; over the elements before its own: their
// bases), runs the slot scan in LDS, ranks and places its own `per_block`
// elements (one wave, on top of those bases) and copies their rows with its
// 16 waves, a wave's first rows loaded before the layout.  Workgroup 0 also writes the scan's
// results (group offsets, kept rows, tile schedule, row count).  The
// recount costs every workgroup a read of the pass's slots (L2-resident),
// which is why the path is kept to passes of at most 8192 elements
// (measured on MI355X with 10 KB rows: 19.7 us against 26.9 us for the
// three-launch path at 4096 elements, 35 us against 39 us at 8192 with one
// row a wave loaded ahead; at 16384
// elements the recount makes it twice as slow, and 512 workgroups of 16
// elements instead of 256 of 32 were 13% slower at 8192).
constexpr int kOneLaunchElems = 8192;  // most elements of a pass
constexpr int kOneLaunchOwn = 64;      // most elements per workgroup
constexpr int kOneLaunchBlocks = 256;  // workgroups aimed for

// PF: 1 KB slices (16 bytes a lane) of the longest row a wave loads before
// the layout; NR: rows a wave loads then (its elements w and w + 16).  Two
// rows of up to 10 KB or one of up to 16 KB keep a wave within the 128
// registers of a 1024-thread workgroup.
template <int PF, int NR>
__global__ __launch_bounds__(1024) void permute_one_launch_kernel(
    Dims d, LayoutSet ls, const int* __restrict__ soa, LayoutBuffers lb,
    const char* __restrict__ x, char* __restrict__ x_sorted, int row_bytes, long long max_rows,
    int per_block) {
  __shared__ int tot[kMaxSlots];
  __shared__ int bef[kMaxSlots];
  __shared__ int excl[kMaxSlots];
  __shared__ int kept_l[kMaxSlots];
  __shared__ int go_l[kMaxSlots];
  __shared__ int tmp[16];
  __shared__ int pos_l[kOneLaunchOwn];
  __shared__ int tok_l[kOneLaunchOwn];
  const PassGeom g = pass_geom(d, ls, 0);
  const int e_lo = blockIdx.x * per_block;
  if (blockIdx.x > 0 && e_lo >= g.nelem) return;  // block-uniform
  const int e_hi = min(g.nelem, e_lo + per_block);
  const int G = d.G_res, k = d.k, lane = lane_id(), w = threadIdx.x >> 6;
  const int nb = key_bits(G);
  // Every slot key the wave needs, read first: the keys of its counting
  // rounds, in wave 0 those of the workgroup's own elements, and that of
  // the wave's own first element (vector loads complete in issue order, so
  // a key read after the row prefetch below would wait for the rows).  The
  // loads are unconditional, element 0's slot standing in for lanes past
  // the elements, so that they issue back to back and are waited for once.
  constexpr int RND = kOneLaunchElems / 1024;
  auto key_of = [&](int e, bool in, int& t) {
    const int ec = in ? e : 0;
    const int tt = elem_token(d, g, ec);  // (garbage when the pass is empty: unused)
    t = in ? tt : 0;
    const int v = soa[(size_t)t * k + (in ? ec % k : 0)];
    return slot_key(d, v) | ((int)in - 1);  // -1 past the elements, no branch
  };
  int kr[RND], tr;
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int e = w * 64 + r * 1024 + lane;
    kr[r] = key_of(e, e < g.nelem, tr);
  }
  int to;
  const int ko = key_of(e_lo + lane, w == 0 && e_lo + lane < e_hi, to);
  int tw[NR];
  bool res_w[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r)
    res_w[r] = key_of(e_lo + w + 16 * r, w + 16 * r < e_hi - e_lo, tw[r]) >= 0;
  // every key landed on every path (s_waitcnt vmcnt(0): the encoding's
  // expcnt and lgkmcnt fields at their maxima), so that no later use of a
  // key waits on the row loads below
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // Each wave's first NR own elements: their source rows are known before
  // the layout, so a resident element's row (at most PF KB) is loaded into
  // registers now and lands while the workgroup recounts and places the
  // keys; it is stored once its position is known.
  typedef int v4i __attribute__((ext_vector_type(4)));
  v4i pf[NR][PF];
  const bool pf_fit = row_bytes <= PF * 1024;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const bool pf_on = pf_fit && w + 16 * r < e_hi - e_lo;
    const bool pf_load = pf_on && res_w[r];
    if (pf_on) {
      const char* src = x + (size_t)tw[r] * row_bytes;
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int o = u * 1024 + lane * 16;
        pf[r][u] = pf_load && o < row_bytes ? *(const v4i*)(src + o) : v4i{0, 0, 0, 0};
      }
    }
  }
  for (int q = threadIdx.x; q < G; q += 1024) tot[q] = bef[q] = 0;
  __syncthreads();
  // the waves take rounds of 64 elements in turn; per round and key the
  // highest peer adds the key's lanes (and those before e_lo)
#pragma unroll
  for (int r = 0; r < RND; ++r) {
    const int base = w * 64 + r * 1024;
    if (base >= g.nelem) break;  // wave-uniform
    const int e = base + lane;
    const bool in = e < g.nelem;
    const int ks = kr[r];
    const unsigned long long peers = wave_peers(ks, ks >= 0, nb);
    const unsigned long long early = __ballot(in && e < e_lo);
    if (ks >= 0 && (peers >> lane) == 1ull) {
      atomicAdd(&tot[ks], __popcll(peers));
      const int nbf = __popcll(peers & early);
      if (nbf > 0) atomicAdd(&bef[ks], nbf);
    }
  }
  __syncthreads();
  slot_scan(d, 0, g.capped && d.cap >= 0, tot, excl, tmp, blockIdx.x == 0, lb, kept_l, go_l);
  __syncthreads();
  if (w == 0) {
    int* roa = lb.row_of_assign + (size_t)layout_set_of(ls, 0) * ((size_t)d.T * k);
    int* sa = lb.sorted_assign + layout_row_base(d, ls, 0);
    {  // the workgroup's own elements (at most 64: one round)
      const int e = e_lo + lane;
      const bool in = e < e_hi;
      const int ks = ko, t = to;
      const int r = wave_rank_step(ks, nb, bef);
      int pos = -1;
      if (ks >= 0 && r < kept_l[ks]) pos = go_l[ks] + r;
      if (in) {
        const int a = t * k + e % k;
        roa[a] = pos;
        if (pos >= 0) sa[pos] = a;
        pos_l[e - e_lo] = pos;
        tok_l[e - e_lo] = t;
      }
    }
  }
  __syncthreads();
  int i = w;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (pf_fit && i < e_hi - e_lo) {
      const int pos = pos_l[i];
      if (pos >= 0 && pos < max_rows) {
        char* dst = x_sorted + (size_t)pos * row_bytes;
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          const int o = u * 1024 + lane * 16;
          if (o < row_bytes) *(v4i*)(dst + o) = pf[r][u];
        }
      }
      i += 16;
    }
  }
  for (; i < e_hi - e_lo; i += 16) {
    const int pos = pos_l[i];
    if (pos < 0 || pos >= max_rows) continue;
    wave_copy_row_deep(x_sorted + (size_t)pos * row_bytes, x + (size_t)tok_l[i] * row_bytes,
                       row_bytes);
  }
}

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// ---------------------------------------------------------------------------
// Buffers and launches
// ---------------------------------------------------------------------------

size_t layout_scratch_bytes(const Dims& d, const LayoutSet& ls) {
  const int np = layout_num_passes(ls);
  const size_t tk = (size_t)d.T * d.k;
  const size_t elems = layout_total_elems(d, ls);
  size_t b = 0;
  b += al256(elems * 4) * 2;                                     // skey, dkey
  b += al256((size_t)np * kSortBlocks * d.G_res * 4);            // bh_slot
  b += al256((size_t)np * kSortBlocks * d.S_res * 4);            // bh_dedup
  b += al256((size_t)np * d.G_res * 4);                          // kept
  b += al256((size_t)np * d.S_res * 4);                          // dedup_kept
  b += al256((size_t)np * (d.G_res + 1) * 4) * 2;                // group_offsets, tile_off
  b += al256((size_t)np * tile_map_len(d) * 4);                  // tile_group
  b += al256((size_t)np * (d.S_res + 1) * 4);                    // dedup_offsets
  b += al256((size_t)np * kLayoutMeta * 4);                      // meta
  b += al256((size_t)layout_num_sets(ls) * tk * 4);              // row_of_assign
  b += al256(elems * 4) * 2;                                     // sorted_assign, expand_idx
  b += al256(layout_total_dedup(d, ls) * 4);                     // dedup_token
  return b;
}

LayoutBuffers carve_layout(const Dims& d, const LayoutSet& ls, void* scratch) {
  const int np = layout_num_passes(ls);
  const size_t tk = (size_t)d.T * d.k;
  const size_t elems = layout_total_elems(d, ls);
  char* p = (char*)scratch;
  LayoutBuffers lb;
  auto take = [&](size_t bytes) {
    char* q = p;
    p += al256(bytes);
    return q;
  };
  lb.skey = (unsigned*)take(elems * 4);
  lb.dkey = (unsigned*)take(elems * 4);
  lb.bh_slot = (int*)take((size_t)np * kSortBlocks * d.G_res * 4);
  lb.bh_dedup = (int*)take((size_t)np * kSortBlocks * d.S_res * 4);
  lb.kept = (int*)take((size_t)np * d.G_res * 4);
  lb.dedup_kept = (int*)take((size_t)np * d.S_res * 4);
  lb.group_offsets = (int*)take((size_t)np * (d.G_res + 1) * 4);
  lb.tile_off = (int*)take((size_t)np * (d.G_res + 1) * 4);
  lb.tile_group = (int*)take((size_t)np * tile_map_len(d) * 4);
  lb.dedup_offsets = (int*)take((size_t)np * (d.S_res + 1) * 4);
  lb.meta = (int*)take((size_t)np * kLayoutMeta * 4);
  lb.row_of_assign = (int*)take((size_t)layout_num_sets(ls) * tk * 4);
  lb.sorted_assign = (int*)take(elems * 4);
  lb.expand_idx = (int*)take(elems * 4);
  lb.dedup_token = (int*)take(layout_total_dedup(d, ls) * 4);
  return lb;
}

bool layout_fused(const Dims& d) {
  return !d.dedup && d.G_res * kSortBlocks <= kFusedBases;
}

hipError_t launch_layout(const Dims& d, const LayoutSet& ls, const int* soa, int home,
                         const LayoutBuffers& lb, const CountArgs* cnt, hipStream_t s) {
  const int np = layout_num_passes(ls);
  const dim3 lgrid(kSortBlocks, np), sb(1024), sgrid(np);
  // waves per sort block: enough for its elements (64 per wave per round),
  // at most 16, and their running counts within the LDS budget
  const int maxe_all = (d.T / d.L) * layout_max_lw(d, ls) * d.k;
  const int blk = (maxe_all + kSortBlocks - 1) / kSortBlocks;
  int nw = (blk + 63) / 64;
  nw = nw < 1 ? 1 : (nw > 16 ? 16 : nw);
  while (nw > 1 && nw * (d.G_res + d.S_res) > kLocalLds) --nw;
  const dim3 lb64(64 * nw);
  const int maxe = (d.T / d.L) * layout_max_lw(d, ls) * d.k;
  if (layout_fused(d)) {
    // with the count step inside, every candidate pass is laid out
    // (liveness would need the flag the count workgroup is computing)
    CountArgs none;
    memset(&none, 0, sizeof(none));
    LayoutSet lsl = ls;
    if (cnt != nullptr) lsl.ovf = nullptr;
    const int pb = (maxe + 1023) / 1024 > 0 ? (maxe + 1023) / 1024 : 1;
    hipLaunchKernelGGL(layout_local_kernel<1>, lgrid, lb64, 0, s, d, lsl, soa, home, lb, 0);
    hipLaunchKernelGGL(layout_scan_place_kernel, dim3(pb, np + (cnt != nullptr ? 1 : 0)), sb, 0,
                       s, d, lsl, lb, cnt != nullptr ? *cnt : none, cnt != nullptr ? 1 : 0);
    return hipGetLastError();
  }
  if (cnt != nullptr) return hipErrorInvalidValue;
  // Static capped + dedup: the cut of each shard's dedup buffer decides which
  // rows drop, so the dedup ranks are scanned before the slot keys.
  const bool two_round = d.dedup && d.cap >= 0 &&
                         ((ls.has_single && ls.single_capped) || (ls.w_cnt && ls.w_capped));
  if (!d.dedup) {
    hipLaunchKernelGGL(layout_local_kernel<1>, lgrid, lb64, 0, s, d, ls, soa, home, lb, 0);
    hipLaunchKernelGGL(layout_scan_kernel, sgrid, sb, 0, s, d, ls, 1, lb);
  } else if (!two_round) {
    hipLaunchKernelGGL(layout_local_kernel<3>, lgrid, lb64, 0, s, d, ls, soa, home, lb, 0);
    hipLaunchKernelGGL(layout_scan_kernel, sgrid, sb, 0, s, d, ls, 3, lb);
  } else {
    hipLaunchKernelGGL(layout_local_kernel<2>, lgrid, lb64, 0, s, d, ls, soa, home, lb, 0);
    hipLaunchKernelGGL(layout_scan_kernel, sgrid, sb, 0, s, d, ls, 2, lb);
    hipLaunchKernelGGL(layout_local_kernel<1>, lgrid, lb64, 0, s, d, ls, soa, home, lb, 1);
    hipLaunchKernelGGL(layout_scan_kernel, sgrid, sb, 0, s, d, ls, 1, lb);
  }
  hipLaunchKernelGGL(layout_place_kernel, dim3((maxe + 255) / 256, np), dim3(256), 0, s, d, ls,
                     soa, home, lb);
  return hipGetLastError();
}

hipError_t launch_permute_one(const Dims& d, const LayoutSet& ls, const int* soa,
                              const LayoutBuffers& lb, const void* x, void* x_sorted,
                              int row_bytes, int64_t max_rows, hipStream_t s) {
  const int nelem = (d.T / d.L) * layout_max_lw(d, ls) * d.k;
  if (d.dedup || layout_num_passes(ls) != 1 || nelem > kOneLaunchElems)
    return hipErrorNotSupported;
  int per = (nelem + kOneLaunchBlocks - 1) / kOneLaunchBlocks;
  per = per < 16 ? 16 : (per + 15) / 16 * 16;
  if (per > kOneLaunchOwn) return hipErrorNotSupported;
  const int nb = nelem > 0 ? (nelem + per - 1) / per : 1;
  if (row_bytes <= 10240 && per > 16)
    hipLaunchKernelGGL((permute_one_launch_kernel<10, 2>), dim3(nb), dim3(1024), 0, s, d, ls,
                       soa, lb, (const char*)x, (char*)x_sorted, row_bytes, (long long)max_rows,
                       per);
  else
    hipLaunchKernelGGL((permute_one_launch_kernel<16, 1>), dim3(nb), dim3(1024), 0, s, d, ls,
                       soa, lb, (const char*)x, (char*)x_sorted, row_bytes, (long long)max_rows,
                       per);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int* count, int count_stride, const int* index,
                              long long index_stride, int div, const void* src, void* dst,
                              int row_bytes, int src_rows, int64_t max_rows, const PassArgs& pa,
                              hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((max_rows + 3) / 4)), dim3(256), 0, s,
                     count, count_stride, index, index_stride, div, (const char*)src, (char*)dst,
                     row_bytes, src_rows, (long long)max_rows, pa);
  return hipGetLastError();
}

}  // namespace moe
