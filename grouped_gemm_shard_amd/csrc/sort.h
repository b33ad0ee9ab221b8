// Stable counting sort on the GPU, without atomics on positions.
//
// A sequence of n elements, each with a key in [0, K) or -1 (skip), is cut
// into kSortBlocks contiguous blocks.  One wavefront per block walks its
// elements 64 at a time: a ballot per key bit finds, for every lane, the
// lanes holding the same key ("peers"); the element's rank is the running
// count of its key in LDS plus the number of lower peers, and the highest
// peer advances the running count.  The result per element is its rank
// among equal keys inside the block (packed with the key), and per block
// the count of every key.  A scan over the blocks then turns counts into
// block bases, so position = key offset + block base + local rank: exactly
// the stable order, independent of scheduling.
#pragma once

#include "common.h"

namespace moe {

// packed element: ((key + 1) << 21) | local_rank, 0 for a skipped element.
constexpr int kRankBits = 21;
__device__ __forceinline__ unsigned pack_key(int key, int rank) {
  return key < 0 ? 0u : (((unsigned)(key + 1)) << kRankBits) | (unsigned)rank;
}
__device__ __forceinline__ int packed_key(unsigned v) { return (int)(v >> kRankBits) - 1; }
__device__ __forceinline__ int packed_rank(unsigned v) { return (int)(v & ((1u << kRankBits) - 1)); }

__host__ __device__ __forceinline__ int sort_block_len(int n) {
  return (n + kSortBlocks - 1) / kSortBlocks;
}

__host__ __device__ __forceinline__ int key_bits(int K) {
  int b = 0;
  while ((1 << b) < K) ++b;
  return b;
}

// Peers of this lane: lanes of the wave with valid keys equal to `key`.
__device__ __forceinline__ unsigned long long wave_peers(int key, bool valid, int nbits) {
  unsigned long long m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    bool bit = valid && ((key >> b) & 1);
    unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return valid ? m : 0ull;
}

// One step of the block walk: ranks 64 elements (one per lane) against the
// running counts `run` (LDS, one int per key).  Must be called by the whole
// wavefront.  Returns the element's rank within the block (or -1).
__device__ __forceinline__ int wave_rank_step(int key, int nbits, int* run) {
  bool valid = key >= 0;
  unsigned long long peers = wave_peers(key, valid, nbits);
  int rank = -1;
  if (valid) {
    int below = __popcll(peers & lanemask_lt());
    rank = run[key] + below;
    if ((peers >> lane_id()) == 1ull) run[key] = rank + 1;  // highest peer advances
  }
  return rank;
}

// Exclusive scan over a 1024-thread block (one value per thread).  `tmp`
// is LDS of at least 16 ints.  Returns the exclusive prefix; *total gets the
// sum over the block.  Contains barriers: every thread must call it.
__device__ __forceinline__ int block_exscan_1024(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < nw) tmp[lane] = t;
  }
  __syncthreads();
  int prefix = w > 0 ? tmp[w - 1] : 0;
  *total = tmp[nw - 1];
  __syncthreads();
  return prefix + x - v;
}

// Turns the block counts of keys [0, K) into exclusive block bases (in
// place) and writes each key's total to totals[key] (LDS).  One wavefront
// per key, one lane per sort block (kSortBlocks == 64).  Contains no
// barrier; the caller synchronises before reading totals.
__device__ __forceinline__ void scan_keys_over_blocks(int* bh, int K, int* totals) {
  static_assert(kSortBlocks == 64, "one lane per sort block");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int key = w; key < K; key += nw) {
    int v = bh[lane * K + key];
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    bh[lane * K + key] = x - v;
    if (lane == 63) totals[key] = x;
  }
}

}  // namespace moe
