// a2 + a3: counts, redundancy plan, reroute, capacity and overflow.
//
// Follows "Support moe_dropless_fallback=layer on the ragged all-to-all MoE
// path" (sections Why / How: each shard's receive buffer holds factor x
// balanced rows, and the check computes from the top-k whether any shard
// would receive more) and "Moe dynamic redundancy" (code review: the greedy
// duplication plan with the has_candidate guard, and the rerouting of a
// planned share of the overloaded expert's tokens to its replica slot).
//
// Counts are order-independent: per-block LDS histograms (left by the route
// kernel in a layer call, else by hist_kernel) are summed by one workgroup.
// Without rerouting, that workgroup also assigns the home slots, counts the
// shards and checks overflow, so the whole step is one launch after route.
// The reroute needs each assignment's rank among the assignments of its
// expert, which comes from the stable counting sort in sort.h.
#include "count_body.h"
#include "sort.h"

namespace moe {

namespace {

// Per-block expert histograms of a caller-supplied top-k (row blockIdx of
// ph) and a per-block flag for out-of-range expert ids.
__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ idx, int n, int E,
                                                   int* __restrict__ ph, int* __restrict__ pbad) {
  __shared__ int hist[kMaxExperts];
  __shared__ int bad;
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int a = blockIdx.x * blockDim.x + threadIdx.x; a < n; a += gridDim.x * blockDim.x) {
    int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    else bad = 1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) ph[(size_t)blockIdx.x * E + e] = hist[e];
  if (threadIdx.x == 0) pbad[blockIdx.x] = bad;
}

// Counts and status for the rerouting path: sums the histograms and clears
// the shard counts and status words the later kernels accumulate into.
__global__ __launch_bounds__(1024) void count_sum_kernel(Dims d, const int* __restrict__ ph,
                                                         const int* __restrict__ pbad, int nb,
                                                         int* expert_counts, int* shard_counts,
                                                         int* status) {
  __shared__ int bad;
  sum_hist(d, ph, pbad, nb, expert_counts, &bad);
  for (int s = threadIdx.x; s < d.S; s += blockDim.x) shard_counts[s] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    status[0] = status[1] = status[2] = 0;
    status[3] = bad ? MOE_ERR_BAD_INDEX : 0;
  }
}

// The greedy plan, in one workgroup.  Loads are assignment counts per shard.
// Each of up to R rounds: r_max = most loaded shard (lowest on ties); its
// hottest expert not yet duplicated (lowest on ties), stop if none; r_min =
// least loaded shard with a free redundant slot (lowest on ties), stop if
// none or if load[r_max] <= load[r_min]; n_div = min(c_e, (load[r_max] -
// load[r_min]) / 2), stop if 0; the replica takes r_min's first free slot.
// Without dedup the final loads are the shard counts.
__global__ __launch_bounds__(1024) void plan_kernel(Dims d, const int* __restrict__ counts,
                                                    int* slot_expert, int* ndiv, int* replica,
                                                    int* dup_id, int* shard_counts) {
  __shared__ int load[kMaxSlots];
  __shared__ int used[kMaxSlots];
  __shared__ unsigned char dup[kMaxExperts];
  for (int s = threadIdx.x; s < d.G; s += blockDim.x) {
    int sh = s / d.spd, i = s - sh * d.spd;
    slot_expert[s] = i < d.El ? sh * d.El + i : -1;
  }
  for (int e = threadIdx.x; e < d.E; e += blockDim.x) {
    ndiv[e] = 0;
    replica[e] = -1;
    dup_id[e] = -1;
    dup[e] = 0;
  }
  for (int sh = threadIdx.x; sh < d.S; sh += blockDim.x) {
    int acc = 0;
    for (int i = 0; i < d.El; ++i) acc += counts[sh * d.El + i];
    load[sh] = acc;
    used[sh] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0 && d.R > 0 && d.B > 0) {
    for (int r = 0; r < d.R; ++r) {
      int rmax = 0;
      for (int sh = 1; sh < d.S; ++sh)
        if (load[sh] > load[rmax]) rmax = sh;
      int cand = -1;
      for (int e = rmax * d.El; e < (rmax + 1) * d.El; ++e) {
        if (dup[e]) continue;
        if (cand < 0 || counts[e] > counts[cand]) cand = e;
      }
      if (cand < 0) break;
      int rmin = -1;
      for (int sh = 0; sh < d.S; ++sh) {
        if (used[sh] >= d.B) continue;
        if (rmin < 0 || load[sh] < load[rmin]) rmin = sh;
      }
      if (rmin < 0 || load[rmax] <= load[rmin]) break;
      int n = min(counts[cand], (load[rmax] - load[rmin]) / 2);
      if (n <= 0) break;
      int s = rmin * d.spd + d.El + used[rmin];
      used[rmin] += 1;
      slot_expert[s] = cand;
      replica[cand] = s;
      ndiv[cand] = n;
      dup_id[cand] = r;
      dup[cand] = 1;
      load[rmax] -= n;
      load[rmin] += n;
    }
  }
  __syncthreads();
  if (!d.dedup)
    for (int sh = threadIdx.x; sh < d.S; sh += blockDim.x) shard_counts[sh] = load[sh];
}


// Ranks every assignment of a duplicated expert among that expert's
// assignments in flat (t, j) order, per block (key = the expert's dup id).
__global__ __launch_bounds__(64) void reroute_rank_kernel(Dims d, const int* __restrict__ idx,
                                                          const int* __restrict__ dup_id,
                                                          unsigned* keys, int* bh) {
  __shared__ int run[kMaxSlots];
  const int n = d.T * d.k, K = d.R, nbits = key_bits(d.R);
  const int blk = sort_block_len(n);
  const int e0 = blockIdx.x * blk, e1 = min(n, e0 + blk);
  for (int q = threadIdx.x; q < K; q += 64) run[q] = 0;
  __syncthreads();
  for (int base = e0; base < e1; base += 64) {
    int a = base + lane_id();
    int key = -1;
    if (a < e1) {
      int e = idx[a];
      if (e >= 0 && e < d.E) key = dup_id[e];
    }
    int rank = wave_rank_step(key, nbits, run);
    if (a < e1) keys[a] = pack_key(key, rank);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < K; q += 64) bh[blockIdx.x * K + q] = run[q];
}

__global__ __launch_bounds__(1024) void reroute_scan_kernel(int K, int* bh) {
  __shared__ int totals[kMaxSlots];
  scan_keys_over_blocks(bh, K, totals);
}

// slot_of_assign: home slot, or the replica slot for the first ndiv[e]
// assignments of a duplicated expert e.
__global__ __launch_bounds__(256) void assign_slots_kernel(Dims d, const int* __restrict__ idx,
                                                           const int* __restrict__ ndiv,
                                                           const int* __restrict__ replica,
                                                           const unsigned* __restrict__ keys,
                                                           const int* __restrict__ bh,
                                                           int* slot_of_assign) {
  const int n = d.T * d.k;
  const int blk = sort_block_len(n);
  for (int a = blockIdx.x * blockDim.x + threadIdx.x; a < n; a += gridDim.x * blockDim.x) {
    int e = idx[a];
    int s = -1;
    if (e >= 0 && e < d.E) {
      s = home_slot(d, e);
      if (keys != nullptr) {
        unsigned v = keys[a];
        int key = packed_key(v);
        if (key >= 0) {
          int rank = bh[(a / blk) * d.R + key] + packed_rank(v);
          if (rank < ndiv[e]) s = replica[e];
        }
      }
    }
    slot_of_assign[a] = s;
  }
}

// Dedup: one buffer row per distinct (token, shard) pair.
__global__ __launch_bounds__(256) void dedup_count_kernel(Dims d,
                                                          const int* __restrict__ slot_of_assign,
                                                          int* shard_counts) {
  __shared__ int hist[kMaxSlots];
  for (int s = threadIdx.x; s < d.S; s += blockDim.x) hist[s] = 0;
  __syncthreads();
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < d.T; t += gridDim.x * blockDim.x) {
    const int* row = slot_of_assign + (size_t)t * d.k;
    for (int j = 0; j < d.k; ++j) {
      int s = row[j];
      if (s < 0) continue;
      int sh = s / d.spd;
      bool first = true;
      for (int jj = 0; jj < j; ++jj) {
        int s2 = row[jj];
        if (s2 >= 0 && s2 / d.spd == sh) first = false;
      }
      if (first) atomicAdd(&hist[sh], 1);
    }
  }
  __syncthreads();
  for (int s = threadIdx.x; s < d.S; s += blockDim.x)
    if (hist[s]) atomicAdd(&shard_counts[s], hist[s]);
}

// status = [cap, overflow, max shard count, error bits]; a strict ">" check.
__global__ __launch_bounds__(1024) void finalize_kernel(Dims d, const int* __restrict__ shard_counts,
                                                        int* status, int* info, int info_mode,
                                                        float* rfactor) {
  __shared__ int red[16];
  int m = 0;
  for (int s = threadIdx.x; s < d.S; s += blockDim.x) m = max(m, shard_counts[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    int mx = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) mx = max(mx, red[w]);
    int ovf = (d.cap >= 0 && mx > d.cap) ? 1 : 0;
    status[0] = d.cap;
    status[1] = ovf;
    status[2] = mx;
    if (info != nullptr) {
      int ran = info_mode == MOE_MODE_FORCE_CHUNKED ? 1 : (info_mode == MOE_MODE_LAYER ? ovf : 0);
      info[0] = ovf;
      info[1] = ran;
      info[2] = d.cap;
      info[3] = mx;
      info[4] = status[3];
    }
    if (rfactor != nullptr) *rfactor = required_factor(d, mx);
  }
}

// The whole count step without rerouting, in one workgroup.
__global__ __launch_bounds__(1024) void count_fused_kernel(Dims d, CountArgs c) {
  count_fused_body(d, c);
}

}  // namespace

inline size_t hist_bytes(const Dims& d) {
  return (((size_t)route_hist_blocks(d) * d.E * 4 + 255) / 256) * 256 +
         (((size_t)route_hist_blocks(d) * 4 + 255) / 256) * 256;
}

int* count_hist_area(const Dims& d, void* scratch) { return (int*)scratch; }

size_t count_scratch_bytes(const Dims& d) {
  size_t n = (size_t)d.T * d.k;
  size_t bytes = hist_bytes(d);
  bytes += ((n * sizeof(unsigned) + 255) / 256) * 256;                          // keys
  bytes += (((size_t)kSortBlocks * (d.R > 0 ? d.R : 1) * 4 + 255) / 256) * 256;  // bh
  bytes += (((size_t)d.E * 4 + 255) / 256) * 256;                               // replica
  bytes += (((size_t)d.E * 4 + 255) / 256) * 256;                               // dup_id
  return bytes;
}

CountArgs layer_count_args(const Dims& d, const int* idx, int* expert_counts, int* slot_expert,
                           int* ndiv, int* shard_counts, int* status, void* scratch, int* info,
                           int info_mode) {
  CountArgs c = {idx, (const int*)scratch, nullptr, route_hist_blocks(d), expert_counts,
                 slot_expert, ndiv, nullptr, shard_counts, status, info, info_mode, nullptr};
  return c;
}

hipError_t launch_count(const Dims& d, const int* idx, int* expert_counts, int* slot_expert,
                        int* ndiv, int* slot_of_assign, int* shard_counts, int* status,
                        void* scratch, int hist_ready, int* info, int info_mode, float* rfactor,
                        hipStream_t st) {
  size_t n = (size_t)d.T * d.k;
  const int nb = route_hist_blocks(d);
  char* p = (char*)scratch;
  int* ph = (int*)p;
  int* pbad = (int*)(p + (((size_t)nb * d.E * 4 + 255) / 256) * 256);
  p += hist_bytes(d);
  unsigned* keys = (unsigned*)p;
  p += ((n * sizeof(unsigned) + 255) / 256) * 256;
  int* bh = (int*)p;
  p += (((size_t)kSortBlocks * (d.R > 0 ? d.R : 1) * 4 + 255) / 256) * 256;
  int* replica = (int*)p;
  p += (((size_t)d.E * 4 + 255) / 256) * 256;
  int* dup_id = (int*)p;

  if (hist_ready) {
    // the route step wrote the histograms; its expert ids are all in range
    pbad = nullptr;
  } else {
    hipLaunchKernelGGL(hist_kernel, dim3(nb), dim3(256), 0, st, idx, (int)n, d.E, ph, pbad);
  }
  const bool reroute = d.R > 0 && d.B > 0;
  if (!reroute) {
    CountArgs c = {idx, ph, pbad, nb, expert_counts, slot_expert, ndiv, slot_of_assign,
                   shard_counts, status, info, info_mode, rfactor};
    hipLaunchKernelGGL(count_fused_kernel, dim3(1), dim3(1024), 0, st, d, c);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(count_sum_kernel, dim3(1), dim3(1024), 0, st, d, ph, pbad, nb,
                     expert_counts, shard_counts, status);
  int nblk = (int)((n + 255) / 256);
  if (nblk > 1024) nblk = 1024;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, d, expert_counts, slot_expert,
                     ndiv, replica, dup_id, shard_counts);
  hipLaunchKernelGGL(reroute_rank_kernel, dim3(kSortBlocks), dim3(64), 0, st, d, idx, dup_id,
                     keys, bh);
  hipLaunchKernelGGL(reroute_scan_kernel, dim3(1), dim3(1024), 0, st, d.R, bh);
  hipLaunchKernelGGL(assign_slots_kernel, dim3(nblk), dim3(256), 0, st, d, idx, ndiv, replica,
                     keys, bh, slot_of_assign);
  if (d.dedup) {
    int tb = (d.T + 255) / 256;
    if (tb > 1024) tb = 1024;
    hipLaunchKernelGGL(dedup_count_kernel, dim3(tb), dim3(256), 0, st, d, slot_of_assign,
                       shard_counts);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, st, d, shard_counts, status, info,
                     info_mode, rfactor);
  return hipGetLastError();
}

}  // namespace moe
