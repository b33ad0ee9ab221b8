// The count step without rerouting as device code, shared by its own
// kernel and by the layout scan kernel, which runs it in one extra
// workgroup when the layer needs no rerouting (the layout then does not
// wait for the counts: it lays out every candidate pass, and only the
// placement reads the overflow flag).
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ int home_slot(const Dims& d, int e) {
  int sh = e / d.El;
  return sh * d.spd + (e - sh * d.El);
}

// Sums the per-block histograms into counts[E] (one thread per expert) and
// ORs the blocks' bad-id flags (pbad may be null: no bad ids) into *bad_out.
__device__ __forceinline__ void sum_hist(const Dims& d, const int* __restrict__ ph,
                                         const int* __restrict__ pbad, int nb, int* counts,
                                         int* bad_out) {
  // blockDim / E partitions of the rows per expert, then a reduction in LDS
  __shared__ int part[1024];
  const int P = max(1, (int)blockDim.x / d.E);
  const int e = threadIdx.x % d.E, q = threadIdx.x / d.E;
  int acc = 0;
  if (q < P) {
#pragma unroll 4
    for (int b = q; b < nb; b += P) acc += ph[(size_t)b * d.E + e];
    part[q * d.E + e] = acc;
  }
  if (threadIdx.x == 0) {
    int bad = 0;
    if (pbad != nullptr)
      for (int b = 0; b < nb; ++b) bad |= pbad[b];
    *bad_out = bad;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < d.E; x += blockDim.x) {
    int sum = 0;
    for (int qq = 0; qq < P; ++qq) sum += part[qq * d.E + x];
    counts[x] = sum;
  }
  __syncthreads();
}

// The smallest buffer factor that would have fit: max shard count over the
// balanced share T*k/S ("Support moe_dropless_fallback=layer on the ragged
// all-to-all MoE path", Shortcomings: the figure the overflow log reports).
__device__ __forceinline__ float required_factor(const Dims& d, int mx) {
  return (float)((double)mx * (double)d.S / ((double)d.T * (double)d.k));
}

__device__ __forceinline__ void write_status(const Dims& d, int mx, int bad, int* status,
                                             int* info, int info_mode, float* rfactor) {
  int ovf = (d.cap >= 0 && mx > d.cap) ? 1 : 0;
  status[0] = d.cap;
  status[1] = ovf;
  status[2] = mx;
  status[3] = bad ? MOE_ERR_BAD_INDEX : 0;
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

// The whole count step without rerouting, in one workgroup: expert counts
// from the per-block histograms, home slots for every assignment, shard
// counts (assignments per shard, or distinct tokens per shard with dedup)
// and the overflow check.
// Runs in one workgroup of 1024 threads.
__device__ __forceinline__ void count_fused_body(const Dims& d, const CountArgs& c) {
  const int* __restrict__ idx = c.idx;
  const int* __restrict__ ph = c.ph;
  const int* __restrict__ pbad = c.pbad;
  const int nb = c.nb;
  int* expert_counts = c.expert_counts;
  int* slot_expert = c.slot_expert;
  int* ndiv = c.ndiv;
  int* slot_of_assign = c.slot_of_assign;
  int* shard_counts = c.shard_counts;
  int* status = c.status;
  int* info = c.info;
  const int info_mode = c.info_mode;
  __shared__ int counts[kMaxExperts];
  __shared__ int load[kMaxSlots];
  __shared__ int bad;
  __shared__ int red[16];
  sum_hist(d, ph, pbad, nb, counts, &bad);
  for (int s = threadIdx.x; s < d.G; s += blockDim.x) {
    int sh = s / d.spd, i = s - sh * d.spd;
    slot_expert[s] = i < d.El ? sh * d.El + i : -1;
  }
  for (int sh = threadIdx.x; sh < d.S; sh += blockDim.x) load[sh] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < d.E; e += blockDim.x) {
    expert_counts[e] = counts[e];
    ndiv[e] = 0;
  }
  const int n = d.T * d.k;
  if (slot_of_assign != nullptr) {
#pragma unroll 4
    for (int a = threadIdx.x; a < n; a += blockDim.x) {
      int e = idx[a];
      slot_of_assign[a] = (e >= 0 && e < d.E) ? home_slot(d, e) : -1;
    }
  }
  if (!d.dedup) {
    for (int sh = threadIdx.x; sh < d.S; sh += blockDim.x) {
      int acc = 0;
      for (int i = 0; i < d.El; ++i) acc += counts[sh * d.El + i];
      load[sh] = acc;
    }
  } else {
    // one buffer row per distinct (token, shard) pair, from the top-k
    for (int t = threadIdx.x; t < d.T; t += blockDim.x) {
      const int* row = idx + (size_t)t * d.k;
      for (int j = 0; j < d.k; ++j) {
        int e = row[j];
        if (e < 0 || e >= d.E) continue;
        int sh = e / d.El;
        bool first = true;
        for (int jj = 0; jj < j; ++jj) {
          int e2 = row[jj];
          if (e2 >= 0 && e2 < d.E && e2 / d.El == sh) first = false;
        }
        if (first) atomicAdd(&load[sh], 1);
      }
    }
  }
  __syncthreads();
  int m = 0;
  for (int sh = threadIdx.x; sh < d.S; sh += blockDim.x) {
    shard_counts[sh] = load[sh];
    m = max(m, load[sh]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    int mx = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) mx = max(mx, red[w]);
    write_status(d, mx, bad, status, info, info_mode, c.rfactor);
  }
}


}  // namespace moe
