// a1: router top-k and gates.
//
// The overflow check of "Support moe_dropless_fallback=layer on the ragged
// all-to-all MoE path" (section How) works from the router's top-k.  One
// wavefront owns one token at a time: each lane holds E/64 logits in
// registers, and k rounds of a wave-wide arg-max (butterfly over 64 lanes)
// pick the experts in descending logit order, equal logits going to the
// lowest index.  The key (value desc, index asc) is a total order over
// distinct indices, so every lane ends each round with the same winner.
//
// With `ph` set, each block also counts the experts it picked in an LDS
// histogram and writes it to row blockIdx of ph [gridDim][E], so the count
// step needs no separate pass over the top-k.  Blocks hold 16 waves; a wave
// takes tokens t, t + 16*gridDim, ..., loading the next token's logits
// while it ranks the current one.
#include "common.h"

namespace moe {

template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ logits, int t, int E,
                                            int lane, float (&v)[VPL]) {
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = i * 64 + lane;
    v[i] = e < E ? row[e] : 0.0f;
  }
}

template <int VPL>
__device__ __forceinline__ void route_token(const float (&v)[VPL], int t, int E, int k, int gate,
                                            int lane, int* __restrict__ idx,
                                            float* __restrict__ gate_out, int* hist) {
  unsigned taken = 0;
  float my_v = 0.0f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = 0.0f;
    int bi = 0x7fffffff;  // no candidate in this lane
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = i * 64 + lane;
      bool ok = e < E && !((taken >> i) & 1u);
      // lanes scan their logits in ascending index: strict > keeps the
      // lowest index among equal values
      if (ok && (bi == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      bool take;
      if (oi == 0x7fffffff) take = false;
      else if (bi == 0x7fffffff) take = true;
      else take = (ov > bv) || (ov == bv && oi < bi);
      if (take) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == r) {
      my_v = bv;
      my_i = bi;
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  float g;
  if (gate == MOE_GATE_SOFTMAX) {
    float l0 = __shfl(my_v, 0);
    float z = lane < k ? __expf(my_v - l0) : 0.0f;
    float sum = z;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    g = z / sum;
  } else {
    g = 1.0f / (1.0f + __expf(-my_v));
  }
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_i;
    gate_out[(size_t)t * k + lane] = g;
    if (hist != nullptr) atomicAdd(&hist[my_i], 1);
  }
}

template <int VPL>
__global__ __launch_bounds__(1024) void route_kernel(const float* __restrict__ logits, int T,
                                                     int E, int k, int gate,
                                                     int* __restrict__ idx,
                                                     float* __restrict__ gate_out,
                                                     int* __restrict__ ph, int* zero,
                                                     int zero_n) {
  __shared__ int hist[kMaxExperts];
  // counters a later launch of the call expects at zero
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero[i] = 0;
  if (ph != nullptr) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
  }
  const int lane = lane_id();
  const int wpb = blockDim.x >> 6;
  const int stride = gridDim.x * wpb;
  int t = blockIdx.x * wpb + (threadIdx.x >> 6);
  float v[VPL], vn[VPL];
  if (t < T) load_logits<VPL>(logits, t, E, lane, v);
  for (; t < T; t += stride) {
    // the next token's logits load while this one is ranked
    if (t + stride < T) load_logits<VPL>(logits, t + stride, E, lane, vn);
    route_token<VPL>(v, t, E, k, gate, lane, idx, gate_out, ph != nullptr ? hist : nullptr);
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] = vn[i];
  }
  if (ph != nullptr) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) ph[(size_t)blockIdx.x * E + e] = hist[e];
  }
}


hipError_t launch_route(const Dims& d, const float* logits, int* idx, float* gate, int* ph,
                        hipStream_t s, int* zero, int zero_n) {
  // with partial histograms: a fixed grid (rows of ph), tokens strided over it
  const int nb = ph != nullptr ? route_hist_blocks(d) : (d.T + 15) / 16;
  dim3 grid(nb), block(1024);
  int vpl = (d.E + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, logits, d.T, d.E, d.k, d.gate, idx, gate, ph, zero, zero_n);
  else if (vpl <= 2)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, logits, d.T, d.E, d.k, d.gate, idx, gate, ph, zero, zero_n);
  else if (vpl <= 4)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, logits, d.T, d.E, d.k, d.gate, idx, gate, ph, zero, zero_n);
  else if (vpl <= 8)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, logits, d.T, d.E, d.k, d.gate, idx, gate, ph, zero, zero_n);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, s, logits, d.T, d.E, d.k, d.gate, idx, gate, ph, zero, zero_n);
  return hipGetLastError();
}

}  // namespace moe
