// a7: gate-weighted combine of one pass.
//
// y[t] = sum over j ascending of gate[t,j] * out[row(t,j)] over the
// assignments that have a row in this pass; a token with none gets 0.  This
// is the combine back to token order of "MoE ring-of-experts: TC Pallas
// ring all-gather for the combine backward + x_sorted remat save" (section
// What), on one device a gather: every output row is written once, by one
// wavefront, with a fixed summation order and no atomics.  Loads and stores
// are 16 bytes per lane; accumulation is fp32.
#include "common.h"

namespace moe {

namespace {

// Output columns [h + u*512, h + u*512 + 8) of one token, u < HU, in bf16:
// the row loads of a batch of KC assignments for all HU column groups are
// issued together, then accumulated in ascending j (the summation order of
// every column stays j = 0, 1, ..., k-1).
template <int KC, int HU>
__device__ __forceinline__ void combine_bf16_cols(const uint16_t* __restrict__ o, const int* rows,
                                                  const float* gts, int j0, int k, int H,
                                                  long long max_rows, int h,
                                                  float (&acc)[HU][8]) {
  uint4 v[KC][HU];
  float gj[KC];
  bool ok[KC];
#pragma unroll
  for (int u = 0; u < KC; ++u) {
    const int j = j0 + u;
    const int r = j < k ? rows[j] : -1;
    ok[u] = r >= 0 && r < max_rows;
    gj[u] = j < k ? gts[j] : 0.0f;
#pragma unroll
    for (int c = 0; c < HU; ++c)
      if (ok[u] && h + c * 512 < H) v[u][c] = *(const uint4*)(o + (size_t)r * H + h + c * 512);
  }
#pragma unroll
  for (int u = 0; u < KC; ++u) {
    if (!ok[u]) continue;
#pragma unroll
    for (int c = 0; c < HU; ++c) {
      if (h + c * 512 >= H) continue;
      const uint32_t w[4] = {v[u][c].x, v[u][c].y, v[u][c].z, v[u][c].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[c][2 * q] = fmaf(gj[u], __uint_as_float(w[q] << 16), acc[c][2 * q]);
        acc[c][2 * q + 1] = fmaf(gj[u], __uint_as_float(w[q] & 0xffff0000u), acc[c][2 * q + 1]);
      }
    }
  }
}

// One token's output row in bf16: column groups of 512 per pass over the
// assignments, KC assignments' loads in flight at a time.
template <int KC, int HU>
__device__ __forceinline__ void combine_bf16_token(const uint16_t* __restrict__ o, const int* rows,
                                                   const float* gts, int k, int H,
                                                   long long max_rows, uint16_t* yr, int lane) {
  for (int h = lane * 8; h < H; h += 512 * HU) {
    float acc[HU][8];
#pragma unroll
    for (int c = 0; c < HU; ++c)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[c][q] = 0.0f;
    // assignments in ascending j, KC at a time: KC x HU row loads in flight
    for (int j0 = 0; j0 < k; j0 += KC) combine_bf16_cols<KC, HU>(o, rows, gts, j0, k, H, max_rows, h, acc);
#pragma unroll
    for (int c = 0; c < HU; ++c) {
      if (h + c * 512 >= H) continue;
      uint4 outv;
      outv.x = (uint32_t)f2bf(acc[c][0]) | ((uint32_t)f2bf(acc[c][1]) << 16);
      outv.y = (uint32_t)f2bf(acc[c][2]) | ((uint32_t)f2bf(acc[c][3]) << 16);
      outv.z = (uint32_t)f2bf(acc[c][4]) | ((uint32_t)f2bf(acc[c][5]) << 16);
      outv.w = (uint32_t)f2bf(acc[c][6]) | ((uint32_t)f2bf(acc[c][7]) << 16);
      *(uint4*)(yr + h + c * 512) = outv;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(Dims d, PassArgs pa, LayoutSet ls,
                                                      const void* __restrict__ out,
                                                      const int* __restrict__ row_of_assign,
                                                      long long roa_stride, long long max_rows,
                                                      const float* __restrict__ gate, void* y) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  row_of_assign += (size_t)layout_set_of(ls, pi.j) * roa_stride;
  const int i = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (i >= pass_tokens(d, pi)) return;
  const int t = pass_token(d, pi, i);
  const int lane = lane_id();
  // the token's rows and gates are wave-uniform (scalar loads)
  const int* rows = row_of_assign + (size_t)t * d.k;
  const float* gts = gate + (size_t)t * d.k;
  if (BF16) {
    const uint16_t* o = (const uint16_t*)out;
    uint16_t* yr = (uint16_t*)y + (size_t)t * d.H;
    // rows of at most 1024 columns: all of a token's (up to 4) assignments
    // in flight at once; wider rows: 4 column groups, 2 assignments
    if (d.H <= 1024)
      combine_bf16_token<4, 2>(o, rows, gts, d.k, d.H, max_rows, yr, lane);
    else
      combine_bf16_token<2, 4>(o, rows, gts, d.k, d.H, max_rows, yr, lane);
  } else {
    const float* o = (const float*)out;
    float* yr = (float*)y + (size_t)t * d.H;
    for (int h = lane * 4; h < d.H; h += 256) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j = 0; j < d.k; ++j) {
        const int r = rows[j];
        const float gj = gts[j];
        if (r < 0 || r >= max_rows) continue;
        float4 v = *(const float4*)(o + (size_t)r * d.H + h);
        acc.x = fmaf(gj, v.x, acc.x);
        acc.y = fmaf(gj, v.y, acc.y);
        acc.z = fmaf(gj, v.z, acc.z);
        acc.w = fmaf(gj, v.w, acc.w);
      }
      *(float4*)(yr + h) = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(const Dims& d, const PassArgs& pa, const LayoutSet& ls, const void* out,
                          const int* row_of_assign, long long roa_stride, int64_t max_rows,
                          const float* gate, void* y, hipStream_t s) {
  const int ntok = pa.ovf != nullptr ? d.T : (d.T / d.L) * pa.lw;
  dim3 grid((ntok + 3) / 4), block(256);
  if (d.bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, s, d, pa, ls, out, row_of_assign,
                       roa_stride, (long long)max_rows, gate, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, s, d, pa, ls, out, row_of_assign,
                       roa_stride, (long long)max_rows, gate, y);
  return hipGetLastError();
}

}  // namespace moe
