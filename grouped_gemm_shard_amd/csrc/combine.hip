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
    // four assignments' row loads in flight; rows of at most 1024 columns
    // take them in 2 column groups of 512, wider rows in 4
    if (d.H <= 1024)
      combine_bf16_token<4, 2>(o, rows, gts, d.k, d.H, max_rows, yr, lane);
    else
      combine_bf16_token<4, 4>(o, rows, gts, d.k, d.H, max_rows, yr, lane);
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

// Return-path dedup.  The rows a wave adds are given per lane (lane j: row
// index or -1, and its weight), for j < k; they are added in ascending j,
// four at a time, with fp32 accumulation, into the wave's output row dst of
// H columns.  Rows are bf16 or fp32 (IN_BF16), the output likewise
// (OUT_BF16); each lane handles 8 consecutive columns per 512.
template <bool IN_BF16>
__device__ __forceinline__ void load8(const void* src, size_t off, float (&v)[8]) {
  if (IN_BF16) {
    const uint4 q = *(const uint4*)((const uint16_t*)src + off);
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(wd[i] << 16);
      v[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *(const float4*)((const float*)src + off);
    const float4 b = *(const float4*)((const float*)src + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* dst, size_t off, const float (&v)[8]) {
  if (OUT_BF16) {
    uint4 q;
    q.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    q.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    q.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    q.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
    *(uint4*)((uint16_t*)dst + off) = q;
  } else {
    *(float4*)((float*)dst + off) = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)((float*)dst + off + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <bool IN_BF16, bool OUT_BF16>
__device__ __forceinline__ void add_lane_rows(const void* __restrict__ src, int r_lane,
                                              float w_lane, int k, int H, void* dst, int lane) {
  constexpr int HU = 2;  // column groups of 512 per pass over the rows
  for (int h = lane * 8; h < H; h += 512 * HU) {
    float acc[HU][8];
#pragma unroll
    for (int c = 0; c < HU; ++c)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[c][q] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 4) {
      float v[4][HU][8];
      int rr[4];
      float ww[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        rr[u] = j < k ? __builtin_amdgcn_readlane(r_lane, j) : -1;
        ww[u] = j < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), j)) : 0.0f;
#pragma unroll
        for (int c = 0; c < HU; ++c)
          if (rr[u] >= 0 && h + c * 512 < H) load8<IN_BF16>(src, (size_t)rr[u] * H + h + c * 512, v[u][c]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (rr[u] < 0) continue;
#pragma unroll
        for (int c = 0; c < HU; ++c) {
          if (h + c * 512 >= H) continue;
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[c][q] = fmaf(ww[u], v[u][c][q], acc[c][q]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < HU; ++c)
      if (h + c * 512 < H) store8<OUT_BF16>(dst, h + c * 512, acc[c]);
  }
}

// Receiving side: one wavefront per dedup row u < *u_count (token t on one
// resident shard).  Lane j keeps assignment j of t when it has a row whose
// dedup row is u (expand_idx[row] == u: its slot is on u's shard); the
// kept rows are added with their gates in ascending j into an fp32 row.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_partial_kernel(
    Dims d, const int* __restrict__ u_count, const int* __restrict__ dedup_token,
    const int* __restrict__ row_of_assign, const int* __restrict__ expand_idx,
    const float* __restrict__ gate, const void* __restrict__ out, long long max_rows,
    long long max_urows, void* partial) {
  const int u = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (u >= *u_count || u >= max_urows) return;
  const int t = dedup_token[u];
  if (t < 0 || t >= d.T) return;
  const int lane = lane_id();
  int r = -1;
  float gj = 0.0f;
  if (lane < d.k) {
    const int rr = row_of_assign[(size_t)t * d.k + lane];
    if (rr >= 0 && rr < max_rows && expand_idx[rr] == u) {
      r = rr;
      gj = gate[(size_t)t * d.k + lane];
    }
  }
  add_lane_rows<BF16, false>(out, r, gj, d.k, d.H, (float*)partial + (size_t)u * d.H, lane);
}

// Source side: one wavefront per token of the pass.  Lane j finds the dedup
// row of assignment j (through its row and expand_idx) and keeps it when no
// lower lane has the same one; the kept fp32 partial rows are added in
// ascending j (each shard's row once, at the token's first assignment
// there) and the sum is stored in the activation dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_from_partials_kernel(
    Dims d, PassArgs pa, const int* __restrict__ row_of_assign,
    const int* __restrict__ expand_idx, const void* __restrict__ partial, long long max_rows,
    long long max_urows, void* y) {
  PassInfo pi = resolve_pass(pa);
  if (!pi.active) return;
  const int i = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (i >= pass_tokens(d, pi)) return;
  const int t = pass_token(d, pi, i);
  const int lane = lane_id();
  int u = -1;
  if (lane < d.k) {
    const int rr = row_of_assign[(size_t)t * d.k + lane];
    if (rr >= 0 && rr < max_rows) {
      const int uu = expand_idx[rr];
      if (uu >= 0 && uu < max_urows) u = uu;
    }
  }
  bool dup = false;
  for (int jj = 0; jj < d.k; ++jj) {
    const int uo = __builtin_amdgcn_readlane(u, jj);
    if (jj < lane && u >= 0 && uo == u) dup = true;
  }
  const size_t es = BF16 ? 2 : 4;
  add_lane_rows<false, BF16>(partial, dup ? -1 : u, 1.0f, d.k, d.H,
                             (char*)y + (size_t)t * d.H * es, lane);
}

}  // namespace

hipError_t launch_combine_partial(const Dims& d, const int* u_count, const int* dedup_token,
                                  const int* row_of_assign, const int* expand_idx,
                                  const float* gate, const void* out, int64_t max_rows,
                                  int64_t max_urows, void* partial, hipStream_t s) {
  if (max_urows <= 0) return hipSuccess;
  dim3 grid((unsigned)((max_urows + 3) / 4)), block(256);
  if (d.bf16)
    hipLaunchKernelGGL(combine_partial_kernel<true>, grid, block, 0, s, d, u_count, dedup_token,
                       row_of_assign, expand_idx, gate, out, (long long)max_rows,
                       (long long)max_urows, partial);
  else
    hipLaunchKernelGGL(combine_partial_kernel<false>, grid, block, 0, s, d, u_count, dedup_token,
                       row_of_assign, expand_idx, gate, out, (long long)max_rows,
                       (long long)max_urows, partial);
  return hipGetLastError();
}

hipError_t launch_combine_from_partials(const Dims& d, const PassArgs& pa,
                                        const int* row_of_assign, const int* expand_idx,
                                        const void* partial, int64_t max_rows, int64_t max_urows,
                                        void* y, hipStream_t s) {
  const int ntok = pa.ovf != nullptr ? d.T : (d.T / d.L) * pa.lw;
  if (ntok <= 0) return hipSuccess;
  dim3 grid((ntok + 3) / 4), block(256);
  if (d.bf16)
    hipLaunchKernelGGL(combine_from_partials_kernel<true>, grid, block, 0, s, d, pa,
                       row_of_assign, expand_idx, partial, (long long)max_rows,
                       (long long)max_urows, y);
  else
    hipLaunchKernelGGL(combine_from_partials_kernel<false>, grid, block, 0, s, d, pa,
                       row_of_assign, expand_idx, partial, (long long)max_rows,
                       (long long)max_urows, y);
  return hipGetLastError();
}

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
